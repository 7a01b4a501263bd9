// Device-side helpers shared by the gfx950 kernels of libmoe355.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ------------------------------------------------------------------ bf16 ---

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Two floats to packed bf16 (lo in bits 0-15), round to nearest even, with
// gfx950's v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
typedef float f32x2_hw __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16_rne(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_hw){lo, hi}, bf16x2_hw));
}

// Value of the neighbouring lane l ^ 1 (DPP quad permutation [1, 0, 3, 2]).
__device__ __forceinline__ float swap_adjacent_lanes(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Element storage traits: F32 = float, BF16 = uint16_t bits.
template <int DT> struct Elem;
template <> struct Elem<0> {  // MOE_F32
  using T = float;
  static constexpr int kBytes = 4;
  __device__ static float load(const T* p, int64_t i) { return p[i]; }
  __device__ static void store(T* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<1> {  // MOE_BF16
  using T = uint16_t;
  static constexpr int kBytes = 2;
  __device__ static float load(const T* p, int64_t i) { return bf16_bits_to_f32(p[i]); }
  __device__ static void store(T* p, int64_t i, float v) { p[i] = (uint16_t)f32_to_bf16_bits(v); }
};

// ------------------------------------------------------- wave reductions ---

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    uint32_t w = (uint32_t)__shfl_xor((int)v, o, 64);
    v = w > v ? w : v;
  }
  return v;
}

// Order-preserving map of a non-NaN float to uint32 (a < b  <=>  key(a) < key(b)).
// -0.0 and +0.0 must be canonicalised by the caller (add 0.0f) to compare equal.
__device__ __forceinline__ uint32_t f32_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- E4M3FN ---

// Four fp32 values to OCP E4M3FN codes (value u in byte u) by the hardware
// conversion: round to nearest even, subnormals at exponent field 0, sign kept
// (tiny negatives give -0).  Callers pass quantised activations
// v / fp32(amax / 448) with |v| <= amax, so |x| <= 448 (1 + 2^-23).  On that
// range the conversion equals the E4M3 rounding rule code for code: every
// code, every midpoint and its neighbouring fp32 values, and the subnormal
// range agree, and 448 < |x| < 464 rounds to 448.  It does not saturate past
// that range (|x| >= 464 gives NaN), which quantised activations never reach.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// SwiGLU: SiLU(g) * u = g / (1 + e^-g) * u, the reciprocal by the hardware's
// v_rcp_f32 (1 ulp) instead of an IEEE division (a dozen instructions); the
// result is rounded to bf16 (or quantised) right after.  Large negative g gives
// e^-g = inf and a reciprocal of 0, the limit -0.
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t s = c & 0x80u, e = (c >> 3) & 0xfu, m = c & 7u;
  float v = (e == 0) ? (float)m * 0.001953125f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return s ? -v : v;
}

// ----------------------------------------------------- workgroup mapping ---

// Work-groups are handed to the 8 XCDs round-robin by id.  Remap a physical id
// P in [0, n) to a logical id so that runs of MOE_XCD_CHUNK consecutive logical
// ids land on one XCD (and share its L2), the runs going to the XCDs in turn;
// the last partial round keeps the hardware order.  MOE_XCD_CHUNK 0: one
// contiguous range per XCD.
#ifndef MOE_XCD_CHUNK
#define MOE_XCD_CHUNK 0
#endif
__device__ __forceinline__ int xcd_remap(int P, int n) {
  constexpr int kXcd = 8;
  if constexpr (MOE_XCD_CHUNK > 0) {
    constexpr int C = MOE_XCD_CHUNK;
    const int full = n / (kXcd * C) * (kXcd * C);
    if (P >= full) return P;
    const int x = P % kXcd, local = P / kXcd;
    return ((local / C) * kXcd + x) * C + local % C;
  } else {
    int q = n / kXcd, r = n % kXcd;
    int x = P % kXcd, local = P / kXcd;
    return x * q + (x < r ? x : r) + local;
  }
}

}  // namespace moe
