// Un-permute + weighted combine (MoE inference walkthrough,
// zhiyuanblog.org/blog/moe-inference, §3.4), small helper kernels, and the
// dynamic 1x128 E4M3 activation quantiser (MoA routing + FP8 inference,
// blog.hotdry.top, FP8 section).
#include "common.h"
#include "kernels.h"

namespace moe {

// out[t] = acc[t] + sum_j w[t,j] * rows[inv[t*k+j]] + shared[t], fp32 sum in
// that order, one rounding.  Block (t, s) covers columns [2048 s, 2048 s + 2048)
// of token t (so a small batch still spreads over the chip), 8 consecutive
// columns per thread, moved with 16-byte loads and stores (H % 8 == 0; row
// starts are 16-byte aligned for every H the ABI accepts).
template <int ADT>
__device__ __forceinline__ void load8(const typename Elem<ADT>::T* p, float v[8]) {
  if constexpr (ADT == MOE_DT_BF16) {
    const u32x4 w = *(const u32x4*)p;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = __uint_as_float(w[q] << 16);
      v[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
    }
  } else {
    const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <int ADT>
__device__ __forceinline__ void store8(typename Elem<ADT>::T* p, const float v[8]) {
  if constexpr (ADT == MOE_DT_BF16) {
    u32x4 w;
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = f32_to_bf16_bits(v[2 * q]) | (f32_to_bf16_bits(v[2 * q + 1]) << 16);
    *(u32x4*)p = w;
  } else {
    *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
    *(float4*)(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
}

template <int ADT>
__global__ __launch_bounds__(256) void combine_kernel(int H, int k, const void* __restrict__ expert_out,
                                                      const float* __restrict__ acc,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ topk_w,
                                                      const void* __restrict__ shared_out, void* __restrict__ out) {
  using T = typename Elem<ADT>::T;
  __shared__ int pos[32];
  __shared__ float wt[32];
  const int t = blockIdx.x;
  const int c_end = min(H, (int)(blockIdx.y + 1) * 2048);
  if (expert_out && threadIdx.x < k) {
    pos[threadIdx.x] = inv[(int64_t)t * k + threadIdx.x];
    wt[threadIdx.x] = topk_w[(int64_t)t * k + threadIdx.x];
  }
  __syncthreads();
  const T* rows = (const T*)expert_out;
  const T* sh = (const T*)shared_out;
  T* o = (T*)out;
  for (int c = blockIdx.y * 2048 + threadIdx.x * 8; c < c_end; c += blockDim.x * 8) {
    float v[8];
    if (acc) {
      const float4 a0 = *(const float4*)(acc + (int64_t)t * H + c);
      const float4 a1 = *(const float4*)(acc + (int64_t)t * H + c + 4);
      v[0] = a0.x; v[1] = a0.y; v[2] = a0.z; v[3] = a0.w;
      v[4] = a1.x; v[5] = a1.y; v[6] = a1.z; v[7] = a1.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
    if (rows) {
      for (int j = 0; j < k; ++j) {
        float r[8];
        load8<ADT>(rows + (int64_t)pos[j] * H + c, r);
        const float w = wt[j];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] += w * r[i];
      }
    }
    if (sh) {
      float r[8];
      load8<ADT>(sh + (int64_t)t * H + c, r);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] += r[i];
    }
    store8<ADT>(o + (int64_t)t * H + c, v);
  }
}

hipError_t launch_combine(int adt, int T, int H, int k, const void* expert_out, const float* acc,
                          const int32_t* inv, const float* topk_w, const void* shared_out, void* out,
                          hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const dim3 grid(T, (H + 2047) / 2048);
  if (adt == MOE_DT_BF16)
    hipLaunchKernelGGL(combine_kernel<MOE_DT_BF16>, grid, dim3(256), 0, s, H, k, expert_out, acc, inv, topk_w,
                       shared_out, out);
  else
    hipLaunchKernelGGL(combine_kernel<MOE_DT_F32>, grid, dim3(256), 0, s, H, k, expert_out, acc, inv, topk_w,
                       shared_out, out);
  return hipGetLastError();
}

// row_w[inv[a]] = topk_w[a]: the routing weight of every permuted row.
__global__ void row_weights_kernel(const float* __restrict__ topk_w, const int32_t* __restrict__ inv, int n,
                                   float* __restrict__ row_w) {
  const int a = blockIdx.x * blockDim.x + threadIdx.x;
  if (a < n) row_w[inv[a]] = topk_w[a];
}

hipError_t launch_row_weights(const float* topk_w, const int32_t* inv, int n, float* row_w, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(row_weights_kernel, dim3((n + 255) / 256), dim3(256), 0, s, topk_w, inv, n, row_w);
  return hipGetLastError();
}

// Zero fill with a kernel (not a memset node, so the sequence can be captured in a graph).
__global__ void fill_zero_kernel(float4* __restrict__ p, int64_t n4) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t n4 = n / 4;  // callers pass multiples of 4
  const int64_t want = (n4 + 255) / 256;
  const int64_t blocks = want < 4096 ? want : 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (float4*)p, n4);
  return hipGetLastError();
}

// Activation quantisation, one 1x128 tile per 8 lanes:
// scale = fp32(amax / 448) (1 if amax == 0), code = E4M3(fp32(v / scale)).
template <int IDT>
__global__ __launch_bounds__(256) void quantize_kernel(int64_t rows, int64_t cols, const void* __restrict__ in,
                                                       uint8_t* __restrict__ codes, float* __restrict__ scales) {
  // 8 lanes per 1x128 tile, 16 consecutive values per lane: two 16-byte (bf16)
  // or four (fp32) loads, issued together, and two 8-byte stores of codes per lane.
  using T = typename Elem<IDT>::T;
  const int lane = threadIdx.x & 63, sub = lane & 7;
  const int64_t tiles_per_row = cols / 128;
  const int64_t tile = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
  if (tile >= rows * tiles_per_row) return;
  const int64_t r = tile / tiles_per_row;
  const int64_t c0 = (tile % tiles_per_row) * 128;
  const int64_t base = r * cols + c0 + 16 * sub;
  float v[16];
  if constexpr (IDT == MOE_DT_BF16) {
    const u32x4 w0 = *(const u32x4*)((const T*)in + base);
    const u32x4 w1 = *(const u32x4*)((const T*)in + base + 8);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = __uint_as_float(w0[q] << 16);
      v[2 * q + 1] = __uint_as_float(w0[q] & 0xffff0000u);
      v[8 + 2 * q] = __uint_as_float(w1[q] << 16);
      v[8 + 2 * q + 1] = __uint_as_float(w1[q] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 w = *(const float4*)((const float*)in + base + 4 * q);
      v[4 * q] = w.x; v[4 * q + 1] = w.y; v[4 * q + 2] = w.z; v[4 * q + 3] = w.w;
    }
  }
  float m = 0.0f;
#pragma unroll
  for (int q = 0; q < 16; ++q) m = fmaxf(m, fabsf(v[q]));
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  const float scale = m > 0.0f ? m / 448.0f : 1.0f;
  // two 8-byte stores: the codes buffer is only required to be 8-byte aligned
  *(uint2*)(codes + base) = make_uint2(e4m3x4(v[0] / scale, v[1] / scale, v[2] / scale, v[3] / scale),
                                       e4m3x4(v[4] / scale, v[5] / scale, v[6] / scale, v[7] / scale));
  *(uint2*)(codes + base + 8) = make_uint2(e4m3x4(v[8] / scale, v[9] / scale, v[10] / scale, v[11] / scale),
                                           e4m3x4(v[12] / scale, v[13] / scale, v[14] / scale, v[15] / scale));
  if (sub == 0) scales[r * tiles_per_row + c0 / 128] = scale;
}

// scales_t[kb * rows + p] = scales[src(p) * nkb + kb]: the activation scales of the
// permuted rows, k-block-major, so a GEMM step reads the scales of a row tile as
// one contiguous run.  src(p) outside [0, src_rows) (rows the expert offsets do
// not cover, or a caller's out-of-range index) reads nothing and gets scale 1.
__global__ __launch_bounds__(256) void gather_scales_t_kernel(const float* __restrict__ scales,
                                                              const int32_t* __restrict__ src, int64_t rows, int nkb,
                                                              int64_t src_rows, float* __restrict__ scales_t) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= rows) return;
  const int64_t sp = src ? (int64_t)src[p] : p;
  if (sp < 0 || sp >= src_rows) {
    for (int kb = 0; kb < nkb; ++kb) scales_t[(int64_t)kb * rows + p] = 1.0f;
    return;
  }
  const float* in = scales + sp * nkb;
  // 16 loads in flight before their stores (each load would otherwise wait
  // for the stores before it: the vector memory counter retires in order)
  int kb = 0;
  for (; kb + 16 <= nkb; kb += 16) {
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = in[kb + u];
#pragma unroll
    for (int u = 0; u < 16; ++u) scales_t[(int64_t)(kb + u) * rows + p] = v[u];
  }
  for (; kb < nkb; ++kb) scales_t[(int64_t)kb * rows + p] = in[kb];
}

hipError_t launch_gather_scales_t(const float* scales, const int32_t* src, int64_t rows, int nkb, int64_t src_rows,
                                  float* scales_t, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_scales_t_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, scales, src,
                     rows, nkb, src_rows, scales_t);
  return hipGetLastError();
}

hipError_t launch_quantize(int in_dt, int64_t rows, int64_t cols, const void* in, uint8_t* codes, float* scales,
                           hipStream_t s) {
  const int64_t tiles = rows * (cols / 128);
  if (tiles <= 0) return hipSuccess;
  const int64_t grid = (tiles + 31) / 32;
  if (in_dt == MOE_DT_BF16)
    hipLaunchKernelGGL(quantize_kernel<MOE_DT_BF16>, dim3((unsigned)grid), dim3(256), 0, s, rows, cols, in, codes,
                       scales);
  else
    hipLaunchKernelGGL(quantize_kernel<MOE_DT_F32>, dim3((unsigned)grid), dim3(256), 0, s, rows, cols, in, codes,
                       scales);
  return hipGetLastError();
}

}  // namespace moe
