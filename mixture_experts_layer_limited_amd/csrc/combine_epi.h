// The layer's un-permute + weighted combine (MoE inference walkthrough,
// zhiyuanblog.org/blog/moe-inference, §3.4-3.5) done by the epilogue of the
// shared expert's down GEMM, the last GEMM of the layer.  That launch is dense
// over the T tokens, so row t of its tile is token t; instead of storing the
// shared expert's row, the epilogue writes the layer output
//   out[t] = sum_j w[t,j] * y[inv[t*k + j]] + shared[t]
// with shared[t] rounded to bf16 first, the fp32 sum in that order and one
// final rounding: the same arithmetic, in the same order, as the stand-alone
// combine kernel, which then has nothing left to do.
#pragma once

#include "common.h"
#include "kernels.h"

namespace moe {

// The gather-combine of chunks q = tid, tid + NT, ... (see combine_staged_tile),
// G chunks at a time, up to G * 8 row gathers of 16 bytes in flight per thread:
// every chunk's routed-row indices and weights first (from LDS when STAGED,
// else from memory), then all its row gathers, then the sums.  Lanes without
// an entry gather a valid row (0) and keep their sum by select, so the loads
// are issued unconditionally and stay in flight together.
template <bool STAGED, int BM, int CPR, int RB, int NT, int G>
__device__ __forceinline__ void combine_chunks(const CombineEpi& cb, const char* lds, const int* pos_l,
                                               const float* w_l, int64_t base, int r0, int rows, int c0, int N,
                                               int tid) {
  const uint16_t* y = (const uint16_t*)cb.rows;
  uint16_t* o = (uint16_t*)cb.out;
  const int k = cb.k;
  for (int q0 = tid; q0 < BM * CPR; q0 += G * NT) {
    int row[G], col[G];
    bool live[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int q = q0 + g * NT;
      row[g] = q / CPR;
      col[g] = c0 + (q % CPR) * 8;
      live[g] = q < BM * CPR && row[g] < rows && col[g] < N;
    }
    float v[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < 8; ++i) v[g][i] = 0.0f;
    for (int j0 = 0; j0 < k; j0 += 8) {
      int pos[G][8];
      float w[G][8];
      bool ok[G][8];
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          ok[g][u] = live[g] && j0 + u < k;
          const int e = ok[g][u] ? row[g] * k + j0 + u : 0;
          const int pe = STAGED ? pos_l[e] : cb.inv[base + e];
          const float we = STAGED ? w_l[e] : cb.w[base + e];
          pos[g][u] = ok[g][u] ? pe : 0;
          w[g][u] = we;
        }
      u32x4 r[G][8];
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int u = 0; u < 8; ++u)
          r[g][u] = *(const u32x4*)(y + (int64_t)pos[g][u] * N + (live[g] ? col[g] : c0));
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const float a = fmaf(w[g][u], __uint_as_float(r[g][u][h] << 16), v[g][2 * h]);
            const float b = fmaf(w[g][u], __uint_as_float(r[g][u][h] & 0xffff0000u), v[g][2 * h + 1]);
            v[g][2 * h] = ok[g][u] ? a : v[g][2 * h];
            v[g][2 * h + 1] = ok[g][u] ? b : v[g][2 * h + 1];
          }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (!live[g]) continue;
      const u32x4 s = *(const u32x4*)(lds + row[g] * RB + (col[g] - c0) * 2);
      u32x4 res;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        v[g][2 * h] += __uint_as_float(s[h] << 16);
        v[g][2 * h + 1] += __uint_as_float(s[h] & 0xffff0000u);
        res[h] = f32_to_bf16_bits(v[g][2 * h]) | (f32_to_bf16_bits(v[g][2 * h + 1]) << 16);
      }
      *(u32x4*)(o + (r0 + row[g]) * (int64_t)N + col[g]) = res;
    }
  }
}

// Second half of a staged bf16 row-store epilogue: the tile's bf16 rows sit in
// LDS (RB bytes per row, BM rows from token r0, columns c0 ..); `spare` bytes of
// LDS after them are free.  Each 8-column chunk of token t's row becomes
// out[t] = sum_j w[t,j] * y[inv[t*k+j]] + tile[t].  The rows' inv_perm entries
// and weights are staged in the spare LDS first when they fit (k <= 14 for
// 256-row tiles), else read from memory.  Every thread of the work-group calls
// it; G is as many chunks per thread as the kernel's free registers allow.
template <int BM, int CPR, int RB, int NT, int G>
__device__ __forceinline__ void combine_staged_tile(const CombineEpi& cb, char* lds, int spare, int r0, int rows,
                                                    int c0, int N, int tid) {
  const int k = cb.k;
  const int64_t base = (int64_t)r0 * k;  // first (token, j) entry of the tile
  int* pos_l = (int*)(lds + BM * RB);
  float* w_l = (float*)(pos_l + BM * k);
  if (BM * k * 8 <= spare) {  // uniform over the work-group
    for (int i = tid; i < rows * k; i += NT) {
      pos_l[i] = cb.inv[base + i];
      w_l[i] = cb.w[base + i];
    }
    __syncthreads();
    combine_chunks<true, BM, CPR, RB, NT, G>(cb, lds, pos_l, w_l, base, r0, rows, c0, N, tid);
  } else {
    combine_chunks<false, BM, CPR, RB, NT, G>(cb, lds, pos_l, w_l, base, r0, rows, c0, N, tid);
  }
}

}  // namespace moe
