// Un-permute + weighted combine (MoE inference walkthrough,
// zhiyuanblog.org/blog/moe-inference, §3.4), small helper kernels, and the
// dynamic 1x128 E4M3 activation quantiser (MoA routing + FP8 inference,
// blog.hotdry.top, FP8 section).
#include "common.h"
#include "kernels.h"

namespace moe {

// out[t] = acc[t] + sum_j w[t,j] * rows[inv[t*k+j]] + shared[t], fp32 sum,
// one rounding.  One block per token, 8 columns per thread per step.
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
  if (expert_out && threadIdx.x < k) {
    pos[threadIdx.x] = inv[(int64_t)t * k + threadIdx.x];
    wt[threadIdx.x] = topk_w[(int64_t)t * k + threadIdx.x];
  }
  __syncthreads();
  const T* rows = (const T*)expert_out;
  const T* sh = (const T*)shared_out;
  T* o = (T*)out;
  for (int c = threadIdx.x * 8; c < H; c += blockDim.x * 8) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    if (acc) {
      const float4 a0 = *(const float4*)(acc + (int64_t)t * H + c);
      const float4 a1 = *(const float4*)(acc + (int64_t)t * H + c + 4);
      v[0] = a0.x; v[1] = a0.y; v[2] = a0.z; v[3] = a0.w;
      v[4] = a1.x; v[5] = a1.y; v[6] = a1.z; v[7] = a1.w;
    }
    if (rows) {
      for (int j = 0; j < k; ++j) {
        const float w = wt[j];
        const int64_t base = (int64_t)pos[j] * H + c;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] += w * Elem<ADT>::load(rows, base + i);
      }
    }
    if (sh) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] += Elem<ADT>::load(sh, (int64_t)t * H + c + i);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) Elem<ADT>::store(o, (int64_t)t * H + c + i, v[i]);
  }
}

hipError_t launch_combine(int adt, int T, int H, int k, const void* expert_out, const float* acc,
                          const int32_t* inv, const float* topk_w, const void* shared_out, void* out,
                          hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (adt == MOE_DT_BF16)
    hipLaunchKernelGGL(combine_kernel<MOE_DT_BF16>, dim3(T), dim3(256), 0, s, H, k, expert_out, acc, inv,
                       topk_w, shared_out, out);
  else
    hipLaunchKernelGGL(combine_kernel<MOE_DT_F32>, dim3(T), dim3(256), 0, s, H, k, expert_out, acc, inv,
                       topk_w, shared_out, out);
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

// One wavefront per (row, 128-column tile), two values per lane:
// scale = fp32(amax / 448) (1 if amax == 0), code = E4M3(fp32(v / scale)).
template <int IDT>
__global__ __launch_bounds__(256) void quantize_kernel(int64_t rows, int64_t cols, const void* __restrict__ in,
                                                       uint8_t* __restrict__ codes, float* __restrict__ scales) {
  using T = typename Elem<IDT>::T;
  const int lane = threadIdx.x & 63;
  const int64_t tiles_per_row = cols / 128;
  const int64_t tile = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tile >= rows * tiles_per_row) return;
  const int64_t r = tile / tiles_per_row, c0 = (tile % tiles_per_row) * 128;
  const int64_t base = r * cols + c0 + 2 * lane;
  const float v0 = Elem<IDT>::load((const T*)in, base);
  const float v1 = Elem<IDT>::load((const T*)in, base + 1);
  const float amax = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
  const float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
  const uint32_t q0 = f32_to_e4m3(v0 / scale);
  const uint32_t q1 = f32_to_e4m3(v1 / scale);
  *(uint16_t*)(codes + base) = (uint16_t)(q0 | (q1 << 8));
  if (lane == 0) scales[r * tiles_per_row + c0 / 128] = scale;
}

hipError_t launch_quantize(int in_dt, int64_t rows, int64_t cols, const void* in, uint8_t* codes, float* scales,
                           hipStream_t s) {
  const int64_t tiles = rows * (cols / 128);
  if (tiles <= 0) return hipSuccess;
  const int64_t grid = (tiles + 3) / 4;
  if (in_dt == MOE_DT_BF16)
    hipLaunchKernelGGL(quantize_kernel<MOE_DT_BF16>, dim3((unsigned)grid), dim3(256), 0, s, rows, cols, in, codes,
                       scales);
  else
    hipLaunchKernelGGL(quantize_kernel<MOE_DT_F32>, dim3((unsigned)grid), dim3(256), 0, s, rows, cols, in, codes,
                       scales);
  return hipGetLastError();
}

}  // namespace moe
