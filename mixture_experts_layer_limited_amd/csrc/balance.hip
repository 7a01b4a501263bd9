// Expert-load statistics of one routed batch and the auxiliary-loss-free bias
// step (DeepSeek V3/R1 overview, xxqk.cn/news/389306, §2.2: an expert that
// received more than its share of tokens has its routing bias lowered by a
// fixed step, one that received less has it raised; V3 lab page,
// gsyq.cn/news/313569, §4: per-expert counts, min / max and the coefficient of
// variation std/mean as the balance measure).
//
// One work-group of 1024 threads, thread e owning expert e (E <= 1024).
#include <limits.h>

#include "common.h"
#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(1024) void load_balance_kernel(const int32_t* __restrict__ offsets, int E,
                                                            float* __restrict__ bias, float gamma,
                                                            moe_load_stats* __restrict__ stats) {
  __shared__ int s_min[1024], s_max[1024], s_empty[1024];
  __shared__ double s_sq[1024];
  const int e = threadIdx.x;
  const bool live = e < E;
  const int rows = offsets[E] - offsets[0];
  const int c = live ? offsets[e + 1] - offsets[e] : 0;
  // the target share and the sign rule in fp32
  const float share = (float)rows / (float)E;
  if (bias && live) {
    const float d = share - (float)c;
    const float step = d > 0.0f ? gamma : (d < 0.0f ? -gamma : 0.0f);
    bias[e] = bias[e] + step;
  }
  if (!stats) return;
  const double mean = (double)rows / E;
  s_min[e] = live ? c : INT_MAX;
  s_max[e] = live ? c : INT_MIN;
  s_empty[e] = live && c == 0;
  s_sq[e] = live ? ((double)c - mean) * ((double)c - mean) : 0.0;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if (e < o) {
      s_min[e] = min(s_min[e], s_min[e + o]);
      s_max[e] = max(s_max[e], s_max[e + o]);
      s_empty[e] += s_empty[e + o];
      s_sq[e] += s_sq[e + o];
    }
    __syncthreads();
  }
  if (e == 0) {
    const double sd = E > 1 ? sqrt(s_sq[0] / (E - 1)) : 0.0;
    moe_load_stats st;
    st.rows = rows;
    st.min = s_min[0];
    st.max = s_max[0];
    st.empty = s_empty[0];
    st.mean = (float)mean;
    st.cv = mean > 0.0 ? (float)(sd / mean) : 0.0f;
    *stats = st;
  }
}

hipError_t launch_load_balance(const int32_t* offsets, int E, float* bias, float gamma, moe_load_stats* stats,
                               hipStream_t s) {
  hipLaunchKernelGGL(load_balance_kernel, dim3(1), dim3(1024), 0, s, offsets, E, bias, gamma, stats);
  return hipGetLastError();
}

}  // namespace moe
