// Scoring and group-limited top-k, one wavefront per token.
//
// Lane l holds experts l*V .. l*V+V-1 (V = ceil(E/64)), so a group of
// contiguous experts spans contiguous lanes and "lowest lane" is "lowest
// expert id".  Every arg-max is a wave-wide max over order-preserving uint32
// keys followed by a ballot that picks the lowest lane holding the max, so
// ties go to the lower expert (or group) id.  Group scores (sum of the two
// largest biased scores of a group) are computed by lane g scanning group g
// from LDS.  (V3 lab page, gsyq.cn/news/313569, §4 route(); MoE inference
// walkthrough, zhiyuanblog.org/blog/moe-inference, §3.1; DeepSeek V3/R1
// overview, xxqk.cn/news/389306, §2.2.)
#include "common.h"
#include "kernels.h"

namespace moe {

// W tokens (waves) per work-group: 1 for small batches, so that the loads
// of a split-K router's partial logits spread over as many CUs as there are
// tokens; 4 for large ones.
// NP: partial-logit slices whose loads are in flight at once (registers:
// NP x V); a launch over few slices takes a small NP, so more waves fit a SIMD.
template <int V, int W, int NP>
__global__ __launch_bounds__(W * 64) void route_kernel(RouteParams p) {
  __shared__ float cs[W][V * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * W + wave;
  const bool active = t < p.T;
  const int E = p.E;

  float s[V], c[V];
  bool valid[V];
  const float* row = p.logits + (int64_t)(active ? t : 0) * E;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int e = lane * V + i;
    valid[i] = active && e < E;
    s[i] = valid[i] ? row[e] : 0.0f;
  }
  // logits of a split-K router GEMM: partial sums of K slices, added in slice
  // order; the loads of up to NP slices are in flight at once, so a decode
  // batch's 50-odd slices take two round trips
  for (int q0 = 1; q0 < p.n_parts; q0 += NP) {
    float part[NP][V];
#pragma unroll
    for (int u = 0; u < NP; ++u)
#pragma unroll
      for (int i = 0; i < V; ++i)
        part[u][i] = (valid[i] && q0 + u < p.n_parts) ? row[(int64_t)(q0 + u) * p.part_stride + lane * V + i] : 0.0f;
#pragma unroll
    for (int u = 0; u < NP; ++u)
#pragma unroll
      for (int i = 0; i < V; ++i)
        if (q0 + u < p.n_parts) s[i] += part[u][i];
  }

  if (!p.scores_given) {
    if (p.scoring == 0) {  // softmax over all E experts
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < V; ++i)
        if (valid[i]) m = fmaxf(m, s[i]);
      m = wave_max(m);
      float sum = 0.0f;
#pragma unroll
      for (int i = 0; i < V; ++i) {
        s[i] = valid[i] ? expf(s[i] - m) : 0.0f;
        sum += s[i];
      }
      sum = wave_sum(sum);
#pragma unroll
      for (int i = 0; i < V; ++i) s[i] = s[i] / sum;
    } else {  // sigmoid
#pragma unroll
      for (int i = 0; i < V; ++i) s[i] = 1.0f / (1.0f + expf(-s[i]));
    }
    if (p.scores_out && active) {
#pragma unroll
      for (int i = 0; i < V; ++i)
        if (valid[i]) p.scores_out[(int64_t)t * E + lane * V + i] = s[i];
    }
  }

  // Selection score c = s + b; adding +0 turns -0 into +0 so the keys compare like floats.
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int e = lane * V + i;
    float v = s[i];
    if (p.bias && valid[i]) v = v + p.bias[e];
    c[i] = v + 0.0f;
  }

  if (p.n_group > 1) {
    const int G = E / p.n_group;
#pragma unroll
    for (int i = 0; i < V; ++i)
      if (lane * V + i < E) cs[wave][lane * V + i] = c[i];
    __syncthreads();
    float gs = 0.0f;
    if (lane < p.n_group) {
      float m1 = -INFINITY, m2 = -INFINITY;
      for (int x = 0; x < G; ++x) {
        const float v = cs[wave][lane * G + x];
        if (v > m1) { m2 = m1; m1 = v; }
        else if (v > m2) { m2 = v; }
      }
      gs = (m1 + m2) + 0.0f;
    }
    uint64_t kept = 0;
    bool taken = false;
    for (int r = 0; r < p.topk_group; ++r) {
      const uint32_t key = (lane < p.n_group && !taken) ? f32_order_key(gs) : 0u;
      const uint32_t mk = wave_max_u32(key);
      const uint64_t who = __ballot(key == mk && lane < p.n_group && !taken);
      const int g = max(__ffsll((unsigned long long)who) - 1, 0);
      kept |= 1ull << g;
      if (lane == g) taken = true;
    }
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int g = (lane * V + i) / G;
      if (!((kept >> g) & 1ull)) c[i] = -INFINITY;
    }
  }

  // Top-k: k rounds of wave arg-max; lane j keeps the j-th winner.
  uint32_t taken_mask = 0;
  int my_id = 0;
  float my_s = 0.0f;
  float wsum = 0.0f;
  for (int j = 0; j < p.k; ++j) {
    uint32_t lkey = 0;
    int li = 0;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      if (valid[i] && !((taken_mask >> i) & 1u)) {
        const uint32_t kk = f32_order_key(c[i]);
        if (kk > lkey) { lkey = kk; li = i; }
      }
    }
    const uint32_t mk = wave_max_u32(lkey);
    const uint64_t who = __ballot(lkey == mk && lkey != 0u);
    const int wl = max(__ffsll((unsigned long long)who) - 1, 0);
    const int e_sel = __shfl(lane * V + li, wl, 64);
    float s_sel = 0.0f;
#pragma unroll
    for (int i = 0; i < V; ++i)
      if (i == li) s_sel = s[i];
    s_sel = __shfl(s_sel, wl, 64);
    if (lane == wl) taken_mask |= 1u << li;
    if (lane == j) { my_id = e_sel; my_s = s_sel; }
    wsum += s_sel;
  }
  if (active && lane < p.k) {
    float w = p.norm ? my_s / wsum : my_s;
    w = w * p.scale;
    p.topk_ids[(int64_t)t * p.k + lane] = my_id;
    p.topk_w[(int64_t)t * p.k + lane] = w;
  }
}

template <int V, int NP>
static hipError_t launch_vp(const RouteParams& p, hipStream_t s) {
  if (p.T <= 2048) {
    hipLaunchKernelGGL((route_kernel<V, 1, NP>), dim3(p.T), dim3(64), 0, s, p);
  } else {
    const int grid = (p.T + 3) / 4;
    hipLaunchKernelGGL((route_kernel<V, 4, NP>), dim3(grid), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

template <int V>
static hipError_t launch_v(const RouteParams& p, hipStream_t s) {
  // up to 4 slices (prefill-sized batches): 4 loads of V each in flight;
  // more (decode): about 112 registers of loads in flight
  if (p.n_parts <= 4) return launch_vp<V, 3>(p, s);
  return launch_vp<V, (112 / V < 32 ? (112 / V > 0 ? 112 / V : 1) : 32)>(p, s);
}

hipError_t launch_route(const RouteParams& p, hipStream_t s) {
  if (p.T <= 0) return hipSuccess;
  const int v = (p.E + 63) / 64;
  if (v <= 1) return launch_v<1>(p, s);
  if (v <= 2) return launch_v<2>(p, s);
  if (v <= 4) return launch_v<4>(p, s);
  if (v <= 8) return launch_v<8>(p, s);
  return launch_v<16>(p, s);
}

}  // namespace moe
