// Token permutation (MoE inference walkthrough, zhiyuanblog.org/blog/moe-inference,
// §3.2): a stable counting sort of the T*k copies by expert.
//
//   1. perm_hist:    per chunk of kChunk copies, an LDS histogram over experts
//   2. perm_scan:    one block turns the (chunk, expert) counts into each
//                    chunk's first slot per expert, and expert_offsets
//   3. perm_scatter: one wavefront per chunk walks its copies in order, 64 at a
//                    time; lanes with equal experts are found with ballots over
//                    the expert id bits, ranked by lane, and placed after the
//                    running count of their expert, so the order is stable and
//                    the result is the same on every run (no atomics decide
//                    a position).
#include "common.h"
#include "kernels.h"
#include "tiles.h"

namespace moe {

constexpr int kChunk = 1024;

int permute_blocks(int n) { return (n + kChunk - 1) / kChunk; }

__global__ __launch_bounds__(256) void perm_hist(const int32_t* __restrict__ ids, int n, int E,
                                                 int32_t* __restrict__ counts) {
  __shared__ int h[1024];
  for (int e = threadIdx.x; e < E; e += blockDim.x) h[e] = 0;
  __syncthreads();
  const int base = blockIdx.x * kChunk;
  for (int i = threadIdx.x; i < kChunk; i += blockDim.x) {
    const int a = base + i;
    if (a < n) {
      const int e = min(max(ids[a], 0), E - 1);
      atomicAdd(&h[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) counts[(int64_t)blockIdx.x * E + e] = h[e];
}

// One block of 1024 threads, thread e owns expert e (E <= 1024).  Rewrites
// counts[b][e] in place into the first permuted slot of chunk b for expert e.
// With t.bm > 0 it also writes the GEMMs' tile lists over the E groups (E + 1
// with the shared expert's ext_T rows as group E).
// When the nb x E counts fit kScanStash entries, all 1024 threads first copy
// them into LDS with coalesced loads, all issued before the first wait, and
// both passes over them read LDS: the stores of the second pass then never
// hold up a load (the vector memory counter retires in order).
constexpr int kScanStash = 32768;  // 128 KB

__global__ __launch_bounds__(1024) void perm_scan(int32_t* __restrict__ counts, int nb, int E,
                                                  int32_t* __restrict__ offsets, int ext_T, TileLists t) {
  __shared__ int scan[1024];
  __shared__ int first[1026];
  __shared__ int stash[kScanStash];
  const int e = threadIdx.x;
  const bool staged = (int64_t)nb * E <= kScanStash;
  const int nall = staged ? nb * E : 0;
  if (staged) {
    int i = e;
    for (; i + 7 * 1024 < nall; i += 8 * 1024) {
      int c[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) c[u] = counts[i + u * 1024];
#pragma unroll
      for (int u = 0; u < 8; ++u) stash[i + u * 1024] = c[u];
    }
    for (; i < nall; i += 1024) stash[i] = counts[i];
    __syncthreads();
  }
  int total = 0;
  if (e < E) {
    if (staged) {
      for (int b = 0; b < nb; ++b) total += stash[b * E + e];
    } else {  // 8 chunks' counts in flight at a time
      int b = 0;
      for (; b + 8 <= nb; b += 8) {
        int c[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) c[u] = counts[(int64_t)(b + u) * E + e];
#pragma unroll
        for (int u = 0; u < 8; ++u) total += c[u];
      }
      for (; b < nb; ++b) total += counts[(int64_t)b * E + e];
    }
  }
  scan[e] = total;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = e >= o ? scan[e - o] : 0;
    __syncthreads();
    scan[e] += v;
    __syncthreads();
  }
  const int excl = scan[e] - total;
  if (e < E) {
    offsets[e] = excl;
    first[e] = excl;
    int run = excl;
    if (staged) {
      for (int b = 0; b < nb; ++b) {
        const int c = stash[b * E + e];
        counts[(int64_t)b * E + e] = run;
        run += c;
      }
    } else {
      int b = 0;
      for (; b + 8 <= nb; b += 8) {
        int c[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) c[u] = counts[(int64_t)(b + u) * E + e];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          counts[(int64_t)(b + u) * E + e] = run;
          run += c[u];
        }
      }
      for (; b < nb; ++b) {
        const int c = counts[(int64_t)b * E + e];
        counts[(int64_t)b * E + e] = run;
        run += c;
      }
    }
  }
  if (e == E - 1) {
    offsets[E] = excl + total;
    first[E] = excl + total;
    first[E + 1] = excl + total + ext_T;
  }
  if (t.bm > 0) {
    __syncthreads();
    write_tile_lists(scan, first, ext_T > 0 ? E + 1 : E, t);
  }
}

__global__ __launch_bounds__(64) void perm_scatter(const int32_t* __restrict__ ids, int n, int k, int E,
                                                   const int32_t* __restrict__ first,
                                                   int32_t* __restrict__ src, int32_t* __restrict__ inv) {
  __shared__ int run[1024];
  // the chunk's experts, loaded up front (the ranking loop's stores would
  // otherwise hold up each of its loads: the vector memory counter retires in order)
  __shared__ int eid[kChunk];
  const int lane = threadIdx.x;
  const int base = blockIdx.x * kChunk;
  {
    int c[kChunk / 64];
#pragma unroll
    for (int u = 0; u < kChunk / 64; ++u) c[u] = ids[min(base + u * 64 + lane, n - 1)];  // n >= 1; copies past n unused
#pragma unroll
    for (int u = 0; u < kChunk / 64; ++u) eid[u * 64 + lane] = min(max(c[u], 0), E - 1);
  }
  for (int e = lane; e < E; e += 64) run[e] = first[(int64_t)blockIdx.x * E + e];
  __syncthreads();
  int bits = 0;
  while ((1 << bits) < E) ++bits;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int g = 0; g < kChunk; g += 64) {
    const int a = base + g + lane;
    const bool ok = a < n;
    const int e = ok ? eid[g + lane] : 0;
    uint64_t same = __ballot(ok);
    for (int b = 0; b < bits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bal = __ballot(bit);
      same &= bit ? bal : ~bal;
    }
    const int rank = __popcll(same & lt);
    const int pos = run[e] + rank;
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): every lane has read run[] before it changes
    __builtin_amdgcn_wave_barrier();
    if (ok && rank == 0) run[e] = pos + __popcll(same);
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    if (ok) {
      src[pos] = a / k;
      inv[a] = pos;
    }
  }
}

// Small batches (n <= kSmallPermute copies): the whole permutation in one
// work-group, one launch instead of three: an LDS histogram, the scan, then
// wave 0 places the copies in order with the ballot ranking of perm_scatter
// (the same stable result); with ext_T > 0 also the shared expert as group E.
// With t.bm > 0 the same work-group writes the GEMMs' tile lists as well.
constexpr int kSmallPermute = 4096;

__global__ __launch_bounds__(1024) void perm_small(const int32_t* __restrict__ ids, int n, int k, int E,
                                                   int32_t* __restrict__ offsets, int32_t* __restrict__ src,
                                                   int32_t* __restrict__ inv, int ext_T, TileLists t) {
  __shared__ int run[1024];  // counts, then the next free slot of each expert
  __shared__ int scan[1024];
  __shared__ int first[1026];  // the groups' first rows (tile lists)
  // Each assignment's expert, kept from the histogram pass: the serial ranking
  // below then issues no global loads, which would each wait (in-order vector
  // memory counter) for every store issued before them.
  __shared__ int eid[kSmallPermute];
  const int tid = threadIdx.x;
  run[tid] = 0;
  __syncthreads();
  for (int a = tid; a < n; a += 1024) {
    const int e = min(max(ids[a], 0), E - 1);
    eid[a] = e;
    atomicAdd(&run[e], 1);
  }
  __syncthreads();
  const int cnt = tid < E ? run[tid] : 0;
  scan[tid] = cnt;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = tid >= o ? scan[tid - o] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  const int excl = scan[tid] - cnt;
  if (tid < E) {
    offsets[tid] = excl;
    run[tid] = excl;
    first[tid] = excl;
  }
  if (tid == E - 1) {
    offsets[E] = excl + cnt;
    first[E] = n;
    first[E + 1] = n + ext_T;
  }
  __syncthreads();
  if (t.bm > 0) write_tile_lists(scan, first, ext_T > 0 ? E + 1 : E, t);
  if (tid < 64) {
    const int lane = tid;
    int bits = 0;
    while ((1 << bits) < E) ++bits;
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int g = 0; g < n; g += 64) {
      const int a = g + lane;
      const bool ok = a < n;
      const int e = ok ? eid[a] : 0;
      uint64_t same = __ballot(ok);
      for (int b = 0; b < bits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t bal = __ballot(bit);
        same &= bit ? bal : ~bal;
      }
      const int rank = __popcll(same & lt);
      const int pos = run[e] + rank;
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): every lane has read run[] before it changes
      __builtin_amdgcn_wave_barrier();
      if (ok && rank == 0) run[e] = pos + __popcll(same);
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
      if (ok) {
        src[pos] = a / k;
        inv[a] = pos;
      }
    }
  }
  if (ext_T > 0) {
    for (int t = tid; t < ext_T; t += 1024) src[n + t] = t;
    if (tid == 0) offsets[E + 1] = n + ext_T;
  }
}

hipError_t launch_permute(const int32_t* ids, int n, int k, int E, int32_t* counts, int32_t* offsets,
                          int32_t* src, int32_t* inv, hipStream_t s, int ext_T, const TileLists* tl,
                          bool* tiles_done) {
  if (tiles_done) *tiles_done = false;
  if (n <= 0) return hipSuccess;
  if (n <= kSmallPermute) {
    const TileLists t = (tl && E + (ext_T > 0 ? 1 : 0) <= 1024) ? *tl : TileLists{};
    hipLaunchKernelGGL(perm_small, dim3(1), dim3(1024), 0, s, ids, n, k, E, offsets, src, inv, ext_T, t);
    const hipError_t e = hipGetLastError();
    if (e == hipSuccess && tiles_done) *tiles_done = t.bm > 0;
    return e;
  }
  const int nb = permute_blocks(n);
  const TileLists t = (tl && E + (ext_T > 0 ? 1 : 0) <= 1024) ? *tl : TileLists{};
  hipLaunchKernelGGL(perm_hist, dim3(nb), dim3(256), 0, s, ids, n, E, counts);
  hipLaunchKernelGGL(perm_scan, dim3(1), dim3(1024), 0, s, counts, nb, E, offsets, ext_T, t);
  hipLaunchKernelGGL(perm_scatter, dim3(nb), dim3(64), 0, s, ids, n, k, E, counts, src, inv);
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess && tiles_done) *tiles_done = t.bm > 0;
  if (e != hipSuccess || ext_T <= 0) return e;
  return launch_extend_shared(offsets, E, n, ext_T, src, s);
}

}  // namespace moe

namespace moe {

// The shared expert as group E of the routed launch: rows [rows, rows + T) of the
// permuted order are the tokens themselves, and the group ends at rows + T.
__global__ __launch_bounds__(256) void extend_shared_kernel(int32_t* __restrict__ offsets, int E, int rows, int T,
                                                           int32_t* __restrict__ src) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t < T) src[rows + t] = t;
  if (t == 0) offsets[E + 1] = rows + T;
}

hipError_t launch_extend_shared(int32_t* offsets, int E, int rows, int T, int32_t* src, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(extend_shared_kernel, dim3((T + 255) / 256), dim3(256), 0, s, offsets, E, rows, T, src);
  return hipGetLastError();
}

}  // namespace moe
