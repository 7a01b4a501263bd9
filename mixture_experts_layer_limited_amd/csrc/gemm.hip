// Grouped "NT" fp32 GEMMs on gfx950 MFMA for fp32 MoE layers: router GEMM,
// routed experts (gate/up GEMM with a fused SiLU*up epilogue, down GEMM with a
// row-store or a weighted scatter-add epilogue) and the shared expert; plus the
// tile-list builder every grouped GEMM uses.
//
// C[p, n] = sum_k A[src(p), k] * B[g][n, k]   for rows p of m-tile (g, r0, r1)
//
// Both operands are K-contiguous (activations (rows, K), weights (out, in)),
// so every lane loads 16-byte K-chunks of one row for both MFMA operands.
// A work-group owns a BM x BN output tile; it stages BK = 128 bytes of K per
// step for A and B in LDS (double-buffered, 16-byte chunks XOR-swizzled by
// row so the fragment reads are bank-conflict free) and prefetches the next
// step into registers while the MFMAs run.  The m-tiles of the routed experts
// come from a device-side list built from expert_offsets, so the launch
// needs no host synchronisation: the grid covers the largest possible tile
// count and surplus work-groups exit at once.
#include "common.h"
#include "kernels.h"
#include "tiles.h"
#include "lds_dma.h"

namespace moe {

// MFMA over one 32-byte K slice per lane pair: lanes 0-31 hold one 16-byte
// chunk, lanes 32-63 the next.  A and B fragments use the same lane -> K map,
// so the K order inside the slice does not matter.  (bf16 layers run the
// pipelined kernels of gemm_pipe.hip; this kernel serves fp32 layers.)
template <int DT> struct Mma;
template <> struct Mma<MOE_DT_F32> {
  __device__ __forceinline__ static void run(f32x16& acc, const u32x4& a, const u32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  }
};


template <int DT, int WM, int WN, int TM, int TN, int EPI, int ODT>
__global__ __launch_bounds__(WM * WN * 64) void gemm_kernel(GemmParams p) {
  constexpr int NT = WM * WN * 64;
  constexpr int BM = WM * TM * 32;
  constexpr int BN = WN * TN * 32;
  constexpr int CA = BM * 8 / NT;  // 16-byte chunks per thread per K step
  constexpr int CB = BN * 8 / NT;
  static_assert(CA * NT == BM * 8 && CB * NT == BN * 8, "tile / thread mismatch");
  static_assert(EPI != EPI_SWIGLU || TN % 2 == 0, "SwiGLU pairs gate and up tiles");
  constexpr int EB = (DT == MOE_DT_BF16) ? 2 : 4;
  constexpr int STAGE = (BM + BN) * 8;  // u32x4 per LDS stage

  extern __shared__ u32x4 lds[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // device list: every (m-tile, n-tile) pair; dense: n_mtiles x ntn tiles
  const int total = p.tiles ? *p.n_mtiles_dev : p.n_mtiles * p.ntn;
  const int P = blockIdx.x;
  if (P >= total) return;
  const int L = xcd_remap(P, total);
  int grp, r0, r1, nt;
  if (p.tiles) {
    const int4 t = p.tiles[L];
    grp = t.x; r0 = t.y; r1 = t.z; nt = t.w;
  } else {
    const int mt = L / p.ntn;
    nt = L - mt * p.ntn;
    grp = 0; r0 = mt * BM; r1 = min(p.M, r0 + BM);
  }
  const int rows = r1 - r0;
  const int64_t kbytes = (int64_t)p.K * EB;
  const char* Bg = (p.B2 && grp == p.b2_group) ? (const char*)p.B2 : (const char*)p.B + (int64_t)grp * p.b_gstride * EB;

  // Global source of every chunk this thread copies (fixed over the K loop).
  const char* aptr[CA];
  bool aok[CA];
  int aoff[CA];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int q = tid + i * NT, r = q >> 3, c = q & 7;
    aok[i] = r < rows;
    int src = 0;
    if (aok[i]) src = p.a_rows ? p.a_rows[r0 + r] : r0 + r;
    aptr[i] = (const char*)p.A + (int64_t)src * kbytes + c * 16;
    aoff[i] = r * 8 + (c ^ (r & 7));
  }
  const char* bptr[CB];
  int boff[CB];
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const int q = tid + i * NT, r = q >> 3, c = q & 7;
    int wrow;
    if constexpr (EPI == EPI_SWIGLU) {
      int j = nt * (BN / 2) + (r % (BN / 2));
      j = min(j, p.N - 1);
      wrow = (r < BN / 2) ? j : p.N + j;
    } else {
      wrow = min(nt * BN + r, p.N - 1);
    }
    bptr[i] = Bg + (int64_t)wrow * kbytes + c * 16;
    boff[i] = (BM + r) * 8 + (c ^ (r & 7));
  }

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // Row blocks of this wave that hold at least one valid row.
  int tm_live = 0;
#pragma unroll
  for (int i = 0; i < TM; ++i)
    if ((wm * TM + i) * 32 < rows) tm_live = i + 1;

  // B row block (of 32) of wave tile column tn.
  auto bblock = [&](int tn) {
    if constexpr (EPI == EPI_SWIGLU)
      return tn < TN / 2 ? wn * (TN / 2) + tn : WN * (TN / 2) + wn * (TN / 2) + (tn - TN / 2);
    else
      return wn * TN + tn;
  };

  const int nk = (int)(kbytes / 128);
  u32x4 ra[CA], rb[CB];

#define MOE_GLOAD(kt_)                                                       \
  do {                                                                       \
    const int64_t ko_ = (int64_t)(kt_) * 128;                                \
    _Pragma("unroll") for (int i = 0; i < CA; ++i) if (aok[i]) ra[i] =       \
        *(const u32x4*)(aptr[i] + ko_);                                      \
    _Pragma("unroll") for (int i = 0; i < CB; ++i) rb[i] =                   \
        *(const u32x4*)(bptr[i] + ko_);                                      \
  } while (0)
#define MOE_SSTORE(buf_)                                                     \
  do {                                                                       \
    u32x4* s_ = lds + (buf_) * STAGE;                                        \
    _Pragma("unroll") for (int i = 0; i < CA; ++i) if (aok[i]) s_[aoff[i]] = ra[i]; \
    _Pragma("unroll") for (int i = 0; i < CB; ++i) s_[boff[i]] = rb[i];      \
  } while (0)

  MOE_GLOAD(0);
  MOE_SSTORE(0);
  __syncthreads();

  const int sw = lane & 7;
  const int lr = lane & 31;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) MOE_GLOAD(kt + 1);
    if (tm_live > 0) {
      const u32x4* s = lds + buf * STAGE;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int ch = (2 * st + (lane >> 5)) ^ sw;
        u32x4 a[TM], b[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) a[i] = s[((wm * TM + i) * 32 + lr) * 8 + ch];
#pragma unroll
        for (int j = 0; j < TN; ++j) b[j] = s[(BM + bblock(j) * 32 + lr) * 8 + ch];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          if (i < tm_live) {
#pragma unroll
            for (int j = 0; j < TN; ++j) Mma<DT>::run(acc[i][j], a[i], b[j]);
          }
        }
      }
    }
    if (kt + 1 < nk) MOE_SSTORE(buf ^ 1);
    __syncthreads();
  }
#undef MOE_GLOAD
#undef MOE_SSTORE

  // Epilogue.  Lane l, register e of a 32x32 tile hold row 8*(e/4) + 4*(l/32) + e%4,
  // column l%32.
  const int hi = lane >> 5;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    if (i >= tm_live) continue;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = (wm * TM + i) * 32 + 8 * (e >> 2) + 4 * hi + (e & 3);
      if (row >= rows) continue;
      const int prow = r0 + row;
      if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int j = 0; j < TN / 2; ++j) {
          const int col = nt * (BN / 2) + (wn * (TN / 2) + j) * 32 + lr;
          if (col < p.N) {
            const float h = silu_mul(acc[i][j][e], acc[i][j + TN / 2][e]);
            Elem<ODT>::store((typename Elem<ODT>::T*)p.C, (int64_t)prow * p.N + col, h);
          }
        }
      } else if constexpr (EPI == EPI_SCATTER) {
        const int tok = p.c_rows ? p.c_rows[prow] : prow;
        const float w = p.row_w[prow];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col = nt * BN + bblock(j) * 32 + lr;
          if (col < p.N) atomicAdd((float*)p.C + (int64_t)tok * p.N + col, w * acc[i][j][e]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col = nt * BN + bblock(j) * 32 + lr;
          if (col < p.N) Elem<ODT>::store((typename Elem<ODT>::T*)p.C, (int64_t)prow * p.N + col, acc[i][j][e]);
        }
      }
    }
  }
}

// ------------------------------------------------------------ m-tile list ---

// One block: the tile lists of a grouped GEMM pair (write_tile_lists).
__global__ __launch_bounds__(1024) void build_tiles_kernel(const int32_t* __restrict__ offsets, int E, TileLists t) {
  __shared__ int scan[1024];
  __shared__ int first[1025];  // offsets[0 .. E]
  const int e = threadIdx.x;
  if (e < E) {
    first[e] = offsets[e];
    if (e == E - 1) first[E] = offsets[E];
  }
  __syncthreads();
  write_tile_lists(scan, first, E, t);
}

// ---------------------------------------------------------------- launch ---

template <int DT, int WM, int WN, int TM, int TN, int EPI, int ODT>
static hipError_t launch_cfg(const GemmParams& p, int grid_m, hipStream_t s) {
  constexpr int BN = WN * TN * 32;
  constexpr int BM = WM * TM * 32;
  constexpr int lds_bytes = 2 * (BM + BN) * 128;
  auto kern = gemm_kernel<DT, WM, WN, TM, TN, EPI, ODT>;
  {
    const hipError_t e = allow_lds<gemm_kernel<DT, WM, WN, TM, TN, EPI, ODT>>(lds_bytes);
    if (e != hipSuccess) return e;
  }
  const int64_t grid = (int64_t)grid_m * p.ntn;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(WM * WN * 64), lds_bytes, s, p);
  return hipGetLastError();
}

// Tile shapes by kind.  Register-staged kernel (fp32):
//   0: 2x2 waves of 2x2 32x32 blocks -> 128 x 128;  1: 1x4 waves of 1x2 -> 32 x 256.
// Pipelined bf16 kernels (gemm_pipe.hip): 12: 128 x 256 single ring; 13: 64 x 256
// single ring of 64-byte K rows, two work-groups per CU (the down GEMM of
// decode-sized groups); 14: 64 x 256 single ring (the gate/up GEMM of
// decode-sized groups and the split-K router); 15: 256 x 256 split rings
// (prefill-sized groups).  MOE_TILE_GEMM1 / MOE_TILE_GEMM2 force a kind for
// the gate/up or down GEMM at build time (tuning).
#ifndef MOE_TILE_GEMM1
#define MOE_TILE_GEMM1 -1
#endif
#ifndef MOE_TILE_GEMM2
#define MOE_TILE_GEMM2 -1
#endif
static int tile_bm(int kind) {
  switch (kind) {
    case 1: return 32;
    case 12: return 128;
    case 13: return 64;
    case 14: return 64;
    case 15: return 256;
    default: return 128;
  }
}
static int tile_bn(int kind) { return kind == 0 ? 128 : 256; }

// which: 0 = gate/up GEMM, 1 = down GEMM, 2 = router GEMM.  rows_hint = mean
// rows per group; tiles256 = the launch's work-groups with 256 x 256 tiles
// (0: not known).  bf16 always takes a pipelined kernel (the ABI bounds the
// activation buffers and every weight matrix below 2^31 bytes, the reach of its
// 32-bit buffer offsets); fp32 takes the register-staged one.
GemmShape gemm_shape(int which, int dt, int rows_hint, int64_t tiles256) {
  int kind;
  if (dt != MOE_DT_BF16) kind = (which != 2 && rows_hint <= 32) ? 1 : 0;
  // router, split K: 64 x 256 tiles, or 128 x 256 for large batches, where the
  // gate weight re-read by every m-tile is most of the bytes
  else if (which == 2) kind = rows_hint >= kRouterWideRows ? 12 : 14;
  else if (rows_hint <= 32) kind = which == 1 ? 13 : 14;
  else if (rows_hint < 128) kind = 12;
  // a launch with fewer 256 x 256 tiles than the chip has CUs leaves CUs idle
  // (one work-group per CU): 128 x 256 tiles double its work-groups
  else if (tiles256 > 0 && tiles256 < kChipCUs) kind = 12;
  else kind = 15;
  if (dt == MOE_DT_BF16) {
    if (which == 0 && MOE_TILE_GEMM1 >= 12 && MOE_TILE_GEMM1 <= 15) kind = MOE_TILE_GEMM1;
    if (which == 1 && MOE_TILE_GEMM2 >= 12 && MOE_TILE_GEMM2 <= 15) kind = MOE_TILE_GEMM2;
  }
  GemmShape g;
  g.kind = kind;
  g.bm = tile_bm(kind);
  g.bn = tile_bn(kind);
  return g;
}

template <int EPI, int ODT>
static hipError_t dispatch_shape(const GemmParams& p, const GemmShape& g, int grid_m, hipStream_t s) {
  if (g.kind == 1) return launch_cfg<MOE_DT_F32, 1, 4, 1, 2, EPI, ODT>(p, grid_m, s);
  return launch_cfg<MOE_DT_F32, 2, 2, 2, 2, EPI, ODT>(p, grid_m, s);
}

hipError_t launch_gemm(int dt, int epi, int odt, const GemmParams& p, const GemmShape& g, int grid_m,
                       hipStream_t s) {
  if (dt == MOE_DT_BF16) {
    if (g.kind < 12) return hipErrorInvalidValue;
    return launch_gemm_pipe(epi, odt, p, g, grid_m, s);
  }
  if (g.kind > 1) return hipErrorInvalidValue;
  switch (epi) {
    case EPI_STORE: return dispatch_shape<EPI_STORE, MOE_DT_F32>(p, g, grid_m, s);
    case EPI_SWIGLU: return dispatch_shape<EPI_SWIGLU, MOE_DT_F32>(p, g, grid_m, s);
    case EPI_SCATTER: return dispatch_shape<EPI_SCATTER, MOE_DT_F32>(p, g, grid_m, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_build_tiles(const int32_t* offsets, int E, int bm, int ntn, int4* tiles, int* n_tiles,
                              hipStream_t s, int bm2, int ntn2, int4* tiles2, int* n_tiles2) {
  TileLists t;
  t.bm = bm; t.ntn = ntn; t.tiles = tiles; t.n_tiles = n_tiles;
  if (tiles2 && bm2 == bm) {  // both lists from one scan
    t.ntn2 = ntn2; t.tiles2 = tiles2; t.n_tiles2 = n_tiles2;
    hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(1024), 0, s, offsets, E, t);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(1024), 0, s, offsets, E, t);
  if (tiles2) {
    TileLists t2;
    t2.bm = bm2; t2.ntn = ntn2; t2.tiles = tiles2; t2.n_tiles = n_tiles2;
    hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(1024), 0, s, offsets, E, t2);
  }
  return hipGetLastError();
}

}  // namespace moe
