// Pipelined grouped bf16 GEMMs for the expert FFNs (gate/up with the SiLU*up
// epilogue, down with the row-store or weighted scatter-add epilogue), after the
// grouped-GEMM step of the MoE inference walkthrough (zhiyuanblog.org/blog/
// moe-inference, §3.3):
//
//   C[p, n] = sum_k A[src(p), k] * B[g][n, k] over the rows p of m-tile (g, r0, r1)
//
// Operand tiles stream straight from memory into LDS rings with buffer_load ...
// lds (no register staging), several K steps ahead of the MFMAs; an explicit
// "s_waitcnt vmcnt(n); s_barrier" per step releases exactly the slot about to be
// read.  Rows are gathered through permuted_src by per-lane buffer offsets, so
// the permuted copy of the activations is never written; rows past a tile and
// the K tail read out of the buffer's range, which fills zeros without traffic.
// 16-byte chunks are XOR-swizzled within each LDS row so the 128-bit fragment
// reads of 8 and of 16 consecutive rows hit distinct banks.
//
// gemm_pipe_kernel: one ring holding A and B (64- or 128-byte K rows), 2 x 2
//   waves; used for decode-sized groups (64 x 256 tiles).
// gemm_split_kernel: separate A and B rings of 128-byte K rows (B runs deeper),
//   k16 sub-steps whose fragment reads overlap the previous sub-step's MFMAs,
//   and an LDS-staged bf16 epilogue with 16-byte row stores; 256 x 256 tiles
//   for prefill-sized groups.
// In both, wave row wm takes row blocks wm, wm+WM, ... so the wave rows stay
// balanced when a tile has fewer live rows than BM; row blocks without live rows
// issue no MFMAs (the live blocks of a wave are a prefix, so the K loop is
// specialised on their count and stays branch-free).
#include "combine_epi.h"
#include "common.h"
#include "kernels.h"
#include "lds_dma.h"

namespace moe {

template <int Q, int M, int LI>
__device__ __forceinline__ void pipe_schedule_mfmas() {
  if constexpr (Q < M) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    constexpr int DE = M / LI > 0 ? M / LI : 1;         // a ring DMA after every DE MFMAs
    if constexpr (LI > 0 && (Q + 1) % DE == 0 && (Q + 1) / DE <= LI) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    pipe_schedule_mfmas<Q + 1, M, LI>();
  }
}

// Instruction order of one K step (a hint to the scheduler): all fragment reads
// of the step, then the MFMAs with the ring DMAs spread evenly among them, so
// the DMAs reach the address unit one at a time while the matrix cores are busy.
template <int NL, int TN, int NSUB, int LI>
__device__ __forceinline__ void pipe_schedule() {
  __builtin_amdgcn_sched_group_barrier(0x100, NSUB * (NL + TN), 0);
  pipe_schedule_mfmas<0, NSUB * NL * TN, LI>();
}

template <int TM, int TN, int S, int OCC, int ROWB, int EPI, int ODT>
__global__ __launch_bounds__(256, OCC) void gemm_pipe_kernel(GemmParams p) {
  constexpr int WM = 2, WN = 2, NW = 4, NT = 256;
  constexpr int BM = WM * TM * 32;
  constexpr int BN = WN * TN * 32;
  constexpr int ROW = ROWB;                     // bytes of K per row per slot (64 or 128)
  constexpr int CPR = ROW / 16;                 // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;                 // rows per DMA instruction (1 KB)
  constexpr int NSUB = ROW / 32;                // k16 MFMA sub-steps per slot
  constexpr int SLOT = (BM + BN) * ROW;         // bytes per ring slot
  constexpr int AI = BM / RPI / NW;             // DMA instructions per wave per slot
  constexpr int BI = BN / RPI / NW;
  constexpr int LI = AI + BI;
  static_assert(ROW == 64 || ROW == 128, "row bytes");
  static_assert(AI * RPI * NW == BM && BI * RPI * NW == BN, "tile / wave mismatch");
  static_assert(EPI != EPI_SWIGLU || TN % 2 == 0, "SwiGLU pairs gate and up tiles");
  static_assert(S >= 2 && S <= 6, "ring depth");

  extern __shared__ __attribute__((aligned(16))) char lds[];
  lds_char* const lds3 = (lds_char*)lds;  // the same memory as an LDS-address-space pointer

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in an SGPR
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
  const int64_t krow = (int64_t)p.K * 2;  // bytes per A / B row
  const char* Bg = (p.B2 && grp == p.b2_group) ? (const char*)p.B2 : (const char*)p.B + (int64_t)grp * p.b_gstride * 2;
  const int b_nrows = (EPI == EPI_SWIGLU) ? 2 * p.N : p.N;
  // split K: this group's slice starts kofs bytes into every row
  const int nsplit = p.ksplit > 1 ? p.ksplit : 1;
  const int64_t kofs = (int64_t)blockIdx.y * (krow / nsplit);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc((const char*)p.A + kofs, p.a_nrows * krow - kofs);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bg + kofs, (int64_t)b_nrows * krow - kofs);

  // Per-lane byte offsets of the rows this lane copies (fixed over K).
  // Lane l of a DMA instruction fills row (l / CPR), slot (l % CPR) of an RPI-row block.
  const int lrow = lane / CPR, lslot = lane % CPR;
  uint32_t voa[AI], vob[BI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int r = (wave * AI + i) * RPI + lrow;
    const int chunk = lslot ^ swz<ROW>(r);
    const int rr = r < rows ? r : 0;  // rows past the tile read row 0 (results discarded)
    const int src = p.a_rows ? p.a_rows[r0 + rr] : r0 + rr;
    voa[i] = (uint32_t)((int64_t)src * krow + chunk * 16);
  }
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int r = (wave * BI + i) * RPI + lrow;
    const int chunk = lslot ^ swz<ROW>(r);
    int wrow;
    if constexpr (EPI == EPI_SWIGLU) {
      const int j = min(nt * (BN / 2) + (r % (BN / 2)), p.N - 1);
      wrow = (r < BN / 2) ? j : p.N + j;
    } else {
      wrow = min(nt * BN + r, p.N - 1);
    }
    vob[i] = (uint32_t)((int64_t)wrow * krow + chunk * 16);
  }

  const int nk = p.K * 2 / nsplit / ROW;

  // Issue the DMA of K step kt into ring slot kt % S; for kt >= nk the offset is
  // out of the buffers' range, so the hardware writes zeros without touching
  // memory (keeps the loop body branch-free and the vmcnt bookkeeping constant).
  // (A macro, not a lambda: device-only builtins inside a lambda would hide the
  // kernel from the host pass.)
#define MOE_PIPE_ISSUE(kt_)                                                                        \
  do {                                                                                             \
    lds_char* slot_ = lds3 + ((kt_) % S) * SLOT;                                                   \
    const uint32_t soff_ = (kt_) < nk ? (uint32_t)(kt_) * ROW : 0x80000000u;                       \
    _Pragma("unroll") for (int i = 0; i < AI; ++i)                                                 \
      dma16(ra, slot_ + (wave * AI + i) * 1024, voa[i], soff_);                                    \
    _Pragma("unroll") for (int i = 0; i < BI; ++i)                                                 \
      dma16(rb, slot_ + BM * ROW + (wave * BI + i) * 1024, vob[i], soff_);                         \
  } while (0)

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  int tm_live = 0;  // row blocks wm, wm+2, ... that hold live rows
#pragma unroll
  for (int i = 0; i < TM; ++i)
    if ((wm + 2 * i) * 32 < rows) tm_live = i + 1;
  tm_live = __builtin_amdgcn_readfirstlane(tm_live);  // wave-uniform: scalar branches only

  auto bblock = [&](int tn) {
    if constexpr (EPI == EPI_SWIGLU)
      return tn < TN / 2 ? wn * (TN / 2) + tn : WN * (TN / 2) + wn * (TN / 2) + (tn - TN / 2);
    else
      return wn * TN + tn;
  };

  const int lr = lane & 31, hi = lane >> 5;
  // (row & 15) == (lr & 15) for every row block, whose starts are multiples of 32
  const int sw = swz<ROW>(lr);

#pragma unroll
  for (int s = 0; s < S - 1; ++s) MOE_PIPE_ISSUE(s);

  // The K loop on the first NL row blocks of this wave; branch-free inside so the
  // accumulators stay in place.  Tiles with at most half their row blocks live
  // run the NL = TM/2 copy.
#define MOE_PIPE_KLOOP                                                                              \
  for (int kt = 0; kt < nk; ++kt) {                                                                 \
    /* slot kt is complete once at most the S-2 later slots' DMAs are pending */                    \
    wait_vm_barrier<(S - 2) * LI>();                                                                \
    const char* slot = lds + (kt % S) * SLOT;                                                       \
    u32x4 a[NSUB][NL], b[NSUB][TN];                                                                 \
    _Pragma("unroll") for (int st = 0; st < NSUB; ++st) {                                           \
      const int coff = ((2 * st + hi) ^ sw) * 16;                                                   \
      _Pragma("unroll") for (int j = 0; j < TN; ++j)                                                \
        b[st][j] = *(const u32x4*)(slot + BM * ROW + (bblock(j) * 32 + lr) * ROW + coff);           \
      _Pragma("unroll") for (int i = 0; i < NL; ++i)                                                \
        a[st][i] = *(const u32x4*)(slot + ((wm + 2 * i) * 32 + lr) * ROW + coff);                   \
    }                                                                                               \
    /* the ring DMAs go after the fragment reads in program order (they may not */                  \
    /* pass LDS reads), then spread among the MFMAs */                                              \
    MOE_PIPE_ISSUE(kt + S - 1);                                                                     \
    _Pragma("unroll") for (int st = 0; st < NSUB; ++st)                                             \
      _Pragma("unroll") for (int i = 0; i < NL; ++i)                                                \
        _Pragma("unroll") for (int j = 0; j < TN; ++j)                                              \
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[st][i]), \
                                                              __builtin_bit_cast(bf16x8, b[st][j]), \
                                                              acc[i][j], 0, 0, 0);                  \
    pipe_schedule<NL, TN, NSUB, LI>();                                                              \
  }

  constexpr int HALF = TM / 2 > 0 ? TM / 2 : 1;
  if (TM > 1 && tm_live <= HALF) {
    constexpr int NL = HALF;
    MOE_PIPE_KLOOP
  } else {
    constexpr int NL = TM;
    MOE_PIPE_KLOOP
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the tail's zero-fill DMAs
#undef MOE_PIPE_KLOOP
#undef MOE_PIPE_ISSUE

  // Epilogue.  Lane l, register e of a 32x32 block: row 8*(e/4) + 4*(l/32) + e%4, column l%32.
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    if (i >= tm_live) continue;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = (wm + 2 * i) * 32 + 8 * (e >> 2) + 4 * hi + (e & 3);
      if (row >= rows) continue;
      const int prow = r0 + row;
      if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int j = 0; j < TN / 2; ++j) {
          const int col = nt * (BN / 2) + (wn * (TN / 2) + j) * 32 + lr;
          if (col < p.N)
            Elem<ODT>::store((typename Elem<ODT>::T*)p.C, (int64_t)prow * p.N + col,
                             silu_mul(acc[i][j][e], acc[i][j + TN / 2][e]));
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
        typename Elem<ODT>::T* C = (typename Elem<ODT>::T*)p.C + (int64_t)blockIdx.y * p.c_split_stride;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col = nt * BN + bblock(j) * 32 + lr;
          if (col < p.N) Elem<ODT>::store(C, (int64_t)prow * p.N + col, acc[i][j][e]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Split-ring kernel for the large prefill GEMMs.  A and B tiles have rings of
// their own (depth SA <= SB slots of 64 bf16 of K), so the weight stream (B,
// mostly HBM misses) runs further ahead than the activation rows (A, mostly L2
// hits shared by every n-tile of the m-tile).  Within a K step the fragment
// reads of sub-step st+1 are issued among the MFMAs of sub-step st, so only the
// first sub-step's LDS latency is exposed per step.
//
// DMA issue order per step: A(kt + SA - 1), then B(kt + SB - 1); the wait at the
// top of step kt leaves exactly the instructions issued after the last one that
// step kt needs in flight (VMN).

template <int WM, int WN, int TM, int TN, int SA, int SB, int EPI, int ODT>
__global__ __launch_bounds__(WM * WN * 64, 1) void gemm_split_kernel(GemmParams p) {
  constexpr int NW = WM * WN;
  constexpr int BM = WM * TM * 32;
  constexpr int BN = WN * TN * 32;
  constexpr int ROW = 128, CPR = 8, RPI = 8, NSUB = 4;  // NSUB is fixed: the K loop names sub-steps 0..3
  constexpr int ASLOT = BM * ROW, BSLOT = BN * ROW;
  constexpr int AI = BM / RPI / NW, BI = BN / RPI / NW;
  constexpr int LI = AI + BI;
  // A(kt) is issued SA-1 steps before step kt; with SB > SA, B(kt) went out even
  // earlier and only B of A(kt)'s step follows it, else B(kt) is that step's last.
  constexpr int VMN = SB > SA ? BI + (SA - 2) * LI : (SA - 2) * LI;
  static_assert(AI * RPI * NW == BM && BI * RPI * NW == BN, "tile / wave mismatch");
  static_assert(SA >= 2 && SB >= SA && VMN < 64, "ring depths");
  static_assert(EPI != EPI_SWIGLU || TN % 2 == 0, "SwiGLU pairs gate and up tiles");

  extern __shared__ __attribute__((aligned(16))) char lds[];
  lds_char* const lds3 = (lds_char*)lds;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

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
  const int64_t krow = (int64_t)p.K * 2;
  const char* Bg = (p.B2 && grp == p.b2_group) ? (const char*)p.B2 : (const char*)p.B + (int64_t)grp * p.b_gstride * 2;
  const int b_nrows = (EPI == EPI_SWIGLU) ? 2 * p.N : p.N;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, p.a_nrows * krow);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bg, (int64_t)b_nrows * krow);

  const int lrow = lane / CPR, lslot = lane % CPR;
  uint32_t voa[AI], vob[BI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int r = (wave * AI + i) * RPI + lrow;
    const int chunk = lslot ^ swz<ROW>(r);
    if (r < rows) {
      const int src = p.a_rows ? p.a_rows[r0 + r] : r0 + r;
      voa[i] = (uint32_t)((int64_t)src * krow + chunk * 16);
    } else {
      voa[i] = 0x40000000u;  // past the tile: out of range (zero fill, no traffic) or harmless
    }
  }
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int r = (wave * BI + i) * RPI + lrow;
    const int chunk = lslot ^ swz<ROW>(r);
    int wrow;
    if constexpr (EPI == EPI_SWIGLU) {
      const int j = min(nt * (BN / 2) + (r % (BN / 2)), p.N - 1);
      wrow = (r < BN / 2) ? j : p.N + j;
    } else {
      wrow = min(nt * BN + r, p.N - 1);
    }
    vob[i] = (uint32_t)((int64_t)wrow * krow + chunk * 16);
  }

  const int nk = p.K * 2 / ROW;
  lds_char* const ring_a = lds3;
  lds_char* const ring_b = lds3 + SA * ASLOT;

  // DMA instructions [lo, hi) of step kt_'s A (or B) slot; the tail steps read
  // out of range (zero fill, no traffic) so the vmcnt bookkeeping stays fixed.
#define MOE_SPLIT_ISSUE_A(kt_, lo_, hi_)                                               \
  do {                                                                                 \
    lds_char* slot_ = ring_a + ((kt_) % SA) * ASLOT;                                   \
    const uint32_t soff_ = (kt_) < nk ? (uint32_t)(kt_) * ROW : 0x80000000u;           \
    _Pragma("unroll") for (int i = (lo_); i < (hi_); ++i)                              \
      dma16(ra, slot_ + (wave * AI + i) * 1024, voa[i], soff_);                        \
  } while (0)
#define MOE_SPLIT_ISSUE_B(kt_, lo_, hi_)                                               \
  do {                                                                                 \
    lds_char* slot_ = ring_b + ((kt_) % SB) * BSLOT;                                   \
    const uint32_t soff_ = (kt_) < nk ? (uint32_t)(kt_) * ROW : 0x80000000u;           \
    _Pragma("unroll") for (int i = (lo_); i < (hi_); ++i)                              \
      dma16(rb, slot_ + (wave * BI + i) * 1024, vob[i], soff_);                        \
  } while (0)

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  int tm_live = 0;  // row blocks wm, wm+2, ... holding live rows form a prefix
#pragma unroll
  for (int i = 0; i < TM; ++i)
    if ((wm + WM * i) * 32 < rows) tm_live = i + 1;
  tm_live = __builtin_amdgcn_readfirstlane(tm_live);

  auto bblock = [&](int tn) {
    if constexpr (EPI == EPI_SWIGLU)
      return tn < TN / 2 ? wn * (TN / 2) + tn : WN * (TN / 2) + wn * (TN / 2) + (tn - TN / 2);
    else
      return wn * TN + tn;
  };

  const int lr = lane & 31, hi = lane >> 5;
  const int sw = swz<ROW>(lr);

  // Prologue: the issues of virtual steps 1-SB .. -1.
#pragma unroll
  for (int v = 1 - SB; v < 0; ++v) {
    if (v + SA - 1 >= 0) MOE_SPLIT_ISSUE_A(v + SA - 1, 0, AI);
    if (v + SB - 1 >= 0) MOE_SPLIT_ISSUE_B(v + SB - 1, 0, BI);
  }

#define MOE_SPLIT_READ(buf_, st_)                                                                   \
  do {                                                                                              \
    const int coff_ = ((2 * (st_) + hi) ^ sw) * 16;                                                 \
    _Pragma("unroll") for (int j = 0; j < TN; ++j)                                                  \
      b[buf_][j] = *(const u32x4*)(sb_ + (bblock(j) * 32 + lr) * ROW + coff_);                      \
    _Pragma("unroll") for (int i = 0; i < NL; ++i)                                                  \
      a[buf_][i] = *(const u32x4*)(sa_ + ((wm + WM * i) * 32 + lr) * ROW + coff_);                   \
  } while (0)

// Sub-step ST issues the reads of sub-step ST+1, its share of the step's ring
// DMAs (A's in the first half of the step, B's in the second, keeping the issue
// order the vmcnt bound assumes) and its MFMAs; a scheduling fence closes it.
#define MOE_SPLIT_SUB(ST)                                                                            \
  do {                                                                                               \
    constexpr int nxt_ = (ST) + 1 < NSUB ? NL + TN : 0;                                              \
    constexpr int h_ = NSUB / 2;                                                                     \
    if constexpr ((ST) + 1 < NSUB) MOE_SPLIT_READ(((ST) + 1) & 1, (ST) + 1);                         \
    if constexpr ((ST) < h_) MOE_SPLIT_ISSUE_A(kt + SA - 1, (ST) * AI / h_, ((ST) + 1) * AI / h_);   \
    else MOE_SPLIT_ISSUE_B(kt + SB - 1, ((ST) - h_) * BI / h_, ((ST) - h_ + 1) * BI / h_);           \
    _Pragma("unroll") for (int i = 0; i < NL; ++i)                                                   \
      _Pragma("unroll") for (int j = 0; j < TN; ++j)                                                 \
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[(ST) & 1][i]), \
                                                            __builtin_bit_cast(bf16x8, b[(ST) & 1][j]), \
                                                            acc[i][j], 0, 0, 0);                     \
    sub_schedule<0, NL * TN, nxt_, ((ST) < h_ ? AI : BI) / h_>();                                    \
    __builtin_amdgcn_sched_barrier(0);                                                               \
  } while (0)

#define MOE_SPLIT_KLOOP                                                                              \
  for (int kt = 0; kt < nk; ++kt) {                                                                  \
    wait_vm_barrier<VMN>();                                                                          \
    const char* sa_ = lds + (kt % SA) * ASLOT;                                                       \
    const char* sb_ = lds + SA * ASLOT + (kt % SB) * BSLOT;                                          \
    u32x4 a[2][NL], b[2][TN];                                                                        \
    MOE_SPLIT_READ(0, 0);                                                                            \
    __builtin_amdgcn_sched_barrier(0);                                                               \
    MOE_SPLIT_SUB(0);                                                                                \
    MOE_SPLIT_SUB(1);                                                                                \
    MOE_SPLIT_SUB(2);                                                                                \
    MOE_SPLIT_SUB(3);                                                                                \
  }

  if (tm_live <= 1) {
    constexpr int NL = 1;
    MOE_SPLIT_KLOOP
  } else if (TM > 2 && tm_live == 2) {
    constexpr int NL = TM > 2 ? 2 : TM;
    MOE_SPLIT_KLOOP
  } else if (TM > 3 && tm_live == 3) {
    constexpr int NL = TM > 3 ? 3 : TM;
    MOE_SPLIT_KLOOP
  } else {
    constexpr int NL = TM;
    MOE_SPLIT_KLOOP
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#undef MOE_SPLIT_KLOOP
#undef MOE_SPLIT_SUB
#undef MOE_SPLIT_READ
#undef MOE_SPLIT_ISSUE_A
#undef MOE_SPLIT_ISSUE_B

  if constexpr (ODT == MOE_DT_BF16 && (EPI == EPI_STORE || EPI == EPI_SWIGLU || EPI == EPI_COMBINE)) {
    // bf16 tile through LDS (the ring is idle now), then 16-byte row-contiguous
    // global stores.  Lanes l and l^1 trade one value per row pair (DPP) so each
    // lane writes two adjacent columns of one row as a dword: even lanes row r,
    // columns c and c+1; odd lanes row r+1, columns c-1 and c.  Rows are padded
    // by 16 bytes.
    constexpr int OC = EPI == EPI_SWIGLU ? BN / 2 : BN;  // output columns of the tile
    constexpr int RB = OC * 2 + 16;                      // LDS bytes per staged row
    constexpr int JO = EPI == EPI_SWIGLU ? TN / 2 : TN;  // output column blocks per wave
    static_assert(BM * RB <= SA * ASLOT + SB * BSLOT, "staging fits the ring");
    const bool odd = lr & 1;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if (i >= tm_live) continue;
#pragma unroll
      for (int jo = 0; jo < JO; ++jo) {
        const int c = (EPI == EPI_SWIGLU ? wn * (TN / 2) + jo : bblock(jo)) * 32 + lr;
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          float v0, v1;
          if constexpr (EPI == EPI_SWIGLU) {
            v0 = silu_mul(acc[i][jo][e], acc[i][jo + TN / 2][e]);
            v1 = silu_mul(acc[i][jo][e + 1], acc[i][jo + TN / 2][e + 1]);
          } else {
            v0 = acc[i][jo][e];
            v1 = acc[i][jo][e + 1];
          }
          const float recv = swap_adjacent_lanes(odd ? v0 : v1);
          const int row = (wm + WM * i) * 32 + 8 * (e >> 2) + 4 * hi + (e & 3) + (odd ? 1 : 0);
          const int col = odd ? c - 1 : c;
          *(uint32_t*)(lds + row * RB + 2 * col) = odd ? pack_bf16_rne(recv, v1) : pack_bf16_rne(v0, recv);
        }
      }
    }
    __syncthreads();
    constexpr int CPRo = OC / 8;  // 16-byte chunks per output row
    const int c0 = nt * OC;
    if constexpr (EPI == EPI_COMBINE) {  // dense launch over tokens: the layer's combine instead of the row store
      combine_staged_tile<BM, CPRo, RB, NW * 64, 4>(p.comb, lds, SA * ASLOT + SB * BSLOT - BM * RB, r0, rows, c0,
                                                   p.N, tid);
      return;
    }
    for (int q = tid; q < BM * CPRo; q += NW * 64) {
      const int row = q / CPRo, ch = q % CPRo;
      const int col = c0 + ch * 8;
      if (row < rows && col < p.N)
        *(u32x4*)((uint16_t*)p.C + (int64_t)(r0 + row) * p.N + col) = *(const u32x4*)(lds + row * RB + ch * 16);
    }
    return;
  }

#pragma unroll
  for (int i = 0; i < TM; ++i) {
    if (i >= tm_live) continue;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = (wm + WM * i) * 32 + 8 * (e >> 2) + 4 * hi + (e & 3);
      if (row >= rows) continue;
      const int prow = r0 + row;
      if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int j = 0; j < TN / 2; ++j) {
          const int col = nt * (BN / 2) + (wn * (TN / 2) + j) * 32 + lr;
          if (col < p.N)
            Elem<ODT>::store((typename Elem<ODT>::T*)p.C, (int64_t)prow * p.N + col,
                             silu_mul(acc[i][j][e], acc[i][j + TN / 2][e]));
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

template <int WM, int WN, int TM, int TN, int SA, int SB, int EPI, int ODT>
static hipError_t launch_split(const GemmParams& p, int grid_m, hipStream_t s) {
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  constexpr int lds_bytes = (SA * BM + SB * BN) * 128;
  static_assert(lds_bytes <= 160 * 1024, "LDS");
  auto kern = gemm_split_kernel<WM, WN, TM, TN, SA, SB, EPI, ODT>;
  {
    const hipError_t e = allow_lds<gemm_split_kernel<WM, WN, TM, TN, SA, SB, EPI, ODT>>(lds_bytes);
    if (e != hipSuccess) return e;
  }
  const int64_t grid = (int64_t)grid_m * p.ntn;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(WM * WN * 64), lds_bytes, s, p);
  return hipGetLastError();
}

template <int TM, int TN, int S, int OCC, int ROWB, int EPI, int ODT>
static hipError_t launch_pipe(const GemmParams& p, int grid_m, hipStream_t s) {
  constexpr int BM = 2 * TM * 32, BN = 2 * TN * 32;
  constexpr int lds_bytes = S * (BM + BN) * ROWB;
  static_assert(lds_bytes * OCC <= 160 * 1024, "LDS");
  auto kern = gemm_pipe_kernel<TM, TN, S, OCC, ROWB, EPI, ODT>;
  {
    const hipError_t e = allow_lds<gemm_pipe_kernel<TM, TN, S, OCC, ROWB, EPI, ODT>>(lds_bytes);
    if (e != hipSuccess) return e;
  }
  const int64_t grid = (int64_t)grid_m * p.ntn;
  if (grid <= 0) return hipSuccess;
  const unsigned nsplit = p.ksplit > 1 ? (unsigned)p.ksplit : 1u;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid, nsplit), dim3(256), lds_bytes, s, p);
  return hipGetLastError();
}

// kind 12: 128 x 256, single ring of 3 slots of 128-byte K rows
// kind 13:  64 x 256, single ring of 4 slots of 64-byte K rows, two work-groups
//           per CU (decode down GEMM: its tiles are short, so one work-group's
//           pipeline fill overlaps the other's stream)
// kind 14:  64 x 256, single ring of 4 slots of 128-byte K rows (split K allowed)
// kind 15: 256 x 256, split rings (A 2 slots + B 3 slots, 160 KB)
template <int EPI, int ODT>
static hipError_t pipe_kind(const GemmParams& p, const GemmShape& g, int grid_m, hipStream_t s) {
  switch (g.kind) {
    case 12: return launch_pipe<2, 4, 3, 1, 128, EPI, ODT>(p, grid_m, s);
    case 13: return launch_pipe<1, 4, 4, 2, 64, EPI, ODT>(p, grid_m, s);
    case 14: return launch_pipe<1, 4, 4, 1, 128, EPI, ODT>(p, grid_m, s);
    case 15: return launch_split<2, 2, 4, 4, 2, 3, EPI, ODT>(p, grid_m, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_pipe(int epi, int odt, const GemmParams& p, const GemmShape& g, int grid_m, hipStream_t s) {
  switch (epi) {
    case EPI_SWIGLU: return pipe_kind<EPI_SWIGLU, MOE_DT_BF16>(p, g, grid_m, s);
    case EPI_SCATTER: return pipe_kind<EPI_SCATTER, MOE_DT_F32>(p, g, grid_m, s);
    case EPI_COMBINE:  // the 256 x 256 split-ring kernel only, dense, bf16 out
      if (g.kind != 15 || odt != MOE_DT_BF16 || p.tiles || !p.comb.rows || !p.comb.inv || !p.comb.w || !p.comb.out ||
          p.comb.k <= 0)
        return hipErrorInvalidValue;
      return launch_split<2, 2, 4, 4, 2, 3, EPI_COMBINE, MOE_DT_BF16>(p, grid_m, s);
    default:
      if (odt == MOE_DT_F32) return pipe_kind<EPI_STORE, MOE_DT_F32>(p, g, grid_m, s);
      return pipe_kind<EPI_STORE, MOE_DT_BF16>(p, g, grid_m, s);
  }
}

}  // namespace moe
