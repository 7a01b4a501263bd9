// FP8 E4M3 grouped GEMM on 256 x 256 tiles for prefill-sized groups (MoA
// routing + FP8 inference, blog.hotdry.top, FP8 section: 1x128 activation
// tiles, 128x128 weight blocks; MoE inference walkthrough, zhiyuanblog.org/
// blog/moe-inference, §3.3: one grouped GEMM over all experts):
//
// C[p, n] = sum_kb sa[src(p), kb] * sb[n/128, kb] * sum_{k in kb} qa[src(p), k] * qb[n, k]
//
// Why 256 x 256: the 128 x 256 kernel (gemm_fp8.hip) streams each weight panel
// once per 128-row m-tile, about four times per expert at 512 rows, and its
// L1->L2 requests run at several times the algorithmic bytes.  A 256-row tile
// halves the weight-panel passes.  Its 64K fp32 accumulators need all 8 waves
// (2 per SIMD, 128 accumulator registers each), so the per-block scale fold
// must not keep a partial per accumulator: each 16 x 16 block's K step is ONE
// v_mfma 16x16x128 (the whole 128-wide scale block) into a fresh partial, and
// the partial folds into the accumulator three MFMAs later, with the product of
// the token's activation scale and the block's weight scale.
//
// Blocks run transposed: weight rows are the MFMA's first operand, so a lane's
// 4 results share one token (lane % 16) and one 128-row weight block, and the
// fold takes one scale product per block and one FMA per accumulator.
//
// Operand staging as in the other pipelined kernels: A (gathered token rows)
// and B (weight rows) stream into LDS rings of 2 and 3 slots of 32 KB by
// buffer_load ... lds; one "s_waitcnt vmcnt; s_barrier" per K step.  The
// activation scales of a step (k-block-major over the permuted rows) go to
// registers by buffer loads issued with the previous step's ring DMAs; a
// tile's weight-block scales sit in one register per wave (lane = K step, so
// K <= 64 * 128), read per step with readlane.
#include "combine_epi.h"
#include "common.h"
#include "kernels.h"
#include "lds_dma.h"

namespace moe {

namespace {

__device__ __forceinline__ f32x4 mma16_fp8(const u32x4& w0, const u32x4& w1, const u32x4& t0, const u32x4& t1) {
  const i32x8 a = {(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w, (int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w};
  const i32x8 b = {(int)t0.x, (int)t0.y, (int)t0.z, (int)t0.w, (int)t1.x, (int)t1.y, (int)t1.z, (int)t1.w};
  const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
  // formats 0/0 = E4M3 for both operands; E8M0 scale 127 = 1.0 (the fp32 block
  // scales are applied outside the MFMA)
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ float buffer_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0));
}

}  // namespace

constexpr int kBigWM = 4, kBigWN = 2, kBigNW = kBigWM * kBigWN;
constexpr int kBigBM = 256, kBigBN = 256;
constexpr int kBigTM = kBigBM / kBigWM / 16;  // 4 token blocks of 16 per wave
constexpr int kBigTN = kBigBN / kBigWN / 16;  // 8 weight blocks of 16 per wave
constexpr int kBigSA = 2, kBigSB = 3;
constexpr int kBigLds = (kBigSA * kBigBM + kBigSB * kBigBN) * 128;

template <int EPI>
__global__ __launch_bounds__(kBigNW * 64, 1) void gemm_fp8_big_kernel(GemmFp8Params p) {
  static_assert(EPI == EPI_SWIGLU || EPI == EPI_STORE || EPI == EPI_COMBINE,
                "transposed blocks: SwiGLU and row-store epilogues");
  constexpr int WM = kBigWM, WN = kBigWN, NW = kBigNW;
  constexpr int BM = kBigBM, BN = kBigBN, TM = kBigTM, TN = kBigTN;
  constexpr int SA = kBigSA, SB = kBigSB;
  constexpr int ROW = 128, CPR = 8, RPI = 8;
  constexpr int ASLOT = BM * ROW, BSLOT = BN * ROW;
  constexpr int AI = BM / RPI / NW, BI = BN / RPI / NW;  // ring DMAs per wave per step (4 + 4)
  // at the top of step kt only B(kt+1) (issued last in step kt-1) may be in flight
  constexpr int VMN = BI;
  // partials in flight: MFMA q is folded NP - 1 MFMAs later, past the MFMA
  // pipeline latency (with NP = 3 the fold waited on it)
  constexpr int NP = 4;
  static_assert(NP == 4, "the K loop folds the last three partials by name");
  static_assert(AI * RPI * NW == BM && BI * RPI * NW == BN, "tile / wave mismatch");

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
  const int64_t krow = p.K;  // bytes per A / B row
  const int nk = p.K / 128;
  const bool g2_ = p.B2 && grp == p.b2_group;
  const uint8_t* Bg = g2_ ? p.B2 : p.B + (int64_t)grp * p.b_gstride;
  const float* SBg = g2_ ? p.b2_scales : p.b_scales + (int64_t)grp * p.bs_gstride;
  const int b_nrows = (EPI == EPI_SWIGLU) ? 2 * p.N : p.N;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, p.a_nrows * krow);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bg, (int64_t)b_nrows * krow);
  // activation scales, k-block-major over the permuted rows: step kt of row p
  // at (kt * as_stride + p) * 4 bytes
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.a_scales, p.as_stride * nk * 4);
  const uint32_t sstep = (uint32_t)(p.as_stride * 4);
  // weight-block scales of this group, [rows / 128][nk]
  const __amdgpu_buffer_rsrc_t rws = make_rsrc(SBg, (int64_t)(b_nrows / 128) * nk * 4);

  // ring DMA offsets (lane l of a DMA instruction: row l / 8 of its 8-row
  // block, 16-byte chunk l % 8, XOR-swizzled)
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
      voa[i] = 0x40000000u;  // past the tile: out of range (zero fill, no traffic)
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

  // This wave's token blocks: tile rows (wm + WM i) * 16 + (lane % 16), i < TM;
  // those holding live rows form a prefix.  Weight blocks j < TN: SwiGLU gate
  // rows wn * 64 + 16 j (j < TN/2) and the matching up rows 128 + wn * 64 +
  // 16 (j - TN/2); row-store rows wn * 128 + 16 j.
  const int lt = lane & 15, lg = lane >> 4;
  int tm_live = 0;
#pragma unroll
  for (int i = 0; i < TM; ++i)
    if ((wm + WM * i) * 16 < rows) tm_live = i + 1;
  tm_live = __builtin_amdgcn_readfirstlane(tm_live);
  // scale offsets of the lane's token in each token block
  uint32_t vos[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int r = (wm + WM * i) * 16 + lt;
    vos[i] = r < rows ? (uint32_t)((r0 + r) * 4) : 0x40000000u;
  }
  auto wblock = [&](int j) {
    if constexpr (EPI == EPI_SWIGLU) return j < TN / 2 ? wn * (TN / 2) + j : WN * (TN / 2) + wn * (TN / 2) + (j - TN / 2);
    else return wn * TN + j;
  };
  // weight-scale rows of this wave: SwiGLU gate and up (two), row-store one
  int srow_g, srow_u;
  if constexpr (EPI == EPI_SWIGLU) {
    srow_g = nt;                         // gate rows nt*128 .. nt*128+127
    srow_u = p.N / 128 + nt;             // up rows N + nt*128 ..
  } else {
    srow_g = min(nt * BN + wn * 128, p.N - 1) / 128;
    srow_u = srow_g;
  }
  const uint32_t vsg = (uint32_t)(srow_g * nk * 4), vsu = (uint32_t)(srow_u * nk * 4);
  // Lane l holds step l's weight-block scales (one load per tile, read per step
  // with readlane): at most 64 K steps, which the launch checks.

  const int sw = swz<ROW>(lt);  // (row & 15) == lt for every 16-row block
  const int c0 = ((2 * lg) ^ sw) * 16, c1 = ((2 * lg + 1) ^ sw) * 16;

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};

  lds_char* const ring_a = lds3;
  lds_char* const ring_b = lds3 + SA * ASLOT;

#define MOE_BIG_ISSUE_A(kt_, slot_)                                                    \
  do {                                                                                 \
    lds_char* dst_ = ring_a + (slot_) * ASLOT;                                         \
    const uint32_t soff_ = (kt_) < nk ? (uint32_t)(kt_) * ROW : 0x80000000u;           \
    _Pragma("unroll") for (int i = 0; i < AI; ++i)                                     \
      dma16(ra, dst_ + (wave * AI + i) * 1024, voa[i], soff_);                         \
  } while (0)
#define MOE_BIG_ISSUE_B(kt_, slot_, lo_, hi_)                                          \
  do {                                                                                 \
    lds_char* dst_ = ring_b + (slot_) * BSLOT;                                         \
    const uint32_t soff_ = (kt_) < nk ? (uint32_t)(kt_) * ROW : 0x80000000u;           \
    _Pragma("unroll") for (int i = (lo_); i < (hi_); ++i)                              \
      dma16(rb, dst_ + (wave * BI + i) * 1024, vob[i], soff_);                         \
  } while (0)
// The scales of step kt_: the lane's activation scale in each token block
// (vector loads, issued with the ring DMAs, so the step's barrier wait covers
// them) and the wave's weight-block scales (gate / up, or the one row), read
// from the tile's scale registers.
#define MOE_BIG_LOAD_SCALES(kt_)                                                       \
  do {                                                                                 \
    const uint32_t so_ = (kt_) < nk ? (uint32_t)(kt_) * sstep : 0x80000000u;           \
    _Pragma("unroll") for (int i = 0; i < TM; ++i) sa_n[i] = buffer_load_f32(rs, vos[i], so_); \
    const int l_ = min((kt_), 63); /* past the last step: a value never used */        \
    sb_n[0] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wsg), l_)); \
    sb_n[1] = EPI == EPI_SWIGLU                                                        \
                  ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wsu), l_)) \
                  : sb_n[0];                                                           \
  } while (0)

  // Prologue: the tile's weight-block scales (lane l: step l), then in the
  // steady state's issue order scales(0), A(0), B(0) and B(1).
  // The scale products of the next step (activation scale x weight scale, per
  // token block: gate sg, up su) are carried from step to step; computing them
  // at the end of a step costs no wait the next barrier would not make anyway.
  float sa_n[TM], sb_n[2], sg_[TM], su_[TM];
  float wsg, wsu = 0.0f;
  wsg = buffer_load_f32(rws, lane < nk ? vsg + (uint32_t)lane * 4u : 0x80000000u, 0);
  if constexpr (EPI == EPI_SWIGLU) wsu = buffer_load_f32(rws, lane < nk ? vsu + (uint32_t)lane * 4u : 0x80000000u, 0);
  __builtin_amdgcn_sched_barrier(0);
  MOE_BIG_LOAD_SCALES(0);
  __builtin_amdgcn_sched_barrier(0);
  MOE_BIG_ISSUE_A(0, 0);
  MOE_BIG_ISSUE_B(0, 0, 0, BI);
  MOE_BIG_ISSUE_B(1, 1, 0, BI);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    sg_[i] = sa_n[i] * sb_n[0];
    su_[i] = sa_n[i] * sb_n[1];
  }

  // Fold of the partial of MFMA q (block i = q % NL, j = q / NL), in slot q % NP.
#define MOE_BIG_FOLD(q)                                                                              \
  do {                                                                                               \
    const int fj_ = (q) / NL, fi_ = (q) % NL;                                                        \
    const float sc_ = (EPI != EPI_SWIGLU || fj_ < TN / 2) ? sg_[fi_] : su_[fi_];                     \
    acc[fi_][fj_] += pt_[(q) % NP] * sc_;                                                            \
  } while (0)

  // The K loop, one 128-wide scale block per step.  Ring slots are wave-uniform
  // counters (A: kt % 2, B: kt % 3).  Per weight block j: its fragment (read one
  // block ahead), NL MFMAs (one per live token block), and the fold of the
  // partial three MFMAs back.
#define MOE_BIG_KLOOP                                                                                \
  {                                                                                                  \
    int sla = 0, slb = 0;                                                                            \
    for (int kt = 0; kt < nk; ++kt) {                                                                \
      wait_vm_barrier<VMN>();                                                                        \
      const char* sa_ = lds + sla * ASLOT;                                                           \
      const char* sb_ = lds + SA * ASLOT + slb * BSLOT;                                              \
      /* reads in the order the first MFMAs consume them (LDS returns in order): */                   \
      /* the first weight block, then the token blocks one by one */                                  \
      u32x4 ta[NL][2], wf[2][2];                                                                     \
      {                                                                                              \
        const char* r_ = sb_ + (wblock(0) * 16 + lt) * ROW;                                          \
        wf[0][0] = *(const u32x4*)(r_ + c0);                                                         \
        wf[0][1] = *(const u32x4*)(r_ + c1);                                                         \
      }                                                                                              \
      __builtin_amdgcn_sched_barrier(0);                                                             \
      _Pragma("unroll") for (int i = 0; i < NL; ++i) {                                               \
        const char* r_ = sa_ + ((wm + WM * i) * 16 + lt) * ROW;                                      \
        ta[i][0] = *(const u32x4*)(r_ + c0);                                                         \
        ta[i][1] = *(const u32x4*)(r_ + c1);                                                         \
        __builtin_amdgcn_sched_barrier(0);                                                           \
      }                                                                                              \
      const int sla_n = sla ^ 1, slb_n2 = slb == 0 ? 2 : slb - 1; /* B slot of step kt + 2 */       \
      /* the next step's scales and A tile go out before any MFMA: the scales must */                 \
      /* be in by this step's end, where the next step's scale products are formed */                 \
      MOE_BIG_LOAD_SCALES(kt + 1);                                                                   \
      MOE_BIG_ISSUE_A(kt + 1, sla_n);                                                                \
      __builtin_amdgcn_sched_barrier(0);                                                             \
      f32x4 pt_[NP];                                                                                 \
      _Pragma("unroll") for (int j = 0; j < TN; ++j) {                                               \
        if (j + 1 < TN) {                                                                            \
          const char* r_ = sb_ + (wblock(j + 1) * 16 + lt) * ROW;                                    \
          wf[(j + 1) & 1][0] = *(const u32x4*)(r_ + c0);                                             \
          wf[(j + 1) & 1][1] = *(const u32x4*)(r_ + c1);                                             \
        }                                                                                            \
        if (j == 1) MOE_BIG_ISSUE_B(kt + SB - 1, slb_n2, 0, BI / 2);                                 \
        if (j == 3) MOE_BIG_ISSUE_B(kt + SB - 1, slb_n2, BI / 2, BI);                                \
        _Pragma("unroll") for (int i = 0; i < NL; ++i) {                                             \
          const int q_ = j * NL + i;                                                                 \
          if (q_ >= NP - 1) MOE_BIG_FOLD(q_ - NP + 1);                                               \
          pt_[q_ % NP] = mma16_fp8(wf[j & 1][0], wf[j & 1][1], ta[i][0], ta[i][1]);                   \
          __builtin_amdgcn_sched_barrier(0); /* keeps each fold NP - 1 MFMAs behind */             \
        }                                                                                            \
      }                                                                                              \
      MOE_BIG_FOLD(NL * TN - 3);                                                                     \
      MOE_BIG_FOLD(NL * TN - 2);                                                                     \
      MOE_BIG_FOLD(NL * TN - 1);                                                                     \
      _Pragma("unroll") for (int i = 0; i < NL; ++i) {                                               \
        sg_[i] = sa_n[i] * sb_n[0];                                                                  \
        su_[i] = sa_n[i] * sb_n[1];                                                                  \
      }                                                                                              \
      sla = sla_n;                                                                                   \
      slb = slb == 2 ? 0 : slb + 1;                                                                  \
    }                                                                                                \
  }

  if (tm_live <= 1) {
    constexpr int NL = 1;
    MOE_BIG_KLOOP
  } else if (tm_live == 2) {
    constexpr int NL = 2;
    MOE_BIG_KLOOP
  } else if (tm_live == 3) {
    constexpr int NL = 3;
    MOE_BIG_KLOOP
  } else {
    constexpr int NL = TM;
    MOE_BIG_KLOOP
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the tail's zero-fill DMAs and scale loads
#undef MOE_BIG_KLOOP
#undef MOE_BIG_FOLD
#undef MOE_BIG_LOAD_SCALES
#undef MOE_BIG_ISSUE_A
#undef MOE_BIG_ISSUE_B

  // Epilogues.  Lane (lt, lg) of block (i, j) holds token row (wm + WM i) * 16
  // + lt and weight rows 4 lg .. 4 lg + 3 of the block.
  if constexpr (EPI == EPI_SWIGLU) {
    // h = SiLU(g) * u leaves as E4M3 codes with 1x128 scales: the tile's 128 h
    // columns are exactly one scale block of each row.  The row's amax meets
    // over the 4 lane groups (shuffles) and the WN waves (LDS); the codes go
    // through LDS to 16-byte row stores.  h is quantised from its fp32 value.
    constexpr int OC = BN / 2;
    constexpr int RQ = OC + 16;                      // LDS bytes per staged row of codes
    static_assert(OC == 128, "one 1x128 scale block per tile row");
    static_assert(BM * RQ + BM * WN * 4 <= SA * ASLOT + SB * BSLOT, "staging fits the rings");
    float* const amax_l = (float*)(lds + BM * RQ);   // [BM][WN] per-wave row maxima
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if (i >= tm_live) continue;
      float m = 0.0f;
#pragma unroll
      for (int j = 0; j < TN / 2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[i][j][e] = silu_mul(acc[i][j][e], acc[i][j + TN / 2][e]);  // h in the gate registers
          m = fmaxf(m, fabsf(acc[i][j][e]));
        }
      m = fmaxf(m, __shfl_xor(m, 16, 64));
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      if (lg == 0) amax_l[((wm + WM * i) * 16 + lt) * WN + wn] = m;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if (i >= tm_live) continue;
      const int row = (wm + WM * i) * 16 + lt;
      float m = 0.0f;
#pragma unroll
      for (int w = 0; w < WN; ++w) m = fmaxf(m, amax_l[row * WN + w]);
      const float scale = m > 0.0f ? m / 448.0f : 1.0f;
#pragma unroll
      for (int j = 0; j < TN / 2; ++j) {
        const int col = wn * (OC / WN) + j * 16 + 4 * lg;
        *(uint32_t*)(lds + row * RQ + col) =
            e4m3x4(acc[i][j][0] / scale, acc[i][j][1] / scale, acc[i][j][2] / scale, acc[i][j][3] / scale);
      }
      if (wn == 0 && lg == 0 && row < rows) p.Cs[(int64_t)nt * p.cs_stride + r0 + row] = scale;  // k-block-major
    }
    __syncthreads();
    constexpr int CPRq = OC / 16;
    for (int q = tid; q < BM * CPRq; q += NW * 64) {
      const int row = q / CPRq, ch = q % CPRq;
      if (row < rows)
        *(u32x4*)(p.Cq + (int64_t)(r0 + row) * p.N + nt * OC + ch * 16) = *(const u32x4*)(lds + row * RQ + ch * 16);
    }
  } else {
    // bf16 tile through LDS, then 16-byte row stores.  Rows padded by 16 bytes.
    constexpr int RB = BN * 2 + 16;
    static_assert(BM * RB <= SA * ASLOT + SB * BSLOT, "staging fits the rings");
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if (i >= tm_live) continue;
      const int row = (wm + WM * i) * 16 + lt;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = wblock(j) * 16 + 4 * lg;
        const uint2 w2 = {pack_bf16_rne(acc[i][j][0], acc[i][j][1]), pack_bf16_rne(acc[i][j][2], acc[i][j][3])};
        *(uint2*)(lds + row * RB + 2 * col) = w2;
      }
    }
    __syncthreads();
    constexpr int CPRo = BN / 8;
    const int cbase = nt * BN;
    if constexpr (EPI == EPI_COMBINE) {  // dense launch over tokens: the layer's combine instead of the row store
      combine_staged_tile<BM, CPRo, RB, NW * 64, 4>(p.comb, lds, SA * ASLOT + SB * BSLOT - BM * RB, r0, rows, cbase,
                                                 p.N, tid);
      return;
    }
    for (int q = tid; q < BM * CPRo; q += NW * 64) {
      const int row = q / CPRo, ch = q % CPRo;
      const int col = cbase + ch * 8;
      if (row < rows && col < p.N)
        *(u32x4*)((uint16_t*)p.C + (int64_t)(r0 + row) * p.N + col) = *(const u32x4*)(lds + row * RB + ch * 16);
    }
  }
}

template <int EPI>
static hipError_t launch_big(const GemmFp8Params& p, int grid_m, hipStream_t s) {
  static_assert(kBigLds <= 160 * 1024, "LDS");
  {
    const hipError_t e = allow_lds<gemm_fp8_big_kernel<EPI>>(kBigLds);
    if (e != hipSuccess) return e;
  }
  const int64_t grid = (int64_t)grid_m * p.ntn;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(gemm_fp8_big_kernel<EPI>, dim3((unsigned)grid), dim3(kBigNW * 64), kBigLds, s, p);
  return hipGetLastError();
}

hipError_t launch_gemm_fp8_big(int epi, const GemmFp8Params& p, int grid_m, hipStream_t s) {
  if (p.as_stride <= 0) return hipErrorInvalidValue;  // k-block-major activation scales only
  if (p.K > kFp8BigMaxK) return hipErrorInvalidValue;  // one weight-scale register per wave
  switch (epi) {
    case EPI_SWIGLU:
      if (!p.Cq || !p.Cs) return hipErrorInvalidValue;
      return launch_big<EPI_SWIGLU>(p, grid_m, s);
    case EPI_STORE: return launch_big<EPI_STORE>(p, grid_m, s);
    case EPI_COMBINE:
      if (!p.comb.rows || !p.comb.inv || !p.comb.w || !p.comb.out || p.comb.k <= 0 || p.tiles)
        return hipErrorInvalidValue;  // dense launches over tokens only
      return launch_big<EPI_COMBINE>(p, grid_m, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
