// Grouped FP8 E4M3 GEMMs with fine-grained fp32 scales (MoA routing + FP8
// inference, blog.hotdry.top, FP8 section: E4M3, 1x128 activation tiles and
// 128x128 weight blocks; V3 lab page, gsyq.cn/news/313569, §3 infer.toml
// weight_block_size [128, 128]).
//
// C[p, n] = sum_kb sa[src(p), kb] * sb[n/128, kb] * sum_{k in kb} qa[src(p), k] * qb[n, k]
//
// One K step is exactly one 128-wide scale block: the two 32x32x64 MFMAs of a
// step accumulate the unscaled partial product in fp32 and the partial is then
// folded into the accumulator with the product of the row's activation scale
// (staged in LDS) and the tile's weight-block scale.  Operand staging, the
// m-tile list and the work-group mapping are those of the bf16 kernel.
#include "common.h"
#include "kernels.h"
#include "lds_dma.h"

namespace moe {

__device__ __forceinline__ f32x16 mma_fp8(const u32x4& a0, const u32x4& a1, const u32x4& b0, const u32x4& b1,
                                          f32x16 c) {
  const i32x8 a = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
  const i32x8 b = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
  // formats 0/0 = E4M3 for both operands; E8M0 scale 127 = 1.0 (the fp32 block
  // scales are applied outside the MFMA)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

typedef __attribute__((address_space(4))) const float cfloat;

// ---------------------------------------------------------------------------
// Pipelined FP8 kernel.  One K step = one 128-wide scale block = 128 bytes of
// every A and B row, streamed straight into LDS rings (A: SA slots, B: SB slots)
// by buffer_load ... lds, as in the bf16 split-ring kernel.  The A slot also
// carries the step's activation scales of the tile's rows (one 4-byte DMA lane
// per row).  Weight-block scales are wave-uniform scalar loads, fetched one step
// ahead.  Per step and 32x32 block: two 32x32x64 MFMAs into a zeroed partial,
// then acc += partial * (sa[row] * sb); the SwiGLU and row-store instances run
// each block transposed so that one scale product serves a lane's 16 results.
template <int WM, int WN, int TM, int TN, int SA, int SB, int EPI>
__global__ __launch_bounds__(WM * WN * 64, 1) void gemm_fp8_split_kernel(GemmFp8Params p) {
  constexpr int NW = WM * WN;
  constexpr int BM = WM * TM * 32;
  constexpr int BN = WN * TN * 32;
  constexpr int ROW = 128, CPR = 8, RPI = 8;
  constexpr int ADATA = BM * ROW;
  constexpr int ASLOT = ADATA + NW * 256;     // + activation scales: 64 lanes x 4 B per wave
  constexpr int BSLOT = BN * ROW;
  constexpr int AI = BM / RPI / NW, BI = BN / RPI / NW;
  constexpr int RW = BM / NW;                 // scale rows per wave (16, 32 or 64)
  constexpr int AL = AI + 1;                  // A instructions per wave per step (data + scales)
  constexpr int LI = AL + BI;
  constexpr int VMN = SB > SA ? BI + (SA - 2) * LI : (SA - 2) * LI;
  static_assert(AI * RPI * NW == BM && BI * RPI * NW == BN, "tile / wave mismatch");
  static_assert(RW == 16 || RW == 32 || RW == 64, "scale rows per wave");
  static_assert(SA >= 2 && SB >= SA && VMN < 64, "ring depths");
  static_assert(EPI != EPI_SWIGLU || TN % 2 == 0, "SwiGLU pairs gate and up tiles");
  // The SwiGLU and row-store instances compute each 32x32 block transposed
  // (weight rows as the MFMA's first operand): a lane's 16 results then share
  // one token and one weight block, so the fold takes one scale product per
  // block and one FMA per accumulator instead of two operations per
  // accumulator.  The scatter instance keeps token rows first, so that its
  // fp32 atomics cover 32 consecutive columns per row.
  constexpr bool TR = EPI != EPI_SCATTER;

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
  const int nkb = p.K / 128;
  const bool g2_ = p.B2 && grp == p.b2_group;
  const uint8_t* Bg = g2_ ? p.B2 : p.B + (int64_t)grp * p.b_gstride;
  // weight scales are read-only for the kernel's lifetime: constant address
  // space, so the wave-uniform loads below become scalar loads
  const cfloat* SBg = (const cfloat*)(g2_ ? p.b2_scales : p.b_scales + (int64_t)grp * p.bs_gstride);
  const int b_nrows = (EPI == EPI_SWIGLU) ? 2 * p.N : p.N;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, p.a_nrows * krow);
  // activation scales: k-block-major over permuted rows (one contiguous run per
  // row tile and step), or row-major over source rows
  const bool st = p.as_stride > 0;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.a_scales, (st ? p.as_stride : p.a_nrows) * nkb * 4);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bg, (int64_t)b_nrows * krow);

  const int lrow = lane / CPR, lslot = lane % CPR;
  uint32_t voa[AI], vob[BI], vos;
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int r = (wave * AI + i) * RPI + lrow;
    const int chunk = lslot ^ swz<ROW>(r);
    if (r < rows) {
      const int src = p.a_rows ? p.a_rows[r0 + r] : r0 + r;
      voa[i] = (uint32_t)((int64_t)src * krow + chunk * 16);
    } else {
      voa[i] = 0x40000000u;
    }
  }
  {
    const int r = wave * RW + lane;  // lanes past RW fill the wave's spare scale words
    if (lane < RW && r < rows) {
      if (st) {
        vos = (uint32_t)((int64_t)(r0 + r) * 4);
      } else {
        const int src = p.a_rows ? p.a_rows[r0 + r] : r0 + r;
        vos = (uint32_t)((int64_t)src * nkb * 4);
      }
    } else {
      vos = 0x40000000u;
    }
  }
  const uint32_t sstep = st ? (uint32_t)(p.as_stride * 4) : 4u;  // scale bytes between K steps
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

  auto bblock = [&](int tn) {
    if constexpr (EPI == EPI_SWIGLU)
      return tn < TN / 2 ? wn * (TN / 2) + tn : WN * (TN / 2) + wn * (TN / 2) + (tn - TN / 2);
    else
      return wn * TN + tn;
  };
  // weight-block row (of 128 output rows) of each wave column block
  int sbrow[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int bb = bblock(j) * 32;
    int wrow;
    if constexpr (EPI == EPI_SWIGLU) {
      const int j0 = min(nt * (BN / 2) + (bb % (BN / 2)), p.N - 1);
      wrow = (bb < BN / 2) ? j0 : p.N + j0;
    } else {
      wrow = min(nt * BN + bb, p.N - 1);
    }
    sbrow[j] = __builtin_amdgcn_readfirstlane(wrow / 128);
  }

  const int nk = nkb;
  lds_char* const ring_a = lds3;
  lds_char* const ring_b = lds3 + SA * ASLOT;

#define MOE_F8_ISSUE_A(kt_, lo_, hi_, scales_)                                         \
  do {                                                                                 \
    lds_char* slot_ = ring_a + ((kt_) % SA) * ASLOT;                                   \
    const uint32_t soff_ = (kt_) < nk ? (uint32_t)(kt_) * ROW : 0x80000000u;           \
    _Pragma("unroll") for (int i = (lo_); i < (hi_); ++i)                              \
      dma16(ra, slot_ + (wave * AI + i) * 1024, voa[i], soff_);                        \
    if (scales_) {                                                                     \
      const uint32_t so4_ = (kt_) < nk ? (uint32_t)(kt_) * sstep : 0x80000000u;        \
      dma4(rs, slot_ + ADATA + wave * 256, vos, so4_);                                 \
    }                                                                                  \
  } while (0)
#define MOE_F8_ISSUE_B(kt_, lo_, hi_)                                                  \
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

  int tm_live = 0;
#pragma unroll
  for (int i = 0; i < TM; ++i)
    if ((wm + WM * i) * 32 < rows) tm_live = i + 1;
  tm_live = __builtin_amdgcn_readfirstlane(tm_live);

  const int lr = lane & 31, hi = lane >> 5;
  const int sw = swz<ROW>(lr);

#pragma unroll
  for (int v = 1 - SB; v < 0; ++v) {
    if (v + SA - 1 >= 0) MOE_F8_ISSUE_A(v + SA - 1, 0, AI, true);
    if (v + SB - 1 >= 0) MOE_F8_ISSUE_B(v + SB - 1, 0, BI);
  }

  // weight-block scales of step 0; each step fetches the next step's
  float sbn[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) sbn[j] = SBg[(int64_t)sbrow[j] * nkb];

  // Fragment of sub-step st (K 64*st .. 64*st+63): lanes 0-31 take 16-byte chunks
  // {4st, 4st+1}, lanes 32-63 take {4st+2, 4st+3} of their row.
#define MOE_F8_READ(st_)                                                                            \
  do {                                                                                              \
    const int c0_ = ((4 * (st_) + 2 * hi) ^ sw) * 16, c1_ = ((4 * (st_) + 2 * hi + 1) ^ sw) * 16;  \
    _Pragma("unroll") for (int j = 0; j < TN; ++j) {                                                \
      const char* r_ = sb_ + (bblock(j) * 32 + lr) * ROW;                                           \
      b[st_][j][0] = *(const u32x4*)(r_ + c0_);                                                     \
      b[st_][j][1] = *(const u32x4*)(r_ + c1_);                                                     \
    }                                                                                               \
    _Pragma("unroll") for (int i = 0; i < NL; ++i) {                                                \
      const char* r_ = sa_ + ((wm + WM * i) * 32 + lr) * ROW;                                        \
      a[st_][i][0] = *(const u32x4*)(r_ + c0_);                                                     \
      a[st_][i][1] = *(const u32x4*)(r_ + c1_);                                                     \
    }                                                                                               \
  } while (0)

// One K step: every LDS read of the step (both sub-steps' fragments and the
// activation scales) first, so none of them follows a ring DMA in program order;
// then A's ring DMAs with the first sub-step's MFMAs, B's with the second's and
// the scaled fold of the partials.  The fold (two VALU operations per
// accumulator and 128-wide K block) costs about as long as the block's MFMAs,
// and the two waves of a SIMD (rows wm = 0 and wm = 1 of one column group)
// leave each step's barrier together.  So the wm = 1 waves run the loop
// rotated (ROT): they fold step kt - 1's partials right after step kt's
// barrier, while their SIMD partner runs step kt's MFMAs, and run their own
// MFMAs while the partner folds.  The partials and scales of step kt - 1 stay
// in the same registers across the back edge; no extra registers are needed.
#define MOE_F8_FOLD()                                                                                \
  _Pragma("unroll") for (int i = 0; i < NL; ++i)                                                     \
    _Pragma("unroll") for (int j = 0; j < TN; ++j) {                                                 \
      if constexpr (TR) {                                                                            \
        const float s_ = sa[i][0] * sbk[j];                                                          \
        _Pragma("unroll") for (int e = 0; e < 16; ++e) acc[i][j][e] += part[i][j][e] * s_;          \
      } else {                                                                                       \
        _Pragma("unroll") for (int e = 0; e < 16; ++e)                                               \
          acc[i][j][e] += part[i][j][e] * (sa[i][e] * sbk[j]);                                       \
      }                                                                                              \
    }
// Step kt = kt0 + OFF_ of the K loop, in ring slot SLOT_ (= kt % SA = kt % SB).
// Unrolled by the ring depth, the slot is a compile-time constant and the
// per-lane LDS addresses of each slot are loop invariant.
#define MOE_F8_STEP(OFF_, SLOT_)                                                                     \
  if (kt0 + (OFF_) < nk) {                                                                           \
    const int kt = kt0 + (OFF_);                                                                     \
    wait_vm_barrier<VMN>();                                                                          \
    const char* sa_ = lds + (SLOT_) * ASLOT;                                                         \
    const char* sb_ = lds + SA * ASLOT + (SLOT_) * BSLOT;                                            \
    float sbc[TN];                                                                                   \
    _Pragma("unroll") for (int j = 0; j < TN; ++j) sbc[j] = sbn[j];                                  \
    {                                                                                                \
      const int kn_ = kt + 1 < nk ? kt + 1 : kt;                                                     \
      _Pragma("unroll") for (int j = 0; j < TN; ++j) sbn[j] = SBg[(int64_t)sbrow[j] * nkb + kn_];    \
    }                                                                                                \
    u32x4 a[2][NL][2], b[2][TN][2];                                                                  \
    MOE_F8_READ(0);                                                                                  \
    MOE_F8_READ(1);                                                                                  \
    if (ROT && kt > 0) MOE_F8_FOLD();                                                                \
    _Pragma("unroll") for (int j = 0; j < TN; ++j) sbk[j] = sbc[j];                                  \
    /* this step's activation scales: transposed, the lane's token (row lr of each */               \
    /* block); else rows 8*(e/4) + 4*hi + (e%4) of each block */                                     \
    _Pragma("unroll") for (int i = 0; i < NL; ++i) {                                                 \
      if constexpr (TR) {                                                                            \
        const int r_ = (wm + WM * i) * 32 + lr;                                                      \
        sa[i][0] = __builtin_bit_cast(float, *(const uint32_t*)(sa_ + ADATA + ((r_ / RW) * 64 + r_ % RW) * 4)); \
      } else {                                                                                       \
        _Pragma("unroll") for (int q = 0; q < 4; ++q) {                                              \
          const int r_ = (wm + WM * i) * 32 + 8 * q + 4 * hi;                                         \
          /* read as u32x4 like the fragments (no wait on the ring DMAs in flight) */              \
          const u32x4 u_ = *(const u32x4*)(sa_ + ADATA + ((r_ / RW) * 64 + r_ % RW) * 4);           \
          const float4 v_ = __builtin_bit_cast(float4, u_);                                          \
          sa[i][4 * q + 0] = v_.x; sa[i][4 * q + 1] = v_.y; sa[i][4 * q + 2] = v_.z; sa[i][4 * q + 3] = v_.w; \
        }                                                                                            \
      }                                                                                              \
    }                                                                                                \
    __builtin_amdgcn_sched_barrier(0);                                                               \
    MOE_F8_ISSUE_A(kt + SA - 1, 0, AI, true);                                                        \
    _Pragma("unroll") for (int i = 0; i < NL; ++i)                                                   \
      _Pragma("unroll") for (int j = 0; j < TN; ++j) {                                               \
        f32x16 z_;                                                                                   \
        _Pragma("unroll") for (int e = 0; e < 16; ++e) z_[e] = 0.0f;                                 \
        part[i][j] = TR ? mma_fp8(b[0][j][0], b[0][j][1], a[0][i][0], a[0][i][1], z_)                \
                        : mma_fp8(a[0][i][0], a[0][i][1], b[0][j][0], b[0][j][1], z_);               \
      }                                                                                              \
    sub_schedule<0, NL * TN, 0, AL>();                                                               \
    __builtin_amdgcn_sched_barrier(0);                                                               \
    MOE_F8_ISSUE_B(kt + SB - 1, 0, BI);                                                              \
    _Pragma("unroll") for (int i = 0; i < NL; ++i)                                                   \
      _Pragma("unroll") for (int j = 0; j < TN; ++j)                                                 \
        part[i][j] = TR ? mma_fp8(b[1][j][0], b[1][j][1], a[1][i][0], a[1][i][1], part[i][j])        \
                        : mma_fp8(a[1][i][0], a[1][i][1], b[1][j][0], b[1][j][1], part[i][j]);       \
    sub_schedule<0, NL * TN, 0, BI>();                                                               \
    if (!ROT) MOE_F8_FOLD();                                                                         \
  }
#define MOE_F8_KLOOP                                                                                 \
  {                                                                                                  \
    static_assert(SA == SB && SA == 3, "the unrolled K loop walks both rings' 3 slots together");    \
    f32x16 part[NL][TN];                                                                             \
    float sa[NL][TR ? 1 : 16], sbk[TN];                                                              \
    for (int kt0 = 0; kt0 < nk; kt0 += 3) {                                                          \
      MOE_F8_STEP(0, 0)                                                                              \
      MOE_F8_STEP(1, 1)                                                                              \
      MOE_F8_STEP(2, 2)                                                                              \
    }                                                                                                \
    if (ROT && nk > 0) MOE_F8_FOLD();                                                                \
  }

  if (tm_live <= 1) {
    constexpr int NL = 1;
    if (wm == 1) {
      constexpr bool ROT = true;
      MOE_F8_KLOOP
    } else {
      constexpr bool ROT = false;
      MOE_F8_KLOOP
    }
  } else {
    constexpr int NL = TM;
    if (wm == 1) {
      constexpr bool ROT = true;
      MOE_F8_KLOOP
    } else {
      constexpr bool ROT = false;
      MOE_F8_KLOOP
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#undef MOE_F8_KLOOP
#undef MOE_F8_STEP
#undef MOE_F8_FOLD
#undef MOE_F8_READ
#undef MOE_F8_ISSUE_A
#undef MOE_F8_ISSUE_B

  if constexpr (EPI == EPI_SWIGLU) {
    // h = SiLU(g) * u leaves as E4M3 codes with their 1x128 scales (the
    // activation rule of the down GEMM's input): the tile's 128 output columns
    // are exactly one scale block of each row.  Per row, the amax meets over the
    // lane pair (hi) and the WN waves of the row (through LDS); then the codes go
    // through LDS to 16-byte row stores.  h is quantised from its fp32 value.
    constexpr int OC = BN / 2;
    constexpr int JO = TN / 2;
    constexpr int RQ = OC + 16;                        // LDS bytes per staged row of codes
    static_assert(OC == 128, "one 1x128 scale block per tile row");
    static_assert(TR, "the epilogue reads transposed blocks");
    static_assert(BM * RQ + BM * WN * 4 <= SA * ASLOT + SB * BSLOT, "staging fits the rings");
    float* const amax_l = (float*)(lds + BM * RQ);     // [BM][WN] per-wave row maxima
    __syncthreads();
    float hv[TM][JO][16];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if (i >= tm_live) continue;
      float m = 0.0f;
#pragma unroll
      for (int jo = 0; jo < JO; ++jo)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          hv[i][jo][e] = silu_mul(acc[i][jo][e], acc[i][jo + TN / 2][e]);
          m = fmaxf(m, fabsf(hv[i][jo][e]));
        }
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      if (hi == 0) amax_l[((wm + WM * i) * 32 + lr) * WN + wn] = m;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if (i >= tm_live) continue;
      const int row = (wm + WM * i) * 32 + lr;
      float m = 0.0f;
#pragma unroll
      for (int w = 0; w < WN; ++w) m = fmaxf(m, amax_l[row * WN + w]);
      const float scale = m > 0.0f ? m / 448.0f : 1.0f;
#pragma unroll
      for (int jo = 0; jo < JO; ++jo) {
        const int cb = (wn * (TN / 2) + jo) * 32 + 4 * hi;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          *(uint32_t*)(lds + row * RQ + cb + 8 * q) =
              e4m3x4(hv[i][jo][4 * q] / scale, hv[i][jo][4 * q + 1] / scale, hv[i][jo][4 * q + 2] / scale,
                     hv[i][jo][4 * q + 3] / scale);
        }
      }
      if (wn == 0 && hi == 0 && row < rows) {
        p.Cs[(int64_t)nt * p.cs_stride + r0 + row] = scale;  // k-block-major
      }
    }
    __syncthreads();
    constexpr int CPRq = OC / 16;
    for (int q = tid; q < BM * CPRq; q += NW * 64) {
      const int row = q / CPRq, ch = q % CPRq;
      if (row < rows)
        *(u32x4*)(p.Cq + (int64_t)(r0 + row) * p.N + nt * OC + ch * 16) = *(const u32x4*)(lds + row * RQ + ch * 16);
    }
    return;
  }

  if constexpr (EPI == EPI_STORE) {
    // bf16 tile through LDS (the rings are idle now) and 16-byte row stores.
    // Rows are padded by 16 bytes.  Transposed blocks: lane (lr, hi) holds token
    // row lr of the block and columns 8q + 4hi .. 8q + 4hi + 3 in results
    // 4q .. 4q + 3, one 8-byte LDS write per q.
    constexpr int RB = BN * 2 + 16;
    static_assert(BM * RB <= SA * ASLOT + SB * BSLOT, "staging fits the rings");
    static_assert(TR, "the staged epilogue reads transposed blocks");
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if (i >= tm_live) continue;
      const int row = (wm + WM * i) * 32 + lr;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int cb = bblock(j) * 32 + 4 * hi;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint2 w2 = {pack_bf16_rne(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                            pack_bf16_rne(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3])};
          *(uint2*)(lds + row * RB + 2 * (cb + 8 * q)) = w2;
        }
      }
    }
    __syncthreads();
    constexpr int CPRo = BN / 8;
    const int c0 = nt * BN;
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
            ((uint16_t*)p.C)[(int64_t)prow * p.N + col] =
                (uint16_t)f32_to_bf16_bits(silu_mul(acc[i][j][e], acc[i][j + TN / 2][e]));
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
          if (col < p.N) ((uint16_t*)p.C)[(int64_t)prow * p.N + col] = (uint16_t)f32_to_bf16_bits(acc[i][j][e]);
        }
      }
    }
  }
}

template <int WM, int WN, int TM, int TN, int SA, int SB, int EPI>
static hipError_t launch8_split(const GemmFp8Params& p, int grid_m, hipStream_t s) {
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  constexpr int lds_bytes = SA * (BM * 128 + WM * WN * 256) + SB * BN * 128;
  static_assert(lds_bytes <= 160 * 1024, "LDS");
  auto kern = gemm_fp8_split_kernel<WM, WN, TM, TN, SA, SB, EPI>;
  {
    const hipError_t e = allow_lds<gemm_fp8_split_kernel<WM, WN, TM, TN, SA, SB, EPI>>(lds_bytes);
    if (e != hipSuccess) return e;
  }
  const int64_t grid = (int64_t)grid_m * p.ntn;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(WM * WN * 64), lds_bytes, s, p);
  return hipGetLastError();
}

// kind 1: pipelined 128 x 256 (A and B buffers addressed with 31-bit offsets;
// the ABI bounds both below 2^31 bytes), 2 x 4 waves of 64 x 64: two waves per
// SIMD, so one wave's scaled fold (VALU) overlaps the other's MFMAs.
// kind 2: 256 x 256 (gemm_fp8_big.hip) for groups of 128 rows and more on
// average, with the SwiGLU or row-store epilogue: half the weight-panel passes
// per group.  The scatter-add epilogue keeps kind 1 (its fp32 atomics want
// token rows first).
#ifndef MOE_FP8_BIG_MIN_ROWS
#define MOE_FP8_BIG_MIN_ROWS 128
#endif
GemmShape gemm_fp8_shape(int rows_hint, int epi, int K) {
  GemmShape g;
  // the 256 x 256 kernel keeps a tile's weight-block scales in one register
  // per wave (one 128-wide K step per lane): K <= 64 * 128
  const bool big = MOE_FP8_BIG_MIN_ROWS > 0 && rows_hint >= MOE_FP8_BIG_MIN_ROWS && epi != EPI_SCATTER &&
                   K <= kFp8BigMaxK;
  g.kind = big ? 2 : 1;
  g.bm = big ? 256 : 128;
  g.bn = 256;
  return g;
}

hipError_t launch_gemm_fp8(int epi, const GemmFp8Params& p, const GemmShape& g, int grid_m, hipStream_t s) {
  if (g.kind == 2) return launch_gemm_fp8_big(epi, p, grid_m, s);
  if (g.kind != 1) return hipErrorInvalidValue;
  if (epi == EPI_SWIGLU && (!p.Cq || !p.Cs)) return hipErrorInvalidValue;  // writes quantised h only
  switch (epi) {
    case EPI_SWIGLU: return launch8_split<2, 4, 2, 2, 3, 3, EPI_SWIGLU>(p, grid_m, s);
    case EPI_SCATTER: return launch8_split<2, 4, 2, 2, 3, 3, EPI_SCATTER>(p, grid_m, s);
    case EPI_STORE: return launch8_split<2, 4, 2, 2, 3, 3, EPI_STORE>(p, grid_m, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
