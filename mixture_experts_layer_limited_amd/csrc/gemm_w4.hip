// Grouped expert GEMMs with 4-bit weights and bf16 activations (W4A16; the
// 4-bit expert-weight format of the MoE inference walkthrough,
// zhiyuanblog.org/blog/moe-inference, §8 quantisation table), for the
// grouped-GEMM step of the same walkthrough (§3.3):
//
//   C[p, n] = sum_g s[g, n] * sum_{k in group g} A[src(p), k] * q[n, k]
//
// with q the signed 4-bit codes (two per byte, the even column in the low
// nibble) and s one fp32 scale per weight row and 128 columns, stored
// group-major.
//
// Design (decode-sized groups, where the weight stream is the whole cost):
//   * tiles of 16 rows (decode experts hold a few rows each);
//   * one K step is two scale groups (256 columns); the packed codes (BN rows
//     x 128 bytes: one whole cache line per weight row) with the 2 x BN
//     scales of the step (two contiguous runs), and the activation rows (16 x
//     512 bytes), stream straight from memory into LDS rings with
//     buffer_load ... lds: the weight ring SB - 1 steps ahead of the MFMAs,
//     the activation ring (mostly L2 hits) SA - 1 steps ahead, so the LDS goes
//     to weight bytes in flight;
//   * codes widen to bf16 with two bit operations per pair: a nibble n, its
//     sign bit flipped (u = n ^ 8 = q + 8), or-ed under the bf16 pattern of
//     128 reads as 128 + u = 136 + q exactly; a pair of nibbles four apart in
//     one dword widens in one and + xor, so the B fragment holds the columns
//     of its 8-column run in the order 0,4,1,5,2,6,3,7 and the activation
//     fragment is permuted to match (a dot product does not see the order);
//   * the offset is removed exactly inside the MFMA chain: each group's
//     accumulation starts from A * (-136) (the same activation fragments
//     against a constant bf16 -136), so the chain ends at sum A*q in fp32;
//     the group's scale then folds into the fp32 accumulator (one FMA per
//     element and group);
//   * the MFMAs are 16 x 16 x 32 (one row block per tile);
//   * 8 waves share the tile's 16 activation rows: wave w owns 2 TN 16-column
//     blocks of weight rows (SwiGLU: TN gate blocks and the matching up
//     blocks, so the SiLU * up epilogue needs no data exchange between
//     column blocks) for group w / 4 of every step; the two waves of a
//     column block share a SIMD, where one's MFMAs overlap the other's code
//     widening, and their sums meet once, through LDS, before the epilogue.
#include "common.h"
#include "kernels.h"
#include "lds_dma.h"

namespace moe {

namespace {

__device__ __forceinline__ float silu_mul_w4(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// Eight 4-bit codes (code i in bits 4i..4i+3 of w) as bf16 values 136 + q_i,
// pairs (0,4), (1,5), (2,6), (3,7).
__device__ __forceinline__ u32x4 widen_w4(uint32_t w) {
  u32x4 r;
  r[0] = (w & 0x000F000Fu) ^ 0x43084308u;
  r[1] = ((w >> 4) & 0x000F000Fu) ^ 0x43084308u;
  r[2] = ((w >> 8) & 0x000F000Fu) ^ 0x43084308u;
  r[3] = ((w >> 12) & 0x000F000Fu) ^ 0x43084308u;
  return r;
}

// Eight consecutive bf16 activations (pairs (0,1), (2,3), (4,5), (6,7)) in
// the order of widen_w4: pairs (0,4), (1,5), (2,6), (3,7).  v_perm_b32 picks
// bytes 0-3 from its second operand and 4-7 from its first.
__device__ __forceinline__ u32x4 reorder_a(u32x4 a) {
  u32x4 r;
  r[0] = __builtin_amdgcn_perm(a[2], a[0], 0x05040100u);
  r[1] = __builtin_amdgcn_perm(a[2], a[0], 0x07060302u);
  r[2] = __builtin_amdgcn_perm(a[3], a[1], 0x05040100u);
  r[3] = __builtin_amdgcn_perm(a[3], a[1], 0x07060302u);
  return r;
}

}  // namespace

// Two waves per SIMD (256 registers each): the MFMAs write VGPRs and the
// scale fold reads them without copies.  LDS holds one work-group per CU.
template <int TN, int SA, int SB, int EPI, int ODT>
__global__ __launch_bounds__(512, 1) void gemm_w4_kernel(GemmW4Params p) {
  constexpr int NW = 8, WN = 4, BM = 16, BN = WN * TN * 32;
  constexpr int G = NW / WN;                      // scale groups per K step, one per wave set
  constexpr int KS = 128 * G;                     // K per step
  constexpr int AROW = KS * 2, BROW = KS / 2;     // bytes per row per step: bf16 / packed 4-bit
  constexpr int ACH = AROW / 16, BCH = BROW / 16; // 16-byte chunks per row
  constexpr int ABYTES = BM * AROW, BBYTES = BN * BROW, SBYTES = G * BN * 4;
  constexpr int ASLOT = ABYTES, BSLOT = BBYTES + SBYTES;  // activation slot; codes + scales slot
  constexpr int BRING = SA * ASLOT;                       // the weight ring follows the activation ring
  constexpr int AI = ABYTES / 1024 / NW;          // 16-byte-per-lane DMAs per wave per slot
  constexpr int BI = BBYTES / 1024 / NW;
  constexpr int SI = SBYTES / 256 / NW;           // 4-byte-per-lane DMAs (scales)
  constexpr int LI = AI + BI + SI;
  // At the top of step kt the last DMAs issued are A(kt) then B(kt + SB - SA);
  // B(kt) went out SB - SA steps before A(kt), so waiting for A(kt) covers it.
  constexpr int VMN = (BI + SI) + (SA - 2) * LI;
  static_assert(AI * 1024 * NW == ABYTES && BI * 1024 * NW == BBYTES && SI * 256 * NW == SBYTES, "tile / wave");
  static_assert(ACH == 32 && BCH == 8 && BN % 64 == 0, "row layout");
  static_assert(EPI != EPI_SWIGLU || TN % 2 == 0, "SwiGLU pairs gate and up blocks");
  static_assert(SA >= 2 && SB >= SA && VMN < 64, "ring depths");

  extern __shared__ __attribute__((aligned(16))) char lds[];
  lds_char* const lds3 = (lds_char*)lds;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % WN, kset = wave / WN;  // column blocks and scale group of this wave

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
  const int64_t arow = (int64_t)p.K * 2;  // bytes per activation row
  const int64_t brow = p.K / 2;           // bytes per packed weight row
  const int ngroups = p.K / 128;          // scale groups per row
  const int nk = (ngroups + G - 1) / G;   // steps; an odd group count leaves the last step half full
  const bool second = p.B2 && grp == p.b2_group;
  const uint8_t* Bg = second ? p.B2 : p.B + (int64_t)grp * p.b_gstride;
  const float* Sg = second ? p.b2_scales : p.b_scales + (int64_t)grp * p.bs_gstride;
  const int b_nrows = (EPI == EPI_SWIGLU) ? 2 * p.N : p.N;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, p.a_nrows * arow);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bg, (int64_t)b_nrows * brow);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(Sg, (int64_t)ngroups * b_nrows * 4);

  // Weight row of tile row r (clamped: rows past N are computed and dropped).
  auto wrow_of = [&](int r) {
    if constexpr (EPI == EPI_SWIGLU) {
      const int j = min(nt * (BN / 2) + (r % (BN / 2)), p.N - 1);
      return (r < BN / 2) ? j : p.N + j;
    } else {
      return min(nt * BN + r, p.N - 1);
    }
  };

  // Per-lane source offsets, fixed over K.  A: 2 rows of 32 chunks per DMA,
  // chunk c of row r stored at chunk c ^ (r & 15); B: 8 rows of 8 chunks,
  // chunk c at c ^ swz<128>(r); scales: 64 consecutive entries of one group
  // per DMA, 4 bytes each (the slot holds group 0's BN scales, then group 1's).
  uint32_t voa[AI], vob[BI], vos[SI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int r = (wave * AI + i) * (64 / ACH) + lane / ACH;
    const int chunk = (lane % ACH) ^ (r & 15);
    if (r < rows) {
      const int src = p.a_rows ? p.a_rows[r0 + r] : r0 + r;
      voa[i] = (uint32_t)((int64_t)src * arow + chunk * 16);
    } else {
      voa[i] = 0x40000000u;  // past the tile's rows: out of range (zero fill, no traffic) or harmless
    }
  }
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int r = (wave * BI + i) * (64 / BCH) + lane / BCH;
    const int chunk = (lane % BCH) ^ swz<128>(r);
    vob[i] = (uint32_t)((int64_t)wrow_of(r) * brow + chunk * 16);
  }
#pragma unroll
  for (int i = 0; i < SI; ++i) {
    const int idx = (wave * SI + i) * 64 + lane;
    vos[i] = (uint32_t)(((int64_t)(idx / BN) * b_nrows + wrow_of(idx % BN)) * 4);
  }

  // Step kt of each ring; past the last step every offset is out of range
  // (zero fill, no traffic), so the instruction count per step stays fixed.
  // In a half-full last step the second group's bytes are not used.
#define MOE_W4_ISSUE_A(kt_)                                                                        \
  do {                                                                                             \
    lds_char* slot_ = lds3 + ((kt_) % SA) * ASLOT;                                                 \
    const uint32_t sa_ = (kt_) < nk ? (uint32_t)(kt_) * AROW : 0x80000000u;                        \
    _Pragma("unroll") for (int i = 0; i < AI; ++i) dma16(ra, slot_ + (wave * AI + i) * 1024, voa[i], sa_); \
  } while (0)
#define MOE_W4_ISSUE_B(kt_)                                                                        \
  do {                                                                                             \
    lds_char* slot_ = lds3 + BRING + ((kt_) % SB) * BSLOT;                                         \
    const bool live_ = (kt_) < nk;                                                                 \
    const uint32_t sb_ = live_ ? (uint32_t)(kt_) * BROW : 0x80000000u;                             \
    const uint32_t ss_ = live_ ? (uint32_t)(kt_) * G * b_nrows * 4 : 0x80000000u;                  \
    _Pragma("unroll") for (int i = 0; i < BI; ++i)                                                 \
      dma16(rb, slot_ + (wave * BI + i) * 1024, vob[i], sb_);                                      \
    _Pragma("unroll") for (int i = 0; i < SI; ++i)                                                 \
      dma4(rs, slot_ + BBYTES + (wave * SI + i) * 256, vos[i], ss_);                               \
  } while (0)

  // 16-column blocks: NB per wave (SwiGLU: NB/2 gate blocks, then the
  // matching up blocks); first B-tile row of block j of this wave.
  constexpr int NB = 2 * TN;
  auto bbase = [&](int j) {
    if constexpr (EPI == EPI_SWIGLU)
      return j < NB / 2 ? (wn * (NB / 2) + j) * 16 : BN / 2 + (wn * (NB / 2) + (j - NB / 2)) * 16;
    else
      return (wn * NB + j) * 16;
  };

  // 16 x 16 x 32 MFMA lanes: l = 16 q + n takes activation row n and weight
  // row n of a block, columns 8 q .. 8 q + 7 of each 32-column sub-step.
  const int n16 = lane & 15, q = lane >> 4;
  const u32x4 kneg = {0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u};  // bf16 -136 everywhere

  f32x4 acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) acc[j] = {0.0f, 0.0f, 0.0f, 0.0f};

  // The issues of the SB - 1 steps before step 0, in steady-state order.
#pragma unroll
  for (int t = -(SB - 1); t < 0; ++t) {
    if (t + SA - 1 >= 0) MOE_W4_ISSUE_A(t + SA - 1);
    MOE_W4_ISSUE_B(t + SB - 1);
  }

  for (int kt = 0; kt < nk; ++kt) {
    wait_vm_barrier<VMN>();  // step kt landed; every wave is done with step kt - 1
    const char* aslot = lds + (kt % SA) * ASLOT;
    const char* bslot = lds + BRING + (kt % SB) * BSLOT;
    const int g = kset;
    const bool live = kt * G + g < ngroups;  // wave-uniform: false only in a half-full last step
    // Lane (n, q) takes columns [32 q, 32 q + 32) of group g: activation
    // chunk 16 g + 4 q + st and code dword st (of chunk 4 g + q) for sub-step st.
    u32x4 a[4];
    u32x4 b[NB];
    float sc[NB];
    if (live) {
#pragma unroll
      for (int st = 0; st < 4; ++st)
        a[st] = *(const u32x4*)(aslot + n16 * AROW + (((16 * g + 4 * q + st) ^ n16) * 16));
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int row = bbase(j) + n16;
        b[j] = *(const u32x4*)(bslot + row * BROW + (((4 * g + q) ^ swz<128>(row)) * 16));
        sc[j] = *(const float*)(bslot + BBYTES + (g * BN + row) * 4);
      }
    }
    // after the reads in program order: refill the slots of step kt - 1
    MOE_W4_ISSUE_A(kt + SA - 1);
    MOE_W4_ISSUE_B(kt + SB - 1);
    if (live) {
      f32x4 base = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int st = 0; st < 4; ++st)
        base = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[st]),
                                                       __builtin_bit_cast(bf16x8, kneg), base, 0, 0, 0);
#pragma unroll
      for (int st = 0; st < 4; ++st) a[st] = reorder_a(a[st]);
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        f32x4 part = base;
#pragma unroll
        for (int st = 0; st < 4; ++st)
          part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[st]),
                                                         __builtin_bit_cast(bf16x8, widen_w4(b[j][st])), part, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[j][r] = fmaf(sc[j], part[r], acc[j][r]);
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the tail's zero-fill DMAs
#undef MOE_W4_ISSUE_A
#undef MOE_W4_ISSUE_B

  // The second wave set hands its sums to the first through the (now idle)
  // ring: block j of lane l of column group wn at (j * WN + wn) * 64 + l.
  __syncthreads();
  f32x4* red = (f32x4*)lds;
  if (kset == 1) {
#pragma unroll
    for (int j = 0; j < NB; ++j) red[(j * WN + wn) * 64 + lane] = acc[j];
  }
  __syncthreads();
  if (kset == 1) return;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const f32x4 v = red[(j * WN + wn) * 64 + lane];
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[j][r] += v[r];
  }

  // Epilogue.  Lane l = 16 q + n, register r of a 16 x 16 block: row 4 q + r, column n.
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * q + r;
    if (row >= rows) continue;
    const int prow = r0 + row;
    if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int j = 0; j < NB / 2; ++j) {
        const int col = nt * (BN / 2) + (wn * (NB / 2) + j) * 16 + n16;
        if (col < p.N)
          Elem<ODT>::store((typename Elem<ODT>::T*)p.C, (int64_t)prow * p.N + col,
                           silu_mul_w4(acc[j][r], acc[j + NB / 2][r]));
      }
    } else if constexpr (EPI == EPI_SCATTER) {
      const int tok = p.c_rows ? p.c_rows[prow] : prow;
      const float w = p.row_w[prow];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int col = nt * BN + bbase(j) + n16;
        if (col < p.N) atomicAdd((float*)p.C + (int64_t)tok * p.N + col, w * acc[j][r]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int col = nt * BN + bbase(j) + n16;
        if (col < p.N) Elem<ODT>::store((typename Elem<ODT>::T*)p.C, (int64_t)prow * p.N + col, acc[j][r]);
      }
    }
  }
}

template <int TN, int SA, int SB, int EPI, int ODT>
static hipError_t launch_w4(const GemmW4Params& p, int grid_m, hipStream_t s) {
  constexpr int BN = 4 * TN * 32;
  constexpr int lds_bytes = SA * 16 * 512 + SB * (BN * 128 + 2 * BN * 4);
  static_assert(lds_bytes <= 160 * 1024, "LDS");
  static_assert(2 * TN * 4 * 64 * 16 <= lds_bytes, "reduction space");
  {
    const hipError_t e = allow_lds<gemm_w4_kernel<TN, SA, SB, EPI, ODT>>(lds_bytes);
    if (e != hipSuccess) return e;
  }
  const int64_t grid = (int64_t)grid_m * p.ntn;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_w4_kernel<TN, SA, SB, EPI, ODT>), dim3((unsigned)grid), dim3(512), lds_bytes, s, p);
  return hipGetLastError();
}

GemmShape gemm_w4_shape() {
  GemmShape g;
  g.bm = 16;
  g.bn = 256;
  g.kind = 0;
  return g;
}

hipError_t launch_gemm_w4(int epi, int odt, const GemmW4Params& p, const GemmShape& g, int grid_m, hipStream_t s) {
  if (g.kind != 0) return hipErrorInvalidValue;
  switch (epi) {
    case EPI_SWIGLU: return launch_w4<2, 2, 4, EPI_SWIGLU, MOE_DT_BF16>(p, grid_m, s);
    case EPI_SCATTER: return launch_w4<2, 2, 4, EPI_SCATTER, MOE_DT_F32>(p, grid_m, s);
    default:
      if (odt == MOE_DT_F32) return launch_w4<2, 2, 4, EPI_STORE, MOE_DT_F32>(p, grid_m, s);
      return launch_w4<2, 2, 4, EPI_STORE, MOE_DT_BF16>(p, grid_m, s);
  }
}

}  // namespace moe
