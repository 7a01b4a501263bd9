// Grouped expert GEMMs with 4-bit weights and bf16 activations (W4A16; the
// 4-bit expert-weight format of the MoE inference walkthrough,
// zhiyuanblog.org/blog/moe-inference, §8 quantisation table), for the
// grouped-GEMM step of the same walkthrough (§3.3):
//
//   C[p, n] = sum_kb s[n, kb] * sum_{k in group kb} A[src(p), k] * q[n, k]
//
// with q the signed 4-bit codes (two per byte, the even column in the low
// nibble) and s one fp32 scale per weight row and 128 columns.
//
// Design (decode-sized groups, where the weight stream is the whole cost):
//   * one K step is one scale group (128 columns): the activation rows (32 x
//     256 bytes), the packed codes (BN x 64 bytes) and the BN scales of the
//     step stream straight from memory into one LDS ring slot with
//     buffer_load ... lds, S - 1 steps ahead of the MFMAs;
//   * codes widen to bf16 with two bit operations per pair: a nibble n, its
//     sign bit flipped (u = n ^ 8 = q + 8), or-ed under the bf16 pattern of
//     128 reads as 128 + u = 136 + q exactly; a pair of nibbles four apart in
//     one dword widens in one and + xor, so the B fragment holds the columns
//     of its 8-column run in the order 0,4,1,5,2,6,3,7 and the activation
//     fragment is reordered to match (a dot product does not see the order);
//   * the offset is removed exactly inside the MFMA chain: each group's
//     accumulation starts from A * (-136) (the same activation fragments
//     against a constant bf16 -136), so the chain ends at sum A*q in fp32;
//     the group's scale then folds into the fp32 accumulator (one FMA per
//     element and group);
//   * 4 waves share the tile's 32 activation rows; wave w owns TN 32-column
//     blocks of weight rows (SwiGLU: TN/2 gate blocks and the matching up
//     blocks), so the SiLU * up epilogue needs no data exchange.
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
// the order of widen_w4: pairs (0,4), (1,5), (2,6), (3,7).
__device__ __forceinline__ u32x4 reorder_a(u32x4 a) {
  u32x4 r;
  r[0] = (a[0] & 0xFFFFu) | (a[2] << 16);
  r[1] = (a[0] >> 16) | (a[2] & 0xFFFF0000u);
  r[2] = (a[1] & 0xFFFFu) | (a[3] << 16);
  r[3] = (a[1] >> 16) | (a[3] & 0xFFFF0000u);
  return r;
}

}  // namespace

template <int TN, int S, int EPI, int ODT>
__global__ __launch_bounds__(256, 1) void gemm_w4_kernel(GemmW4Params p) {
  constexpr int NW = 4, BM = 32, BN = NW * TN * 32;
  constexpr int KS = 128;                        // K per step = one scale group
  constexpr int AROW = KS * 2, BROW = KS / 2;    // bytes per row per step: bf16 / packed 4-bit
  constexpr int ABYTES = BM * AROW, BBYTES = BN * BROW, SBYTES = BN * 4;
  constexpr int SLOT = ABYTES + BBYTES + SBYTES;
  constexpr int AI = ABYTES / 1024 / NW;         // 16-byte-per-lane DMAs per wave per slot
  constexpr int BI = BBYTES / 1024 / NW;
  constexpr int SI = SBYTES / 256 / NW;          // 4-byte-per-lane DMAs (scales)
  constexpr int LI = AI + BI + SI;
  static_assert(AI * 1024 * NW == ABYTES && BI * 1024 * NW == BBYTES && SI * 256 * NW == SBYTES, "tile / wave");
  static_assert(EPI != EPI_SWIGLU || TN % 2 == 0, "SwiGLU pairs gate and up blocks");
  static_assert(S >= 2 && (S - 2) * LI < 64, "ring depth");

  extern __shared__ __attribute__((aligned(16))) char lds[];
  lds_char* const lds3 = (lds_char*)lds;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

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
  const int nk = p.K / KS;                // steps = scale groups per row
  const bool second = p.B2 && grp == p.b2_group;
  const uint8_t* Bg = second ? p.B2 : p.B + (int64_t)grp * p.b_gstride;
  const float* Sg = second ? p.b2_scales : p.b_scales + (int64_t)grp * p.bs_gstride;
  const int b_nrows = (EPI == EPI_SWIGLU) ? 2 * p.N : p.N;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, p.a_nrows * arow);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bg, (int64_t)b_nrows * brow);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(Sg, (int64_t)b_nrows * nk * 4);

  // Weight row of tile row r (clamped: rows past N are computed and dropped).
  auto wrow_of = [&](int r) {
    if constexpr (EPI == EPI_SWIGLU) {
      const int j = min(nt * (BN / 2) + (r % (BN / 2)), p.N - 1);
      return (r < BN / 2) ? j : p.N + j;
    } else {
      return min(nt * BN + r, p.N - 1);
    }
  };

  // Per-lane source offsets, fixed over K.  A: 4 rows of 16 chunks per DMA,
  // chunk c of row r stored at chunk c ^ (r & 15); B: 16 rows of 4 chunks,
  // chunk c at c ^ swz<64>(r); scales: 64 rows per DMA, 4 bytes each.
  uint32_t voa[AI], vob[BI], vos[SI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int r = (wave * AI + i) * 4 + (lane >> 4);
    const int chunk = (lane & 15) ^ (r & 15);
    if (r < rows) {
      const int src = p.a_rows ? p.a_rows[r0 + r] : r0 + r;
      voa[i] = (uint32_t)((int64_t)src * arow + chunk * 16);
    } else {
      voa[i] = 0x40000000u;  // past the tile's rows: out of range (zero fill, no traffic) or harmless
    }
  }
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int r = (wave * BI + i) * 16 + (lane >> 2);
    const int chunk = (lane & 3) ^ swz<64>(r);
    vob[i] = (uint32_t)((int64_t)wrow_of(r) * brow + chunk * 16);
  }
#pragma unroll
  for (int i = 0; i < SI; ++i) vos[i] = (uint32_t)((int64_t)wrow_of((wave * SI + i) * 64 + lane) * nk * 4);

  // Step kt into slot kt % S; past the last step every offset is out of range
  // (zero fill, no traffic), so the instruction count per step stays fixed.
#define MOE_W4_ISSUE(kt_)                                                                          \
  do {                                                                                             \
    lds_char* slot_ = lds3 + ((kt_) % S) * SLOT;                                                   \
    const bool live_ = (kt_) < nk;                                                                 \
    const uint32_t sa_ = live_ ? (uint32_t)(kt_) * AROW : 0x80000000u;                             \
    const uint32_t sb_ = live_ ? (uint32_t)(kt_) * BROW : 0x80000000u;                             \
    const uint32_t ss_ = live_ ? (uint32_t)(kt_) * 4 : 0x80000000u;                                \
    _Pragma("unroll") for (int i = 0; i < AI; ++i) dma16(ra, slot_ + (wave * AI + i) * 1024, voa[i], sa_); \
    _Pragma("unroll") for (int i = 0; i < BI; ++i)                                                 \
      dma16(rb, slot_ + ABYTES + (wave * BI + i) * 1024, vob[i], sb_);                             \
    _Pragma("unroll") for (int i = 0; i < SI; ++i)                                                 \
      dma4(rs, slot_ + ABYTES + BBYTES + (wave * SI + i) * 256, vos[i], ss_);                      \
  } while (0)

  auto bblock = [&](int j) {
    if constexpr (EPI == EPI_SWIGLU)
      return j < TN / 2 ? wave * (TN / 2) + j : NW * (TN / 2) + wave * (TN / 2) + (j - TN / 2);
    else
      return wave * TN + j;
  };

  const int lr = lane & 31, hi = lane >> 5;
  const u32x4 kneg = {0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u};  // bf16 -136 everywhere

  f32x16 acc[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;

#pragma unroll
  for (int s = 0; s < S - 1; ++s) MOE_W4_ISSUE(s);

  for (int kt = 0; kt < nk; ++kt) {
    wait_vm_barrier<(S - 2) * LI>();  // slot kt landed; every wave is done with slot kt - 1
    const char* slot = lds + (kt % S) * SLOT;
    // Lane (row lr, half hi) takes columns [64 hi, 64 hi + 64) of the group:
    // activation chunk 8 hi + st and code dword st for sub-step st.
    u32x4 a[8];
#pragma unroll
    for (int st = 0; st < 8; ++st)
      a[st] = *(const u32x4*)(slot + lr * AROW + (((8 * hi + st) ^ (lr & 15)) * 16));
    u32x4 b[TN][2];
    float sc[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int row = bblock(j) * 32 + lr;
#pragma unroll
      for (int c = 0; c < 2; ++c)
        b[j][c] = *(const u32x4*)(slot + ABYTES + row * BROW + (((2 * hi + c) ^ swz<64>(row)) * 16));
      sc[j] = *(const float*)(slot + ABYTES + BBYTES + row * 4);
    }
    MOE_W4_ISSUE(kt + S - 1);  // after the reads in program order: refills slot kt - 1

    f32x16 base;
#pragma unroll
    for (int e = 0; e < 16; ++e) base[e] = 0.0f;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      a[st] = reorder_a(a[st]);
      base = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[st]),
                                                     __builtin_bit_cast(bf16x8, kneg), base, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      f32x16 part = base;
#pragma unroll
      for (int st = 0; st < 8; ++st)
        part = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[st]),
                                                       __builtin_bit_cast(bf16x8, widen_w4(b[j][st >> 2][st & 3])),
                                                       part, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][e] = fmaf(sc[j], part[e], acc[j][e]);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the tail's zero-fill DMAs
#undef MOE_W4_ISSUE

  // Epilogue.  Lane l, register e of a 32x32 block: row 8*(e/4) + 4*(l/32) + e%4, column l%32.
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int row = 8 * (e >> 2) + 4 * hi + (e & 3);
    if (row >= rows) continue;
    const int prow = r0 + row;
    if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int j = 0; j < TN / 2; ++j) {
        const int col = nt * (BN / 2) + (wave * (TN / 2) + j) * 32 + lr;
        if (col < p.N)
          Elem<ODT>::store((typename Elem<ODT>::T*)p.C, (int64_t)prow * p.N + col,
                           silu_mul_w4(acc[j][e], acc[j + TN / 2][e]));
      }
    } else if constexpr (EPI == EPI_SCATTER) {
      const int tok = p.c_rows ? p.c_rows[prow] : prow;
      const float w = p.row_w[prow];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = nt * BN + bblock(j) * 32 + lr;
        if (col < p.N) atomicAdd((float*)p.C + (int64_t)tok * p.N + col, w * acc[j][e]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = nt * BN + bblock(j) * 32 + lr;
        if (col < p.N) Elem<ODT>::store((typename Elem<ODT>::T*)p.C, (int64_t)prow * p.N + col, acc[j][e]);
      }
    }
  }
}

template <int TN, int S, int EPI, int ODT>
static hipError_t launch_w4(const GemmW4Params& p, int grid_m, hipStream_t s) {
  constexpr int BN = 4 * TN * 32;
  constexpr int lds_bytes = S * (32 * 256 + BN * 64 + BN * 4);
  static_assert(lds_bytes <= 160 * 1024, "LDS");
  {
    const hipError_t e = allow_lds<gemm_w4_kernel<TN, S, EPI, ODT>>(lds_bytes);
    if (e != hipSuccess) return e;
  }
  const int64_t grid = (int64_t)grid_m * p.ntn;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_w4_kernel<TN, S, EPI, ODT>), dim3((unsigned)grid), dim3(256), lds_bytes, s, p);
  return hipGetLastError();
}

GemmShape gemm_w4_shape() {
  GemmShape g;
  g.bm = 32;
  g.bn = 256;
  g.kind = 0;
  return g;
}

hipError_t launch_gemm_w4(int epi, int odt, const GemmW4Params& p, const GemmShape& g, int grid_m, hipStream_t s) {
  if (g.kind != 0) return hipErrorInvalidValue;
  switch (epi) {
    case EPI_SWIGLU: return launch_w4<2, 6, EPI_SWIGLU, MOE_DT_BF16>(p, grid_m, s);
    case EPI_SCATTER: return launch_w4<2, 6, EPI_SCATTER, MOE_DT_F32>(p, grid_m, s);
    default:
      if (odt == MOE_DT_F32) return launch_w4<2, 6, EPI_STORE, MOE_DT_F32>(p, grid_m, s);
      return launch_w4<2, 6, EPI_STORE, MOE_DT_BF16>(p, grid_m, s);
  }
}

}  // namespace moe
