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
//   * tiles of 16 rows x 256 weight rows (decode experts hold a few rows each);
//   * persistent work-groups, one per CU: work-group b walks a list of tiles,
//     and its LDS rings stream straight across tile boundaries, so a tile's
//     first weight bytes are in flight while the previous tile finishes (a
//     fresh pipeline per tile would wait one memory latency per tile);
//   * one K step is two scale groups (256 columns); the packed codes (256
//     rows x 128 bytes: one whole cache line per weight row) with the 512
//     scales of the step (two contiguous runs), and the activation rows (16 x
//     512 bytes), stream from memory into LDS rings with buffer_load ... lds:
//     the weight ring SB - 1 steps ahead of the MFMAs, the activation ring
//     (mostly L2 hits) SA - 1 steps ahead, so the LDS goes to weight bytes
//     in flight;
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
//   * 16 x 16 x 32 MFMAs; 8 waves: wave w owns four 16-column blocks of
//     weight rows (SwiGLU: two gate blocks and the matching up blocks, so the
//     SiLU * up epilogue needs no data exchange between blocks) for group
//     w / 4 of every step; the two waves of a column group share a SIMD,
//     where one's MFMAs overlap the other's code widening, and add their sums
//     through LDS at the end of each tile.
#include <atomic>

#include "common.h"
#include "kernels.h"
#include "lds_dma.h"

namespace moe {

namespace {

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

typedef __attribute__((address_space(4))) const int cint32;  // uniform data read with scalar loads

// LDS writes done, then meet the other waves; the DMAs in flight stay in flight
// (a __syncthreads fence would also wait for them).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

struct W4Tile {
  int grp, r0, r1, nt;
};

__device__ __forceinline__ W4Tile w4_tile(const GemmW4Params& p, int L, int bm) {
  if (p.tiles) {
    const cint32* t = (cint32*)p.tiles + 4 * (int64_t)L;
    return {t[0], t[1], t[2], t[3]};
  }
  const int mt = L / p.ntn;
  return {0, mt * bm, min(p.M, mt * bm + bm), L - mt * p.ntn};
}

}  // namespace

template <int SA, int SB, int EPI, int ODT>
__global__ __launch_bounds__(512, 1) void gemm_w4_kernel(GemmW4Params p) {
  constexpr int NW = 8, WN = 4, NB = 4, BM = 16, BN = WN * NB * 16;  // 16 rows x 256 weight rows
  constexpr int G = 2;                            // scale groups per K step
  constexpr int KS = 128 * G;                     // K per step
  constexpr int AROW = KS * 2, BROW = KS / 2;     // bytes per row per step: bf16 / packed 4-bit
  constexpr int ACH = AROW / 16, BCH = BROW / 16; // 16-byte chunks per row
  constexpr int ABYTES = BM * AROW, BBYTES = BN * BROW, SBYTES = G * BN * 4;
  constexpr int ASLOT = ABYTES, BSLOT = BBYTES + SBYTES;  // activation slot; codes + scales slot
  constexpr int BRING = SA * ASLOT;                       // the weight ring follows the activation ring
  constexpr int RED = BRING + SB * BSLOT;                 // 8 KB: the wave sets' sums meet here, half at a time
  constexpr int AI = ABYTES / 1024 / NW;          // 16-byte-per-lane DMAs per wave per step
  constexpr int BI = BBYTES / 1024 / NW;
  constexpr int SI = SBYTES / 256 / NW;           // 4-byte-per-lane DMAs (scales)
  // At the top of step c the DMAs issued after A(c) are B(c + SB - 2) and, when
  // step c - 1 ended a tile, the NST stores of that tile's epilogue in the
  // waves of the first set (every store instruction is issued; lanes without
  // an element store out of range).  B(c) went out before A(c), so waiting for
  // A(c) covers it.
  constexpr int VMN = BI + SI;
  constexpr int NST = EPI == EPI_SWIGLU ? 4 * NB / 2 : (EPI == EPI_STORE ? 4 * NB : 0);
  static_assert(AI * 1024 * NW == ABYTES && BI * 1024 * NW == BBYTES && SI * 256 * NW == SBYTES, "tile / wave");
  static_assert(ACH == 32 && BCH == 8, "row layout");
  static_assert(SA == 2 && SB >= SA && VMN + NST < 64, "ring depths");

  extern __shared__ __attribute__((aligned(16))) char lds[];
  lds_char* const lds3 = (lds_char*)lds;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % WN, kset = wave / WN;  // column group and scale group of this wave

  // This work-group's tiles.  XCD x (work-groups b with b % 8 == x) takes a
  // contiguous eighth of the list and its work-groups take that range round
  // robin, so the work-groups of an XCD run neighbouring tiles (the m-tiles
  // that share a weight tile) together and read the weights once into its L2.
  const int total = p.tiles ? *(cint32*)p.n_mtiles_dev : p.n_mtiles * p.ntn;
  const int nxcd = gridDim.x < 8 ? (int)gridDim.x : 8;
  const int x = blockIdx.x % nxcd, wj = blockIdx.x / nxcd;
  const int nx = ((int)gridDim.x - x + nxcd - 1) / nxcd;  // work-groups on this XCD
  const int xbeg = x * (total / nxcd) + min(x, total % nxcd);
  const int xlen = total / nxcd + (x < total % nxcd ? 1 : 0);
  const int my_n = wj < xlen ? (xlen - wj + nx - 1) / nx : 0;
  if (my_n == 0) return;
  auto tile_of = [&](int ti) { return w4_tile(p, xbeg + wj + ti * nx, BM); };

  const int64_t arow = (int64_t)p.K * 2;  // bytes per activation row
  const int64_t brow = p.K / 2;           // bytes per packed weight row
  const int ngroups = p.K / 128;          // scale groups per row
  const int nk = (ngroups + G - 1) / G;   // steps per tile; an odd group count leaves the last half full
  const int b_nrows = (EPI == EPI_SWIGLU) ? 2 * p.N : p.N;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, p.a_nrows * arow);

  // Weight row of tile row r of n-tile nt (clamped: rows past N are computed and dropped).
  auto wrow_of = [&](int r, int nt) {
    if constexpr (EPI == EPI_SWIGLU) {
      const int jj = min(nt * (BN / 2) + (r % (BN / 2)), p.N - 1);
      return (r < BN / 2) ? jj : p.N + jj;
    } else {
      return min(nt * BN + r, p.N - 1);
    }
  };

  // Activation stream: per-lane offsets of its current tile.  A DMA fills 2
  // rows of 32 chunks; chunk c of row r is stored at chunk c ^ (r & 15).
  int a_t = 0, a_k = 0, a_i = 0;
  uint32_t voa[AI];
  auto set_a = [&](int ti) {
    const W4Tile t = tile_of(ti);
    const int rows = t.r1 - t.r0;
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      const int rb = (wave * AI + i) * 2;  // this DMA's rows rb, rb + 1 (wave-uniform: scalar loads)
      int s0 = 0, s1 = 0;
      if (rb < rows) s0 = p.a_rows ? ((cint32*)p.a_rows)[t.r0 + rb] : t.r0 + rb;
      if (rb + 1 < rows) s1 = p.a_rows ? ((cint32*)p.a_rows)[t.r0 + rb + 1] : t.r0 + rb + 1;
      const int r = rb + lane / ACH;
      const int chunk = (lane % ACH) ^ (r & 15);
      voa[i] = r < rows ? (uint32_t)((int64_t)(lane < ACH ? s0 : s1) * arow + chunk * 16)
                        : 0x40000000u;  // past the tile's rows: out of range (zero fill, no traffic) or harmless
    }
  };
  // Weight stream: codes and scales of its current tile's group.  A DMA fills
  // 8 rows of 8 chunks (chunk c of row r at c ^ swz<128>(r)); a scale DMA 64
  // consecutive entries of one group (the slot holds group 0's 256 scales, then group 1's).
  int b_t = 0, b_k = 0, b_i = 0;
  uint32_t vob[BI], vos[SI];
  const uint8_t* bg = nullptr;
  const float* sg = nullptr;
  auto set_b = [&](int ti) {
    const W4Tile t = tile_of(ti);
    const bool second = p.B2 && t.grp == p.b2_group;
    bg = second ? p.B2 : p.B + (int64_t)t.grp * p.b_gstride;
    sg = second ? p.b2_scales : p.b_scales + (int64_t)t.grp * p.bs_gstride;
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      const int r = (wave * BI + i) * (64 / BCH) + lane / BCH;
      const int chunk = (lane % BCH) ^ swz<128>(r);
      vob[i] = (uint32_t)((int64_t)wrow_of(r, t.nt) * brow + chunk * 16);
    }
#pragma unroll
    for (int i = 0; i < SI; ++i) {
      const int idx = (wave * SI + i) * 64 + lane;
      vos[i] = (uint32_t)(((int64_t)(idx / BN) * b_nrows + wrow_of(idx % BN, t.nt)) * 4);
    }
  };

  // One step of each stream; past this work-group's last step every offset is
  // out of range (zero fill, no traffic), so the instruction count per step
  // stays fixed.  In a half-full last step the second group's bytes are not used.
#define MOE_W4_ISSUE_A()                                                                           \
  do {                                                                                             \
    lds_char* slot_ = lds3 + (a_i % SA) * ASLOT;                                                   \
    const uint32_t so_ = a_t < my_n ? (uint32_t)a_k * AROW : 0x80000000u;                          \
    _Pragma("unroll") for (int i = 0; i < AI; ++i) dma16(ra, slot_ + (wave * AI + i) * 1024, voa[i], so_); \
    ++a_i;                                                                                         \
    if (++a_k == nk) {                                                                             \
      a_k = 0;                                                                                     \
      if (++a_t < my_n) set_a(a_t);                                                                \
    }                                                                                              \
  } while (0)
#define MOE_W4_ISSUE_B()                                                                           \
  do {                                                                                             \
    lds_char* slot_ = lds3 + BRING + (b_i % SB) * BSLOT;                                           \
    const bool live_ = b_t < my_n;                                                                 \
    const uint32_t sb_ = live_ ? (uint32_t)b_k * BROW : 0x80000000u;                               \
    const uint32_t ss_ = live_ ? (uint32_t)b_k * G * b_nrows * 4 : 0x80000000u;                    \
    const __amdgpu_buffer_rsrc_t rb_ = make_rsrc(bg, (int64_t)b_nrows * brow);                     \
    const __amdgpu_buffer_rsrc_t rs_ = make_rsrc(sg, (int64_t)ngroups * b_nrows * 4);              \
    _Pragma("unroll") for (int i = 0; i < BI; ++i) dma16(rb_, slot_ + (wave * BI + i) * 1024, vob[i], sb_); \
    _Pragma("unroll") for (int i = 0; i < SI; ++i)                                                 \
      dma4(rs_, slot_ + BBYTES + (wave * SI + i) * 256, vos[i], ss_);                              \
    ++b_i;                                                                                         \
    if (++b_k == nk) {                                                                             \
      b_k = 0;                                                                                     \
      if (++b_t < my_n) set_b(b_t);                                                                \
    }                                                                                              \
  } while (0)

  // 16-column blocks of this wave: first B-tile row of block jb (SwiGLU: NB/2
  // gate blocks, then the matching up blocks).
  auto bbase = [&](int jb) {
    if constexpr (EPI == EPI_SWIGLU)
      return jb < NB / 2 ? (wn * (NB / 2) + jb) * 16 : BN / 2 + (wn * (NB / 2) + jb - NB / 2) * 16;
    else
      return (wn * NB + jb) * 16;
  };
  // 16 x 16 x 32 MFMA lanes: l = 16 q + n takes activation row n and weight
  // row n of a block, columns 8 q .. 8 q + 7 of each 32-column sub-step.
  const int n16 = lane & 15, q = lane >> 4;
  const u32x4 kneg = {0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u};  // bf16 -136 everywhere

  set_a(0);
  set_b(0);
  // The issues of the SB - 1 steps before step 0, in steady-state order.
#pragma unroll
  for (int t = -(SB - 1); t < 0; ++t) {
    if (t + SA - 1 >= 0) MOE_W4_ISSUE_A();
    MOE_W4_ISSUE_B();
  }

  f32x4 acc[NB];
#pragma unroll
  for (int jb = 0; jb < NB; ++jb) acc[jb] = {0.0f, 0.0f, 0.0f, 0.0f};
  W4Tile ct = tile_of(0);  // the tile being computed (its epilogue needs the rows and n-tile)
  int c_t = 0, c_k = 0;
  bool after_epi = false;
  const int steps = my_n * nk;
  for (int cs = 0; cs < steps; ++cs) {
    // step cs landed; every wave is done with step cs - 1
    if (EPI != EPI_SCATTER && after_epi && kset == 0) wait_vm_barrier<VMN + NST>();
    else wait_vm_barrier<VMN>();
    const char* aslot = lds + (cs % SA) * ASLOT;
    const char* bslot = lds + BRING + (cs % SB) * BSLOT;
    const int g = kset;
    const bool live = c_k * G + g < ngroups;  // wave-uniform: false only in a half-full last step
    // Lane (n, q) takes columns [32 q, 32 q + 32) of group g: activation
    // chunk 16 g + 4 q + st and code dword st (of chunk 4 g + q) for sub-step st.
    u32x4 a[4], b[NB];
    float sc[NB];
    if (live) {
#pragma unroll
      for (int st = 0; st < 4; ++st)
        a[st] = *(const u32x4*)(aslot + n16 * AROW + (((16 * g + 4 * q + st) ^ n16) * 16));
#pragma unroll
      for (int jb = 0; jb < NB; ++jb) {
        const int row = bbase(jb) + n16;
        b[jb] = *(const u32x4*)(bslot + row * BROW + (((4 * g + q) ^ swz<128>(row)) * 16));
        sc[jb] = *(const float*)(bslot + BBYTES + (g * BN + row) * 4);
      }
    }
    // after the reads in program order: refill the slots of step cs - 1
    MOE_W4_ISSUE_A();
    MOE_W4_ISSUE_B();
    asm volatile("" ::: "memory");  // the epilogue's stores stay behind these DMAs
    if (live) {
      f32x4 base = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int st = 0; st < 4; ++st)
        base = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[st]),
                                                       __builtin_bit_cast(bf16x8, kneg), base, 0, 0, 0);
#pragma unroll
      for (int st = 0; st < 4; ++st) a[st] = reorder_a(a[st]);
      // the NB chains run interleaved (sub-step outer), so consecutive MFMAs
      // do not wait on each other; each chain keeps its own order
      f32x4 part[NB];
#pragma unroll
      for (int jb = 0; jb < NB; ++jb) part[jb] = base;
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int jb = 0; jb < NB; ++jb)
          part[jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[st]),
                                                             __builtin_bit_cast(bf16x8, widen_w4(b[jb][st])),
                                                             part[jb], 0, 0, 0);
#pragma unroll
      for (int jb = 0; jb < NB; ++jb)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[jb][r] = fmaf(sc[jb], part[jb][r], acc[jb][r]);
    }
    after_epi = false;
    if (++c_k < nk) continue;

    // End of tile ct: the second wave set adds its sums into the first's,
    // half of the blocks at a time through the 8 KB region (block jb of lane
    // l of column group wn at ((jb % (NB / 2)) * WN + wn) * 64 + l).
    f32x4* red = (f32x4*)(lds + RED);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (half) lds_barrier();  // the first half has been read
      if (kset == 1) {
#pragma unroll
        for (int jb = 0; jb < NB / 2; ++jb) red[(jb * WN + wn) * 64 + lane] = acc[half * (NB / 2) + jb];
      }
      lds_barrier();
      if (kset == 0) {
#pragma unroll
        for (int jb = 0; jb < NB / 2; ++jb) {
          const f32x4 v = red[(jb * WN + wn) * 64 + lane];
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[half * (NB / 2) + jb][r] += v[r];
        }
      }
    }

    // Epilogue of tile ct.  Lane l = 16 q + n, register r of a 16 x 16 block:
    // row 4 q + r, column n.  Stores go through a buffer resource over the
    // tile's rows: every store instruction is issued (a fixed count per
    // tile), lanes without an element write out of range and are dropped.
    // Only the first wave set holds the sums.  (The scatter path's row indices
    // and weights are vector loads: waiting for them also waits for the ring
    // DMAs in flight, one drain per tile on that path.)
    const int rows = ct.r1 - ct.r0;
    if (kset == 0 && EPI == EPI_SCATTER) {
      const int col0 = ct.nt * BN;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * q + r;
        if (row >= rows) continue;
        const int prow = ct.r0 + row;
        const int tok = p.c_rows ? p.c_rows[prow] : prow;
        const float w = p.row_w[prow];
#pragma unroll
        for (int jb = 0; jb < NB; ++jb) {
          const int col = col0 + bbase(jb) + n16;
          if (col < p.N) atomicAdd((float*)p.C + (int64_t)tok * p.N + col, w * acc[jb][r]);
        }
      }
    } else if (kset == 0) {
      constexpr int EB = EPI == EPI_SWIGLU ? 2 : Elem<ODT>::kBytes;
      const __amdgpu_buffer_rsrc_t rc =
          make_rsrc((const char*)p.C + (int64_t)ct.r0 * p.N * EB, (int64_t)rows * p.N * EB);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * q + r;
        if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
          for (int jb = 0; jb < NB / 2; ++jb) {
            const int col = ct.nt * (BN / 2) + (wn * (NB / 2) + jb) * 16 + n16;
            const uint32_t off = (row < rows && col < p.N) ? (uint32_t)((row * p.N + col) * 2) : 0x80000000u;
            __builtin_amdgcn_raw_buffer_store_b16(
                (unsigned short)f32_to_bf16_bits(silu_mul(acc[jb][r], acc[jb + NB / 2][r])), rc, off, 0, 0);
          }
        } else {
#pragma unroll
          for (int jb = 0; jb < NB; ++jb) {
            const int col = ct.nt * BN + bbase(jb) + n16;
            const uint32_t off = (row < rows && col < p.N) ? (uint32_t)((row * p.N + col) * EB) : 0x80000000u;
            if constexpr (ODT == MOE_DT_BF16)
              __builtin_amdgcn_raw_buffer_store_b16((unsigned short)f32_to_bf16_bits(acc[jb][r]), rc, off, 0, 0);
            else
              __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, acc[jb][r]), rc, off, 0, 0);
          }
        }
      }
    }
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) acc[jb] = {0.0f, 0.0f, 0.0f, 0.0f};
    c_k = 0;
    after_epi = true;
    if (++c_t < my_n) ct = tile_of(c_t);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the tail's zero-fill DMAs
#undef MOE_W4_ISSUE_A
#undef MOE_W4_ISSUE_B
}

// Compute units of the current device, queried once per device (64 devices at most are remembered).
static hipError_t device_cus(int* cus) {
  static std::atomic<int> known[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64) {
    const int v = known[dev].load(std::memory_order_relaxed);
    if (v > 0) {
      *cus = v;
      return hipSuccess;
    }
  }
  e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess && dev >= 0 && dev < 64) known[dev].store(*cus, std::memory_order_relaxed);
  return e;
}

template <int SA, int SB, int EPI, int ODT>
static hipError_t launch_w4(const GemmW4Params& p, int grid_m, hipStream_t s) {
  constexpr int BN = 256;
  constexpr int lds_bytes = SA * 16 * 512 + SB * (BN * 128 + 2 * BN * 4) + 8192;
  static_assert(lds_bytes <= 160 * 1024, "LDS");
  {
    const hipError_t e = allow_lds<gemm_w4_kernel<SA, SB, EPI, ODT>>(lds_bytes);
    if (e != hipSuccess) return e;
  }
  // one persistent work-group per CU (LDS holds one), at most one per tile
  int cus = 0;
  {
    const hipError_t e = device_cus(&cus);
    if (e != hipSuccess) return e;
  }
  const int64_t tiles = (int64_t)grid_m * p.ntn;
  const int64_t grid = tiles < cus ? tiles : cus;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_w4_kernel<SA, SB, EPI, ODT>), dim3((unsigned)grid), dim3(512), lds_bytes, s, p);
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
    case EPI_SWIGLU: return launch_w4<2, 4, EPI_SWIGLU, MOE_DT_BF16>(p, grid_m, s);
    case EPI_SCATTER: return launch_w4<2, 4, EPI_SCATTER, MOE_DT_F32>(p, grid_m, s);
    default:
      if (odt == MOE_DT_F32) return launch_w4<2, 4, EPI_STORE, MOE_DT_F32>(p, grid_m, s);
      return launch_w4<2, 4, EPI_STORE, MOE_DT_BF16>(p, grid_m, s);
  }
}

}  // namespace moe
