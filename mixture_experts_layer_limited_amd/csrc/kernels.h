// Internal launch interface between the C-ABI layer (api.cpp) and the
// kernels (*.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe355.h"

namespace moe {

enum { MOE_DT_F32 = 0, MOE_DT_BF16 = 1, MOE_DT_FP8 = 2 };
// EPI_COMBINE: a row store over the T tokens of a dense launch (the shared
// expert's down GEMM) whose tile is combined with the routed rows (CombineEpi)
// and written as the layer output; 256 x 256 bf16 and FP8 kernels only.
enum { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_SCATTER = 2, EPI_COMBINE = 3 };

// The EPI_COMBINE epilogue's inputs: it writes
// out[t] = sum_j w[t*k+j] * rows[inv[t*k+j]] + C-tile[t] (bf16), the layer's
// weighted un-permute + combine, instead of storing the launch's own rows.
struct CombineEpi {
  const void* rows = nullptr;   // routed expert rows in permuted order, [T*k, N] bf16
  const int32_t* inv = nullptr; // inv_perm [T*k]
  const float* w = nullptr;     // routing weights [T*k]
  int k = 0;
  void* out = nullptr;          // [T, N] bf16
};

struct GemmParams {
  const void* A;          // activations: row src(p) at A + src(p) * K elements
  const int32_t* a_rows;  // src(p) = a_rows[p]; NULL: src(p) = p
  const void* B;          // weights of group g at B + g * b_gstride elements, (out, in)
  int64_t b_gstride;
  const void* B2;         // if not NULL: the weights of group b2_group (the shared expert
  int b2_group;           // run as one more group of the routed launch)
  int K;                  // reduction length (elements)
  int N;                  // output columns; SwiGLU: h columns (B holds 2N rows)
  void* C;                // output: rows p (store, SwiGLU) or rows c_rows[p] (scatter)
  const int32_t* c_rows;  // scatter: output row of row p; NULL: p
  const float* row_w;     // scatter: weight of row p
  const int4* tiles;      // tiles {group, row0, row1, n-tile}; NULL: dense rows [0, M)
  const int* n_mtiles_dev; // number of entries of `tiles`
  int n_mtiles;           // dense: number of m-tiles
  int M;                  // dense: rows
  int ntn;                // number of n-tiles
  int64_t a_nrows;        // rows of A (bounds of the activation buffer)
  // Split K (pipelined single-ring kernel, store epilogue only): grid.y = ksplit
  // slices of K / ksplit columns each; slice z writes C + z * c_split_stride.
  int ksplit;             // 0 or 1: no split
  int64_t c_split_stride; // elements between the slices' outputs
  CombineEpi comb;        // EPI_COMBINE
};

struct GemmShape {
  int bm = 128;
  int bn = 128;  // weight rows per tile (SwiGLU: bn/2 h columns)
  int kind = 0;
};

// MI355X: 256 compute units.
constexpr int kChipCUs = 256;
// Batches from this many tokens up take 128 x 256 router tiles.
constexpr int kRouterWideRows = 4096;
GemmShape gemm_shape(int which, int dt, int rows_hint, int64_t tiles256 = 0);
hipError_t launch_gemm(int dt, int epi, int odt, const GemmParams& p, const GemmShape& g, int grid_m,
                       hipStream_t s);
// Pipelined bf16 kernel (LDS ring filled by direct-to-LDS buffer loads).
hipError_t launch_gemm_pipe(int epi, int odt, const GemmParams& p, const GemmShape& g, int grid_m, hipStream_t s);
// The tile list of a grouped GEMM; with tiles2, a second list (another n-tile
// count) in the same launch when bm2 == bm, else in a launch of its own.
// Where the tile lists of a grouped GEMM pair go: m-tiles of bm rows, ntn
// n-tiles in the first list and ntn2 (0: none) in the second.
struct TileLists {
  int bm = 0;
  int ntn = 0;
  int4* tiles = nullptr;
  int* n_tiles = nullptr;
  int ntn2 = 0;
  int4* tiles2 = nullptr;
  int* n_tiles2 = nullptr;
};
hipError_t launch_build_tiles(const int32_t* offsets, int E, int bm, int ntn, int4* tiles, int* n_tiles,
                              hipStream_t s, int bm2 = 0, int ntn2 = 0, int4* tiles2 = nullptr,
                              int* n_tiles2 = nullptr);

// FP8 grouped GEMM: A = E4M3 codes with 1x128 fp32 scales, B = E4M3 codes with
// 128x128 fp32 block scales.
struct GemmFp8Params {
  const uint8_t* A;
  const float* a_scales;  // [rowsA, K/128], or k-block-major when as_stride > 0
  int64_t as_stride;      // > 0: scale of permuted row p, k-block kb at a_scales[kb * as_stride + p]
  const int32_t* a_rows;
  const uint8_t* B;
  const float* b_scales;  // group g: b_scales + g * bs_gstride, [Nrows/128, K/128]
  int64_t b_gstride;      // bytes between groups
  int64_t bs_gstride;     // floats between groups
  const uint8_t* B2;      // if not NULL: codes and scales of group b2_group
  const float* b2_scales;
  int b2_group;
  int K;
  int N;
  void* C;                // store: bf16 [rows, N]; scatter: fp32 [T, N]
  uint8_t* Cq;            // SwiGLU: E4M3 codes of h [rows, N] ...
  float* Cs;              // ... and their 1x128 scales, k-block-major: Cs[kb * cs_stride + row]
  int64_t cs_stride;
  const int32_t* c_rows;
  const float* row_w;
  const int4* tiles;
  const int* n_mtiles_dev;
  int n_mtiles;
  int M;
  int ntn;
  int64_t a_nrows;        // rows of A and of its scales (bounds of the activation buffers)
  CombineEpi comb;        // EPI_COMBINE
};
// rows_hint = mean rows per group; epi = the epilogue the launch will use
constexpr int kFp8BigMaxK = 64 * 128;
GemmShape gemm_fp8_shape(int rows_hint, int epi, int K);
hipError_t launch_gemm_fp8(int epi, const GemmFp8Params& p, const GemmShape& g, int grid_m, hipStream_t s);
// 256 x 256 tiles (SwiGLU and row-store epilogues; k-block-major activation scales)
hipError_t launch_gemm_fp8_big(int epi, const GemmFp8Params& p, int grid_m, hipStream_t s);

// Grouped GEMM with 4-bit weights (two's-complement codes, two per byte, the
// even column in the low nibble) and one fp32 scale per weight row and 128
// columns; bf16 activations.
struct GemmW4Params {
  const void* A;          // bf16 activations, row src(p) at A + src(p) * K elements
  const int32_t* a_rows;
  const uint8_t* B;       // group g: packed codes at B + g * b_gstride bytes, [Nrows, K/2]
  const float* b_scales;  // group g: b_scales + g * bs_gstride, [Nrows, K/128]
  int64_t b_gstride;
  int64_t bs_gstride;
  const uint8_t* B2;      // if not NULL: codes and scales of group b2_group
  const float* b2_scales;
  int b2_group;
  int K;
  int N;
  void* C;
  const int32_t* c_rows;
  const float* row_w;
  const int4* tiles;
  const int* n_mtiles_dev;
  int n_mtiles;
  int M;
  int ntn;
  int64_t a_nrows;
};
GemmShape gemm_w4_shape();
hipError_t launch_gemm_w4(int epi, int odt, const GemmW4Params& p, const GemmShape& g, int grid_m, hipStream_t s);

struct RouteParams {
  const float* logits;    // [T,E] router logits, or scores when scores_given;
                          // n_parts > 1: partial logits of K slices, part_stride apart
  int n_parts;
  int64_t part_stride;
  int scores_given;
  const float* bias;      // [E] or NULL
  float* scores_out;      // [T,E] or NULL
  int32_t* topk_ids;
  float* topk_w;
  int T, E, k, n_group, topk_group, scoring, norm;
  float scale;
};
hipError_t launch_route(const RouteParams& p, hipStream_t s);

// ext_T > 0: also offsets[E+1] = n + ext_T and src[n + t] = t (the shared
// expert as group E).
// tl (optional): the GEMMs' tile lists over the E (+1 with ext_T) groups, also
// written when the batch is small enough for the one-work-group permutation;
// *tiles_done tells whether they were.
hipError_t launch_permute(const int32_t* ids, int n, int k, int E, int32_t* counts, int32_t* offsets,
                          int32_t* src, int32_t* inv, hipStream_t s, int ext_T = 0, const TileLists* tl = nullptr,
                          bool* tiles_done = nullptr);
int permute_blocks(int n);
// offsets[E+1] = rows + T and src[rows + t] = t: the shared expert as group E.
hipError_t launch_extend_shared(int32_t* offsets, int E, int rows, int T, int32_t* src, hipStream_t s);

hipError_t launch_row_weights(const float* topk_w, const int32_t* inv, int n, float* row_w, hipStream_t s);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s);
hipError_t launch_combine(int adt, int T, int H, int k, const void* expert_out, const float* acc,
                          const int32_t* inv, const float* topk_w, const void* shared_out, void* out,
                          hipStream_t s);
hipError_t launch_load_balance(const int32_t* offsets, int E, float* bias, float gamma, ::moe_load_stats* stats,
                               hipStream_t s);
// codes [rows, cols] E4M3, scales [rows, cols/128]
hipError_t launch_quantize(int in_dt, int64_t rows, int64_t cols, const void* in, uint8_t* codes,
                           float* scales, hipStream_t s);
// scales_t[kb * rows + p] = scales[src(p) * nkb + kb], src(p) = src[p] or p; a
// row whose src(p) lies outside [0, src_rows) gets scale 1 (its activation
// loads in the GEMM are out of range and read zeros)
hipError_t launch_gather_scales_t(const float* scales, const int32_t* src, int64_t rows, int nkb,
                                  int64_t src_rows, float* scales_t, hipStream_t s);

}  // namespace moe
