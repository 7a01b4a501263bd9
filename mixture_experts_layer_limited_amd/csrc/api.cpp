// C ABI of libmoe355 (include/moe355.h): argument validation, workspace
// carving and the launch sequence of every entry point.  No allocation, no
// host synchronisation: each call enqueues kernels on the caller's stream.
#include "moe355.h"

#include <math.h>
#include <stddef.h>

#include <mutex>

#include "kernels.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Sequential carving of the caller's workspace; with base == nullptr it only
// measures.
struct Carver {
  char* base;
  size_t used = 0;
  explicit Carver(void* b) : base((char*)b) {}
  template <class T>
  T* take(size_t count) {
    const size_t off = used;
    used = align_up(used + count * sizeof(T));
    return base ? (T*)(base + off) : nullptr;
  }
};

bool is_fp8(const moe_config* c) { return c->weight_dtype == MOE_FP8_E4M3; }
bool is_w4(const moe_config* c) { return c->weight_dtype == MOE_INT4; }
// weights that come with scale tensors
bool has_scales(const moe_config* c) { return is_fp8(c) || is_w4(c); }
int act_dt(const moe_config* c) { return c->act_dtype == MOE_F32 ? MOE_DT_F32 : MOE_DT_BF16; }
size_t act_bytes(const moe_config* c) { return c->act_dtype == MOE_F32 ? 4 : 2; }

int check_cfg(const moe_config* c) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->scoring != MOE_SCORE_SOFTMAX && c->scoring != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID_ARG;
  if (c->norm_topk_prob != 0 && c->norm_topk_prob != 1) return MOE_ERR_INVALID_ARG;
  if (c->act_dtype != MOE_F32 && c->act_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (c->weight_dtype != MOE_F32 && c->weight_dtype != MOE_BF16 && c->weight_dtype != MOE_FP8_E4M3 &&
      c->weight_dtype != MOE_INT4)
    return MOE_ERR_INVALID_ARG;
  if (c->out_dtype != MOE_F32 && c->out_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (c->hidden <= 0 || c->inter <= 0 || c->n_experts <= 0 || c->top_k <= 0 || c->n_group <= 0 ||
      c->topk_group <= 0 || c->shared_inter < 0)
    return MOE_ERR_CONFIG;
  if (!isfinite(c->routed_scaling_factor)) return MOE_ERR_CONFIG;
  if (c->n_experts % c->n_group) return MOE_ERR_CONFIG;
  if (c->topk_group > c->n_group) return MOE_ERR_CONFIG;
  const int G = c->n_experts / c->n_group;
  if (c->n_group > 1 && G < 2) return MOE_ERR_CONFIG;
  if (c->top_k > c->n_experts) return MOE_ERR_CONFIG;
  if (c->n_group > 1 && c->top_k > c->topk_group * G) return MOE_ERR_CONFIG;
  // Limits of this implementation.
  if (c->n_experts > 1024 || c->top_k > 32 || c->n_group > 64) return MOE_ERR_UNSUPPORTED;
  if (c->out_dtype != c->act_dtype) return MOE_ERR_UNSUPPORTED;
  if (c->weight_dtype != c->act_dtype && !(has_scales(c) && c->act_dtype == MOE_BF16)) return MOE_ERR_UNSUPPORTED;
  const int mult = has_scales(c) ? 128 : 64;
  if (c->hidden % mult || c->inter % mult || c->shared_inter % mult) return MOE_ERR_UNSUPPORTED;
  // The GEMMs address one weight matrix (an expert's w13 or w2, the shared
  // expert's, the router's) with 32-bit buffer offsets: each spans < 2^31 bytes.
  const int64_t lim = (int64_t)1 << 31;
  const int64_t wide = c->shared_inter > c->inter ? c->shared_inter : c->inter;
  const int64_t w13_elems = 2 * wide * (int64_t)c->hidden;
  const int64_t w13_bytes = is_w4(c) ? w13_elems / 2 : w13_elems * (is_fp8(c) ? 1 : (int64_t)act_bytes(c));
  if (w13_bytes >= lim) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)c->n_experts * c->hidden * (int64_t)act_bytes(c) >= lim) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int check_T(const moe_config* c, int64_t T) {
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (T * (int64_t)c->top_k >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED;
  if (T * (int64_t)c->n_experts >= (int64_t)1 << 40) return MOE_ERR_UNSUPPORTED;
  // The GEMMs address their activation operands (hidden rows, the
  // intermediate rows) with 32-bit buffer offsets.
  const int64_t lim = (int64_t)1 << 31;
  const int64_t eb = c->act_dtype == MOE_F32 ? 4 : 2;
  const int64_t wide = c->shared_inter > c->inter ? c->shared_inter : c->inter;
  if (T * c->hidden * eb >= lim) return MOE_ERR_UNSUPPORTED;
  if ((T * c->top_k + T) * wide * eb >= lim) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Activation, weight and output tensors are moved with 16-byte vector accesses.
bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool al16(const void* a, const void* b, const void* c = nullptr, const void* d = nullptr,
          const void* e = nullptr, const void* f = nullptr, const void* g = nullptr) {
  return al16(a) && al16(b) && al16(c) && al16(d) && al16(e) && al16(f) && al16(g);
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  (void)hipGetLastError();
  return MOE_ERR_HIP;
}

#define MOE_TRY(expr)                 \
  do {                                \
    const int _st = (expr);           \
    if (_st != MOE_OK) return _st;    \
  } while (0)
#define HIP_TRY(expr) MOE_TRY(hip_status(expr))

int ntiles_n(int n, int bn) { return (n + bn - 1) / bn; }

int max_mtiles(int64_t rows, int bm, int groups) {
  if (rows <= 0) return 0;
  const int64_t bound = rows / bm + groups;
  return (int)(bound < rows ? bound : rows);
}

// ------------------------------------------------------------- workspace ---

// K slices of the router GEMM: enough work-groups for the whole chip when T is
// small (a divisor of H/64, at most 64).
GemmShape router_shape(const moe_config* c, int64_t T) {
  return gemm_shape(2, act_dt(c), (int)T);
}

int router_splits(const moe_config* c, int64_t T) {
  const GemmShape sh = router_shape(c, T);
  if (sh.kind < 10) return 1;  // only the pipelined kernel splits K
  const int64_t tiles = ((T + sh.bm - 1) / sh.bm) * ((c->n_experts + sh.bn - 1) / sh.bn);
  const int nk = c->hidden / 64;
  // two rounds of 64-row tiles over the chip's CUs, or one of 128-row tiles
  const int64_t groups = sh.bm >= 128 ? kChipCUs : 2 * kChipCUs;
  int want = (int)((groups + tiles - 1) / tiles);
  if (want > 64) want = 64;
  int best = 1;
  for (int d = 1; d <= nk && d <= want; ++d)
    if (nk % d == 0) best = d;
  return best;
}

struct RouteWs { float* logits; };
void carve_route(Carver& cv, const moe_config* c, int64_t T, RouteWs& w) {
  w.logits = cv.take<float>((size_t)router_splits(c, T) * T * c->n_experts);
}

struct PermuteWs { int32_t* counts; };
void carve_permute(Carver& cv, const moe_config* c, int64_t T, PermuteWs& w) {
  const int nb = permute_blocks((int)(T * c->top_k));
  w.counts = cv.take<int32_t>((size_t)nb * c->n_experts);
}

// Tile shapes of the gate/up and down GEMMs of one grouped SwiGLU.
// A dense call (one group) passes its 256 x 256 tile count, so that a launch
// too small to fill the chip can take smaller tiles.
GemmShape shape1(const moe_config* c, int64_t rows, int groups, int I) {
  const int64_t t256 = groups == 1 ? ((rows + 255) / 256) * ntiles_n(I, 128) : 0;
  return gemm_shape(0, act_dt(c), (int)(rows / groups), t256);
}
GemmShape shape2(const moe_config* c, int64_t rows, int groups) {
  const int64_t t256 = groups == 1 ? ((rows + 255) / 256) * ntiles_n(c->hidden, 256) : 0;
  return gemm_shape(1, act_dt(c), (int)(rows / groups), t256);
}

GemmShape tile_shape1(const moe_config* c, int64_t rows, int groups, int I) {
  if (is_fp8(c)) return gemm_fp8_shape((int)(rows / groups), EPI_SWIGLU, c->hidden);
  if (is_w4(c)) return gemm_w4_shape();
  return shape1(c, rows, groups, I);
}
GemmShape tile_shape2(const moe_config* c, int64_t rows, int groups, int I, bool scatter) {
  if (is_fp8(c)) return gemm_fp8_shape((int)(rows / groups), scatter ? EPI_SCATTER : EPI_STORE, I);
  if (is_w4(c)) return gemm_w4_shape();
  return shape2(c, rows, groups);
}

// Workspace of one grouped SwiGLU over `rows` permuted rows of `groups` experts
// with intermediate size I.
struct SwigluWs {
  int4* tiles1; int* ntiles1;
  int4* tiles2; int* ntiles2;
  void* h;                    // intermediate, act dtype (bf16 and fp32 weights, 4-bit weights: bf16)
  uint8_t* hq; float* h_scales; // FP8: E4M3 intermediate + 1x128 scales, k-block-major
  uint8_t* xq; float* xs;
  float* xs_t;                // FP8: activation scales of the permuted rows, k-block-major
  float* row_w;
};
void carve_swiglu(Carver& cv, const moe_config* c, int64_t T, int64_t rows, int groups, int I,
                  bool quantize_x, bool scatter, SwigluWs& w) {
  const GemmShape g1 = tile_shape1(c, rows, groups, I);
  const GemmShape g2 = tile_shape2(c, rows, groups, I, scatter);
  // tile lists: every (m-tile, n-tile) pair of the gate/up and of the down GEMM
  w.tiles1 = cv.take<int4>((size_t)max_mtiles(rows, g1.bm, groups) * ntiles_n(I, g1.bn / 2) + 1);
  w.ntiles1 = cv.take<int>(1);
  w.tiles2 = cv.take<int4>((size_t)max_mtiles(rows, g2.bm, groups) * ntiles_n(c->hidden, g2.bn) + 1);
  w.ntiles2 = cv.take<int>(1);
  if (is_fp8(c)) {
    // the gate/up kernel writes h already quantised
    w.h = nullptr;
    w.hq = cv.take<uint8_t>((size_t)rows * I);
    w.h_scales = cv.take<float>((size_t)rows * (I / 128));
    if (quantize_x) {
      w.xq = cv.take<uint8_t>((size_t)T * c->hidden);
      w.xs = cv.take<float>((size_t)T * (c->hidden / 128));
    } else {
      w.xq = nullptr; w.xs = nullptr;
    }
    w.xs_t = cv.take<float>((size_t)rows * (c->hidden / 128));
  } else {
    w.h = cv.take<char>((size_t)rows * I * act_bytes(c));
    w.hq = nullptr; w.h_scales = nullptr; w.xq = nullptr; w.xs = nullptr; w.xs_t = nullptr;
  }
  w.row_w = scatter ? cv.take<float>((size_t)rows) : nullptr;
}

// The shared expert runs as group E of the routed launch (no launches of its
// own, no separate output) when it has the routed experts' width, the routed
// rows are stored rather than scatter-added, and T is small: a dense launch of
// at most 4 x I/128 tiles of 256 rows cannot fill the chip, while for large T
// the separate dense launch keeps its activation rows in L2 better than the
// expert-ordered grouped launch does.
constexpr int64_t kMergeSharedMaxT = 1024;
bool merge_shared(const moe_config* c, int64_t T, bool scatter) {
  // E + 1 groups must fit the tile builder's one-thread-per-group scan (1024)
  return !scatter && c->shared_inter > 0 && c->shared_inter == c->inter && c->n_experts < 1024 &&
         T <= kMergeSharedMaxT;
}

// The shared expert as a dense SwiGLU of its own: n_experts = 1, top-k 1.
moe_config shared_config(const moe_config* c) {
  moe_config sc = *c;
  sc.n_experts = 1; sc.top_k = 1; sc.inter = c->shared_inter; sc.n_group = 1; sc.topk_group = 1;
  return sc;
}

// Stored rows and the shared expert in dense launches of its own on a 256 x 256
// kernel (bf16 or FP8): the shared down GEMM runs last and its EPI_COMBINE
// epilogue also does the layer's combine, so the shared rows never reach HBM
// and the combine kernel is not launched.
bool fuse_combine(const moe_config* c, int64_t T, bool scatter) {
  if (scatter || c->shared_inter <= 0 || merge_shared(c, T, scatter)) return false;
  if (act_dt(c) != MOE_DT_BF16 || is_w4(c)) return false;
  const moe_config sc = shared_config(c);
  const GemmShape g = tile_shape2(&sc, T, 1, c->shared_inter, false);
  return is_fp8(c) ? g.kind == 2 : g.kind == 15;
}

struct ForwardWs {
  RouteWs route;
  PermuteWs perm;
  SwigluWs routed, shared;
  float* scores; int32_t* ids; float* topw;
  int32_t* offsets; int32_t* src; int32_t* inv;
  void* y; float* acc;
  void* sh_out;
};
void carve_forward(Carver& cv, const moe_config* c, int64_t T, bool scatter, ForwardWs& w) {
  const int64_t rows = T * c->top_k;
  w.scores = cv.take<float>((size_t)T * c->n_experts);
  if (router_splits(c, T) > 1) carve_route(cv, c, T, w.route);
  else w.route.logits = nullptr;
  w.ids = cv.take<int32_t>((size_t)rows);
  w.topw = cv.take<float>((size_t)rows);
  const bool merged = merge_shared(c, T, scatter);
  const int64_t rows_all = rows + (merged ? T : 0);
  w.offsets = cv.take<int32_t>((size_t)c->n_experts + 2);
  w.src = cv.take<int32_t>((size_t)rows_all);
  w.inv = cv.take<int32_t>((size_t)rows);
  carve_permute(cv, c, T, w.perm);
  carve_swiglu(cv, c, T, rows_all, c->n_experts + (merged ? 1 : 0), c->inter, true, scatter, w.routed);
  if (scatter) {
    w.y = nullptr;
    w.acc = cv.take<float>((size_t)T * c->hidden);
  } else {
    w.y = cv.take<char>((size_t)rows_all * c->hidden * act_bytes(c));
    w.acc = nullptr;
  }
  if (c->shared_inter > 0 && !merged) {
    carve_swiglu(cv, c, T, T, 1, c->shared_inter, false, false, w.shared);
    w.sh_out = cv.take<char>((size_t)T * c->hidden * act_bytes(c));
  } else {
    w.sh_out = nullptr;
  }
}

// ------------------------------------------------------------ sequences ---

int do_route(const moe_config* c, int64_t T, const void* hidden, const void* gate_w, const float* bias,
             const float* scores_in, float* scores_out, int32_t* ids, float* topw, float* logits_ws,
             hipStream_t s) {
  RouteParams rp{};
  rp.bias = bias;
  rp.topk_ids = ids;
  rp.topk_w = topw;
  rp.T = (int)T; rp.E = c->n_experts; rp.k = c->top_k;
  rp.n_group = c->n_group; rp.topk_group = c->topk_group;
  rp.scoring = c->scoring; rp.norm = c->norm_topk_prob; rp.scale = c->routed_scaling_factor;
  if (scores_in) {
    rp.logits = scores_in;
    rp.scores_given = 1;
    rp.scores_out = nullptr;
  } else {
    // Logits land in the workspace (all K slices), or, unsplit, where the
    // scores go (in place per element).
    const int parts = logits_ws ? router_splits(c, T) : 1;
    float* logits = (scores_out && parts == 1) ? scores_out : logits_ws;
    GemmParams g{};
    g.A = hidden; g.a_rows = nullptr;
    g.B = gate_w; g.b_gstride = 0;
    g.K = c->hidden; g.N = c->n_experts;
    g.C = logits;
    g.tiles = nullptr;
    g.ksplit = parts;
    g.c_split_stride = T * c->n_experts;
    const GemmShape sh = router_shape(c, T);
    g.M = (int)T;
    g.a_nrows = T;
    g.n_mtiles = (int)((T + sh.bm - 1) / sh.bm);
    g.ntn = (c->n_experts + sh.bn - 1) / sh.bn;
    HIP_TRY(launch_gemm(act_dt(c), EPI_STORE, MOE_DT_F32, g, sh, g.n_mtiles, s));
    rp.logits = logits;
    rp.n_parts = parts;
    rp.part_stride = T * c->n_experts;
    rp.scores_given = 0;
    rp.scores_out = scores_out;
  }
  HIP_TRY(launch_route(rp, s));
  return MOE_OK;
}

// m-tiles from the device list, or dense rows [0, rows) when there are no offsets.
template <class P>
void set_tiles(P& p, bool dense, int64_t rows, int bm, const int4* tiles, const int* ntiles) {
  if (dense) {
    p.tiles = nullptr; p.n_mtiles_dev = nullptr;
    p.M = (int)rows; p.n_mtiles = (int)((rows + bm - 1) / bm);
  } else {
    p.tiles = tiles; p.n_mtiles_dev = ntiles;
  }
}

// Weights of the shared expert when it runs as one more group of the routed launch.
struct SharedGroup {
  const void* w13; const float* w13_s;
  const void* w2; const float* w2_s;
  int group;
};

// One grouped SwiGLU: routed experts (offsets given) or a dense FFN over all
// rows (offsets == nullptr, the shared expert).  phase 1 launches only the
// gate/up GEMM, phase 2 only the down GEMM (0: both).
int do_swiglu(const moe_config* c, int64_t T, int64_t rows, int groups, int I, const void* hidden,
              const float* hidden_scales, const int32_t* src, const int32_t* offsets, const void* w13,
              const float* w13_s, const void* w2, const float* w2_s, int epi, const float* topk_w,
              const int32_t* inv, void* out, float* acc, const SwigluWs& w, hipStream_t s,
              hipEvent_t const* ev = nullptr, const SharedGroup* sg = nullptr, bool tiles_ready = false,
              const CombineEpi* cb = nullptr, int phase = 0) {
  auto mark = [&](int i) -> int {
    if (ev && ev[i]) return hip_status(hipEventRecord(ev[i], s));
    return MOE_OK;
  };
  const int H = c->hidden;
  if (is_fp8(c)) {
    const uint8_t* xq = (const uint8_t*)hidden;
    const float* xs = hidden_scales;
    if (!hidden_scales) {  // quantise the activations first
      HIP_TRY(launch_quantize(act_dt(c), T, H, hidden, w.xq, w.xs, s));
      xq = w.xq; xs = w.xs;
    }
    const GemmShape g1 = tile_shape1(c, rows, groups, I);
    const GemmShape g2 = tile_shape2(c, rows, groups, I, epi == MOE_EPI_SCATTER_ADD);
    const bool dense = offsets == nullptr;
    const int ntn1 = ntiles_n(I, g1.bn / 2), ntn2 = ntiles_n(H, g2.bn);
    if (!dense && !tiles_ready) {
      HIP_TRY(launch_build_tiles(offsets, groups, g1.bm, ntn1, w.tiles1, w.ntiles1, s, g2.bm, ntn2, w.tiles2,
                                 w.ntiles2));
    }
    GemmFp8Params p{};
    // the kernel reads the activation scales k-block-major over the permuted rows
    if (phase != 2) HIP_TRY(launch_gather_scales_t(xs, src, rows, H / 128, T, w.xs_t, s));
    p.A = xq; p.a_scales = w.xs_t; p.as_stride = rows; p.a_rows = src;
    p.B = (const uint8_t*)w13; p.b_scales = w13_s;
    p.b_gstride = (int64_t)2 * I * H; p.bs_gstride = (int64_t)(2 * I / 128) * (H / 128);
    if (sg) { p.B2 = (const uint8_t*)sg->w13; p.b2_scales = sg->w13_s; p.b2_group = sg->group; }
    p.K = H; p.N = I;
    // the epilogue quantises h (E4M3 + k-block-major 1x128 scales)
    p.Cq = w.hq; p.Cs = w.h_scales; p.cs_stride = rows;
    p.a_nrows = T;
    set_tiles(p, dense, rows, g1.bm, w.tiles1, w.ntiles1);
    p.ntn = ntn1;
    const int gm1 = dense ? p.n_mtiles : max_mtiles(rows, g1.bm, groups);
    MOE_TRY(mark(0));
    if (phase != 2) HIP_TRY(launch_gemm_fp8(EPI_SWIGLU, p, g1, gm1, s));
    MOE_TRY(mark(1));
    GemmFp8Params q{};
    q.A = w.hq; q.a_scales = w.h_scales; q.a_rows = nullptr; q.as_stride = rows;
    q.B = (const uint8_t*)w2; q.b_scales = w2_s;
    q.b_gstride = (int64_t)H * I; q.bs_gstride = (int64_t)(H / 128) * (I / 128);
    if (sg) { q.B2 = (const uint8_t*)sg->w2; q.b2_scales = sg->w2_s; q.b2_group = sg->group; }
    q.K = I; q.N = H;
    q.a_nrows = rows;
    set_tiles(q, dense, rows, g2.bm, w.tiles2, w.ntiles2);
    q.ntn = ntn2;
    const int gm2 = dense ? q.n_mtiles : max_mtiles(rows, g2.bm, groups);
    if (epi == MOE_EPI_SCATTER_ADD) {
      HIP_TRY(launch_row_weights(topk_w, inv, (int)rows, w.row_w, s));
      q.C = acc; q.c_rows = src; q.row_w = w.row_w;
      MOE_TRY(mark(2));
      HIP_TRY(launch_gemm_fp8(EPI_SCATTER, q, g2, gm2, s));
    } else {
      q.C = out;
      if (cb) q.comb = *cb;
      MOE_TRY(mark(2));
      if (phase != 1) HIP_TRY(launch_gemm_fp8(cb ? EPI_COMBINE : EPI_STORE, q, g2, gm2, s));
    }
    return mark(3);
  }
  if (is_w4(c)) {
    const GemmShape g1 = gemm_w4_shape(), g2 = gemm_w4_shape();
    const bool dense = offsets == nullptr;
    const int ntn1 = ntiles_n(I, g1.bn / 2), ntn2 = ntiles_n(H, g2.bn);
    if (!dense && !tiles_ready) {
      HIP_TRY(launch_build_tiles(offsets, groups, g1.bm, ntn1, w.tiles1, w.ntiles1, s, g2.bm, ntn2, w.tiles2,
                                 w.ntiles2));
    }
    GemmW4Params p{};
    p.A = hidden; p.a_rows = src;
    p.B = (const uint8_t*)w13; p.b_scales = w13_s;
    p.b_gstride = (int64_t)2 * I * (H / 2); p.bs_gstride = (int64_t)2 * I * (H / 128);
    if (sg) { p.B2 = (const uint8_t*)sg->w13; p.b2_scales = sg->w13_s; p.b2_group = sg->group; }
    p.K = H; p.N = I; p.C = w.h;
    p.a_nrows = T;
    set_tiles(p, dense, rows, g1.bm, w.tiles1, w.ntiles1);
    p.ntn = ntn1;
    MOE_TRY(mark(0));
    HIP_TRY(launch_gemm_w4(EPI_SWIGLU, MOE_DT_BF16, p, g1, dense ? p.n_mtiles : max_mtiles(rows, g1.bm, groups), s));
    MOE_TRY(mark(1));
    GemmW4Params q{};
    q.A = w.h; q.a_rows = nullptr;
    q.B = (const uint8_t*)w2; q.b_scales = w2_s;
    q.b_gstride = (int64_t)H * (I / 2); q.bs_gstride = (int64_t)H * (I / 128);
    if (sg) { q.B2 = (const uint8_t*)sg->w2; q.b2_scales = sg->w2_s; q.b2_group = sg->group; }
    q.K = I; q.N = H;
    q.a_nrows = rows;
    set_tiles(q, dense, rows, g2.bm, w.tiles2, w.ntiles2);
    q.ntn = ntn2;
    const int gm2 = dense ? q.n_mtiles : max_mtiles(rows, g2.bm, groups);
    if (epi == MOE_EPI_SCATTER_ADD) {
      HIP_TRY(launch_row_weights(topk_w, inv, (int)rows, w.row_w, s));
      q.C = acc; q.c_rows = src; q.row_w = w.row_w;
      MOE_TRY(mark(2));
      HIP_TRY(launch_gemm_w4(EPI_SCATTER, MOE_DT_F32, q, g2, gm2, s));
    } else {
      q.C = out;
      MOE_TRY(mark(2));
      HIP_TRY(launch_gemm_w4(EPI_STORE, MOE_DT_BF16, q, g2, gm2, s));
    }
    return mark(3);
  }
  const int dt = act_dt(c);
  const GemmShape g1 = shape1(c, rows, groups, I);
  const GemmShape g2 = shape2(c, rows, groups);
  const bool dense = offsets == nullptr;
  const int ntn1 = ntiles_n(I, g1.bn / 2), ntn2 = ntiles_n(H, g2.bn);
  if (!dense && !tiles_ready) {
    HIP_TRY(launch_build_tiles(offsets, groups, g1.bm, ntn1, w.tiles1, w.ntiles1, s, g2.bm, ntn2, w.tiles2,
                               w.ntiles2));
  }
  GemmParams p{};
  p.A = hidden; p.a_rows = src;
  p.B = w13; p.b_gstride = (int64_t)2 * I * H;
  if (sg) { p.B2 = sg->w13; p.b2_group = sg->group; }
  p.K = H; p.N = I; p.C = w.h;
  p.a_nrows = T;
  set_tiles(p, dense, rows, g1.bm, w.tiles1, w.ntiles1);
  p.ntn = ntn1;
  MOE_TRY(mark(0));
  if (phase != 2)
    HIP_TRY(launch_gemm(dt, EPI_SWIGLU, dt, p, g1, dense ? p.n_mtiles : max_mtiles(rows, g1.bm, groups), s));
  MOE_TRY(mark(1));

  GemmParams q{};
  q.A = w.h; q.a_rows = nullptr;
  q.B = w2; q.b_gstride = (int64_t)H * I;
  if (sg) { q.B2 = sg->w2; q.b2_group = sg->group; }
  q.K = I; q.N = H;
  q.a_nrows = rows;
  set_tiles(q, dense, rows, g2.bm, w.tiles2, w.ntiles2);
  q.ntn = ntn2;
  const int gm2 = dense ? q.n_mtiles : max_mtiles(rows, g2.bm, groups);
  if (epi == MOE_EPI_SCATTER_ADD) {
    HIP_TRY(launch_row_weights(topk_w, inv, (int)rows, w.row_w, s));
    q.C = acc; q.c_rows = src; q.row_w = w.row_w;
    MOE_TRY(mark(2));
    HIP_TRY(launch_gemm(dt, EPI_SCATTER, MOE_DT_F32, q, g2, gm2, s));
  } else {
    q.C = out;
    if (cb) q.comb = *cb;
    MOE_TRY(mark(2));
    if (phase != 1) HIP_TRY(launch_gemm(dt, cb ? EPI_COMBINE : EPI_STORE, dt, q, g2, gm2, s));
  }
  return mark(3);
}

}  // namespace

// ================================================================== ABI ===

extern "C" {

int moe_version(void) { return MOE355_VERSION; }

const char* moe_strerror(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_CONFIG: return "inconsistent layer configuration";
    case MOE_ERR_UNSUPPORTED: return "configuration not supported by this library";
    case MOE_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case MOE_ERR_HIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

int moe_validate_config(const moe_config* cfg) { return check_cfg(cfg); }

size_t moe_workspace_size(const moe_config* c, int64_t T, int32_t op) {
  if (check_cfg(c) != MOE_OK || T < 0 || check_T(c, T) != MOE_OK) return 0;
  if (T == 0) return 0;
  Carver cv(nullptr);
  switch (op) {
    case MOE_OP_ROUTE: { RouteWs w; carve_route(cv, c, T, w); break; }
    case MOE_OP_PERMUTE: { PermuteWs w; carve_permute(cv, c, T, w); break; }
    case MOE_OP_GROUPED_SWIGLU: {
      // Sized for the routed experts and for a one-group shared call of the same T.
      SwigluWs w;
      Carver a(nullptr), b(nullptr);
      carve_swiglu(a, c, T, T * c->top_k, c->n_experts, c->inter, true, true, w);
      if (c->shared_inter > 0) carve_swiglu(b, c, T, T, 1, c->shared_inter, true, true, w);
      return a.used > b.used ? a.used : b.used;
    }
    case MOE_OP_COMBINE: return 0;
    case MOE_OP_FORWARD: {
      ForwardWs a, b;
      Carver ca(nullptr), cb(nullptr);
      carve_forward(ca, c, T, false, a);
      carve_forward(cb, c, T, true, b);
      return ca.used > cb.used ? ca.used : cb.used;
    }
    default: return 0;
  }
  return cv.used;
}

static int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return MOE_OK;
  if (!ws || ((uintptr_t)ws % kAlign) || ws_bytes < need) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

int moe_route(const moe_config* c, int64_t T, const void* hidden, const void* gate_w, const float* bias,
              const float* scores_in, float* scores_out, int32_t* topk_ids, float* topk_w, void* ws,
              size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_cfg(c));
  MOE_TRY(check_T(c, T));
  if (!topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
  if (!scores_in && (!hidden || !gate_w)) return MOE_ERR_INVALID_ARG;
  if (!scores_in && !al16(hidden, gate_w)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  RouteWs w{};
  // Without scores_out the logits need the workspace; with scores_out a
  // workspace is optional and only enables the split-K router GEMM.
  if (!scores_in && (!scores_out || ws)) {
    Carver probe(nullptr);
    carve_route(probe, c, T, w);
    MOE_TRY(check_ws(ws, ws_bytes, probe.used));
    Carver cv(ws);
    carve_route(cv, c, T, w);
  }
  return do_route(c, T, hidden, gate_w, bias, scores_in, scores_out, topk_ids, topk_w, w.logits, stream);
}

int moe_permute(const moe_config* c, int64_t T, const int32_t* topk_ids, int32_t* expert_offsets,
                int32_t* permuted_src, int32_t* inv_perm, void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_cfg(c));
  MOE_TRY(check_T(c, T));
  if (!topk_ids || !expert_offsets || !permuted_src || !inv_perm) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  Carver probe(nullptr);
  PermuteWs w;
  carve_permute(probe, c, T, w);
  MOE_TRY(check_ws(ws, ws_bytes, probe.used));
  Carver cv(ws);
  carve_permute(cv, c, T, w);
  HIP_TRY(launch_permute(topk_ids, (int)(T * c->top_k), c->top_k, c->n_experts, w.counts, expert_offsets,
                         permuted_src, inv_perm, stream));
  return MOE_OK;
}

int moe_grouped_swiglu(const moe_config* c, int64_t T, const void* hidden, const float* hidden_scales,
                       const int32_t* permuted_src, const int32_t* expert_offsets, const void* w13,
                       const float* w13_scales, const void* w2, const float* w2_scales, int32_t epilogue,
                       const float* topk_w, const int32_t* inv_perm, void* expert_out, float* acc, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_cfg(c));
  MOE_TRY(check_T(c, T));
  if (epilogue != MOE_EPI_STORE_ROWS && epilogue != MOE_EPI_SCATTER_ADD) return MOE_ERR_INVALID_ARG;
  if (!hidden || !expert_offsets || !w13 || !w2) return MOE_ERR_INVALID_ARG;
  if (has_scales(c) && (!w13_scales || !w2_scales)) return MOE_ERR_INVALID_ARG;
  if (hidden_scales && !is_fp8(c)) return MOE_ERR_INVALID_ARG;
  if (epilogue == MOE_EPI_STORE_ROWS && !expert_out) return MOE_ERR_INVALID_ARG;
  if (epilogue == MOE_EPI_SCATTER_ADD && (!acc || !topk_w || !inv_perm)) return MOE_ERR_INVALID_ARG;
  if (!al16(hidden, w13, w2, expert_out, acc)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  const int64_t rows = T * c->top_k;
  const bool scatter = epilogue == MOE_EPI_SCATTER_ADD;
  Carver probe(nullptr);
  SwigluWs w;
  carve_swiglu(probe, c, T, rows, c->n_experts, c->inter, hidden_scales == nullptr, scatter, w);
  MOE_TRY(check_ws(ws, ws_bytes, probe.used));
  Carver cv(ws);
  carve_swiglu(cv, c, T, rows, c->n_experts, c->inter, hidden_scales == nullptr, scatter, w);
  return do_swiglu(c, T, rows, c->n_experts, c->inter, hidden, hidden_scales, permuted_src, expert_offsets, w13,
                   w13_scales, w2, w2_scales, epilogue, topk_w, inv_perm, expert_out, acc, w, stream);
}

int moe_combine(const moe_config* c, int64_t T, const void* expert_out, const float* acc, const int32_t* inv_perm,
                const float* topk_w, const void* shared_out, void* out, hipStream_t stream) {
  MOE_TRY(check_cfg(c));
  MOE_TRY(check_T(c, T));
  if (!out) return MOE_ERR_INVALID_ARG;
  if (expert_out && (!inv_perm || !topk_w)) return MOE_ERR_INVALID_ARG;
  if (!al16(expert_out, acc, shared_out, out)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  HIP_TRY(launch_combine(act_dt(c), (int)T, c->hidden, c->top_k, expert_out, acc, inv_perm, topk_w, shared_out,
                         out, stream));
  return MOE_OK;
}

int moe_forward(const moe_config* c, int64_t T, const void* hidden, const void* gate_w, const float* bias,
                const void* w13, const float* w13_scales, const void* w2, const float* w2_scales,
                const void* sh_w13, const float* sh_w13_scales, const void* sh_w2, const float* sh_w2_scales,
                void* out, const moe_forward_opts* opts, void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_cfg(c));
  MOE_TRY(check_T(c, T));
  if (!hidden || !gate_w || !w13 || !w2 || !out) return MOE_ERR_INVALID_ARG;
  if (has_scales(c) && (!w13_scales || !w2_scales)) return MOE_ERR_INVALID_ARG;
  if (c->shared_inter > 0 && (!sh_w13 || !sh_w2)) return MOE_ERR_INVALID_ARG;
  if (c->shared_inter > 0 && has_scales(c) && (!sh_w13_scales || !sh_w2_scales)) return MOE_ERR_INVALID_ARG;
  if (!al16(hidden, gate_w, w13, w2, sh_w13, sh_w2, out)) return MOE_ERR_INVALID_ARG;
  const int epi = opts ? opts->epilogue : MOE_EPI_STORE_ROWS;
  if (epi != MOE_EPI_STORE_ROWS && epi != MOE_EPI_SCATTER_ADD) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  const bool scatter = epi == MOE_EPI_SCATTER_ADD;
  Carver probe(nullptr);
  ForwardWs w;
  carve_forward(probe, c, T, scatter, w);
  MOE_TRY(check_ws(ws, ws_bytes, probe.used));
  Carver cv(ws);
  carve_forward(cv, c, T, scatter, w);

  const bool merged = merge_shared(c, T, scatter);
  const int E = c->n_experts;
  float* scores = (opts && opts->scores) ? opts->scores : w.scores;
  int32_t* ids = (opts && opts->topk_ids) ? opts->topk_ids : w.ids;
  float* topw = (opts && opts->topk_w) ? opts->topk_w : w.topw;
  // merged: the permutation is extended by the shared group, so it lives in the
  // workspace and is copied out when asked for
  int32_t* offsets = (!merged && opts && opts->expert_offsets) ? opts->expert_offsets : w.offsets;
  int32_t* src = (!merged && opts && opts->permuted_src) ? opts->permuted_src : w.src;
  int32_t* inv = (opts && opts->inv_perm) ? opts->inv_perm : w.inv;
  const int64_t rows = T * c->top_k;
  const int64_t rows_all = rows + (merged ? T : 0);

  MOE_TRY(do_route(c, T, hidden, gate_w, bias, nullptr, scores, ids, topw, w.route.logits, stream));
  // Small batches: the permutation's one work-group also writes both GEMMs' tile
  // lists (when their m-tiles have one height).
  const int groups = E + (merged ? 1 : 0);
  const GemmShape g1 = tile_shape1(c, rows_all, groups, c->inter);
  const GemmShape g2 = tile_shape2(c, rows_all, groups, c->inter, scatter);
  TileLists tl;
  if (g1.bm == g2.bm) {
    tl.bm = g1.bm;
    tl.ntn = ntiles_n(c->inter, g1.bn / 2); tl.tiles = w.routed.tiles1; tl.n_tiles = w.routed.ntiles1;
    tl.ntn2 = ntiles_n(c->hidden, g2.bn); tl.tiles2 = w.routed.tiles2; tl.n_tiles2 = w.routed.ntiles2;
  }
  bool tiles_ready = false;
  HIP_TRY(launch_permute(ids, (int)rows, c->top_k, E, w.perm.counts, offsets, src, inv, stream,
                         merged ? (int)T : 0, tl.bm > 0 ? &tl : nullptr, &tiles_ready));
  if (merged) {
    if (opts && opts->expert_offsets)
      HIP_TRY(hipMemcpyAsync(opts->expert_offsets, offsets, (size_t)(E + 1) * sizeof(int32_t),
                             hipMemcpyDeviceToDevice, stream));
    if (opts && opts->permuted_src)
      HIP_TRY(hipMemcpyAsync(opts->permuted_src, src, (size_t)rows * sizeof(int32_t), hipMemcpyDeviceToDevice,
                             stream));
  }

  // Shared expert first: its quantised activations (FP8) are reused by the routed experts.
  const float* xs = nullptr;
  const void* xin = hidden;
  if (is_fp8(c)) {
    HIP_TRY(launch_quantize(act_dt(c), T, c->hidden, hidden, w.routed.xq, w.routed.xs, stream));
    xin = w.routed.xq;
    xs = w.routed.xs;
  }
  const bool fused = fuse_combine(c, T, scatter);
  const moe_config sc = shared_config(c);
  if (c->shared_inter > 0 && !merged) {
    MOE_TRY(do_swiglu(&sc, T, T, 1, c->shared_inter, xin, xs, nullptr, nullptr, sh_w13, sh_w13_scales, sh_w2,
                      sh_w2_scales, MOE_EPI_STORE_ROWS, nullptr, nullptr, w.sh_out, nullptr, w.shared, stream,
                      nullptr, nullptr, false, nullptr, fused ? 1 : 0));
  }
  if (scatter) HIP_TRY(launch_fill_zero(w.acc, T * c->hidden, stream));
  const SharedGroup sg{sh_w13, sh_w13_scales, sh_w2, sh_w2_scales, E};
  MOE_TRY(do_swiglu(c, T, rows_all, groups, c->inter, xin, xs, src, offsets, w13, w13_scales, w2, w2_scales, epi,
                    topw, inv, w.y, w.acc, w.routed, stream, opts ? opts->events : nullptr, merged ? &sg : nullptr,
                    tiles_ready));
  if (fused) {
    // the shared down GEMM last: its epilogue combines the routed rows with its
    // own and writes the layer output (its gate/up GEMM ran before the routed
    // GEMMs, which measured slightly faster than running it here)
    CombineEpi cb;
    cb.rows = w.y; cb.inv = inv; cb.w = topw; cb.k = c->top_k; cb.out = out;
    return do_swiglu(&sc, T, T, 1, c->shared_inter, xin, xs, nullptr, nullptr, sh_w13, sh_w13_scales, sh_w2,
                     sh_w2_scales, MOE_EPI_STORE_ROWS, nullptr, nullptr, w.sh_out, nullptr, w.shared, stream, nullptr,
                     nullptr, false, &cb, 2);
  }
  const void* shared_rows = merged ? (const void*)((const char*)w.y + rows * c->hidden * act_bytes(c)) : w.sh_out;
  HIP_TRY(launch_combine(act_dt(c), (int)T, c->hidden, c->top_k, w.y, w.acc, inv, topw, shared_rows, out, stream));
  return MOE_OK;
}

}  // extern "C"

// --------------------------------------------- forward without allocation ---

namespace {

// The scratch of moe_forward_static: one copy on every device the library
// runs on, held until the process ends.  Host code never passes `scratch`
// itself to a kernel (on the host it names a stand-in, not device memory);
// it uses the device address hipGetSymbolAddress returns for each device.
static __device__ __align__(256) char scratch[MOE_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of this device's scratch, looked up once per device with
// that device current.
int scratch_for(int dev, void** ptr) {
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return MOE_ERR_HIP;
    }
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_forward_static(const moe_config* c, int64_t T, const void* hidden, const void* gate_w, const float* bias,
                       const void* w13, const float* w13_scales, const void* w2, const float* w2_scales,
                       const void* sh_w13, const float* sh_w13_scales, const void* sh_w2, const float* sh_w2_scales,
                       void* out, const moe_forward_opts* opts, hipStream_t stream) {
  MOE_TRY(check_cfg(c));
  MOE_TRY(check_T(c, T));
  const int epi = opts ? opts->epilogue : MOE_EPI_STORE_ROWS;
  if (epi != MOE_EPI_STORE_ROWS && epi != MOE_EPI_SCATTER_ADD) return MOE_ERR_INVALID_ARG;
  if (T == 0) return moe_forward(c, T, hidden, gate_w, bias, w13, w13_scales, w2, w2_scales, sh_w13, sh_w13_scales,
                                 sh_w2, sh_w2_scales, out, opts, nullptr, 0, stream);
  // The batch must fit the static scratch: rejected before touching the device.
  Carver probe(nullptr);
  ForwardWs w;
  carve_forward(probe, c, T, epi == MOE_EPI_SCATTER_ADD, w);
  if (probe.used > (size_t)MOE_STATIC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  int cur = 0;
  HIP_TRY(hipGetDevice(&cur));
  if (stream) {
    hipDevice_t sdev = 0;
    HIP_TRY(hipStreamGetDevice(stream, &sdev));
    if ((int)sdev != cur) return MOE_ERR_INVALID_ARG;
  }
  void* ws = nullptr;
  MOE_TRY(scratch_for(cur, &ws));
  return moe_forward(c, T, hidden, gate_w, bias, w13, w13_scales, w2, w2_scales, sh_w13, sh_w13_scales, sh_w2,
                     sh_w2_scales, out, opts, ws, (size_t)MOE_STATIC_SCRATCH_BYTES, stream);
}

int moe_load_balance(const moe_config* c, const int32_t* expert_offsets, float* bias, float gamma,
                     moe_load_stats* stats, hipStream_t stream) {
  MOE_TRY(check_cfg(c));
  if (!expert_offsets) return MOE_ERR_INVALID_ARG;
  if (!isfinite(gamma) || gamma < 0.0f) return MOE_ERR_INVALID_ARG;
  if (!bias && !stats) return MOE_OK;
  HIP_TRY(launch_load_balance(expert_offsets, c->n_experts, bias, gamma, stats, stream));
  return MOE_OK;
}

int moe_quantize_fp8_1x128(int64_t rows, int64_t cols, const void* in, int32_t in_dtype, uint8_t* codes,
                           float* scales, hipStream_t stream) {
  if (rows < 0 || cols < 0 || (cols % 128)) return MOE_ERR_INVALID_ARG;
  if (in_dtype != MOE_F32 && in_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (rows == 0 || cols == 0) return MOE_OK;
  if (!in || !codes || !scales) return MOE_ERR_INVALID_ARG;
  if (!al16(in) || ((uintptr_t)codes & 7u)) return MOE_ERR_INVALID_ARG;
  HIP_TRY(launch_quantize(in_dtype == MOE_F32 ? MOE_DT_F32 : MOE_DT_BF16, rows, cols, in, codes, scales, stream));
  return MOE_OK;
}

}  // extern "C"
