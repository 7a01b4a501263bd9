/*
 * moe355.h - C ABI of a DeepSeek-style mixture-of-experts layer forward for
 * AMD MI355X (gfx950).
 *
 * The layer (MoE inference walkthrough, zhiyuanblog.org/blog/moe-inference, §3;
 * DeepSeek-V3 MoE/MLA lab, gsyq.cn/news/313569, §4 route()):
 *   1. router GEMM          logits = hidden_states @ gate.weight^T       (T,E)
 *   2. scoring + top-k      softmax, or sigmoid with a score-correction bias,
 *                           group-limited top-k, optional renormalisation,
 *                           routed_scaling_factor
 *   3. permutation          copies of every token ordered by expert
 *   4. grouped SwiGLU GEMM  per expert: SiLU(x W1^T) * (x W3^T) W2^T,
 *                           plus the always-on shared expert
 *   5. combine              out[t] = sum_j w[t,j] y(t, e_j) + shared(t)
 *
 * Conventions, for every entry point:
 *   - every tensor pointer is a DEVICE pointer owned by the caller; tensors are
 *     row-major and contiguous; the library never allocates, frees or keeps
 *     device memory, and never synchronises the host;
 *   - every call enqueues its kernels on `stream` and returns at once; results
 *     are ready when the stream reaches that point;
 *   - weights are stored (out, in): gate.weight (E,H); w13 (E,2I,H) with the
 *     gate projection (w1) in rows [0,I) and the up projection (w3) in rows
 *     [I,2I); w2 (E,H,I); shared gate_up (2Is,H) split the same way; shared
 *     down (H,Is) (walkthrough §2.2-§2.3 stacked storage, §3.3 x @ w.T);
 *   - index tensors are int32; T*k < 2^31; the hidden rows (T*H elements) and
 *     the intermediate rows ((T*k + T) * max(I, Is) elements) span less than
 *     2^31 bytes in the activation dtype, and so does every weight matrix (one
 *     expert's w13 or w2, the shared expert's, gate.weight) in its storage
 *     type (MOE_ERR_UNSUPPORTED otherwise): the GEMMs address each with 32-bit
 *     buffer offsets;
 *   - activation, weight and output tensors (hidden, gate_w, w13, w2, sh_w13,
 *     sh_w2, expert_out, acc, shared_out, out, quantiser input) start on a
 *     16-byte boundary, E4M3 code outputs on an 8-byte boundary, every other
 *     array on a 4-byte boundary (MOE_ERR_INVALID_ARG otherwise);
 *   - arguments are validated before anything is launched; a failed check
 *     returns a negative moe_status and launches nothing; T == 0 returns MOE_OK
 *     and launches nothing; a failed launch returns MOE_ERR_HIP (the HIP error
 *     is cleared);
 *   - workspace: `ws` is device memory of at least moe_workspace_size(cfg, T,
 *     op) bytes, 256-byte aligned, owned by the caller; its contents on entry
 *     do not matter and on return are unspecified.  Calls that share one
 *     workspace must be ordered on one stream.
 */
#ifndef MOE355_H
#define MOE355_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE355_VERSION 1

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* NULL required pointer, negative size, bad enum   */
  MOE_ERR_CONFIG = -2,      /* routing config inconsistent (E % n_group, k, ...) */
  MOE_ERR_UNSUPPORTED = -3, /* valid layer this library does not implement       */
  MOE_ERR_WORKSPACE = -4,   /* workspace NULL, too small or misaligned           */
  MOE_ERR_HIP = -5          /* a kernel launch failed                            */
} moe_status;

typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_scoring;

/* MOE_INT4: signed 4-bit expert weights (walkthrough §8 quantisation table,
 * W4A16), two's complement in [-8, 7], two per byte: input column 2j in the
 * low nibble (bits 0-3) of byte j of its row, column 2j+1 in the high nibble;
 * a weight matrix stored (out, in) is (out, in/2) bytes, with one fp32 scale
 * per output row and 128 input columns, stored group-major, (in/128, out);
 * value = q * scale. */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2, MOE_INT4 = 3 } moe_dtype;

typedef enum { MOE_EPI_STORE_ROWS = 0, MOE_EPI_SCATTER_ADD = 1 } moe_epilogue;

typedef enum {
  MOE_OP_ROUTE = 0,
  MOE_OP_PERMUTE = 1,
  MOE_OP_GROUPED_SWIGLU = 2,
  MOE_OP_COMBINE = 3,
  MOE_OP_FORWARD = 4
} moe_op;

/*
 * Layer configuration (walkthrough §1.3 MoE config keys; V3 lab page §3
 * moe_router.json).
 *   hidden, inter        H and I; multiples of 64 (of 128 for FP8 and
 *                        4-bit weights)
 *   n_experts            E, 1..1024
 *   top_k                k, 1..min(E, 32)
 *   n_group, topk_group  E % n_group == 0; 1 <= topk_group <= n_group; when
 *                        n_group > 1 every group holds >= 2 experts and
 *                        k <= topk_group * E / n_group.  n_group == 1 is plain
 *                        (greedy) top-k.
 *   shared_inter         Is = n_shared * shared expert intermediate size;
 *                        0 = no shared expert; multiple of 64 (128 for FP8
 *                        and 4-bit weights)
 *   scoring              moe_scoring
 *   norm_topk_prob       0/1: divide the k weights by their sum
 *   routed_scaling_factor  multiplies every routing weight
 *   act_dtype            dtype of hidden_states, gate.weight and the output:
 *                        MOE_F32 or MOE_BF16
 *   weight_dtype         dtype of routed and shared expert weights: equal to
 *                        act_dtype, or MOE_FP8_E4M3 with act_dtype MOE_BF16
 *                        (E4M3 codes + one fp32 scale per 128x128 block;
 *                        activations are then quantised to E4M3 per 1x128 tile
 *                        inside the layer; the router stays in bf16), or
 *                        MOE_INT4 with act_dtype MOE_BF16 (4-bit codes + one
 *                        fp32 scale per weight row and 128 input columns;
 *                        activations stay bf16, the intermediate is rounded
 *                        to bf16; the router stays in bf16)
 *   out_dtype            must equal act_dtype
 */
typedef struct moe_config {
  int32_t hidden;
  int32_t inter;
  int32_t n_experts;
  int32_t top_k;
  int32_t n_group;
  int32_t topk_group;
  int32_t shared_inter;
  int32_t scoring;
  int32_t norm_topk_prob;
  float routed_scaling_factor;
  int32_t act_dtype;
  int32_t weight_dtype;
  int32_t out_dtype;
} moe_config;

/* Optional outputs and options of moe_forward.  Every pointer may be NULL. */
typedef struct moe_forward_opts {
  int32_t epilogue;        /* moe_epilogue used for the routed experts         */
  float* scores;           /* [T,E] fp32 scores after softmax/sigmoid, pre-bias */
  int32_t* topk_ids;       /* [T,k]                                             */
  float* topk_w;           /* [T,k]                                             */
  int32_t* expert_offsets; /* [E+1]                                             */
  int32_t* permuted_src;   /* [T*k]                                             */
  int32_t* inv_perm;       /* [T*k]                                             */
  /* Timing hooks: events the caller created with hipEventCreate; any may be
   * NULL.  events[0]/[1] are recorded on `stream` right before/after the
   * routed experts' gate/up GEMM (with its SiLU*up epilogue), events[2]/[3]
   * right before/after their down GEMM.  When shared_inter == inter, E < 1024,
   * T <= 1024 and the rows are stored, the shared expert runs as one more group
   * of these two launches, so the events bracket it too. */
  hipEvent_t events[4];
} moe_forward_opts;

/* Bytes of workspace `op` needs for T tokens (0 when none); 0 also for an
 * invalid config (moe_validate_config tells why). */
size_t moe_workspace_size(const moe_config* cfg, int64_t T, int32_t op);

/* MOE_OK or the moe_status a call with this config would return. */
int moe_validate_config(const moe_config* cfg);

/*
 * Router GEMM + scoring + group-limited top-k + routing weights
 * (walkthrough §2.1, §3.1; V3 lab page §4 route(); DeepSeek V3/R1 overview,
 * xxqk.cn/news/389306, §2.2).
 *   hidden     [T,H] act_dtype (ignored when scores_in != NULL)
 *   gate_w     [E,H] act_dtype (ignored when scores_in != NULL)
 *   bias       [E] fp32 e_score_correction_bias, or NULL (= 0)
 *   scores_in  [T,E] fp32 scores, or NULL; when given, the GEMM and the
 *              scoring are skipped and selection runs on these scores
 *   scores_out [T,E] fp32 scores (softmax or sigmoid, before the bias), or NULL
 *   topk_ids   [T,k] selected experts, by descending s+b, ties to the lower id
 *   topk_w     [T,k] s[e] (unbiased) / sum_j s[e_j] if norm_topk_prob, times
 *              routed_scaling_factor
 * Selection: c = fp32(s + b); for n_group > 1 a group scores
 * fp32(c_first + c_second) of its two largest c; the topk_group best groups
 * (ties to the lower group) are kept; the k best c in kept groups win.
 * The router GEMM accumulates in fp32; given a workspace, for bf16 it may
 * split H into slices whose partial logits (kept in ws) are added in slice
 * order: the logits are deterministic for a given config and T, and those of
 * moe_forward equal those of moe_route with a workspace.
 *   ws         moe_workspace_size(cfg, T, MOE_OP_ROUTE) bytes; unused when
 *              scores_in is given; optional when scores_out is given (NULL
 *              keeps the router GEMM unsplit and writes the logits in place)
 */
int moe_route(const moe_config* cfg, int64_t T, const void* hidden, const void* gate_w,
              const float* bias, const float* scores_in, float* scores_out,
              int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes,
              hipStream_t stream);

/*
 * Token permutation (walkthrough §3.2): a stable sort of the T*k copies
 * a = t*k + j by expert topk_ids[a].
 *   topk_ids        [T,k] int32 in [0,E); a token lists k distinct experts
 *   expert_offsets  [E+1] bucket starts (expert_first_token_offset), empty
 *                   experts included; expert_offsets[E] = T*k
 *   permuted_src    [T*k] token of every permuted row
 *   inv_perm        [T*k] permuted row of copy a (inv_permuted_idx)
 * Deterministic: rows inside a bucket are in ascending token order.
 * Ids outside [0,E) are a caller error; they are clamped, not reported.
 */
int moe_permute(const moe_config* cfg, int64_t T, const int32_t* topk_ids,
                int32_t* expert_offsets, int32_t* permuted_src, int32_t* inv_perm,
                void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Grouped SwiGLU expert FFN over the permuted rows (walkthrough §3.3.1 and its
 * one-kernel grouped GEMM segmented by expert offsets): for every expert e and
 * row p in [expert_offsets[e], expert_offsets[e+1]):
 *   x_p = hidden[permuted_src[p]]   (permuted_src == NULL: x_p = hidden[p],
 *                                    which needs expert_offsets[E] <= T)
 *   y_p = (SiLU(x_p w13[e][0:I]^T) * (x_p w13[e][I:2I]^T)) w2[e]^T
 * in fp32 accumulation, SiLU and product in fp32, the intermediate rounded to
 * the activation dtype (bf16, or E4M3 with 1x128 scales for FP8 weights;
 * bf16 for 4-bit weights, whose codes are applied exactly: each 128-column
 * group's dot product is accumulated in fp32 and multiplied by its scale).
 *   hidden         [T,H] act_dtype, or E4M3 codes when hidden_scales != NULL
 *   hidden_scales  [T,H/128] fp32 1x128 scales of E4M3 codes, or NULL
 *   permuted_src, expert_offsets   as produced by moe_permute; the number of
 *                  rows is expert_offsets[E] <= T*k; a permuted_src entry
 *                  outside [0,T) is a caller error: its row reads zeros (no
 *                  access outside hidden or hidden_scales), it is not reported
 *   w13, w2        weight_dtype; w13_scales [E,2I/128,H/128] and
 *                  w2_scales [E,H/128,I/128] fp32 for FP8 weights;
 *                  4-bit weights: w13 [E,2I,H/2] and w2 [E,H,I/2] bytes with
 *                  w13_scales [E,H/128,2I] and w2_scales [E,I/128,H] fp32;
 *                  NULL for bf16 / fp32 weights
 *   epilogue       MOE_EPI_STORE_ROWS: expert_out[p] = y_p, [T*k,H] act_dtype
 *                  MOE_EPI_SCATTER_ADD: acc[permuted_src[p]] += w_p * y_p with
 *                  w_p = topk_w[a] for the copy a with inv_perm[a] = p; acc is
 *                  [T,H] fp32 and is added to, not overwritten; fp32 atomics,
 *                  so the summation order is not fixed
 * The shared expert is this call with a config whose n_experts = 1,
 * top_k = 1, inter = shared_inter, expert_offsets = {0, T} and
 * permuted_src = NULL.
 */
int moe_grouped_swiglu(const moe_config* cfg, int64_t T, const void* hidden,
                       const float* hidden_scales, const int32_t* permuted_src,
                       const int32_t* expert_offsets, const void* w13,
                       const float* w13_scales, const void* w2, const float* w2_scales,
                       int32_t epilogue, const float* topk_w, const int32_t* inv_perm,
                       void* expert_out, float* acc, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/*
 * Un-permute and combine (walkthrough §3.4):
 *   out[t] = acc[t] + sum_j topk_w[t,j] * expert_out[inv_perm[t*k+j]] + shared_out[t]
 * with each of the three terms left out when its pointer is NULL, summed in
 * fp32 and rounded once to act_dtype.
 *   expert_out [T*k,H] act_dtype or NULL (then inv_perm, topk_w may be NULL)
 *   acc        [T,H] fp32 or NULL
 *   shared_out [T,H] act_dtype or NULL
 *   out        [T,H] act_dtype; may alias neither input
 */
int moe_combine(const moe_config* cfg, int64_t T, const void* expert_out, const float* acc,
                const int32_t* inv_perm, const float* topk_w, const void* shared_out,
                void* out, hipStream_t stream);

/*
 * The whole layer (walkthrough §3: routing §3.1, permutation §3.2, grouped
 * expert GEMMs and the shared expert §3.3, combine §3.4, the shape timeline
 * of §3.5; V3 lab page §4 route()): moe_route, moe_permute,
 * moe_grouped_swiglu for the routed experts and for the shared expert,
 * moe_combine, all on `stream`.  With FP8 weights x is quantised once
 * (1x128) for the routed and the shared experts, the router reads the
 * unquantised x (walkthrough §8: the gate is not quantised), and h is
 * quantised after SiLU(gate) * up.
 *   hidden [T,H], gate_w [E,H] act_dtype; bias [E] fp32 or NULL;
 *   w13, w2 (+ scales) as in moe_grouped_swiglu; sh_w13 [2Is,H], sh_w2 [H,Is]
 *   (+ scales [2Is/128,H/128], [H/128,Is/128] for FP8; packed [2Is,H/2],
 *   [H,Is/2] with scales [H/128,2Is], [Is/128,H] for 4-bit weights), NULL
 *   when Is == 0;
 *   out [T,H] act_dtype; opts may be NULL (store-rows epilogue, no extra
 *   outputs).
 * The result equals that of the staged calls bit for bit.  Where the shared
 * expert runs as dense launches of 256 x 256 tiles with stored rows, its down
 * GEMM runs last and does the combine in its epilogue (same sums, same order),
 * so no combine launch and no shared-expert rows in memory.
 */
int moe_forward(const moe_config* cfg, int64_t T, const void* hidden, const void* gate_w,
                const float* bias, const void* w13, const float* w13_scales, const void* w2,
                const float* w2_scales, const void* sh_w13, const float* sh_w13_scales,
                const void* sh_w2, const float* sh_w2_scales, void* out,
                const moe_forward_opts* opts, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, results and launch sequence as moe_forward, without `ws`: the
 * workspace is a static device buffer of MOE_STATIC_SCRATCH_BYTES inside the
 * library, one copy per device, held until the process ends.  The call
 * allocates nothing (no hipMalloc, no hipFree, no allocating library routine).
 *   - a batch whose workspace (moe_workspace_size(cfg, T, MOE_OP_FORWARD) for
 *     the epilogue in opts) exceeds MOE_STATIC_SCRATCH_BYTES is rejected with
 *     MOE_ERR_WORKSPACE before anything touches the device; at V3 dimensions
 *     (H 7168, E 256, I = Is = 2048, k 8) that allows T up to 256 in bf16;
 *   - `stream` must belong to the current device (MOE_ERR_INVALID_ARG
 *     otherwise); the buffer's device address is looked up once per device
 *     (MOE_ERR_HIP if that fails);
 *   - every call on one device shares that device's buffer: calls that
 *     overlap on one device (other streams, other host threads) race, so
 *     order them on one stream.  The buffer keeps the last call's contents;
 *     the layer clears what it needs cleared with kernels of its own.
 */
#define MOE_STATIC_SCRATCH_BYTES (64u << 20)
int moe_forward_static(const moe_config* cfg, int64_t T, const void* hidden, const void* gate_w,
                       const float* bias, const void* w13, const float* w13_scales, const void* w2,
                       const float* w2_scales, const void* sh_w13, const float* sh_w13_scales,
                       const void* sh_w2, const float* sh_w2_scales, void* out,
                       const moe_forward_opts* opts, hipStream_t stream);

/*
 * Dynamic 1x128 E4M3 quantisation of activations (MoA routing + FP8
 * inference, blog.hotdry.top, FP8 section: 1x128 activation tiles; V3 lab
 * page §3 activation_scheme dynamic): per row and 128-column tile,
 * scale = fp32(amax / 448) (1 for an all-zero tile) and
 * code = E4M3FN(fp32(v / scale)), rounded to nearest even, saturated to +-448.
 *   in     [rows, cols] in_dtype (MOE_F32 or MOE_BF16); cols % 128 == 0
 *   codes  [rows, cols] uint8;  scales [rows, cols/128] fp32
 */
int moe_quantize_fp8_1x128(int64_t rows, int64_t cols, const void* in, int32_t in_dtype,
                           uint8_t* codes, float* scales, hipStream_t stream);

/* Expert load of one routed batch (V3 lab page §4 balance check). */
typedef struct moe_load_stats {
  int32_t rows;   /* expert_offsets[E] - expert_offsets[0]                      */
  int32_t min;    /* smallest per-expert count                                  */
  int32_t max;    /* largest per-expert count                                   */
  int32_t empty;  /* experts with no rows                                       */
  float mean;     /* rows / E                                                   */
  float cv;       /* std / mean, std with n - 1 (0 when E == 1 or rows == 0)    */
} moe_load_stats;

/*
 * Auxiliary-loss-free balancing step and load statistics (DeepSeek V3/R1
 * overview, xxqk.cn/news/389306, §2.2: the routing bias of an overloaded
 * expert is lowered by a fixed step, that of an underloaded one raised; V3 lab
 * page §4: per-expert counts, min, max and coefficient of variation).
 *   expert_offsets [E+1] as produced by moe_permute (or moe_forward's opts)
 *   bias   [E] fp32 e_score_correction_bias, updated in place, or NULL:
 *          share = fp32(rows / E), b_e = fp32(b_e + gamma * sign(share - count_e))
 *   gamma  step size, finite and >= 0
 *   stats  one moe_load_stats in device memory, or NULL
 * One kernel on `stream`; needs no workspace.  E <= 1024.
 */
int moe_load_balance(const moe_config* cfg, const int32_t* expert_offsets, float* bias, float gamma,
                     moe_load_stats* stats, hipStream_t stream);

/* Static text for a moe_status value. */
const char* moe_strerror(int status);

/* MOE355_VERSION of the built library. */
int moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE355_H */
