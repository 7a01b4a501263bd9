"""fp64 numpy oracle of the MoE layer forward (test infrastructure only).

Notation: T tokens, H hidden, E routed experts, I expert intermediate size,
k experts per token, Is shared intermediate size, G = E / n_group experts per
group.  Weights are stored (out, in): gate.weight (E,H), w13 (E,2I,H) with the
gate rows first and the up rows second, w2 (E,H,I), shared gate_up (2Is,H),
shared down (H,Is) (MoE inference walkthrough, zhiyuanblog.org/blog/moe-inference,
§2.1-§2.3 and the x @ w.T products of §3.3).

Readings of points the pages leave open (each applies everywhere below):
  * the score-correction bias enters expert *selection* only; output weights
    come from the unbiased scores;
  * experts of a group that is not kept are excluded with -inf (not 0.0),
    so a negative biased score can never pull in an expert of a dropped group;
  * every tie (between groups, between experts) goes to the lower index;
  * the k experts of a token are listed by descending selection score;
  * routed_scaling_factor is folded into the routing weights;
  * no token is dropped (no capacity limit).
"""
from __future__ import annotations

from typing import Callable, Optional, Tuple

import numpy as np


# ---------------------------------------------------------------- routing ---

def router_logits(x: np.ndarray, gate_w: np.ndarray) -> np.ndarray:
    """logits (T,E) = x (T,H) @ gate.weight (E,H)^T, fp64, no bias term
    (walkthrough §2.1 "有无 bias: 无" and §3.1 step 1)."""
    return np.asarray(x, np.float64) @ np.asarray(gate_w, np.float64).T


def score(logits: np.ndarray, scoring: str) -> np.ndarray:
    """Scores from router logits.

    softmax: over all E experts of a token (walkthrough §3.1 step 2), computed
    with the row maximum subtracted (exact in real arithmetic).
    sigmoid: 1 / (1 + e^-z) per expert (V3 lab page, gsyq.cn/news/313569,
    §3 scoring_func and §4 route(); walkthrough §3.3.1 defines sigma)."""
    z = np.asarray(logits, np.float64)
    if scoring == "softmax":
        z = z - z.max(axis=-1, keepdims=True)
        e = np.exp(z)
        return e / e.sum(axis=-1, keepdims=True)
    if scoring == "sigmoid":
        with np.errstate(over="ignore"):
            return 1.0 / (1.0 + np.exp(-z))
    raise ValueError(f"unknown scoring function {scoring!r}")


def select_experts(s: np.ndarray, bias: Optional[np.ndarray], top_k: int,
                   n_group: int = 1, topk_group: int = 1,
                   dtype=np.float64) -> np.ndarray:
    """Group-limited top-k selection (V3 lab page §4 route(); V3/R1 overview,
    xxqk.cn/news/389306, §2.2; greedy case: walkthrough §3.1 step 3).

    1. selection score c = s + b, evaluated in `dtype` (b = 0 when absent);
    2. if n_group > 1: experts form n_group contiguous groups of G; a group's
       score is the sum of its two largest c; the topk_group groups with the
       largest group score are kept and every other expert gets c = -inf;
    3. the k experts with the largest c, listed by descending c.
    Ties go to the lower index at both stages.  `dtype` fixes the precision of
    c and of the group sums: float32 reproduces a single-precision evaluation
    bit for bit (IEEE round-to-nearest-even), float64 is the exact reading.
    Returns int64 ids (T, k)."""
    s = np.asarray(s)
    T, E = s.shape
    c = s.astype(dtype)
    if bias is not None:
        c = c + np.asarray(bias).astype(dtype)[None, :]
    if n_group > 1:
        G = E // n_group
        grouped = c.reshape(T, n_group, G)
        two = np.sort(grouped, axis=-1)[..., -2:]
        gscore = two[..., 1] + two[..., 0]
        keep = np.argsort(-gscore, axis=-1, kind="stable")[:, :topk_group]
        allowed = np.zeros((T, n_group), dtype=bool)
        np.put_along_axis(allowed, keep, True, axis=-1)
        c = np.where(np.repeat(allowed, G, axis=1), c, np.array(-np.inf, dtype=dtype))
    return np.argsort(-c, axis=-1, kind="stable")[:, :top_k]


def routing_weights(s: np.ndarray, ids: np.ndarray, norm_topk_prob: bool,
                    routed_scaling_factor: float) -> np.ndarray:
    """w[t,j] = s[t, ids[t,j]] (unbiased score), divided by the sum over the
    token's k experts when norm_topk_prob, then times routed_scaling_factor
    (V3 lab page §4 route(); walkthrough §3.1 step 4).  fp64."""
    w = np.take_along_axis(np.asarray(s, np.float64), np.asarray(ids), axis=-1)
    if norm_topk_prob:
        w = w / w.sum(axis=-1, keepdims=True)
    return w * float(routed_scaling_factor)


def route(x, gate_w, bias, *, scoring, top_k, n_group=1, topk_group=1,
          norm_topk_prob=False, routed_scaling_factor=1.0, scores=None,
          select_dtype=np.float64):
    """Whole routing step.  With `scores` given (a (T,E) score tensor, e.g. the
    float32 one another implementation produced) the GEMM and scoring are
    skipped and selection runs on those scores.  Returns (s, ids, w)."""
    s = score(router_logits(x, gate_w), scoring) if scores is None else np.asarray(scores)
    ids = select_experts(s, bias, top_k, n_group, topk_group, dtype=select_dtype)
    w = routing_weights(s, ids, norm_topk_prob, routed_scaling_factor)
    return s, ids, w


# ------------------------------------------------------------ permutation ---

def permute(ids: np.ndarray, n_experts: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Token permutation into per-expert buckets (walkthrough §3.2).

    Every token is replicated k times; copy a = t*k + j goes to expert
    ids[t,j].  Copies are ordered by expert and, inside one expert, by a
    (ascending token, as in the page's example).
      offsets (E+1,)      : expert_first_token_offset, empty experts included;
      permuted_src (T*k,) : token index of every permuted row;
      inv_perm (T*k,)     : permuted row of copy a (inv_permuted_idx).
    A stable sort by expert id is exactly this order."""
    flat = np.asarray(ids, np.int64).reshape(-1)
    k = ids.shape[1]
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=n_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    inv_perm = np.empty_like(order)
    inv_perm[order] = np.arange(order.size)
    return offsets, order // k, inv_perm


# ----------------------------------------------------------------- experts ---

def _sigmoid(v):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-v))


def swiglu_ffn(xrows: np.ndarray, w13: np.ndarray, w2: np.ndarray,
               quantize_h: Optional[Callable[[np.ndarray], np.ndarray]] = None) -> np.ndarray:
    """One SwiGLU expert on rows (M,H): gate_up = x @ w13^T (M,2I); chunk(2)
    into gate and up; h = SiLU(gate) * up with SiLU(v) = v * sigmoid(v);
    out = h @ w2^T (M,H) (walkthrough §3.3.1 and its SwiGLU definition).
    `quantize_h`, when given, replaces h by its quantise-dequantise image
    before the down projection (the FP8 path)."""
    xr = np.asarray(xrows, np.float64)
    w13 = np.asarray(w13, np.float64)
    I = w13.shape[0] // 2
    gu = xr @ w13.T
    gate, up = gu[:, :I], gu[:, I:]
    h = gate * _sigmoid(gate) * up
    if quantize_h is not None:
        h = quantize_h(h)
    return h @ np.asarray(w2, np.float64).T


def expert_outputs(x: np.ndarray, offsets: np.ndarray, permuted_src: np.ndarray,
                   get_expert: Callable[[int], Tuple[np.ndarray, np.ndarray]],
                   quantize_h=None, quantize_x=None) -> np.ndarray:
    """permuted_output (T*k, H): row p = expert e's FFN applied to token
    permuted_src[p], for p in [offsets[e], offsets[e+1]) (walkthrough §3.3.1,
    the grouped GEMM segmented by expert_offsets).  `get_expert(e)` returns
    (w13[e], w2[e]) so that weights can be fetched one expert at a time."""
    xin = np.asarray(x, np.float64) if quantize_x is None else quantize_x(x)
    E = offsets.size - 1
    out = np.zeros((permuted_src.size, xin.shape[1]), np.float64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        w13, w2 = get_expert(e)
        out[lo:hi] = swiglu_ffn(xin[permuted_src[lo:hi]], w13, w2, quantize_h)
    return out


def combine(expert_out: np.ndarray, inv_perm: np.ndarray, w: np.ndarray,
            shared_out: Optional[np.ndarray]) -> np.ndarray:
    """out[t] = sum_j w[t,j] * expert_out[inv_perm[t*k+j]] (+ shared_out[t])
    (walkthrough §3.4 steps 1-2)."""
    T, k = w.shape
    rows = np.asarray(expert_out, np.float64)[np.asarray(inv_perm).reshape(T, k)]
    out = np.einsum("tj,tjh->th", np.asarray(w, np.float64), rows)
    if shared_out is not None:
        out = out + shared_out
    return out


def moe_layer(x, gate_w, bias, w13, w2, sh_w13, sh_w2, *, scoring, top_k,
              n_group=1, topk_group=1, norm_topk_prob=False,
              routed_scaling_factor=1.0, scores=None, select_dtype=np.float64,
              quantize_x=None, quantize_h=None):
    """The whole layer on all T tokens (walkthrough §3, V3 lab page §4).
    Router on the unquantised x; experts on quantize_x(x) when given.
    Returns (out (T,H), info dict with s, ids, w, offsets, permuted_src, inv_perm)."""
    x = np.asarray(x, np.float64)
    s, ids, w = route(x, gate_w, bias, scoring=scoring, top_k=top_k, n_group=n_group,
                      topk_group=topk_group, norm_topk_prob=norm_topk_prob,
                      routed_scaling_factor=routed_scaling_factor, scores=scores,
                      select_dtype=select_dtype)
    E = np.asarray(w13).shape[0]
    offsets, src, inv = permute(ids, E)
    y = expert_outputs(x, offsets, src, lambda e: (w13[e], w2[e]), quantize_h, quantize_x)
    sh = None
    if sh_w13 is not None:
        xin = x if quantize_x is None else quantize_x(x)
        sh = swiglu_ffn(xin, sh_w13, sh_w2, quantize_h)
    out = combine(y, inv, w, sh)
    return out, dict(s=s, ids=ids, w=w, offsets=offsets, permuted_src=src, inv_perm=inv)


def moe_layer_rows(tokens, x, ids, w, get_expert, get_shared=None,
                   quantize_x=None, quantize_h=None) -> np.ndarray:
    """Output rows of the selected tokens only, given their routing (ids, w for
    all T tokens).  Same arithmetic as moe_layer, one token at a time, each
    expert's weights fetched once through get_expert(e) -> (w13[e], w2[e]);
    get_shared() -> (sh_w13, sh_w2) or None.  Used at sizes where the whole
    layer does not fit in fp64 on the host."""
    tokens = np.asarray(tokens, np.int64)
    xs = np.asarray(x, np.float64)[tokens]
    if quantize_x is not None:
        xs = quantize_x(xs)
    out = np.zeros_like(xs)
    need = {}
    for r, t in enumerate(tokens):
        for j in range(ids.shape[1]):
            need.setdefault(int(ids[t, j]), []).append((r, float(w[t, j])))
    for e in sorted(need):
        w13, w2 = get_expert(e)
        rs = [r for r, _ in need[e]]
        ys = swiglu_ffn(xs[rs], w13, w2, quantize_h)
        for (r, wt), yrow in zip(need[e], ys):
            out[r] += wt * yrow
    if get_shared is not None:
        sh = get_shared()
        if sh is not None:
            out += swiglu_ffn(xs, sh[0], sh[1], quantize_h)
    return out


# ------------------------------------------------------- load statistics ---

def load_stats(ids: np.ndarray, n_experts: int) -> dict:
    """Expert activation counts (bincount) with min / max / mean and the
    coefficient of variation std/mean, std with n-1 (V3 lab page §4 script)."""
    counts = np.bincount(np.asarray(ids).reshape(-1), minlength=n_experts).astype(np.float64)
    mean = counts.mean()
    std = counts.std(ddof=1) if counts.size > 1 else 0.0
    return dict(counts=counts.astype(np.int64), min=int(counts.min()), max=int(counts.max()),
                mean=float(mean), cv=float(std / mean) if mean > 0 else 0.0,
                empty=int((counts == 0).sum()))


def bias_update(bias: np.ndarray, load: np.ndarray, target: np.ndarray, gamma: float) -> np.ndarray:
    """Bias-based balancing step (V3/R1 overview §2.2): an expert that received
    more tokens than its target has its bias lowered by gamma, one that
    received fewer has it raised, one on target keeps it."""
    return np.asarray(bias, np.float64) + gamma * np.sign(
        np.asarray(target, np.float64) - np.asarray(load, np.float64))
