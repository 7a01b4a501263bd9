"""Pins of the oracle's routing step against things other than itself:
closed forms, a brute-force enumeration of the two-stage group-limited
selection, a different library routine for the greedy case, and the
invariants the pages state for routing logs and weights."""
import heapq
import itertools
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle


# --------------------------------------------------------------- scoring ---

def test_softmax_closed_forms():
    rng = np.random.default_rng(1)
    z = rng.normal(size=(7, 13)) * 4
    s = oracle.score(z, "softmax")
    np.testing.assert_allclose(s.sum(-1), 1.0, rtol=0, atol=1e-15)
    # shift invariance, and the two-expert case is the logistic function
    np.testing.assert_allclose(oracle.score(z + 3.25, "softmax"), s, rtol=1e-14, atol=0)
    z2 = np.array([[0.7, -0.4]])
    np.testing.assert_allclose(oracle.score(z2, "softmax")[0, 0], 1 / (1 + math.exp(-1.1)), rtol=1e-15)
    # equal logits give the uniform distribution
    np.testing.assert_array_equal(oracle.score(np.zeros((1, 8)), "softmax"), np.full((1, 8), 0.125))


def test_sigmoid_closed_forms():
    z = np.array([[0.0, 1.0, -1.0, 40.0, -800.0]])
    s = oracle.score(z, "sigmoid")
    assert s[0, 0] == 0.5
    assert abs(s[0, 1] - 0.7310585786300049) < 1e-16
    assert abs(s[0, 1] + s[0, 2] - 1.0) < 1e-16          # sigma(-x) = 1 - sigma(x)
    assert s[0, 4] == 0.0 and 0.0 < s[0, 3] <= 1.0


def test_router_logits_is_a_plain_product():
    # gate rows that pick single coordinates of x return those coordinates
    x = np.arange(12.0).reshape(3, 4)
    gw = np.array([[0, 0, 1, 0], [1, 0, 0, 0], [0, 0, 0, 2.0]])
    np.testing.assert_array_equal(oracle.router_logits(x, gw), np.stack([x[:, 2], x[:, 0], 2 * x[:, 3]], 1))


# ---------------------------------------------- brute-force group top-k ---

def _brute_force(c, k, n_group, topk_group):
    """Enumerates the two-stage definition on one token: group score = best
    pair sum inside the group (all pairs), kept groups = the max-sum set of
    topk_group groups (lexicographically first on ties), experts = the max-sum
    k-subset of the kept groups' experts (lexicographically first on ties),
    listed by descending c then ascending index."""
    E = len(c)
    G = E // n_group
    if n_group > 1:
        gs = [max(c[a] + c[b] for a, b in itertools.combinations(range(g * G, (g + 1) * G), 2))
              for g in range(n_group)]
        best = None
        for S in itertools.combinations(range(n_group), topk_group):
            v = sum(gs[g] for g in S)
            if best is None or v > best[0]:
                best = (v, S)
        allowed = [e for g in best[1] for e in range(g * G, (g + 1) * G)]
    else:
        allowed = list(range(E))
    best = None
    for S in itertools.combinations(sorted(allowed), k):
        v = sum(c[e] for e in S)
        if best is None or v > best[0]:
            best = (v, S)
    return sorted(best[1], key=lambda e: (-c[e], e))


@settings(max_examples=300, deadline=None)
@given(st.sampled_from([(8, 2, 1), (8, 2, 2), (8, 4, 2), (12, 3, 2), (12, 4, 3), (16, 4, 2), (16, 2, 1), (9, 1, 1)]),
       st.integers(1, 6), st.integers(0, 2 ** 31 - 1), st.booleans())
def test_group_limited_topk_matches_brute_force(shape, k, seed, ties):
    E, n_group, topk_group = shape
    G = E // n_group
    k = min(k, topk_group * G)
    rng = np.random.default_rng(seed)
    # scores on a coarse dyadic grid force ties; sums stay exact in fp64
    c = rng.integers(-6, 7, size=E) / 4.0 if ties else rng.normal(size=E)
    got = oracle.select_experts(c[None, :], None, k, n_group, topk_group)[0].tolist()
    assert got == _brute_force(c.tolist(), k, n_group, topk_group)


def test_two_stage_differs_from_best_k_within_any_groups():
    # groups are kept by their top-2 sums first: group 0 = {5, 0} sums to 5,
    # group 1 = {3, 3} sums to 6, so group 1 is kept and the single best
    # expert (0) is out of reach; plain top-1 over all experts picks it
    c = np.array([5.0, 0.0, 3.0, 3.0])
    assert oracle.select_experts(c[None], None, 1, n_group=2, topk_group=1)[0].tolist() == [2]
    assert oracle.select_experts(c[None], None, 1)[0].tolist() == [0]


def test_greedy_matches_heapq():
    rng = np.random.default_rng(3)
    c = np.round(rng.normal(size=(50, 64)), 1)            # many ties
    ids = oracle.select_experts(c, None, 6)
    for t in range(c.shape[0]):
        ref = heapq.nlargest(6, range(64), key=lambda e: (c[t, e], -e))
        assert ids[t].tolist() == ref


@settings(max_examples=150, deadline=None)
@given(st.integers(0, 2 ** 31 - 1))
def test_selection_invariants(seed):
    rng = np.random.default_rng(seed)
    T, E, n_group, topk_group, k = 16, 64, 8, 3, 6
    s = rng.uniform(size=(T, E))
    b = rng.normal(size=E) * 0.3
    ids = oracle.select_experts(s, b, k, n_group, topk_group)
    c = s + b
    for t in range(T):
        sel = ids[t]
        assert len(set(sel.tolist())) == k
        groups = set((sel // (E // n_group)).tolist())
        assert len(groups) <= topk_group
        # descending order
        assert all(c[t, sel[j]] >= c[t, sel[j + 1]] for j in range(k - 1))
        # nothing unselected inside a kept group beats the worst selected expert
        kept = set()
        gs = [np.sort(c[t, g * 8:(g + 1) * 8])[-2:].sum() for g in range(n_group)]
        order = sorted(range(n_group), key=lambda g: (-gs[g], g))[:topk_group]
        kept = {e for g in order for e in range(g * 8, g * 8 + 8)}
        assert groups <= {g for g in order}
        rest = [c[t, e] for e in kept if e not in set(sel.tolist())]
        assert not rest or min(c[t, sel]) >= max(rest)


def test_masked_groups_use_minus_infinity():
    # all biased scores negative: a 0.0 fill would let an expert of a dropped
    # group beat every kept expert; -inf never does
    s = np.full((1, 8), 0.1)
    b = np.array([-0.5, -0.6, -0.2, -0.3, -0.9, -0.9, -0.9, -0.9])
    ids = oracle.select_experts(s, b, 4, n_group=4, topk_group=2)[0]
    assert sorted(ids.tolist()) == [0, 1, 2, 3]


def test_float32_selection_rounds_like_float32():
    # 1 + 2^-25 is a quarter ulp above 1: exact in fp64, rounds to 1 in fp32,
    # where the two experts tie and the lower index wins
    s = np.array([[1.0, 1.0]])
    b = np.array([0.0, 2.0 ** -25])
    assert oracle.select_experts(s, b, 1, dtype=np.float64)[0].tolist() == [1]
    assert oracle.select_experts(s.astype(np.float32), b.astype(np.float32), 1,
                                 dtype=np.float32)[0].tolist() == [0]


# --------------------------------------------------------------- weights ---

@settings(max_examples=100, deadline=None)
@given(st.integers(0, 2 ** 31 - 1), st.floats(0.5, 20.0))
def test_weight_invariants(seed, scale):
    rng = np.random.default_rng(seed)
    s = oracle.score(rng.normal(size=(9, 32)), "softmax")
    ids = oracle.select_experts(s, None, 5)
    w = oracle.routing_weights(s, ids, True, scale)
    np.testing.assert_allclose(w.sum(-1), scale, rtol=1e-13)
    wr = oracle.routing_weights(s, ids, False, scale)
    assert np.all(wr.sum(-1) <= scale * (1 + 1e-12))
    np.testing.assert_allclose(wr, np.take_along_axis(s, ids, -1) * scale, rtol=1e-15)


def test_k_equals_e_returns_the_softmax():
    rng = np.random.default_rng(5)
    s = oracle.score(rng.normal(size=(4, 8)), "softmax")
    ids = oracle.select_experts(s, None, 8)
    w = oracle.routing_weights(s, ids, True, 1.0)
    back = np.zeros_like(s)
    np.put_along_axis(back, ids, w, -1)
    np.testing.assert_allclose(back, s, rtol=1e-14)


def test_unnormalised_weights_of_the_walkthrough_token():
    # walkthrough §3.1 token "深": top-6 softmax weights 0.053 .. 0.033 sum to 0.25
    top = np.array([0.053, 0.048, 0.041, 0.039, 0.036, 0.033])
    rest = (1.0 - top.sum()) / 58
    s = np.full((1, 64), rest)
    s[0, [47, 12, 3, 58, 21, 7]] = top
    ids = oracle.select_experts(s, None, 6)
    assert ids[0].tolist() == [47, 12, 3, 58, 21, 7]
    w = oracle.routing_weights(s, ids, False, 1.0)
    assert abs(w.sum() - 0.25) < 1e-12
    np.testing.assert_allclose(w[0], top, rtol=1e-15)


def test_routing_log_invariants():
    # routing-log check (mhpn.cn/news/2412747 §4.1): k entries, normalised weights sum to 1
    rng = np.random.default_rng(11)
    s = oracle.score(rng.normal(size=(32, 256)), "sigmoid")
    ids = oracle.select_experts(s, np.zeros(256), 8, 8, 4)
    w = oracle.routing_weights(s, ids, True, 1.0)
    assert ids.shape == (32, 8)
    np.testing.assert_allclose(w.sum(-1), 1.0, rtol=1e-14)


def test_bias_changes_selection_not_weights():
    s = np.array([[0.9, 0.8, 0.1, 0.05]])
    b = np.array([0.0, 0.0, 2.0, 0.0])
    _, ids, w = oracle.route(None, None, b, scoring="sigmoid", top_k=2, scores=s,
                             norm_topk_prob=False, routed_scaling_factor=1.0)
    assert ids[0].tolist() == [2, 0]
    np.testing.assert_array_equal(w[0], [0.1, 0.9])


def test_bias_update_sign_rule():
    b = oracle.bias_update(np.zeros(4), load=np.array([10, 4, 5, 0]), target=np.array([5, 5, 5, 5]), gamma=0.01)
    np.testing.assert_array_equal(b, [-0.01, 0.01, 0.0, 0.01])


def test_load_stats_matches_page_formula():
    ids = np.array([[0, 1], [0, 2], [0, 1]])
    st_ = oracle.load_stats(ids, 4)
    assert st_["counts"].tolist() == [3, 2, 1, 0]
    assert st_["min"] == 0 and st_["max"] == 3 and st_["empty"] == 1
    assert abs(st_["cv"] - np.std([3, 2, 1, 0], ddof=1) / 1.5) < 1e-15
