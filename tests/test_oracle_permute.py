"""Pins of the oracle's permutation: the walkthrough's worked example (a golden
vector) and the invariants of a stable bucket sort, checked on random and
adversarial routings."""
import json
import os

import numpy as np
from hypothesis import given, settings, strategies as st

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "permute_example.json")


def test_walkthrough_worked_example():
    with open(GOLDEN) as f:
        g = json.load(f)
    ids = np.array(g["topk_ids"])
    offsets, src, inv = oracle.permute(ids, g["n_experts"])
    assert offsets.tolist() == g["offsets"]
    assert src.tolist() == g["permuted_src"]
    assert inv.tolist() == g["inv_perm"]
    # the page's compact offsets are the distinct boundaries of used experts
    used = sorted({int(e) for e in ids.reshape(-1)})
    assert [int(offsets[e]) for e in used] + [int(offsets[-1])] == g["compact_offsets"]
    # the page's buckets, expert by expert
    for e, toks in g["buckets"].items():
        e = int(e)
        assert src[offsets[e]:offsets[e + 1]].tolist() == toks


def _check_invariants(ids, E):
    T, k = ids.shape
    offsets, src, inv = oracle.permute(ids, E)
    n = T * k
    assert offsets[0] == 0 and offsets[-1] == n
    assert np.all(np.diff(offsets) >= 0)
    assert sorted(inv.tolist()) == list(range(n))                 # bijection
    flat = ids.reshape(-1)
    for a in range(n):
        p = inv[a]
        assert src[p] == a // k                                   # row p holds token t
        assert offsets[flat[a]] <= p < offsets[flat[a] + 1]       # inside its expert's bucket
    for e in range(E):
        rows = src[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(rows) > 0)                          # ascending tokens (stable)
        assert rows.size == int((flat == e).sum())


@settings(max_examples=200, deadline=None)
@given(st.integers(1, 40), st.integers(1, 8), st.integers(0, 2 ** 31 - 1), st.sampled_from(["random", "one", "skew"]))
def test_permutation_invariants(T, k, seed, mode):
    E = 16
    k = min(k, E)
    rng = np.random.default_rng(seed)
    if mode == "random":
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    elif mode == "one":                       # every token picks experts 0..k-1 (all on the same few)
        ids = np.tile(np.arange(k), (T, 1))
    else:                                     # Zipf-like skew, many empty experts
        p = 1.0 / np.arange(1, E + 1) ** 2
        ids = np.stack([rng.choice(E, size=k, replace=False, p=p / p.sum()) for _ in range(T)])
    _check_invariants(ids, E)


def test_brute_force_order():
    # plain double loop over (expert, copy index) reproduces permuted_src and inv_perm
    rng = np.random.default_rng(9)
    T, k, E = 23, 3, 7
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    offsets, src, inv = oracle.permute(ids, E)
    order = [a for e in range(E) for a in range(T * k) if ids[a // k, a % k] == e]
    assert src.tolist() == [a // k for a in order]
    assert inv.tolist() == [order.index(a) for a in range(T * k)]
