"""Pins of the oracle's expert, shared-expert and combine arithmetic: a
hand-computed scalar SwiGLU, special cases in which the layer reduces to a
dense FFN, the shared-expert merge identity, linearity, equivariance and the
walkthrough's shape table."""
import json
import math

import numpy as np
import pytest

import oracle


def _layer(x, gw, b, w13, w2, sh13, sh2, **kw):
    return oracle.moe_layer(x, gw, b, w13, w2, sh13, sh2, **kw)[0]


def _rand_layer(rng, T=12, H=16, E=6, I=8, Is=8):
    x = rng.normal(size=(T, H))
    gw = rng.normal(size=(E, H)) / math.sqrt(H)
    w13 = rng.normal(size=(E, 2 * I, H)) / math.sqrt(H)
    w2 = rng.normal(size=(E, H, I)) / math.sqrt(I)
    sh13 = rng.normal(size=(2 * Is, H)) / math.sqrt(H)
    sh2 = rng.normal(size=(H, Is)) / math.sqrt(Is)
    return x, gw, w13, w2, sh13, sh2


def test_scalar_swiglu_by_hand():
    # H = I = 1: out = c * SiLU(a x) * (b x), SiLU(v) = v / (1 + e^-v)
    a, b, c, x = 0.7, -1.3, 2.1, 0.9
    g, u = a * x, b * x
    expect = c * (g / (1.0 + math.exp(-g))) * u
    got = oracle.swiglu_ffn(np.array([[x]]), np.array([[a], [b]]), np.array([[c]]))
    assert abs(got[0, 0] - expect) < 1e-15


def test_silu_values():
    # SiLU(1) = sigma(1) = 0.7310585786300049..., SiLU(0) = 0, SiLU(-x) = -x*sigma(-x)
    out = oracle.swiglu_ffn(np.array([[1.0], [0.0], [-2.0]]), np.array([[1.0], [1.0]]), np.array([[1.0]]))
    # third row: SiLU(-2) * (-2) = 4 * sigma(-2)
    np.testing.assert_allclose(out[:, 0], [0.7310585786300049, 0.0, 4.0 / (1 + math.exp(2.0))], rtol=1e-15)


def test_single_expert_reduces_to_dense_ffn():
    rng = np.random.default_rng(0)
    x, gw, w13, w2, sh13, sh2 = _rand_layer(rng, E=1)
    for scale in (1.0, 2.5):
        out = _layer(x, gw, None, w13, w2, sh13, sh2, scoring="softmax", top_k=1,
                     norm_topk_prob=True, routed_scaling_factor=scale)
        dense = oracle.swiglu_ffn(x, w13[0], w2[0])
        shared = oracle.swiglu_ffn(x, sh13, sh2)
        np.testing.assert_allclose(out, scale * dense + shared, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("scoring,ng,tg,k", [("softmax", 1, 1, 2), ("sigmoid", 3, 2, 3)])
def test_identical_experts_make_routing_irrelevant(scoring, ng, tg, k):
    rng = np.random.default_rng(1)
    x, gw, w13, w2, sh13, sh2 = _rand_layer(rng, E=6)
    w13[:] = w13[0]
    w2[:] = w2[0]
    out = _layer(x, gw, rng.normal(size=6) if scoring == "sigmoid" else None, w13, w2, None, None,
                 scoring=scoring, top_k=k, n_group=ng, topk_group=tg, norm_topk_prob=True,
                 routed_scaling_factor=2.5)
    np.testing.assert_allclose(out, 2.5 * oracle.swiglu_ffn(x, w13[0], w2[0]), rtol=1e-12, atol=1e-13)


def test_zero_down_projection_leaves_the_shared_expert():
    rng = np.random.default_rng(2)
    x, gw, w13, w2, sh13, sh2 = _rand_layer(rng)
    out = _layer(x, gw, None, w13, np.zeros_like(w2), sh13, sh2, scoring="softmax", top_k=2)
    np.testing.assert_allclose(out, oracle.swiglu_ffn(x, sh13, sh2), rtol=1e-14, atol=0)


def test_linear_in_routed_scaling_factor():
    rng = np.random.default_rng(3)
    x, gw, w13, w2, sh13, sh2 = _rand_layer(rng)
    kw = dict(scoring="sigmoid", top_k=2, n_group=2, topk_group=1, norm_topk_prob=True)
    b = np.zeros(6)
    o1 = _layer(x, gw, b, w13, w2, sh13, sh2, routed_scaling_factor=1.0, **kw)
    o3 = _layer(x, gw, b, w13, w2, sh13, sh2, routed_scaling_factor=3.0, **kw)
    sh = oracle.swiglu_ffn(x, sh13, sh2)
    np.testing.assert_allclose(o3 - sh, 3.0 * (o1 - sh), rtol=1e-12, atol=1e-13)


def test_token_permutation_equivariance():
    rng = np.random.default_rng(4)
    x, gw, w13, w2, sh13, sh2 = _rand_layer(rng, T=17)
    kw = dict(scoring="softmax", top_k=3, norm_topk_prob=False)
    out = _layer(x, gw, None, w13, w2, sh13, sh2, **kw)
    perm = rng.permutation(17)
    outp = _layer(x[perm], gw, None, w13, w2, sh13, sh2, **kw)
    np.testing.assert_allclose(outp, out[perm], rtol=1e-13, atol=1e-14)


def test_shared_expert_merge_identity():
    # two I-wide experts equal one 2I-wide expert built by stacking their gate
    # rows, their up rows, and concatenating their down columns (walkthrough §2.3)
    rng = np.random.default_rng(5)
    H, I = 16, 8
    x = rng.normal(size=(9, H))
    a13, b13 = rng.normal(size=(2, 2 * I, H))
    a2, b2 = rng.normal(size=(2, H, I))
    merged13 = np.concatenate([a13[:I], b13[:I], a13[I:], b13[I:]])
    merged2 = np.concatenate([a2, b2], axis=1)
    np.testing.assert_allclose(oracle.swiglu_ffn(x, merged13, merged2),
                               oracle.swiglu_ffn(x, a13, a2) + oracle.swiglu_ffn(x, b13, b2),
                               rtol=1e-12, atol=1e-12)


def test_rows_api_matches_whole_layer():
    rng = np.random.default_rng(6)
    x, gw, w13, w2, sh13, sh2 = _rand_layer(rng, T=20, E=8)
    kw = dict(scoring="sigmoid", top_k=3, n_group=4, topk_group=2, norm_topk_prob=True,
              routed_scaling_factor=2.5)
    b = rng.normal(size=8) * 0.1
    out, info = oracle.moe_layer(x, gw, b, w13, w2, sh13, sh2, **kw)
    toks = [0, 7, 19, 3]
    rows = oracle.moe_layer_rows(toks, x, info["ids"], info["w"], lambda e: (w13[e], w2[e]),
                                 lambda: (sh13, sh2))
    np.testing.assert_allclose(rows, out[toks], rtol=1e-13, atol=1e-14)


def test_walkthrough_shape_table():
    # walkthrough §3.5: 32 tokens through a V2-Lite layer (H 2048, E 64, I 1408, k 6, Is 2816)
    rng = np.random.default_rng(7)
    T, H, E, I, k, Is = 32, 2048, 64, 1408, 6, 2816
    x = rng.normal(size=(T, H))
    gw = rng.normal(size=(E, H)) / math.sqrt(H)
    logits = oracle.router_logits(x, gw)
    assert logits.shape == (32, 64)
    s = oracle.score(logits, "softmax")
    ids = oracle.select_experts(s, None, k)
    w = oracle.routing_weights(s, ids, False, 1.0)
    assert ids.shape == (32, 6) and w.shape == (32, 6)
    offsets, src, inv = oracle.permute(ids, E)
    assert offsets.shape == (65,) and inv.shape == (192,) and src.shape == (192,)
    small = np.random.default_rng(8)

    def get_expert(e):
        return (small.normal(size=(2 * I, H)) / math.sqrt(H), small.normal(size=(H, I)) / math.sqrt(I))
    y = oracle.expert_outputs(x, offsets, src, get_expert)
    assert y.shape == (192, 2048)
    sh13 = small.normal(size=(2 * Is, H)) / math.sqrt(H)
    sh2 = small.normal(size=(H, Is)) / math.sqrt(Is)
    assert (x @ sh13.T).shape == (32, 5632)
    sh = oracle.swiglu_ffn(x, sh13, sh2)
    assert sh.shape == (32, 2048)
    out = oracle.combine(y, inv, w, sh)
    assert out.shape == (32, 2048)
