"""GPU parity of every step of the layer against the oracle, through the C ABI.

Bars: routing ids and the permutation bit-exact (both sides select from the
same fp32 score tensor, in fp32); the E4M3 quantiser bit-exact; layer
outputs within max|y-r|/max|r| <= 1e-2 (bf16), 3e-2 (FP8), 1e-4 (fp32).
Element-wise checks run at sizes the oracle finishes in seconds that span
several tiles and a ragged tail; the full workloads are checked on sampled
tokens, with routing and permutation compared on every token."""
import sys

import numpy as np
import pytest
import torch

import mixture_experts_layer_limited_amd as moe
import oracle
from moe_inputs import PRESETS, layer_inputs
from helpers import (TOL, ExpertSource, binding_config, f64, fp8_quantizers, oracle_forward_rows,
                     oracle_routing, rel_err, u8)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def i32(shape):
    return torch.empty(shape, dtype=torch.int32, device=DEV)


def f32(shape):
    return torch.empty(shape, dtype=torch.float32, device=DEV)


# ------------------------------------------------------------------ route ---

ROUTE_CASES = [
    # (T, E, k, n_group, topk_group, bias)
    (64, 8, 2, 1, 1, None),
    (1, 8, 8, 1, 1, None),                # k = E
    (333, 64, 6, 1, 1, None),
    (1000, 256, 8, 8, 4, "zero"),
    (1000, 256, 8, 8, 4, "neg"),          # negative biased scores: masked groups must use -inf
    (517, 160, 10, 5, 2, "rand"),         # 3 experts per lane, groups of 32
    (200, 1024, 32, 64, 16, "rand"),      # largest E, k, n_group
    (77, 96, 4, 12, 3, "rand"),           # groups of 8 spanning lane boundaries
]


@pytest.mark.parametrize("T,E,k,ng,tg,bias", ROUTE_CASES)
@pytest.mark.parametrize("ties", [False, True])
def test_route_selection_bit_exact(T, E, k, ng, tg, bias, ties):
    say(f"route selection T={T} E={E} k={k} groups={ng}/{tg} bias={bias} ties={ties}")
    rng = np.random.default_rng(T * 7 + E + k)
    s = rng.uniform(0.0, 1.0, size=(T, E)).astype(np.float32)
    if ties:
        s = (np.round(s * 8) / 8).astype(np.float32)
    b = None
    if bias == "zero":
        b = np.zeros(E, np.float32)
    elif bias == "neg":
        b = (-1.5 - rng.uniform(size=E)).astype(np.float32)
    elif bias == "rand":
        b = (rng.normal(size=E) * 0.2).astype(np.float32)
        if ties:
            b = (np.round(b * 8) / 8).astype(np.float32)
    cfg = moe.make_config(hidden=64, inter=64, n_experts=E, top_k=k, n_group=ng, topk_group=tg,
                          scoring="sigmoid", norm_topk_prob=True, routed_scaling_factor=2.5)
    ids, w = i32((T, k)), f32((T, k))
    bt = None if b is None else torch.from_numpy(b).to(DEV)
    moe.route(cfg, T, None, None, bt, torch.from_numpy(s).to(DEV), None, ids, w)
    torch.cuda.synchronize()
    ref = oracle.select_experts(s, b, k, ng, tg, dtype=np.float32)
    got = ids.cpu().numpy()
    assert np.array_equal(got, ref), f"{(got != ref).any(1).sum()} tokens differ"
    wref = oracle.routing_weights(s.astype(np.float64), ref, True, 2.5)
    np.testing.assert_allclose(w.cpu().numpy(), wref, rtol=2e-6, atol=1e-7)


@pytest.mark.parametrize("name", ["tiny_fp32", "v2_lite_bf16", "v3_prefill_bf16", "v3_decode_bf16", "v3_fp8",
                                  "v3_prefill_bf16@4173", "v3_prefill_bf16@4095"])
def test_route_from_hidden(name):
    """Router GEMM + scoring + selection on the workload's own x and gate
    weight (full T): scores against the fp64 oracle, selection bit-exact from
    the GPU scores, and the fraction of tokens whose fp64 routing differs.
    "name@T" runs the workload's layer on T tokens: 4173 gives the 128-row
    router tiles a ragged last tile, 4095 is the last batch on 64-row tiles."""
    base, _, t = name.partition("@")
    cfg = PRESETS[base] if not t else PRESETS[base].replace(tokens=int(t))
    say(f"route from hidden {name} T={cfg.tokens}")
    from moe_inputs import routing_inputs
    r = routing_inputs(cfg, 0)
    x, gw = r["x"].to(DEV), r["gate_w"].to(DEV)
    bias = None if r["bias"] is None else r["bias"].to(DEV)
    c = binding_config(cfg)
    T, E, k = cfg.tokens, cfg.n_experts, cfg.top_k
    scores, ids, w = f32((T, E)), i32((T, k)), f32((T, k))
    moe.route(c, T, x, gw, bias, None, scores, ids, w)
    torch.cuda.synchronize()
    s_gpu = scores.cpu().numpy()
    s_ref = oracle.score(oracle.router_logits(f64(r["x"]), f64(r["gate_w"])), cfg.scoring)
    err = np.abs(s_gpu - s_ref).max()
    say(f"  max |score - fp64 score| = {err:.3g}")
    assert err < 2e-5
    ids_ref, w_ref = oracle_routing(cfg, s_gpu, r["bias"])
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    np.testing.assert_allclose(w.cpu().numpy(), w_ref, rtol=2e-6, atol=1e-7)
    own = oracle.select_experts(s_ref, None if r["bias"] is None else r["bias"].double().numpy(), k,
                                cfg.n_group, cfg.topk_group)
    differ = float((np.sort(own, 1) != np.sort(ids_ref, 1)).any(1).mean())
    say(f"  tokens whose fp64 routing picks another expert set: {differ:.4%}")
    assert differ < 0.01
    # with a workspace the bf16 router GEMM splits H into slices (summed in order)
    ws = moe.workspace(c, T, moe.MOE_OP_ROUTE)
    scores2, ids2, w2 = f32((T, E)), i32((T, k)), f32((T, k))
    moe.route(c, T, x, gw, bias, None, scores2, ids2, w2, ws)
    torch.cuda.synchronize()
    s2 = scores2.cpu().numpy()
    err2 = np.abs(s2 - s_ref).max()
    say(f"  split-K router: max |score - fp64 score| = {err2:.3g}")
    assert err2 < 2e-5
    ids2_ref, w2_ref = oracle_routing(cfg, s2, r["bias"])
    assert np.array_equal(ids2.cpu().numpy(), ids2_ref)
    np.testing.assert_allclose(w2.cpu().numpy(), w2_ref, rtol=2e-6, atol=1e-7)


# ---------------------------------------------------------------- permute ---

def _permute(ids_np, E):
    T, k = ids_np.shape
    cfg = moe.make_config(hidden=64, inter=64, n_experts=E, top_k=k)
    ids = torch.from_numpy(ids_np.astype(np.int32)).to(DEV)
    off, src, inv = i32(E + 1), i32(T * k), i32(T * k)
    ws = moe.workspace(cfg, T, moe.MOE_OP_PERMUTE)
    moe.permute(cfg, T, ids, off, src, inv, ws)
    torch.cuda.synchronize()
    return off.cpu().numpy(), src.cpu().numpy(), inv.cpu().numpy()


def test_permute_walkthrough_example():
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "permute_example.json")))
    off, src, inv = _permute(np.array(g["topk_ids"]), g["n_experts"])
    assert off.tolist() == g["offsets"] and src.tolist() == g["permuted_src"] and inv.tolist() == g["inv_perm"]


@pytest.mark.parametrize("T,E,k,mode", [
    (1, 8, 2, "random"), (61, 8, 2, "random"), (4096, 64, 6, "random"), (8192, 256, 8, "random"),
    (16384, 256, 8, "random"), (777, 1024, 32, "random"), (3000, 64, 6, "one"), (128, 256, 8, "skew"),
    (129, 3, 2, "random"),
    (512, 64, 8, "random"), (513, 64, 8, "random"),   # 4096 copies (one work-group) and just past it
    # chunk x expert counts: 16384 x 256 fills the scan's LDS copy exactly; 4500 x 1024 overflows it
    (4500, 1024, 8, "random"),
])
def test_permute_bit_exact(T, E, k, mode):
    say(f"permute T={T} E={E} k={k} {mode}")
    rng = np.random.default_rng(T + E + k)
    if mode == "random":
        ids = np.argsort(rng.uniform(size=(T, E)), axis=1)[:, :k]
    elif mode == "one":
        ids = np.tile(np.arange(k), (T, 1))
    else:
        p = 1.0 / np.arange(1, E + 1) ** 1.1
        ids = np.stack([rng.choice(E, size=k, replace=False, p=p / p.sum()) for _ in range(T)])
    got = _permute(ids, E)
    ref = oracle.permute(ids, E)
    for a, b, name in zip(got, ref, ("offsets", "permuted_src", "inv_perm")):
        assert np.array_equal(a, b), name
    again = _permute(ids, E)
    assert all(np.array_equal(a, b) for a, b in zip(got, again))


# --------------------------------------------------------------- quantise ---

@pytest.mark.parametrize("rows,cols,dt", [(37, 256, torch.bfloat16), (300, 1024, torch.bfloat16),
                                          (16, 7168, torch.float32)])
def test_quantize_bit_exact(rows, cols, dt):
    say(f"quantize {rows}x{cols} {dt}")
    g = torch.Generator().manual_seed(rows)
    x = torch.randn(rows, cols, generator=g) * torch.exp(torch.randn(rows, 1, generator=g) * 3)
    x[0, :128] = 0.0                                       # all-zero tile
    x[1, :] *= 1e-7                                        # codes in the subnormal range
    x[2, 5] = 1e4                                          # outlier
    x = x.to(dt)
    codes = torch.empty(rows, cols, dtype=torch.uint8, device=DEV)
    scales = f32((rows, cols // 128))
    moe.quantize_fp8_1x128(x.to(DEV).contiguous(), codes, scales)
    torch.cuda.synchronize()
    rc, rs = oracle.quantize_1x128(x.float().numpy())
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    got = codes.cpu().numpy()
    assert np.array_equal(got, rc), f"{(got != rc).sum()} codes differ"


def test_quantize_every_code_and_midpoint():
    """Every E4M3 value, every midpoint between neighbours and the fp32 values
    two ulps around each, both signs, through the 1x128 quantiser: each tile
    holds 448 so its scale is exactly 1 and the codes are the rounding rule's
    own, compared bit for bit with the oracle's encoder."""
    pos = np.unique(oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8)).astype(np.float64))
    pts = np.concatenate([pos, (pos[1:] + pos[:-1]) / 2]).astype(np.float32)
    vals = [pts]
    for _ in range(2):
        vals.append(np.nextafter(vals[-1], np.float32(np.inf)))
    vals.append(np.nextafter(pts, np.float32(-np.inf)))
    vals.append(np.nextafter(vals[-1], np.float32(-np.inf)))
    v = np.concatenate(vals)
    v = v[(v >= 0) & (v <= 448)]
    v = np.concatenate([v, -v]).astype(np.float32)
    n_tiles = -(-v.size // 127)
    x = np.zeros((n_tiles, 128), np.float32)
    x[:, 0] = 448.0
    flat = x[:, 1:].reshape(-1)
    flat[:v.size] = v
    x[:, 1:] = flat.reshape(n_tiles, 127)
    say(f"quantize every code: {v.size} values in {n_tiles} tiles")
    codes = torch.empty(n_tiles, 128, dtype=torch.uint8, device=DEV)
    scales = f32((n_tiles, 1))
    moe.quantize_fp8_1x128(torch.from_numpy(x).to(DEV), codes, scales)
    torch.cuda.synchronize()
    rc, rs = oracle.quantize_1x128(x)
    assert np.all(rs == 1.0)
    got = codes.cpu().numpy()
    assert np.array_equal(got, rc), f"{(got != rc).sum()} codes differ"


# -------------------------------------------------- grouped SwiGLU + combine ---

def _reduced(name, **kw):
    return PRESETS[name].replace(**kw)


SMALL = {
    "tiny_fp32": _reduced("tiny_fp32"),
    "tiny_fp32_ragged": _reduced("tiny_fp32", tokens=61),
    "v2_lite_small": _reduced("v2_lite_bf16", tokens=203),
    "v3_small": _reduced("v3_prefill_bf16", tokens=300, hidden=1024, inter=256, n_experts=64, shared_inter=256),
    "v3_small_t1": _reduced("v3_prefill_bf16", tokens=1, hidden=1024, inter=256, n_experts=64, shared_inter=256),
    # about 300 rows per expert: the 256-row tiles, two ragged m-tiles per expert
    "v3_mid": _reduced("v3_prefill_bf16", tokens=1203, hidden=512, inter=384, n_experts=32, shared_inter=128),
    # H and I not multiples of the 256-wide n-tiles; shared expert as one more group
    "odd_dims": _reduced("v3_prefill_bf16", tokens=333, hidden=576, inter=192, n_experts=16, n_group=4,
                         topk_group=2, top_k=4, shared_inter=192),
    # the largest expert count and top-k the library takes (1024, 32): many empty
    # experts, 1024 groups in the tile builder, 32 rows per token in the combine
    "max_experts_top_k": _reduced("v3_prefill_bf16", tokens=150, hidden=256, inter=128, n_experts=1024,
                                  top_k=32, shared_inter=128),
    # shared expert of the routed width at T > 1024: its own dense launches
    "wide_shared_large_t": _reduced("v3_prefill_bf16", tokens=1100, hidden=512, inter=256, n_experts=32,
                                    shared_inter=256),
    "fp8_small": _reduced("v3_fp8", tokens=300, hidden=1024, inter=256, n_experts=64, shared_inter=256),
    "fp8_small_ragged": _reduced("v3_fp8", tokens=45, hidden=512, inter=384, n_experts=64, shared_inter=128),
    # FP8 groups of ~275 rows: the 256-row FP8 tiles (two ragged m-tiles per expert), the
    # shared expert of the routed width in its own dense launches (T > 1024)
    "fp8_big": _reduced("v3_fp8", tokens=1100, hidden=512, inter=256, n_experts=16, n_group=4, topk_group=2,
                        top_k=4, shared_inter=256),
    # FP8 with k = 16: the shared down GEMM's combine epilogue reads the routed rows'
    # indices and weights from memory (16 per token do not fit its spare LDS)
    "fp8_big_top_k16": _reduced("v3_fp8", tokens=1100, hidden=512, inter=256, n_experts=32, n_group=1,
                                topk_group=1, top_k=16, shared_inter=256),
    # 256-row FP8 tiles with H a ragged number of 256-column n-tiles and I of 128-column ones
    "fp8_big_ragged": _reduced("v3_fp8", tokens=777, hidden=640, inter=384, n_experts=8, n_group=1, topk_group=1,
                               top_k=3, shared_inter=128),
    # 256-row FP8 tiles, one group each (~250 rows: every token block of a tile live)
    "fp8_big_full_tiles": _reduced("v3_fp8", tokens=500, hidden=768, inter=256, n_experts=8, n_group=1,
                                   topk_group=1, top_k=4, shared_inter=256),
    # FP8 with H past the 64 K steps whose weight-block scales the 256-row kernel keeps in
    # one register: the gate/up GEMM takes the 128 x 256 kernel, the down GEMM (K = I) the
    # 256 x 256 one, so the two GEMMs use tile lists of different heights
    "fp8_wide_k": _reduced("v3_fp8", tokens=600, hidden=8320, inter=256, n_experts=8, n_group=1,
                           topk_group=1, top_k=4, shared_inter=256),
    # bf16 shared expert in dense launches of 256 x 256 tiles (at least one per CU), whose
    # down GEMM's epilogue also does the layer's combine; ragged last m-tile and n-tile
    "dense_shared_256": _reduced("v3_prefill_bf16", tokens=2100, hidden=8256, inter=128, n_experts=16, n_group=4,
                              topk_group=2, top_k=2, shared_inter=128),
    # 4-bit weights: shared expert merged as one more group (Is == I, T <= 1024)
    "w4_small": _reduced("v3_decode_w4a16", tokens=300, hidden=1024, inter=256, n_experts=64, shared_inter=256,
                         bias="zero"),
    # 4-bit weights: H a ragged number of 256-row n-tiles, a separate shared expert (Is != I)
    "w4_ragged": _reduced("v3_decode_w4a16", tokens=45, hidden=640, inter=384, n_experts=16, n_group=4,
                          topk_group=2, top_k=4, shared_inter=128, bias="zero"),
    # 4-bit weights, decode batch with the Zipf-skewed load: many empty and one-row experts
    "w4_decode_like": _reduced("v3_decode_w4a16", hidden=1024, inter=256, shared_inter=256),
    # 4-bit weights with the largest expert count and top-k: 1024 groups in the tile list
    "w4_max_experts_top_k": _reduced("v3_decode_w4a16", tokens=150, hidden=256, inter=128, n_experts=1024,
                                     top_k=32, shared_inter=128, bias="zero"),
    # 4-bit weights at T > 1024: the shared expert of the routed width runs its own dense launches
    "w4_large_t": _reduced("v3_decode_w4a16", tokens=1100, hidden=512, inter=256, n_experts=32, shared_inter=256,
                           bias="zero"),
}


def _oracle_full(cfg, inp, ids, w):
    """fp64 oracle of the whole layer for all T tokens, from the given routing."""
    T = cfg.tokens
    return oracle_forward_rows(cfg, inp, ids, w, np.arange(T))


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("epi", [moe.MOE_EPI_STORE_ROWS, moe.MOE_EPI_SCATTER_ADD])
def test_forward_small(name, epi):
    cfg = SMALL[name]
    say(f"forward {name} T={cfg.tokens} epilogue={epi}")
    inp = layer_inputs(cfg, 0, DEV)
    c = binding_config(cfg)
    T, E, k, H = cfg.tokens, cfg.n_experts, cfg.top_k, cfg.hidden
    out = torch.empty(T, H, dtype=inp["x"].dtype, device=DEV)
    aux = moe.ForwardOutputs(scores=f32((T, E)), topk_ids=i32((T, k)), topk_w=f32((T, k)),
                             expert_offsets=i32(E + 1), permuted_src=i32(T * k), inv_perm=i32(T * k))
    ws = moe.workspace(c, T)
    moe.forward(c, T, inp["x"], inp["gate_w"], inp["bias"], inp["w13"], inp["w13_s"], inp["w2"], inp["w2_s"],
                inp["sh_w13"], inp["sh_w13_s"], inp["sh_w2"], inp["sh_w2_s"], out, ws, epilogue=epi, aux=aux)
    torch.cuda.synchronize()
    s_gpu = aux.scores.cpu().numpy()
    ids, w = oracle_routing(cfg, s_gpu, inp["bias"])
    assert np.array_equal(aux.topk_ids.cpu().numpy(), ids)
    off, src, inv = oracle.permute(ids, E)
    assert np.array_equal(aux.expert_offsets.cpu().numpy(), off)
    assert np.array_equal(aux.permuted_src.cpu().numpy(), src)
    assert np.array_equal(aux.inv_perm.cpu().numpy(), inv)
    ref = _oracle_full(cfg, inp, ids, w)
    err = rel_err(f64(out), ref)
    say(f"  max rel err {err:.3e} (tol {TOL[cfg.dtype]})")
    assert err <= TOL[cfg.dtype]


_BASE_PRESET = {"bf16": "v3_prefill_bf16", "fp8": "v3_fp8", "w4a16": "v3_decode_w4a16", "f32": "tiny_fp32"}


def _random_layer(seed):
    """A random valid layer: storage format, H, I, E, k, groups, shared width,
    T from 1 to 1500, scoring, bias, renormalisation, scaling and epilogue;
    T is halved until the fp64 oracle runs in about a second."""
    rng = np.random.default_rng(seed)
    dt = str(rng.choice(["bf16", "bf16", "fp8", "w4a16", "f32"]))
    mult = 128 if dt in ("fp8", "w4a16") else 64
    H = mult * int(rng.integers(1, 9))
    I = mult * int(rng.integers(1, 7))
    E = int(rng.choice([2, 3, 8, 16, 40, 64, 96, 160, 256, 300]))
    ng = int(rng.choice([g for g in (1, 2, 4, 5, 8, 16) if E % g == 0 and (g == 1 or E // g >= 2)]))
    tg = int(rng.integers(1, ng + 1))
    kmax = E if ng == 1 else min(E, tg * (E // ng))
    k = int(rng.integers(1, min(kmax, 32) + 1))
    T = int(rng.choice([1, 2, 7, 33, 100, 257, 700, 1025, 1500]))
    while T > 1 and T * k * H * I > 2e9:
        T //= 2
    scoring = "sigmoid" if (ng > 1 or rng.random() < 0.5) else "softmax"
    cfg = PRESETS[_BASE_PRESET[dt]].replace(
        name=f"random{seed}", tokens=T, hidden=H, inter=I, n_experts=E, top_k=k, n_group=ng, topk_group=tg,
        shared_inter=int(rng.choice([0, I, 2 * I, mult])), scoring=scoring,
        bias=str(rng.choice(["none", "zero"])) if scoring == "sigmoid" else "none",
        norm_topk_prob=bool(rng.random() < 0.5), routed_scaling_factor=float(rng.choice([1.0, 2.5])))
    return cfg, int(rng.integers(0, 2)), int(rng.integers(0, 1 << 30))


@pytest.mark.parametrize("seed", range(32))
def test_forward_random_layer(seed):
    cfg, epi, input_seed = _random_layer(seed)
    T, E, k, H = cfg.tokens, cfg.n_experts, cfg.top_k, cfg.hidden
    say(f"forward random{seed}: {cfg.dtype} T={T} H={H} I={cfg.inter} E={E} k={k} groups={cfg.n_group}/"
        f"{cfg.topk_group} Is={cfg.shared_inter} {cfg.scoring} bias={cfg.bias} epilogue={epi}")
    inp = layer_inputs(cfg, input_seed, DEV)
    c = binding_config(cfg)
    out = torch.empty(T, H, dtype=inp["x"].dtype, device=DEV)
    aux = moe.ForwardOutputs(scores=f32((T, E)), topk_ids=i32((T, k)), topk_w=f32((T, k)),
                             expert_offsets=i32(E + 1), permuted_src=i32(T * k), inv_perm=i32(T * k))
    moe.forward(c, T, inp["x"], inp["gate_w"], inp["bias"], inp["w13"], inp["w13_s"], inp["w2"], inp["w2_s"],
                inp["sh_w13"], inp["sh_w13_s"], inp["sh_w2"], inp["sh_w2_s"], out, moe.workspace(c, T),
                epilogue=epi, aux=aux)
    torch.cuda.synchronize()
    ids, w = oracle_routing(cfg, aux.scores.cpu().numpy(), inp["bias"])
    assert np.array_equal(aux.topk_ids.cpu().numpy(), ids)
    off, src, inv = oracle.permute(ids, E)
    assert np.array_equal(aux.expert_offsets.cpu().numpy(), off)
    assert np.array_equal(aux.permuted_src.cpu().numpy(), src)
    assert np.array_equal(aux.inv_perm.cpu().numpy(), inv)
    err = rel_err(f64(out), _oracle_full(cfg, inp, ids, w))
    say(f"  max rel err {err:.3e} (tol {TOL[cfg.dtype]})")
    assert err <= TOL[cfg.dtype]


def test_forward_zero_tokens_is_a_no_op():
    cfg = SMALL["v3_small"]
    c = binding_config(cfg)
    inp = layer_inputs(cfg.replace(tokens=4), 0, DEV)
    out = torch.full((4, cfg.hidden), 7.0, dtype=torch.bfloat16, device=DEV)
    moe.forward(c, 0, inp["x"], inp["gate_w"], inp["bias"], inp["w13"], None, inp["w2"], None,
                inp["sh_w13"], None, inp["sh_w2"], None, out, None)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("mode", ["one_expert", "two_experts_empty_rest", "mixed"])
def test_grouped_swiglu_skewed(mode, dtype):
    """All rows on one expert (many m-tiles of one group), most experts empty,
    and a mix of group sizes whose tiles hold 1 to 16 token blocks (FP8: the
    256-row tiles run every live-block count of their K loop)."""
    base = "v3_prefill_bf16" if dtype == "bf16" else "v3_fp8"
    cfg = _reduced(base, tokens=700, hidden=512, inter=384, n_experts=32, n_group=1, topk_group=1,
                   top_k=2, shared_inter=0)
    if mode == "mixed":
        cfg = cfg.replace(n_experts=8)
    say(f"grouped swiglu skew {mode} {dtype}")
    inp = layer_inputs(cfg, 1, DEV)
    T, E, k, H, I = cfg.tokens, cfg.n_experts, cfg.top_k, cfg.hidden, cfg.inter
    if mode == "one_expert":                       # every token: expert 3 plus one other
        other = np.arange(T) % (E - 1)
        ids = np.stack([np.full(T, 3), other + (other >= 3)], 1)
    elif mode == "two_experts_empty_rest":         # experts 5 and 9 only, 30 empty experts
        ids = np.tile(np.array([5, 9]), (T, 1))
    else:                                          # 600, 300, 249, 130, 40, 37, 43 and 1 rows
        first = np.concatenate([np.zeros(600), np.ones(100)]).astype(int)
        second = np.concatenate([np.full(200, 1), np.full(249, 2), np.full(130, 3), np.full(40, 4),
                                 np.full(37, 5), np.full(43, 6), np.full(1, 7)]).astype(int)
        ids = np.stack([first, second], 1)
        assert (ids[:, 0] != ids[:, 1]).all()
    c = binding_config(cfg)
    off, src, inv = oracle.permute(ids, E)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).astype(np.int32)).to(DEV)
    rows = torch.empty(T * k, H, dtype=torch.bfloat16, device=DEV)
    ws = moe.workspace(c, T, moe.MOE_OP_GROUPED_SWIGLU)
    moe.grouped_swiglu(c, T, inp["x"], None, dev(src), dev(off), inp["w13"], inp["w13_s"], inp["w2"], inp["w2_s"],
                       moe.MOE_EPI_STORE_ROWS, None, None, rows, None, ws)
    torch.cuda.synchronize()
    srcx = ExpertSource(inp, cfg.dtype)
    qx, qh = fp8_quantizers(cfg)
    ref = oracle.expert_outputs(f64(inp["x"]), off, src, srcx.expert, qh, qx)
    err = rel_err(f64(rows), ref)
    say(f"  max rel err {err:.3e}")
    assert err <= TOL[cfg.dtype]
    # every group on its own, so that a small group's error cannot hide under a large one's scale
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            assert rel_err(f64(rows[lo:hi]), ref[lo:hi]) <= TOL[cfg.dtype], e


def test_shared_expert_through_grouped_call():
    """The shared expert as a one-group grouped SwiGLU (n_experts = 1, offsets {0, T}, identity rows)."""
    cfg = SMALL["v2_lite_small"]
    inp = layer_inputs(cfg, 2, DEV)
    T, H, Is = cfg.tokens, cfg.hidden, cfg.shared_inter
    c = moe.make_config(hidden=H, inter=Is, n_experts=1, top_k=1, dtype="bf16")
    off = torch.tensor([0, T], dtype=torch.int32, device=DEV)
    rows = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    ws = moe.workspace(c, T, moe.MOE_OP_GROUPED_SWIGLU)
    moe.grouped_swiglu(c, T, inp["x"], None, None, off, inp["sh_w13"][None], None, inp["sh_w2"][None], None,
                       moe.MOE_EPI_STORE_ROWS, None, None, rows, None, ws)
    torch.cuda.synchronize()
    ref = oracle.swiglu_ffn(f64(inp["x"]), f64(inp["sh_w13"]), f64(inp["sh_w2"]))
    assert rel_err(f64(rows), ref) <= TOL["bf16"]


@pytest.mark.parametrize("name", ["v3_small", "dense_shared_256", "fp8_big", "fp8_big_ragged", "fp8_big_top_k16",
                                  "v3_prefill_bf16", "v3_fp8"])
def test_staged_calls_match_forward(name):
    """route -> permute -> grouped_swiglu (routed and shared) -> combine gives
    the same layer output as moe_forward, bit for bit, and both match the
    oracle.  Inside moe_forward, v3_small runs the shared expert as one more
    routed group; in the others its down GEMM runs on a 256 x 256 kernel whose
    epilogue also does the combine (dense_shared_256: bf16; fp8_big,
    fp8_big_ragged with a ragged n-tile, fp8_big_top_k16 with k = 16: FP8),
    which the staged combine kernel checks bit for bit.  v3_prefill_bf16 and
    v3_fp8 run the full-size workloads (the launches the benchmark times),
    compared bit for bit over the whole output; their oracle comparison is
    test_forward_full_size_sampled's."""
    full = name in PRESETS
    cfg = PRESETS[name] if full else SMALL[name]
    inp = layer_inputs(cfg, 3, DEV)
    c = binding_config(cfg)
    T, E, k, H, Is = cfg.tokens, cfg.n_experts, cfg.top_k, cfg.hidden, cfg.shared_inter
    say(f"staged calls vs forward {name} T={T} H={H} Is={Is}")
    scores, ids, w = f32((T, E)), i32((T, k)), f32((T, k))
    # with a workspace, as moe_forward has one: the same split-K router GEMM
    moe.route(c, T, inp["x"], inp["gate_w"], inp["bias"], None, scores, ids, w,
              moe.workspace(c, T, moe.MOE_OP_ROUTE))
    off, src, inv = i32(E + 1), i32(T * k), i32(T * k)
    moe.permute(c, T, ids, off, src, inv, moe.workspace(c, T, moe.MOE_OP_PERMUTE))
    rows = torch.empty(T * k, H, dtype=torch.bfloat16, device=DEV)
    ws = moe.workspace(c, T, moe.MOE_OP_GROUPED_SWIGLU)
    moe.grouped_swiglu(c, T, inp["x"], None, src, off, inp["w13"], inp["w13_s"], inp["w2"], inp["w2_s"],
                       moe.MOE_EPI_STORE_ROWS, None, None, rows, None, ws)
    sc = moe.make_config(hidden=H, inter=Is, n_experts=1, top_k=1, dtype=cfg.dtype)
    sh = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    scale = lambda t: None if t is None else t[None]
    moe.grouped_swiglu(sc, T, inp["x"], None, None, torch.tensor([0, T], dtype=torch.int32, device=DEV),
                       inp["sh_w13"][None], scale(inp["sh_w13_s"]), inp["sh_w2"][None], scale(inp["sh_w2_s"]),
                       moe.MOE_EPI_STORE_ROWS, None, None, sh, None, moe.workspace(sc, T, moe.MOE_OP_GROUPED_SWIGLU))
    out = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    moe.combine(c, T, rows, None, inv, w, sh, out)
    out2 = torch.empty_like(out)
    moe.forward(c, T, inp["x"], inp["gate_w"], inp["bias"], inp["w13"], inp["w13_s"], inp["w2"], inp["w2_s"],
                inp["sh_w13"], inp["sh_w13_s"], inp["sh_w2"], inp["sh_w2_s"], out2, moe.workspace(c, T))
    torch.cuda.synchronize()
    assert torch.equal(out, out2), f"{(out != out2).sum().item()} elements differ"
    assert bool(torch.isfinite(out.float()).all())
    if not full:
        ids_r, w_r = oracle_routing(cfg, scores.cpu().numpy(), inp["bias"])
        assert rel_err(f64(out), _oracle_full(cfg, inp, ids_r, w_r)) <= TOL[cfg.dtype]


# ------------------------------------------------------ full-size workloads ---

FULL_SIZE = [
    ("v2_lite_bf16", 8, moe.MOE_EPI_STORE_ROWS),
    ("v2_lite_bf16", 8, moe.MOE_EPI_SCATTER_ADD),
    ("v3_prefill_bf16", 6, moe.MOE_EPI_STORE_ROWS),
    ("v3_prefill_bf16", 6, moe.MOE_EPI_SCATTER_ADD),
    ("v3_decode_bf16", 8, moe.MOE_EPI_STORE_ROWS),
    ("v3_decode_bf16", 8, moe.MOE_EPI_SCATTER_ADD),
    ("v3_fp8", 4, moe.MOE_EPI_STORE_ROWS),
    ("v3_fp8", 4, moe.MOE_EPI_SCATTER_ADD),
    ("v3_decode_w4a16", 8, moe.MOE_EPI_STORE_ROWS),
    ("v3_decode_w4a16", 8, moe.MOE_EPI_SCATTER_ADD),
]


@pytest.mark.parametrize("name,samples,epi", FULL_SIZE)
def test_forward_full_size_sampled(name, samples, epi):
    """The workload at its full size, in the launch configuration the
    benchmark times (and with the scatter-add combine): routing and
    permutation bit-exact on every token, layer output on sampled tokens
    within tolerance."""
    cfg = PRESETS[name]
    say(f"full-size forward {name} T={cfg.tokens} epilogue={epi}: drawing inputs")
    inp = layer_inputs(cfg, 0, DEV)
    c = binding_config(cfg)
    T, E, k, H = cfg.tokens, cfg.n_experts, cfg.top_k, cfg.hidden
    out = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    aux = moe.ForwardOutputs(scores=f32((T, E)), topk_ids=i32((T, k)), topk_w=f32((T, k)),
                             expert_offsets=i32(E + 1), permuted_src=i32(T * k), inv_perm=i32(T * k))
    say("  running the layer")
    moe.forward(c, T, inp["x"], inp["gate_w"], inp["bias"], inp["w13"], inp["w13_s"], inp["w2"], inp["w2_s"],
                inp["sh_w13"], inp["sh_w13_s"], inp["sh_w2"], inp["sh_w2_s"], out, moe.workspace(c, T),
                epilogue=epi, aux=aux)
    torch.cuda.synchronize()
    s_gpu = aux.scores.cpu().numpy()
    ids, w = oracle_routing(cfg, s_gpu, inp["bias"])
    assert np.array_equal(aux.topk_ids.cpu().numpy(), ids)
    np.testing.assert_allclose(aux.topk_w.cpu().numpy(), w, rtol=2e-6, atol=1e-7)
    off, src, inv = oracle.permute(ids, E)
    assert np.array_equal(aux.expert_offsets.cpu().numpy(), off)
    assert np.array_equal(aux.permuted_src.cpu().numpy(), src)
    assert np.array_equal(aux.inv_perm.cpu().numpy(), inv)
    st = oracle.load_stats(ids, E)
    say(f"  expert load: min {st['min']} max {st['max']} cv {st['cv']:.3f} empty {st['empty']}")
    rng = np.random.default_rng(5 + epi)
    toks = np.sort(rng.choice(T, size=samples, replace=False))
    say(f"  oracle on tokens {toks.tolist()}")
    ref = oracle_forward_rows(cfg, inp, ids, w, toks)
    err = rel_err(f64(out[torch.from_numpy(toks).to(DEV)]), ref)
    say(f"  max rel err {err:.3e} (tol {TOL[cfg.dtype]})")
    assert err <= TOL[cfg.dtype]
    assert bool(torch.isfinite(out.float()).all())


@pytest.mark.parametrize("name,n_top", [("v3_prefill_bf16", 3), ("v3_fp8", 2), ("v2_lite_bf16", 2)])
def test_most_loaded_experts_every_row(name, n_top):
    """Every row of the most-loaded experts at full size: these experts span
    several m-tiles of the grouped GEMMs at the full K (two 256-row tiles at
    V3 prefill and V2-Lite, four or five 128-row tiles at V3 FP8), so the
    row split between m-tiles and the second tile's rows are all compared,
    through the grouped SwiGLU call with stored rows."""
    cfg = PRESETS[name]
    say(f"most-loaded experts {name}: drawing inputs")
    inp = layer_inputs(cfg, 0, DEV)
    c = binding_config(cfg)
    T, E, k, H = cfg.tokens, cfg.n_experts, cfg.top_k, cfg.hidden
    scores, ids_d, w_d = f32((T, E)), i32((T, k)), f32((T, k))
    moe.route(c, T, inp["x"], inp["gate_w"], inp["bias"], None, scores, ids_d, w_d,
              moe.workspace(c, T, moe.MOE_OP_ROUTE))
    off_d, src_d, inv_d = i32(E + 1), i32(T * k), i32(T * k)
    moe.permute(c, T, ids_d, off_d, src_d, inv_d, moe.workspace(c, T, moe.MOE_OP_PERMUTE))
    rows = torch.empty(T * k, H, dtype=torch.bfloat16, device=DEV)
    moe.grouped_swiglu(c, T, inp["x"], None, src_d, off_d, inp["w13"], inp["w13_s"], inp["w2"], inp["w2_s"],
                       moe.MOE_EPI_STORE_ROWS, None, None, rows, None,
                       moe.workspace(c, T, moe.MOE_OP_GROUPED_SWIGLU))
    torch.cuda.synchronize()
    off, src = off_d.cpu().numpy().astype(np.int64), src_d.cpu().numpy().astype(np.int64)
    counts = np.diff(off)
    top = np.argsort(-counts, kind="stable")[:n_top]
    say(f"  experts {top.tolist()} with {counts[top].tolist()} rows")
    # the selected experts' rows as a small grouped problem of their own
    sub_src = np.concatenate([src[off[e]:off[e + 1]] for e in top])
    sub_off = np.concatenate([[0], np.cumsum(counts[top])])
    x_sub = f64(inp["x"][torch.from_numpy(sub_src).to(DEV)])
    exp = ExpertSource(inp, cfg.dtype)
    qx, qh = fp8_quantizers(cfg)
    ref = oracle.expert_outputs(x_sub, sub_off, np.arange(sub_src.size), lambda g: exp.expert(int(top[g])),
                                qh, qx)
    got = f64(torch.cat([rows[int(off[e]):int(off[e + 1])] for e in top]))
    for g, e in enumerate(top):
        lo, hi = int(sub_off[g]), int(sub_off[g + 1])
        err = rel_err(got[lo:hi], ref[lo:hi])
        say(f"  expert {int(e)}: {hi - lo} rows, max rel err {err:.3e} (tol {TOL[cfg.dtype]})")
        assert err <= TOL[cfg.dtype]


def test_fp8_hand_built_layer_is_exact():
    """A one-token FP8 layer whose every intermediate value is exact (built
    by hand in tests/test_oracle_fp8_layer.py, where the oracle is pinned to
    it): the GPU must produce exactly 1, 28, 448, 28, 448 in columns 10, 11,
    12, 20, 21 and zeros elsewhere.  It checks on the device what the CPU
    test checks of the oracle: the router reads the raw x, the routed and the
    shared experts read the 1x128-quantised x, and h is quantised after
    SiLU(gate) * up."""
    import test_oracle_fp8_layer as hand
    x, gate_w, w13, w2, sh13, sh2 = hand._hand_layer()
    H, I = hand.H, hand.I
    enc = lambda a: torch.from_numpy(oracle.e4m3_encode(a)).to(DEV)
    ones = lambda *shape: torch.ones(shape, dtype=torch.float32, device=DEV)
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).to(DEV).to(torch.bfloat16)
    c = moe.make_config(hidden=H, inter=I, n_experts=2, top_k=1, shared_inter=hand.IS, scoring="softmax",
                        norm_topk_prob=True, routed_scaling_factor=1.0, dtype="fp8")
    out = torch.empty(1, H, dtype=torch.bfloat16, device=DEV)
    aux = moe.ForwardOutputs(topk_ids=i32((1, 1)))
    moe.forward(c, 1, bf(x), bf(gate_w), None, enc(w13), ones(2, 2, 1), enc(w2), ones(2, 1, 1), enc(sh13),
                ones(2, 1), enc(sh2), ones(1, 1), out, moe.workspace(c, 1), aux=aux)
    torch.cuda.synchronize()
    assert aux.topk_ids.cpu().numpy().tolist() == [[1]]
    np.testing.assert_array_equal(f64(out), hand._expected())


# ----------------------------------------------------- load balance step ---

def _ids_for(mode, T, E, k, rng):
    if T == 0:
        return np.zeros((0, k), dtype=np.int64)
    if mode == "uniform":          # k distinct experts per token, uniformly
        return np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
    if mode == "skewed":           # Zipf-like preference, many empty experts
        p = 1.0 / np.arange(1, E + 1) ** 1.1
        p /= p.sum()
        return np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)])
    if mode == "one_expert":       # E = 1: cv is 0 by definition
        return np.zeros((T, 1), dtype=np.int64)
    raise ValueError(mode)


@pytest.mark.parametrize("mode,T,E,k", [("uniform", 900, 256, 8), ("skewed", 128, 256, 8),
                                        ("uniform", 77, 1024, 32), ("one_expert", 50, 1, 1),
                                        ("uniform", 0, 64, 6)])
def test_load_balance_matches_oracle(mode, T, E, k):
    """Bias step bit-exact against the oracle's sign rule in fp32; load statistics
    against the oracle's counts, min, max, empty (exact) and mean, cv (fp32)."""
    say(f"load balance {mode} T={T} E={E} k={k}")
    rng = np.random.default_rng(11)
    ids = _ids_for(mode, T, E, k, rng).reshape(T, k)
    off, _, _ = oracle.permute(ids, E)
    cfgd = dict(hidden=128, inter=128, n_experts=E, top_k=k, dtype="bf16")
    if E >= 8:
        cfgd.update(n_group=8, topk_group=8)
    c = moe.make_config(**cfgd)
    bias0 = (rng.standard_normal(E) * 0.05).astype(np.float32)
    gamma = np.float32(1e-3)
    bias = torch.from_numpy(bias0).to(DEV)
    stats = torch.zeros(moe.LOAD_STATS_BYTES, dtype=torch.uint8, device=DEV)
    moe.load_balance(c, torch.from_numpy(off.astype(np.int32)).to(DEV), bias, float(gamma), stats)
    torch.cuda.synchronize()
    rows = int(off[-1])
    share = np.float32(rows) / np.float32(E)
    counts = np.diff(off)
    want = oracle.bias_update(bias0.astype(np.float64), counts, np.full(E, share, np.float64),
                              float(gamma)).astype(np.float32)
    got = bias.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    st = moe.load_stats_from(stats)
    ref = oracle.load_stats(ids, E)
    say(f"  rows {st.rows} min {st.min} max {st.max} empty {st.empty} mean {st.mean:.3f} cv {st.cv:.4f}")
    assert (st.rows, st.min, st.max, st.empty) == (rows, ref["min"], ref["max"], ref["empty"])
    assert st.mean == pytest.approx(ref["mean"], rel=1e-7, abs=0)
    assert st.cv == pytest.approx(ref["cv"], rel=1e-6, abs=1e-12)


@pytest.mark.parametrize("name", ["v3_small", "fp8_small", "v2_lite_small", "w4_small"])
def test_forward_is_deterministic(name):
    """With the row-store epilogue the layer output is bitwise reproducible:
    fixed split-K slice order in the router, fixed K order in every GEMM and a
    fixed summation order in the combine (no atomics)."""
    cfg = SMALL[name]
    inp = layer_inputs(cfg, 4, DEV)
    c = binding_config(cfg)
    T, H = cfg.tokens, cfg.hidden
    ws = moe.workspace(c, T)
    outs = []
    for _ in range(3):
        out = torch.empty(T, H, dtype=inp["x"].dtype, device=DEV)
        moe.forward(c, T, inp["x"], inp["gate_w"], inp["bias"], inp["w13"], inp["w13_s"], inp["w2"], inp["w2_s"],
                    inp["sh_w13"], inp["sh_w13_s"], inp["sh_w2"], inp["sh_w2_s"], out, ws)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


@pytest.mark.parametrize("entry", ["forward", "forward_static"])
@pytest.mark.parametrize("name", ["v3_small", "fp8_small", "w4_small"])
def test_forward_in_a_hip_graph(name, entry):
    """moe_forward allocates nothing and never synchronises, so a whole layer can
    be captured into a HIP graph: every replay, with eager work in between,
    equals the eager forward.  The same holds for moe_forward_static, whose
    scratch is the library's own static buffer (the caller it serves is code
    under graph capture)."""
    cfg = SMALL[name]
    inp = layer_inputs(cfg, 5, DEV)
    c = binding_config(cfg)
    T, H = cfg.tokens, cfg.hidden
    ws = moe.workspace(c, T)
    args = (inp["x"], inp["gate_w"], inp["bias"], inp["w13"], inp["w13_s"], inp["w2"], inp["w2_s"],
            inp["sh_w13"], inp["sh_w13_s"], inp["sh_w2"], inp["sh_w2_s"])
    if entry == "forward":
        run = lambda o: moe.forward(c, T, *args, o, ws)
    else:
        assert moe.workspace_size(c, T) <= moe.STATIC_SCRATCH_BYTES
        run = lambda o: moe.forward_static(c, T, *args, o)
    ref = torch.empty(T, H, dtype=inp["x"].dtype, device=DEV)
    moe.forward(c, T, *args, ref, ws)
    torch.cuda.synchronize()
    out = torch.empty_like(ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                      # warm-up on the capture stream
        run(out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(out)
    for rep in range(3):
        out.zero_()
        noise = torch.randn(1 << 20, device=DEV).sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep} differs from the eager forward"
        del noise
