"""GPU parity of the grouped SwiGLU with 4-bit expert weights against the
oracle, through the C ABI, on codes drawn uniformly from all 256 byte values
(so every 4-bit value, -8 included, sits at every nibble position) and scales
of both signs, in ragged shapes: K a few 128-column groups, N a ragged number
of 256-row tiles, empty experts, one-row experts and T = 1."""
import sys

import numpy as np
import pytest
import torch

import mixture_experts_layer_limited_amd as moe
import oracle
from helpers import TOL, f64, rel_err

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _random_w4(rng, E, n_out, n_in):
    codes = rng.integers(0, 256, size=(E, n_out, n_in // 2), dtype=np.uint8)
    mag = rng.uniform(0.5, 1.5, size=(E, n_in // 128, n_out)) / (4.0 * np.sqrt(n_in))
    sign = np.where(rng.uniform(size=mag.shape) < 0.25, -1.0, 1.0)
    return codes, (mag * sign).astype(np.float32)


CASES = [
    # (T, H, I, E, k, routing)
    (77, 640, 384, 8, 2, "random"),      # H: two full 256-row down tiles and a half one
    (300, 1024, 256, 64, 6, "random"),
    (1, 256, 128, 4, 4, "random"),       # one token: four one-row experts
    (40, 384, 640, 16, 2, "skewed"),     # most rows on two experts, most experts empty
]


@pytest.mark.parametrize("T,H,I,E,k,routing", CASES)
@pytest.mark.parametrize("epi", [moe.MOE_EPI_STORE_ROWS, moe.MOE_EPI_SCATTER_ADD])
def test_w4_grouped_swiglu_every_code(T, H, I, E, k, routing, epi):
    say(f"w4 grouped swiglu T={T} H={H} I={I} E={E} k={k} {routing} epilogue={epi}")
    rng = np.random.default_rng(T * 131 + H + I + E + k)
    x = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16)
    if routing == "random":
        ids = np.argsort(rng.uniform(size=(T, E)), axis=1)[:, :k]
    else:
        ids = np.stack([np.array([3, 11])[:k] for _ in range(T)])
    w = rng.uniform(0.1, 1.0, size=(T, k)).astype(np.float32)
    off, src, inv = oracle.permute(ids, E)
    c13, s13 = _random_w4(rng, E, 2 * I, H)
    c2, s2 = _random_w4(rng, E, H, I)
    c = moe.make_config(hidden=H, inter=I, n_experts=E, top_k=k, dtype="w4a16")
    dev = lambda a, dt=torch.int32: torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(DEV)
    ws = moe.workspace(c, T, moe.MOE_OP_GROUPED_SWIGLU)
    rows = acc = None
    if epi == moe.MOE_EPI_STORE_ROWS:
        rows = torch.empty(T * k, H, dtype=torch.bfloat16, device=DEV)
    else:
        acc = torch.zeros(T, H, dtype=torch.float32, device=DEV)
    moe.grouped_swiglu(c, T, x.to(DEV), None, dev(src), dev(off), dev(c13, torch.uint8), dev(s13, torch.float32),
                       dev(c2, torch.uint8), dev(s2, torch.float32), epi, dev(w, torch.float32), dev(inv), rows, acc,
                       ws)
    torch.cuda.synchronize()
    experts = lambda e: (oracle.dequantize_int4_groups(c13[e], s13[e]), oracle.dequantize_int4_groups(c2[e], s2[e]))
    y = oracle.expert_outputs(f64(x), off, src, experts)
    if epi == moe.MOE_EPI_STORE_ROWS:
        err = rel_err(f64(rows), y)
    else:
        err = rel_err(acc.cpu().double().numpy(), oracle.combine(y, inv, w, None))
    say(f"  max rel err {err:.3e} (tol {TOL['w4a16']})")
    assert err <= TOL["w4a16"]


def test_w4_structured_weights():
    """One expert with small-integer activations and codes and power-of-two
    gate/up scales (the gate/up dot products are exact in fp32 on both sides),
    and a down projection that selects h column n % I with weight 1: the
    output is bf16(SiLU(g) * u) up to SiLU in fp32, the bf16 rounding of h and
    the fp32 rounding of the down GEMM."""
    T, H, I, E = 32, 256, 128, 1
    rng = np.random.default_rng(9)
    xi = rng.integers(-3, 4, size=(T, H)).astype(np.float32)
    q13 = rng.integers(-8, 8, size=(2 * I, H))
    nib = (q13 & 0xF).astype(np.uint8)
    c13 = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)[None]
    s13 = np.full((1, H // 128, 2 * I), 2.0 ** -6, np.float32)
    q2 = np.zeros((H, I), np.int64)
    q2[np.arange(H), np.arange(H) % I] = 1
    nib2 = (q2 & 0xF).astype(np.uint8)
    c2 = (nib2[:, 0::2] | (nib2[:, 1::2] << 4)).astype(np.uint8)[None]
    s2 = np.ones((1, I // 128, H), np.float32)
    c = moe.make_config(hidden=H, inter=I, n_experts=E, top_k=1, dtype="w4a16")
    dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(DEV)
    off = torch.tensor([0, T], dtype=torch.int32, device=DEV)
    rows = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    moe.grouped_swiglu(c, T, dev(xi, torch.bfloat16), None, None, off, dev(c13, torch.uint8),
                       dev(s13, torch.float32), dev(c2, torch.uint8), dev(s2, torch.float32),
                       moe.MOE_EPI_STORE_ROWS, None, None, rows, None, moe.workspace(c, T, moe.MOE_OP_GROUPED_SWIGLU))
    torch.cuda.synchronize()
    w13 = oracle.dequantize_int4_groups(c13[0], s13[0])
    assert np.array_equal(w13, q13 * 2.0 ** -6)
    h = oracle.swiglu_ffn(xi.astype(np.float64), w13, np.eye(I))
    want = torch.from_numpy(h.astype(np.float32)).to(torch.bfloat16).double().numpy()[:, np.arange(H) % I]
    got = f64(rows)
    dev_ = np.abs(got - want)
    say(f"  max |out - bf16(h)| = {dev_.max():.3e} (max |h| {np.abs(want).max():.3f})")
    assert np.all(dev_ <= np.abs(want) * 2.0 ** -7 + 1e-4 * np.abs(want).max())
