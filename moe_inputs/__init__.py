"""Seeded synthetic inputs for the DeepSeek-style MoE layer forward.

This module is shared by the tests, the benchmark and the oracle's checks.
It draws inputs only: shapes, seeds, value distributions and storage
formats.  It holds none of the layer's arithmetic (no routing, no
permutation, no expert FFN, no activation quantisation).

Layer configurations follow the layer description of the MoE inference
walkthrough (zhiyuanblog.org/blog/moe-inference, §1.3 MoE config) for
DeepSeek-V2-Lite and the DeepSeek-V3 router config of the V3 lab page
(gsyq.cn/news/313569, §3 moe_router.json).

Distributions:
  * x ~ N(0, 1); the FP8 workload multiplies a Bernoulli(1e-3) subset of
    elements by 20 (sign kept) to plant outliers.
  * every weight matrix ~ N(0, 1/fan_in), fan_in = the matrix's input
    dimension (H for the router, w13 and the shared gate/up matrix; I for
    w2; Is for the shared down matrix).
  * values are drawn in fp32 and rounded once (round-to-nearest-even) to
    the storage dtype; both sides of every check receive the same bits.
  * FP8 workloads store expert weights as E4M3 codes plus one fp32 scale per
    128x128 block, as checkpoints do (V3 lab page §3 infer.toml
    weight_block_size [128, 128]); the conversion is done here, offline,
    with torch's float8_e4m3fn cast: it is part of preparing the weights,
    not part of the layer.
  * W4A16 workloads store expert weights as signed 4-bit integers, two per
    byte (even input column in the low nibble), with one fp32 scale per
    output row and 128 input columns, stored group-major (in/128, out)
    (walkthrough §8 quantisation table names the format; the packing and
    grouping are this library's reading).
    The conversion is done here, offline: symmetric, scale = amax / 7 (1 for
    an all-zero group), q = round-half-even(w / scale), clamped to [-8, 7].

Routing inputs (x, gate weight, bias) are always drawn on the CPU so that
they are identical wherever the layer runs; expert weights are drawn on the
device the caller names, one independent generator per expert, so any
expert can be drawn alone.
"""
from __future__ import annotations

import dataclasses
import json
import os
import zlib
from dataclasses import dataclass
from typing import Dict, Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
REPO_ROOT = os.path.dirname(_HERE)
DECODE_BIAS_FIXTURE = os.path.join(REPO_ROOT, "tests", "golden", "v3_decode_bias_seed0.json")


@dataclass(frozen=True)
class LayerConfig:
    """Shape, routing configuration and storage format of one MoE layer."""

    name: str
    tokens: int          # T
    hidden: int          # H
    inter: int           # I, routed expert intermediate size
    n_experts: int       # E
    top_k: int           # k
    n_group: int
    topk_group: int
    shared_inter: int    # Is = n_shared * I_shared (0 = no shared expert)
    scoring: str         # "softmax" | "sigmoid"
    norm_topk_prob: bool
    routed_scaling_factor: float
    dtype: str           # "f32" | "bf16" | "fp8" | "w4a16"
    bias: str            # "none" | "zero" | "zipf"
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)

    @property
    def group_size(self) -> int:
        return self.n_experts // self.n_group

    @property
    def rows(self) -> int:
        return self.tokens * self.top_k


PRESETS: Dict[str, LayerConfig] = {
    # Tiny fp32 layer: softmax greedy, norm true, scale 1.0, 1 shared expert.
    "tiny_fp32": LayerConfig(
        "tiny_fp32", tokens=64, hidden=128, inter=64, n_experts=8, top_k=2,
        n_group=1, topk_group=1, shared_inter=64, scoring="softmax",
        norm_topk_prob=True, routed_scaling_factor=1.0, dtype="f32", bias="none"),
    # DeepSeek-V2-Lite MoE layer (walkthrough §1.3): 2 shared experts fused.
    "v2_lite_bf16": LayerConfig(
        "v2_lite_bf16", tokens=4096, hidden=2048, inter=1408, n_experts=64, top_k=6,
        n_group=1, topk_group=1, shared_inter=2816, scoring="softmax",
        norm_topk_prob=False, routed_scaling_factor=1.0, dtype="bf16", bias="none"),
    # DeepSeek-V3 MoE layer, prefill batch (V3 lab page §3 moe_router.json).
    "v3_prefill_bf16": LayerConfig(
        "v3_prefill_bf16", tokens=8192, hidden=7168, inter=2048, n_experts=256, top_k=8,
        n_group=8, topk_group=4, shared_inter=2048, scoring="sigmoid",
        norm_topk_prob=True, routed_scaling_factor=2.5, dtype="bf16", bias="zero"),
    # Same layer, decode batch; bias skews expert load toward Zipf(1.1).
    "v3_decode_bf16": LayerConfig(
        "v3_decode_bf16", tokens=128, hidden=7168, inter=2048, n_experts=256, top_k=8,
        n_group=8, topk_group=4, shared_inter=2048, scoring="sigmoid",
        norm_topk_prob=True, routed_scaling_factor=2.5, dtype="bf16", bias="zipf"),
    # Same layer, FP8 E4M3 expert weights and activations.
    "v3_fp8": LayerConfig(
        "v3_fp8", tokens=16384, hidden=7168, inter=2048, n_experts=256, top_k=8,
        n_group=8, topk_group=4, shared_inter=2048, scoring="sigmoid",
        norm_topk_prob=True, routed_scaling_factor=2.5, dtype="fp8", bias="zero",
        outlier_frac=1e-3, outlier_scale=20.0),
    # V3 decode batch with 4-bit expert weights and bf16 activations (walkthrough §8).
    "v3_decode_w4a16": LayerConfig(
        "v3_decode_w4a16", tokens=128, hidden=7168, inter=2048, n_experts=256, top_k=8,
        n_group=8, topk_group=4, shared_inter=2048, scoring="sigmoid",
        norm_topk_prob=True, routed_scaling_factor=2.5, dtype="w4a16", bias="zipf"),
}


def stream_seed(seed: int, name: str, index: int = 0) -> int:
    """Seed of one independent generator stream, stable across runs and machines."""
    return (seed * 1_000_003 + zlib.crc32(name.encode()) * 65_537 + index) % (2 ** 62)


def _gen(seed: int, name: str, index: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(stream_seed(seed, name, index))
    return g


def _store_dtype(cfg: LayerConfig) -> torch.dtype:
    return torch.float32 if cfg.dtype == "f32" else torch.bfloat16


def _normal(shape, std: float, seed: int, name: str, index: int, device) -> torch.Tensor:
    g = _gen(seed, name, index, device)
    t = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    return t.mul_(std)


def load_decode_bias(n_experts: int) -> torch.Tensor:
    with open(DECODE_BIAS_FIXTURE) as f:
        fx = json.load(f)
    b = torch.tensor(fx["bias"], dtype=torch.float32)
    if b.numel() != n_experts:
        raise ValueError(f"decode bias fixture holds {b.numel()} experts, need {n_experts}")
    return b


def routing_inputs(cfg: LayerConfig, seed: int = 0) -> Dict[str, Optional[torch.Tensor]]:
    """x (T,H), gate weight (E,H) and score-correction bias (E,) on the CPU."""
    sd = _store_dtype(cfg)
    x = _normal((cfg.tokens, cfg.hidden), 1.0, seed, "x", 0, "cpu")
    if cfg.outlier_frac > 0:
        g = _gen(seed, "outlier_mask", 0, "cpu")
        mask = torch.rand(cfg.tokens, cfg.hidden, generator=g) < cfg.outlier_frac
        x = torch.where(mask, x * cfg.outlier_scale, x)
    gate_w = _normal((cfg.n_experts, cfg.hidden), cfg.hidden ** -0.5, seed, "gate_w", 0, "cpu")
    if cfg.bias == "none":
        bias = None
    elif cfg.bias == "zero":
        bias = torch.zeros(cfg.n_experts, dtype=torch.float32)
    elif cfg.bias == "zipf":
        bias = load_decode_bias(cfg.n_experts)
    else:
        raise ValueError(cfg.bias)
    return {"x": x.to(sd), "gate_w": gate_w.to(sd), "bias": bias}


def fp8_block_quantize(w: torch.Tensor):
    """E4M3 codes + fp32 scale per 128x128 block of a 2-D fp32 weight (checkpoint format)."""
    n, k = w.shape
    if n % 128 or k % 128:
        raise ValueError("FP8 weights need both dims to be multiples of 128")
    blk = w.reshape(n // 128, 128, k // 128, 128)
    amax = blk.abs().amax(dim=(1, 3))
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (blk / scale[:, None, :, None]).clamp_(-448.0, 448.0)
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8).reshape(n, k)
    return codes.contiguous(), scale.contiguous()


def int4_group_quantize(w: torch.Tensor):
    """Packed signed 4-bit codes (n, k/2) uint8 and fp32 scales (k/128, n) of a
    2-D fp32 weight: one symmetric scale per row and 128 columns."""
    n, k = w.shape
    if k % 128:
        raise ValueError("4-bit weights need a multiple of 128 input columns")
    g = w.reshape(n, k // 128, 128)
    amax = g.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / 7.0, torch.ones_like(amax))
    q = torch.round(g / scale[:, :, None]).clamp_(-8, 7).to(torch.int16).reshape(n, k)
    nib = q & 0xF
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).to(torch.uint8)
    return packed.contiguous(), scale.t().contiguous()


def _stacked(cfg: LayerConfig, name: str, n_out: int, n_in: int, count: int, seed: int,
             device, fp8: bool):
    """count matrices (n_out, n_in) ~ N(0, 1/n_in), one generator per matrix."""
    std = n_in ** -0.5
    if cfg.dtype == "w4a16":
        codes = torch.empty(count, n_out, n_in // 2, dtype=torch.uint8, device=device)
        scales = torch.empty(count, n_in // 128, n_out, dtype=torch.float32, device=device)
        for e in range(count):
            c, s = int4_group_quantize(_normal((n_out, n_in), std, seed, name, e, device))
            codes[e].copy_(c)
            scales[e].copy_(s)
        return codes, scales
    if fp8:
        codes = torch.empty(count, n_out, n_in, dtype=torch.uint8, device=device)
        scales = torch.empty(count, n_out // 128, n_in // 128, dtype=torch.float32, device=device)
        for e in range(count):
            c, s = fp8_block_quantize(_normal((n_out, n_in), std, seed, name, e, device))
            codes[e].copy_(c)
            scales[e].copy_(s)
        return codes, scales
    out = torch.empty(count, n_out, n_in, dtype=_store_dtype(cfg), device=device)
    for e in range(count):
        out[e].copy_(_normal((n_out, n_in), std, seed, name, e, device))
    return out, None


def expert_weights(cfg: LayerConfig, seed: int = 0, device="cpu") -> Dict[str, Optional[torch.Tensor]]:
    """Stacked routed weights w13 (E,2I,H), w2 (E,H,I) and the shared expert's
    gate_up (2Is,H) / down (H,Is), all (out,in).  Gate rows are [0,I) of w13 and
    up rows [I,2I) (walkthrough §2.2, §3.3.1).  FP8 configs also return block
    scales w13_s (E,2I/128,H/128), w2_s (E,H/128,I/128), sh_w13_s, sh_w2_s.
    W4A16 configs return packed codes w13 (E,2I,H/2), w2 (E,H,I/2) and group
    scales w13_s (E,H/128,2I), w2_s (E,I/128,H) (shared: without the E axis)."""
    fp8 = cfg.dtype == "fp8"
    E, H, I, Is = cfg.n_experts, cfg.hidden, cfg.inter, cfg.shared_inter
    w13, w13_s = _stacked(cfg, "w13", 2 * I, H, E, seed, device, fp8)
    w2, w2_s = _stacked(cfg, "w2", H, I, E, seed, device, fp8)
    out = {"w13": w13, "w13_s": w13_s, "w2": w2, "w2_s": w2_s,
           "sh_w13": None, "sh_w13_s": None, "sh_w2": None, "sh_w2_s": None}
    if Is > 0:
        a, a_s = _stacked(cfg, "sh_w13", 2 * Is, H, 1, seed, device, fp8)
        b, b_s = _stacked(cfg, "sh_w2", H, Is, 1, seed, device, fp8)
        out.update(sh_w13=a[0], sh_w2=b[0],
                   sh_w13_s=None if a_s is None else a_s[0],
                   sh_w2_s=None if b_s is None else b_s[0])
    return out


def layer_inputs(cfg: LayerConfig, seed: int = 0, device="cpu") -> Dict[str, Optional[torch.Tensor]]:
    """All inputs of one layer: routing inputs moved to `device`, expert weights drawn there."""
    r = routing_inputs(cfg, seed)
    d = {k: (None if v is None else v.to(device)) for k, v in r.items()}
    d.update(expert_weights(cfg, seed, device))
    return d
