"""Glue shared by the GPU parity tests: moving tensors to numpy, composing the
oracle's steps for one layer, and the error metric.  No layer arithmetic
lives here: every number on the reference side comes from oracle/."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from moe_inputs import LayerConfig

TOL = {"f32": 1e-4, "bf16": 1e-2, "fp8": 3e-2, "w4a16": 1e-2}


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.uint8)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max |ref| over the whole tensor (normwise infinity)."""
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


def binding_config(cfg: LayerConfig):
    import mixture_experts_layer_limited_amd as moe
    return moe.make_config(hidden=cfg.hidden, inter=cfg.inter, n_experts=cfg.n_experts, top_k=cfg.top_k,
                           n_group=cfg.n_group, topk_group=cfg.topk_group, shared_inter=cfg.shared_inter,
                           scoring=cfg.scoring, norm_topk_prob=cfg.norm_topk_prob,
                           routed_scaling_factor=cfg.routed_scaling_factor, dtype=cfg.dtype)


class ExpertSource:
    """Per-expert fp64 weights for the oracle, decoded one expert at a time
    from the tensors the GPU received (bf16/fp32 values, E4M3 codes with
    128x128 block scales, or packed 4-bit codes with per-row 128-column
    group scales)."""

    def __init__(self, inp: dict, dtype: str):
        self.inp, self.dtype = inp, dtype
        self.cache = {}

    def _w(self, name, e=None):
        t = self.inp[name] if e is None else self.inp[name][e]
        if self.dtype not in ("fp8", "w4a16"):
            return f64(t)
        s = self.inp[name + "_s"] if e is None else self.inp[name + "_s"][e]
        if self.dtype == "fp8":
            return oracle.dequantize_blocks(u8(t), s.float().cpu().numpy())
        return oracle.dequantize_int4_groups(u8(t), s.float().cpu().numpy())

    def expert(self, e: int):
        if e not in self.cache:
            if len(self.cache) > 16:
                self.cache.clear()
            self.cache[e] = (self._w("w13", e), self._w("w2", e))
        return self.cache[e]

    def shared(self):
        if self.inp["sh_w13"] is None:
            return None
        return self._w("sh_w13"), self._w("sh_w2")


def fp8_quantizers(cfg: LayerConfig):
    if cfg.dtype != "fp8":
        return None, None
    return oracle.quantize_dequantize_1x128, oracle.quantize_dequantize_1x128


def oracle_routing(cfg: LayerConfig, gpu_scores: np.ndarray, bias):
    """Selection and weights from the GPU's fp32 score tensor, in fp32 (the
    precision both sides take the integer decision in)."""
    b = None if bias is None else bias.float().cpu().numpy()
    ids = oracle.select_experts(gpu_scores.astype(np.float32), b, cfg.top_k, cfg.n_group, cfg.topk_group,
                                dtype=np.float32)
    w = oracle.routing_weights(gpu_scores, ids, cfg.norm_topk_prob, cfg.routed_scaling_factor)
    return ids, w


def oracle_forward_rows(cfg: LayerConfig, inp: dict, ids, w, tokens):
    src = ExpertSource(inp, cfg.dtype)
    qx, qh = fp8_quantizers(cfg)
    return oracle.moe_layer_rows(tokens, f64(inp["x"]), ids, w, src.expert, src.shared, quantize_x=qx,
                                 quantize_h=qh)
