"""Python binding of libmoe355, the MI355X (gfx950) MoE layer forward.

Argument marshalling only: every function takes torch tensors (device
memory) or None, passes their data pointers and the current HIP stream to
the C ABI declared in include/moe355.h, and raises MoeError on a non-zero
status.  All computation happens in the library's HIP kernels; there is no
fallback of any kind: without the built library nothing here runs.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE355_LIB names another build of the same library (e.g. a tuning variant).
LIB_PATH = os.environ.get("MOE355_LIB", os.path.join(_HERE, "libmoe355.so"))

MOE_F32, MOE_BF16, MOE_FP8_E4M3, MOE_INT4 = 0, 1, 2, 3
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID = 0, 1
MOE_EPI_STORE_ROWS, MOE_EPI_SCATTER_ADD = 0, 1
MOE_OP_ROUTE, MOE_OP_PERMUTE, MOE_OP_GROUPED_SWIGLU, MOE_OP_COMBINE, MOE_OP_FORWARD = range(5)
STATUS = {0: "MOE_OK", -1: "MOE_ERR_INVALID_ARG", -2: "MOE_ERR_CONFIG", -3: "MOE_ERR_UNSUPPORTED",
          -4: "MOE_ERR_WORKSPACE", -5: "MOE_ERR_HIP"}

EXPORTS = ("moe_workspace_size", "moe_validate_config", "moe_route", "moe_permute", "moe_grouped_swiglu",
           "moe_combine", "moe_forward", "moe_forward_static", "moe_load_balance", "moe_quantize_fp8_1x128",
           "moe_strerror", "moe_version")


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str, text: str):
        super().__init__(f"{where}: {STATUS.get(status, status)} ({text})")
        self.status = status


class MoeConfig(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32),
                ("shared_inter", ctypes.c_int32), ("scoring", ctypes.c_int32),
                ("norm_topk_prob", ctypes.c_int32), ("routed_scaling_factor", ctypes.c_float),
                ("act_dtype", ctypes.c_int32), ("weight_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32)]


class ForwardOpts(ctypes.Structure):
    _fields_ = [("epilogue", ctypes.c_int32), ("scores", ctypes.c_void_p), ("topk_ids", ctypes.c_void_p),
                ("topk_w", ctypes.c_void_p), ("expert_offsets", ctypes.c_void_p),
                ("permuted_src", ctypes.c_void_p), ("inv_perm", ctypes.c_void_p),
                ("events", ctypes.c_void_p * 4)]


def make_config(*, hidden, inter, n_experts, top_k, n_group=1, topk_group=1, shared_inter=0,
                scoring="softmax", norm_topk_prob=False, routed_scaling_factor=1.0,
                dtype="bf16") -> MoeConfig:
    """dtype: "f32" (everything fp32), "bf16" (bf16 activations and weights),
    "fp8" (bf16 activations and router, E4M3 expert weights) or "w4a16" (bf16
    activations and router, 4-bit expert weights)."""
    act = MOE_F32 if dtype == "f32" else MOE_BF16
    wdt = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8_E4M3, "w4a16": MOE_INT4}[dtype]
    return MoeConfig(hidden, inter, n_experts, top_k, n_group, topk_group, shared_inter,
                     MOE_SCORE_SOFTMAX if scoring == "softmax" else MOE_SCORE_SIGMOID,
                     int(bool(norm_topk_prob)), float(routed_scaling_factor), act, wdt, act)


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m mixture_experts_layer_limited_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        cfgp = ctypes.POINTER(MoeConfig)
        L.moe_workspace_size.argtypes = [cfgp, i64, i32]
        L.moe_workspace_size.restype = sz
        L.moe_validate_config.argtypes = [cfgp]
        L.moe_route.argtypes = [cfgp, i64, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_permute.argtypes = [cfgp, i64, vp, vp, vp, vp, vp, sz, vp]
        L.moe_grouped_swiglu.argtypes = [cfgp, i64, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, sz,
                                         vp]
        L.moe_combine.argtypes = [cfgp, i64, vp, vp, vp, vp, vp, vp, vp]
        L.moe_forward.argtypes = [cfgp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                  ctypes.POINTER(ForwardOpts), vp, sz, vp]
        L.moe_forward_static.argtypes = [cfgp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                         ctypes.POINTER(ForwardOpts), vp]
        L.moe_load_balance.argtypes = [cfgp, vp, vp, ctypes.c_float, vp, vp]
        L.moe_quantize_fp8_1x128.argtypes = [i64, i64, vp, i32, vp, vp, vp]
        L.moe_strerror.argtypes = [ctypes.c_int]
        L.moe_strerror.restype = ctypes.c_char_p
        L.moe_version.argtypes = []
        for name in ("moe_validate_config", "moe_route", "moe_permute", "moe_grouped_swiglu", "moe_combine",
                     "moe_forward", "moe_forward_static", "moe_load_balance", "moe_quantize_fp8_1x128",
                     "moe_version"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmoe355 must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(status: int, where: str):
    if status != 0:
        raise MoeError(status, where, lib().moe_strerror(status).decode())


def validate_config(cfg: MoeConfig) -> int:
    return lib().moe_validate_config(ctypes.byref(cfg))


def workspace_size(cfg: MoeConfig, T: int, op: int = MOE_OP_FORWARD) -> int:
    return lib().moe_workspace_size(ctypes.byref(cfg), T, op)


def workspace(cfg: MoeConfig, T: int, op: int = MOE_OP_FORWARD, device="cuda") -> torch.Tensor:
    """A uint8 device tensor large enough for `op` (torch allocations are 256-byte aligned)."""
    return torch.empty(max(workspace_size(cfg, T, op), 1), dtype=torch.uint8, device=device)


def _ws(ws):
    return (None, 0) if ws is None else (_ptr(ws), ws.numel() * ws.element_size())


def route(cfg, T, hidden, gate_w, bias, scores_in, scores_out, topk_ids, topk_w, ws=None, stream=None):
    wp, wb = _ws(ws)
    _check(lib().moe_route(ctypes.byref(cfg), T, _ptr(hidden), _ptr(gate_w), _ptr(bias), _ptr(scores_in),
                           _ptr(scores_out), _ptr(topk_ids), _ptr(topk_w), wp, wb, _stream(stream)), "moe_route")


def permute(cfg, T, topk_ids, expert_offsets, permuted_src, inv_perm, ws=None, stream=None):
    wp, wb = _ws(ws)
    _check(lib().moe_permute(ctypes.byref(cfg), T, _ptr(topk_ids), _ptr(expert_offsets), _ptr(permuted_src),
                             _ptr(inv_perm), wp, wb, _stream(stream)), "moe_permute")


def grouped_swiglu(cfg, T, hidden, hidden_scales, permuted_src, expert_offsets, w13, w13_scales, w2, w2_scales,
                   epilogue, topk_w, inv_perm, expert_out, acc, ws=None, stream=None):
    wp, wb = _ws(ws)
    _check(lib().moe_grouped_swiglu(ctypes.byref(cfg), T, _ptr(hidden), _ptr(hidden_scales), _ptr(permuted_src),
                                    _ptr(expert_offsets), _ptr(w13), _ptr(w13_scales), _ptr(w2), _ptr(w2_scales),
                                    epilogue, _ptr(topk_w), _ptr(inv_perm), _ptr(expert_out), _ptr(acc), wp, wb,
                                    _stream(stream)), "moe_grouped_swiglu")


def combine(cfg, T, expert_out, acc, inv_perm, topk_w, shared_out, out, stream=None):
    _check(lib().moe_combine(ctypes.byref(cfg), T, _ptr(expert_out), _ptr(acc), _ptr(inv_perm), _ptr(topk_w),
                             _ptr(shared_out), _ptr(out), _stream(stream)), "moe_combine")


@dataclass
class ForwardOutputs:
    """Optional intermediate outputs of forward(); any field may stay None."""
    scores: Optional[torch.Tensor] = None
    topk_ids: Optional[torch.Tensor] = None
    topk_w: Optional[torch.Tensor] = None
    expert_offsets: Optional[torch.Tensor] = None
    permuted_src: Optional[torch.Tensor] = None
    inv_perm: Optional[torch.Tensor] = None
    events: Optional[tuple] = None      # up to 4 raw hipEvent_t handles (ints) for the timing hooks


def forward(cfg, T, hidden, gate_w, bias, w13, w13_scales, w2, w2_scales, sh_w13, sh_w13_scales, sh_w2,
            sh_w2_scales, out, ws, epilogue=MOE_EPI_STORE_ROWS, aux: Optional[ForwardOutputs] = None,
            stream=None):
    aux = aux or ForwardOutputs()
    ev = (ctypes.c_void_p * 4)(*[(aux.events[i] if aux.events and i < len(aux.events) else None)
                                 for i in range(4)])
    opts = ForwardOpts(epilogue, _ptr(aux.scores), _ptr(aux.topk_ids), _ptr(aux.topk_w), _ptr(aux.expert_offsets),
                       _ptr(aux.permuted_src), _ptr(aux.inv_perm), ev)
    wp, wb = _ws(ws)
    _check(lib().moe_forward(ctypes.byref(cfg), T, _ptr(hidden), _ptr(gate_w), _ptr(bias), _ptr(w13),
                             _ptr(w13_scales), _ptr(w2), _ptr(w2_scales), _ptr(sh_w13), _ptr(sh_w13_scales),
                             _ptr(sh_w2), _ptr(sh_w2_scales), _ptr(out), ctypes.byref(opts), wp, wb,
                             _stream(stream)), "moe_forward")


def forward_static(cfg, T, hidden, gate_w, bias, w13, w13_scales, w2, w2_scales, sh_w13, sh_w13_scales, sh_w2,
                   sh_w2_scales, out, epilogue=MOE_EPI_STORE_ROWS, aux: Optional[ForwardOutputs] = None,
                   stream=None):
    """moe_forward_static: forward() with the library's static scratch instead of a workspace."""
    aux = aux or ForwardOutputs()
    ev = (ctypes.c_void_p * 4)(*[(aux.events[i] if aux.events and i < len(aux.events) else None)
                                 for i in range(4)])
    opts = ForwardOpts(epilogue, _ptr(aux.scores), _ptr(aux.topk_ids), _ptr(aux.topk_w), _ptr(aux.expert_offsets),
                       _ptr(aux.permuted_src), _ptr(aux.inv_perm), ev)
    _check(lib().moe_forward_static(ctypes.byref(cfg), T, _ptr(hidden), _ptr(gate_w), _ptr(bias), _ptr(w13),
                                    _ptr(w13_scales), _ptr(w2), _ptr(w2_scales), _ptr(sh_w13), _ptr(sh_w13_scales),
                                    _ptr(sh_w2), _ptr(sh_w2_scales), _ptr(out), ctypes.byref(opts),
                                    _stream(stream)), "moe_forward_static")


STATIC_SCRATCH_BYTES = 64 << 20   # MOE_STATIC_SCRATCH_BYTES of include/moe355.h


class LoadStats(ctypes.Structure):
    """moe_load_stats: expert load of one routed batch."""
    _fields_ = [("rows", ctypes.c_int32), ("min", ctypes.c_int32), ("max", ctypes.c_int32),
                ("empty", ctypes.c_int32), ("mean", ctypes.c_float), ("cv", ctypes.c_float)]


LOAD_STATS_BYTES = ctypes.sizeof(LoadStats)


def load_stats_from(buf: torch.Tensor) -> LoadStats:
    """Decode the moe_load_stats a device byte buffer received."""
    raw = bytes(buf.detach().cpu().numpy().tobytes()[:LOAD_STATS_BYTES])
    return LoadStats.from_buffer_copy(raw)


def load_balance(cfg: MoeConfig, expert_offsets: torch.Tensor, bias: Optional[torch.Tensor], gamma: float,
                 stats: Optional[torch.Tensor], stream=None):
    """moe_load_balance: bias [E] fp32 updated in place (or None); stats is a
    device uint8 buffer of at least LOAD_STATS_BYTES (or None)."""
    _check(lib().moe_load_balance(ctypes.byref(cfg), _ptr(expert_offsets), _ptr(bias), float(gamma), _ptr(stats),
                                  _stream(stream)), "moe_load_balance")


def quantize_fp8_1x128(x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, stream=None):
    dt = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16}[x.dtype]
    _check(lib().moe_quantize_fp8_1x128(x.shape[0], x.shape[1], _ptr(x), dt, _ptr(codes), _ptr(scales),
                                        _stream(stream)), "moe_quantize_fp8_1x128")
