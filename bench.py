"""Benchmark of the MoE layer forward on one MI355X.

Default workload: the DeepSeek-V3 MoE layer, prefill batch of 8192 tokens
(H 7168, 256 routed experts of intermediate 2048, top-8 with sigmoid scores,
zero score-correction bias and 8/4 group limit, norm_topk_prob, scale 2.5, one
shared expert), bf16, synthetic seeded inputs resident in HBM.  One step is
one whole layer forward (router GEMM, scoring + top-k, permutation, routed
grouped SwiGLU GEMMs, shared expert, combine) through the C ABI.

Prints one JSON line.  `value` is layer tokens/s; `roofline` is for the
dominant kernel, the routed experts' gate/up GEMM with its SiLU*up epilogue,
timed live with HIP events the library records around it on the layer's
stream; `grouped_gemm` covers both routed GEMMs (gate/up and down);
`cpu_baseline` times the fp64 CPU oracle on a sample of the same workload.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X dense MFMA (fp32: vector/matrix fp32); 4-bit weights are widened to bf16 for the MFMAs
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3, "fp8": 5000.0, "w4a16": 2500.0}
PEAK_HBM_GBS = 8000.0
METRIC = "MoE layer tokens/s + grouped-GEMM TFLOPS (% MFMA peak) at V3 shape, 1 GPU"


def csrc_sha256():
    """Hash of the kernel sources: counter figures taken on other sources are stale."""
    d = os.path.join(ROOT, "mixture_experts_layer_limited_amd", "csrc")
    h = hashlib.sha256()
    for fn in sorted(os.listdir(d)):
        if fn.endswith((".hip", ".h", ".cpp")):
            h.update(fn.encode())
            with open(os.path.join(d, fn), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def measured_traffic(config):
    """HBM bytes per launch of the routed gate/up GEMM from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary of this workload (calibrated
    against a plain copy), or None when there is none or the kernels changed."""
    path = os.path.join(ROOT, "profiles", f"gemm_traffic_{config}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            k, sep, v = line.partition(":")
            if sep and k.strip() and " " not in k.strip():
                fields[k.strip()] = v.strip()
    if fields.get("csrc_sha256") != csrc_sha256() or "routed_gate_up_traffic_bytes" not in fields:
        return None
    return float(fields["routed_gate_up_traffic_bytes"])


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", default="v3_prefill_bf16")
    p.add_argument("--epilogue", choices=["store", "scatter"], default="store")
    p.add_argument("--cpu-sample", type=int, default=None,
                   help="tokens in the oracle's timed sample (0 = skip; default: about 10-30 s of host work)")
    return p.parse_args()


class HipEvents:
    """Raw hipEvent_t handles (the library records them on the layer's stream)."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(h.value)

    def ms(self, a, b):
        out = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return out.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


def cpu_baseline(cfg, inp, n_tokens):
    """The fp64 oracle, as it stands, on the first n_tokens tokens of the batch:
    fp64 router GEMM + scoring + group-limited top-k for those tokens, then
    their expert FFNs and the shared expert with weights decoded from the
    stored bf16 / E4M3 / 4-bit values.  Weights of the experts the sample
    needs are copied to host memory first (not timed)."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info

    x = inp["x"][:n_tokens].float().cpu().double().numpy()
    gw = inp["gate_w"].float().cpu().double().numpy()
    bias = None if inp["bias"] is None else inp["bias"].cpu().double().numpy()
    s, ids, w = oracle.route(x, gw, bias, scoring=cfg.scoring, top_k=cfg.top_k, n_group=cfg.n_group,
                             topk_group=cfg.topk_group, norm_topk_prob=cfg.norm_topk_prob,
                             routed_scaling_factor=cfg.routed_scaling_factor)
    need = sorted({int(e) for e in ids.reshape(-1)})
    fp8 = cfg.dtype == "fp8"
    scaled = cfg.dtype in ("fp8", "w4a16")
    host = {e: tuple(inp[n][e].cpu() for n in (("w13", "w13_s", "w2", "w2_s") if scaled else ("w13", "w2")))
            for e in need}
    sh = tuple(inp[n].cpu() for n in (("sh_w13", "sh_w13_s", "sh_w2", "sh_w2_s") if scaled else ("sh_w13", "sh_w2")))

    def dec(t, sc=None):
        if sc is None:
            return t.float().double().numpy()
        if fp8:
            return oracle.dequantize_blocks(t.numpy(), sc.numpy())
        return oracle.dequantize_int4_groups(t.numpy(), sc.numpy())

    def get_expert(e):
        h = host[e]
        return (dec(h[0], h[1]), dec(h[2], h[3])) if scaled else (dec(h[0]), dec(h[1]))

    def get_shared():
        return (dec(sh[0], sh[1]), dec(sh[2], sh[3])) if scaled else (dec(sh[0]), dec(sh[1]))

    q = None
    if fp8:
        def q(v):
            return oracle.dequantize_1x128(*oracle.quantize_1x128(v))
    t0 = time.perf_counter()
    s, ids, w = oracle.route(x, gw, bias, scoring=cfg.scoring, top_k=cfg.top_k, n_group=cfg.n_group,
                             topk_group=cfg.topk_group, norm_topk_prob=cfg.norm_topk_prob,
                             routed_scaling_factor=cfg.routed_scaling_factor)
    oracle.permute(ids, cfg.n_experts)
    oracle.moe_layer_rows(np.arange(n_tokens), x, ids, w, get_expert, get_shared, quantize_x=q, quantize_h=q)
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    return {"value": n_tokens / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "seconds": dt,
            "sample": f"first {n_tokens} tokens of the {cfg.tokens}-token batch: fp64 routing of those tokens, "
                      f"their {len(need)} routed expert FFNs and the shared expert, weights decoded to fp64 "
                      f"from the stored values"}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU: the layer runs on one MI355X here and --gpus {a.gpus} is not "
              f"supported (data parallelism over tokens needs no exchange; see the sharding notes)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import mixture_experts_layer_limited_amd as moe
    from moe_inputs import PRESETS, layer_inputs

    cfg = PRESETS[a.config]
    dev = "cuda"
    print(f"[bench] drawing inputs for {cfg.name} on {torch.cuda.get_device_name(0)}", file=sys.stderr, flush=True)
    inp = layer_inputs(cfg, 0, dev)
    c = moe.make_config(hidden=cfg.hidden, inter=cfg.inter, n_experts=cfg.n_experts, top_k=cfg.top_k,
                        n_group=cfg.n_group, topk_group=cfg.topk_group, shared_inter=cfg.shared_inter,
                        scoring=cfg.scoring, norm_topk_prob=cfg.norm_topk_prob,
                        routed_scaling_factor=cfg.routed_scaling_factor, dtype=cfg.dtype)
    T, E, k, H, I, Is = cfg.tokens, cfg.n_experts, cfg.top_k, cfg.hidden, cfg.inter, cfg.shared_inter
    epi = moe.MOE_EPI_SCATTER_ADD if a.epilogue == "scatter" else moe.MOE_EPI_STORE_ROWS
    out = torch.empty(T, H, dtype=inp["x"].dtype, device=dev)
    ws = moe.workspace(c, T, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)

    def step(events=None):
        moe.forward(c, T, inp["x"], inp["gate_w"], inp["bias"], inp["w13"], inp["w13_s"], inp["w2"], inp["w2_s"],
                    inp["sh_w13"], inp["sh_w13_s"], inp["sh_w2"], inp["sh_w2_s"], out, ws, epilogue=epi,
                    aux=moe.ForwardOutputs(expert_offsets=offsets, events=events))

    step()
    torch.cuda.synchronize()
    counts = np.diff(offsets.cpu().numpy())
    non_empty = int((counts > 0).sum())
    for _ in range(a.warmup):
        step()
    ev = HipEvents(4 * a.steps)
    torch.cuda.synchronize()
    # one event between consecutive steps: the whole region and every step's own time
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)]
    marks[0].record()
    for i in range(a.steps):
        step(tuple(ev.ev[4 * i:4 * i + 4]))
        marks[i + 1].record()
    torch.cuda.synchronize()
    ms = marks[0].elapsed_time(marks[-1]) / a.steps
    per_step = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(a.steps)])
    g1 = float(np.mean([ev.ms(ev.ev[4 * i], ev.ev[4 * i + 1]) for i in range(a.steps)]))
    g2 = float(np.mean([ev.ms(ev.ev[4 * i + 2], ev.ev[4 * i + 3]) for i in range(a.steps)]))
    ev.close()

    eb = {"f32": 4, "bf16": 2, "fp8": 1, "w4a16": 0.5}[cfg.dtype]   # bytes per expert weight
    ab = 4 if cfg.dtype == "f32" else 2
    # With the routed experts' width, stored rows and T <= 1024, the shared expert runs
    # as one more group of the routed GEMM launches, so the timed grouped GEMMs include it.
    merged = Is == I and Is > 0 and a.epilogue == "store" and E < 1024 and T <= 1024
    groups = non_empty + (1 if merged else 0)
    rows = T * k + (T if merged else 0)
    flops1 = 2.0 * rows * (2 * I) * H
    flops2 = 2.0 * rows * H * I
    # algorithmic bytes: weights of the groups that received rows, activations in, results out
    bytes1 = groups * 2 * I * H * eb + T * H * ab + rows * I * ab
    bytes2 = groups * H * I * eb + rows * I * ab + rows * H * ab
    if cfg.dtype == "fp8":
        bytes1 += groups * (2 * I // 128) * (H // 128) * 4 + T * (H // 128) * 4
        bytes2 += groups * (H // 128) * (I // 128) * 4
    if cfg.dtype == "w4a16":  # one fp32 scale per weight row and 128 columns
        bytes1 += groups * (2 * I) * (H // 128) * 4
        bytes2 += groups * H * (I // 128) * 4
    peak = PEAK_TFLOPS[cfg.dtype]
    ridge = peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    intensity = flops1 / bytes1
    if intensity < ridge:
        achieved = bytes1 / (g1 * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS}
    else:
        achieved = flops1 / (g1 * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak}
    roof.update({"traffic": measured_traffic(cfg.name),
                 "kernel": "gate/up grouped GEMM with the SiLU*up epilogue (routed experts"
                           + (" + the shared expert as one more group)" if merged else ")"),
                 "ms": g1, "algorithmic_bytes": bytes1, "algorithmic_flops": flops1})
    gg_tflops = (flops1 + flops2) / ((g1 + g2) * 1e-3) / 1e12
    result = {
        "metric": METRIC,
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "step_ms": {"median": float(np.median(per_step)), "p10": float(np.percentile(per_step, 10)),
                    "p90": float(np.percentile(per_step, 90))},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "w4a16" else cfg.dtype,
        "data": "synthetic (seeded N(0,1) activations, N(0,1/fan_in) weights)",
        "config": {"workload": f"{cfg.name}: T={T} H={H} E={E} I={I} k={k} groups {cfg.n_group}/{cfg.topk_group} "
                               f"{cfg.scoring} shared Is={Is}", "tokens": T, "hidden": H, "experts": E,
                   "inter": I, "top_k": k, "shared_inter": Is, "epilogue": a.epilogue,
                   "expert_weights": {"f32": "fp32", "bf16": "bf16", "fp8": "E4M3 + 128x128 fp32 scales",
                                      "w4a16": "int4 + fp32 scale per row and 128 columns"}[cfg.dtype],
                   "non_empty_experts": non_empty},
        "grouped_gemm": {"ms_gate_up": g1, "ms_down": g2, "shared_expert_included": merged,
                         "tflops": gg_tflops, "peak_tflops": peak,
                         "frac_mfma_peak": gg_tflops / peak,
                         "gb_s": (bytes1 + bytes2) / ((g1 + g2) * 1e-3) / 1e9},
        "roofline": roof,
    }
    # 4-bit weights are unpacked in numpy, which makes the oracle's per-token cost higher
    sample = a.cpu_sample if a.cpu_sample is not None else (24 if cfg.dtype == "w4a16" else 40)
    if sample > 0:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(cfg, inp, sample)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
