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
stream; `grouped_gemm` covers both routed GEMMs (gate/up and down); `decode` times
the V3 decode-shaped layer (T = 128, Zipf-skewed routing) the same way, as
weight streaming against the HBM peak; `cpu_baseline` times the fp64 CPU
oracle on a sample of the same workload shaped like the real batch.
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
    p.add_argument("--cpu-seconds", type=float, default=12.5,
                   help="about this much timed host work for the oracle's sample (0 = skip)")
    p.add_argument("--decode-steps", type=int, default=200,
                   help="timed forwards of the V3 decode layer reported beside the default workload (0 = skip)")
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


def _blas_info():
    from threadpoolctl import threadpool_info
    blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    threads = max([i.get("num_threads", 1) for i in blas] or [1])
    vendor = ", ".join(sorted({f"{i.get('internal_api')} {i.get('version') or ''}".strip() for i in blas})) or "none"
    return int(threads), vendor


def cpu_baseline(cfg, inp, min_seconds=10.0, max_experts=None):
    """The fp64 oracle, as it stands, on a bounded sample shaped like the real
    batch.  Timed: routing and permutation of all T tokens (fp64 router GEMM,
    scoring, group-limited top-k); then, expert by expert in id order, the
    expert FFN over every row the expert received (its real row count) until
    about min_seconds of work (or max_experts experts); then the shared expert
    on the same number of tokens as the sample's routed rows / k.  Decoding the
    stored bf16 / E4M3 / 4-bit weights to fp64 is not timed.  The layer time
    is extrapolated per routed row (T*k rows) and per shared-expert token (T);
    the combine (k*H multiply-adds per token, well under 1 % of the flops) is
    left out."""
    import numpy as np
    import oracle

    T, H, I, Is, E, k = cfg.tokens, cfg.hidden, cfg.inter, cfg.shared_inter, cfg.n_experts, cfg.top_k
    fp8 = cfg.dtype == "fp8"
    scaled = cfg.dtype in ("fp8", "w4a16")
    x = inp["x"].float().cpu().double().numpy()
    gw = inp["gate_w"].float().cpu().double().numpy()
    bias = None if inp["bias"] is None else inp["bias"].cpu().double().numpy()

    def dec(name, e=None):
        t = inp[name] if e is None else inp[name][e]
        if not scaled:
            return t.float().cpu().double().numpy()
        sc = (inp[name + "_s"] if e is None else inp[name + "_s"][e]).cpu().numpy()
        if fp8:
            return oracle.dequantize_blocks(t.cpu().numpy(), sc)
        return oracle.dequantize_int4_groups(t.cpu().numpy(), sc)

    q = oracle.quantize_dequantize_1x128 if fp8 else None
    t0 = time.perf_counter()
    s, ids, w = oracle.route(x, gw, bias, scoring=cfg.scoring, top_k=k, n_group=cfg.n_group,
                             topk_group=cfg.topk_group, norm_topk_prob=cfg.norm_topk_prob,
                             routed_scaling_factor=cfg.routed_scaling_factor)
    off, src, inv = oracle.permute(ids, E)
    t_route = time.perf_counter() - t0
    t_exp, rows, n_exp, flops = 0.0, 0, 0, 0.0
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        w13, w2 = dec("w13", e), dec("w2", e)
        xs = x[src[lo:hi]]
        t1 = time.perf_counter()
        oracle.expert_outputs(xs, np.array([0, hi - lo]), np.arange(hi - lo), lambda g: (w13, w2), q, q)
        t_exp += time.perf_counter() - t1
        rows += hi - lo
        n_exp += 1
        flops += 6.0 * (hi - lo) * H * I
        if t_route + t_exp >= 0.8 * min_seconds or (max_experts is not None and n_exp >= max_experts):
            break
    n_sh, t_sh = 0, 0.0
    if Is > 0:
        n_sh = min(T, max(1, rows // k))
        sh13, sh2 = dec("sh_w13"), dec("sh_w2")
        t1 = time.perf_counter()
        oracle.swiglu_ffn(x[:n_sh] if q is None else q(x[:n_sh]), sh13, sh2, q)
        t_sh = time.perf_counter() - t1
        flops += 6.0 * n_sh * H * Is
    est = t_route + t_exp * (T * k / rows) + (t_sh * T / n_sh if n_sh else 0.0)
    threads, vendor = _blas_info()
    whole = rows == T * k
    return {"value": T / est, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "seconds": t_route + t_exp + t_sh, "gflops_fp64": flops / (t_exp + t_sh) / 1e9, "blas": vendor,
            "extrapolated": not whole,
            "sample": (f"fp64 routing + permutation of all {T} tokens; routed expert FFNs of experts in id order "
                       f"over every row each received: {n_exp} experts, {rows} of {T * k} rows (real per-expert "
                       f"counts); shared expert on {n_sh} tokens; weights decoded to fp64 untimed"
                       + ("" if whole else "; layer time extrapolated per routed row and per shared token"))}


def oracle_check(cfg, inp, routing, out, samples=4):
    """Part of the oracle leg, outside any timed region: the benchmarked
    forward's routing and permutation against the oracle's selection from the
    same fp32 score tensor (bit-exact), and its output rows on a few sampled
    tokens against the oracle's fp64 layer (max |got - ref| / max |ref|)."""
    import numpy as np
    import oracle

    bias = None if inp["bias"] is None else inp["bias"].float().cpu().numpy()
    s = routing["scores"]
    ids = oracle.select_experts(s.astype(np.float32), bias, cfg.top_k, cfg.n_group, cfg.topk_group, dtype=np.float32)
    w = oracle.routing_weights(s, ids, cfg.norm_topk_prob, cfg.routed_scaling_factor)
    off, src, inv = oracle.permute(ids, cfg.n_experts)
    routing_exact = bool(np.array_equal(routing["topk_ids"], ids))
    perm_exact = bool(np.array_equal(routing["expert_offsets"], off) and np.array_equal(routing["permuted_src"], src)
                      and np.array_equal(routing["inv_perm"], inv))
    fp8 = cfg.dtype == "fp8"
    scaled = cfg.dtype in ("fp8", "w4a16")

    def dec(name, e=None):
        t = inp[name] if e is None else inp[name][e]
        if not scaled:
            return t.float().cpu().double().numpy()
        sc = (inp[name + "_s"] if e is None else inp[name + "_s"][e]).cpu().numpy()
        if fp8:
            return oracle.dequantize_blocks(t.cpu().numpy(), sc)
        return oracle.dequantize_int4_groups(t.cpu().numpy(), sc)

    rng = np.random.default_rng(11)
    toks = np.sort(rng.choice(cfg.tokens, size=min(samples, cfg.tokens), replace=False))
    q = oracle.quantize_dequantize_1x128 if fp8 else None
    shared = (lambda: (dec("sh_w13"), dec("sh_w2"))) if cfg.shared_inter > 0 else None
    ref = oracle.moe_layer_rows(toks, inp["x"].float().cpu().double().numpy(), ids, w,
                                lambda e: (dec("w13", e), dec("w2", e)), shared, quantize_x=q, quantize_h=q)
    got = out[toks].float().cpu().double().numpy()
    err = float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))
    tol = {"f32": 1e-4, "bf16": 1e-2, "fp8": 3e-2, "w4a16": 1e-2}[cfg.dtype]
    return {"routing_bit_exact": routing_exact, "permutation_bit_exact": perm_exact,
            "sampled_tokens": [int(t) for t in toks], "max_rel_err": err, "tol": tol, "within_tol": err <= tol}


def time_layer(moe, torch, np, cfg, inp, epilogue, steps, warmup):
    """Warm-up, then `steps` timed forwards of the layer: the region's mean per
    forward, every forward's own time, and the routed gate/up and down GEMMs'
    times from the events the library records on its stream."""
    dev = "cuda"
    c = moe.make_config(hidden=cfg.hidden, inter=cfg.inter, n_experts=cfg.n_experts, top_k=cfg.top_k,
                        n_group=cfg.n_group, topk_group=cfg.topk_group, shared_inter=cfg.shared_inter,
                        scoring=cfg.scoring, norm_topk_prob=cfg.norm_topk_prob,
                        routed_scaling_factor=cfg.routed_scaling_factor, dtype=cfg.dtype)
    T, E, H = cfg.tokens, cfg.n_experts, cfg.hidden
    epi = moe.MOE_EPI_SCATTER_ADD if epilogue == "scatter" else moe.MOE_EPI_STORE_ROWS
    out = torch.empty(T, H, dtype=inp["x"].dtype, device=dev)
    ws = moe.workspace(c, T, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)

    def step(events=None, aux=None):
        moe.forward(c, T, inp["x"], inp["gate_w"], inp["bias"], inp["w13"], inp["w13_s"], inp["w2"], inp["w2_s"],
                    inp["sh_w13"], inp["sh_w13_s"], inp["sh_w2"], inp["sh_w2_s"], out, ws, epilogue=epi,
                    aux=aux or moe.ForwardOutputs(expert_offsets=offsets, events=events))

    # first (untimed) call: the routing and permutation of this batch, for the load summary and the checks
    k = cfg.top_k
    first = moe.ForwardOutputs(scores=torch.empty(T, E, dtype=torch.float32, device=dev),
                               topk_ids=torch.empty(T, k, dtype=torch.int32, device=dev),
                               topk_w=torch.empty(T, k, dtype=torch.float32, device=dev), expert_offsets=offsets,
                               permuted_src=torch.empty(T * k, dtype=torch.int32, device=dev),
                               inv_perm=torch.empty(T * k, dtype=torch.int32, device=dev))
    step(aux=first)
    torch.cuda.synchronize()
    routing = {f: getattr(first, f).cpu().numpy() for f in ("scores", "topk_ids", "topk_w", "expert_offsets",
                                                            "permuted_src", "inv_perm")}
    counts = np.diff(routing["expert_offsets"]).astype(np.float64)
    non_empty = int((counts > 0).sum())
    for _ in range(warmup):
        step()
    ev = HipEvents(4 * steps)
    torch.cuda.synchronize()
    # one event between consecutive steps: the whole region and every step's own time
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    marks[0].record()
    for i in range(steps):
        step(tuple(ev.ev[4 * i:4 * i + 4]))
        marks[i + 1].record()
    torch.cuda.synchronize()
    ms = marks[0].elapsed_time(marks[-1]) / steps
    per_step = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(steps)])
    g1 = float(np.mean([ev.ms(ev.ev[4 * i], ev.ev[4 * i + 1]) for i in range(steps)]))
    g2 = float(np.mean([ev.ms(ev.ev[4 * i + 2], ev.ev[4 * i + 3]) for i in range(steps)]))
    ev.close()
    load = {"min": int(counts.min()), "max": int(counts.max()), "mean": float(counts.mean()),
            "cv": float(counts.std(ddof=1) / counts.mean()) if counts.size > 1 and counts.mean() > 0 else 0.0,
            "empty": int((counts == 0).sum())}
    return ms, per_step, g1, g2, non_empty, load, routing, out


def work(cfg, epilogue, non_empty):
    """Algorithmic flops and bytes of the routed gate/up GEMM (1), the routed
    down GEMM (2) and the whole layer: each non-empty expert's weights once,
    activations in, results out (padding rows, permuted copies and re-reads
    are not counted)."""
    T, E, k, H, I, Is = cfg.tokens, cfg.n_experts, cfg.top_k, cfg.hidden, cfg.inter, cfg.shared_inter
    eb = {"f32": 4, "bf16": 2, "fp8": 1, "w4a16": 0.5}[cfg.dtype]   # bytes per expert weight
    ab = 4 if cfg.dtype == "f32" else 2                              # bytes per activation (x, out)
    qb = 1 if cfg.dtype == "fp8" else ab                             # bytes per GEMM operand (x, h)
    # With the routed experts' width, stored rows and T <= 1024, the shared expert runs
    # as one more group of the routed GEMM launches, so the timed grouped GEMMs include it.
    merged = Is == I and Is > 0 and epilogue == "store" and E < 1024 and T <= 1024
    groups = non_empty + (1 if merged else 0)
    rows = T * k + (T if merged else 0)
    flops1 = 2.0 * rows * (2 * I) * H
    flops2 = 2.0 * rows * H * I
    bytes1 = groups * 2 * I * H * eb + T * H * qb + rows * I * qb
    bytes2 = groups * H * I * eb + rows * I * qb + rows * H * ab
    if cfg.dtype == "fp8":   # 128x128 weight-block scales, 1x128 activation scales (x in, h out, h in)
        bytes1 += groups * (2 * I // 128) * (H // 128) * 4 + T * (H // 128) * 4 + rows * (I // 128) * 4
        bytes2 += groups * (H // 128) * (I // 128) * 4 + rows * (I // 128) * 4
    if cfg.dtype == "w4a16":  # one fp32 scale per weight row and 128 columns
        bytes1 += groups * (2 * I) * (H // 128) * 4
        bytes2 += groups * H * (I // 128) * 4
    # the whole layer: router weight, every non-empty expert and the shared expert once, x in, out
    sh_bytes = 3 * H * Is * eb if Is > 0 else 0
    layer_bytes = E * H * ab + non_empty * 3 * I * H * eb + sh_bytes + 2 * T * H * ab
    return dict(merged=merged, rows=rows, flops1=flops1, flops2=flops2, bytes1=bytes1, bytes2=bytes2,
                layer_bytes=layer_bytes)


def decode_object(moe, torch, np, layer_inputs, PRESETS, steps, warmup):
    """The decode-shaped layer (V3 dims, T = 128, Zipf-skewed routing) timed the
    same way: weight streaming against the HBM peak."""
    cfg = PRESETS["v3_decode_bf16"]
    print(f"[bench] drawing inputs for {cfg.name}", file=sys.stderr, flush=True)
    inp = layer_inputs(cfg, 0, "cuda")
    ms, per_step, g1, g2, non_empty, load, _, _ = time_layer(moe, torch, np, cfg, inp, "store", steps, warmup)
    w = work(cfg, "store", non_empty)
    gemm_bytes = w["bytes1"] + w["bytes2"]
    del inp
    torch.cuda.empty_cache()
    return {"workload": f"{cfg.name}: T={cfg.tokens} H={cfg.hidden} E={cfg.n_experts} I={cfg.inter} "
                        f"k={cfg.top_k} groups {cfg.n_group}/{cfg.topk_group} sigmoid + Zipf(1.1)-calibrated bias, "
                        f"shared Is={cfg.shared_inter}, bf16",
            "steps": steps, "warmup": warmup, "ms_per_step": ms, "tokens_per_s": cfg.tokens / (ms * 1e-3),
            "step_ms_median": float(np.median(per_step)), "non_empty_experts": non_empty, "expert_load": load,
            "layer_bytes": w["layer_bytes"], "layer_gb_s": w["layer_bytes"] / (ms * 1e-3) / 1e9,
            "layer_hbm_frac": w["layer_bytes"] / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "ms_gate_up": g1, "ms_down": g2, "grouped_gemm_bytes": gemm_bytes,
            "grouped_gemm_gb_s": gemm_bytes / ((g1 + g2) * 1e-3) / 1e9,
            "grouped_gemm_hbm_frac": gemm_bytes / ((g1 + g2) * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "shared_expert_included": w["merged"]}


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
    print(f"[bench] drawing inputs for {cfg.name} on {torch.cuda.get_device_name(0)}", file=sys.stderr, flush=True)
    inp = layer_inputs(cfg, 0, "cuda")
    T, E, k, H, I, Is = cfg.tokens, cfg.n_experts, cfg.top_k, cfg.hidden, cfg.inter, cfg.shared_inter
    ms, per_step, g1, g2, non_empty, load, routing, out = time_layer(moe, torch, np, cfg, inp, a.epilogue, a.steps,
                                                                      a.warmup)
    w = work(cfg, a.epilogue, non_empty)
    flops1, flops2, bytes1, bytes2, merged = w["flops1"], w["flops2"], w["bytes1"], w["bytes2"], w["merged"]
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
                 "ms": g1, "algorithmic_bytes": bytes1, "algorithmic_flops": flops1,
                 "mfma_frac": flops1 / (g1 * 1e-3) / 1e12 / peak})
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
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) activations, N(0,1/fan_in) weights)",
        "config": {"workload": f"{cfg.name}: T={T} H={H} E={E} I={I} k={k} groups {cfg.n_group}/{cfg.topk_group} "
                               f"{cfg.scoring} shared Is={Is}", "tokens": T, "hidden": H, "experts": E,
                   "inter": I, "top_k": k, "shared_inter": Is, "epilogue": a.epilogue,
                   "expert_weights": {"f32": "fp32", "bf16": "bf16", "fp8": "E4M3 + 128x128 fp32 scales",
                                      "w4a16": "int4 + fp32 scale per row and 128 columns, bf16 MFMAs"}[cfg.dtype],
                   "non_empty_experts": non_empty, "expert_load": load},
        "grouped_gemm": {"ms_gate_up": g1, "ms_down": g2, "shared_expert_included": merged,
                         "tflops": gg_tflops, "peak_tflops": peak,
                         "frac_mfma_peak": gg_tflops / peak,
                         "gb_s": (bytes1 + bytes2) / ((g1 + g2) * 1e-3) / 1e9},
        "roofline": roof,
    }
    if a.cpu_seconds > 0:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(cfg, inp, min_seconds=a.cpu_seconds)
        result["cpu_baseline"]["check"] = oracle_check(cfg, inp, routing, out)
    if a.config == "v3_prefill_bf16" and a.decode_steps > 0:
        del inp
        torch.cuda.empty_cache()
        result["decode"] = decode_object(moe, torch, np, layer_inputs, PRESETS, a.decode_steps, a.warmup)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
