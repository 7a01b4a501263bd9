"""Writes v3_decode_bias_seed0.json: the score-correction bias of the V3 decode
workload (128 tokens), calibrated so that expert load follows Zipf(s = 1.1).

The calibration runs the bias rule of the DeepSeek V3/R1 overview
(xxqk.cn/news/389306, §2.2: lower the bias of an expert that got more tokens
than its target, raise it for one that got fewer) on the oracle's routing of
the seeded decode batch:
  * a seeded permutation pi ranks the experts; expert of rank r (1-based) has
    target round(min(T, T*k * r^-1.1 / sum_r' r'^-1.1)) tokens;
  * b starts at 0; 300 rounds of b += 0.01 * sign(target - load);
  * b is frozen and stored as float32.
Only oracle/ does arithmetic here; moe_inputs draws the batch.

Run from the repository root:  python tests/golden/make_decode_bias.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from moe_inputs import PRESETS, routing_inputs, stream_seed  # noqa: E402

ZIPF_S = 1.1
GAMMA = 0.01
ROUNDS = 300


def main():
    cfg = PRESETS["v3_decode_bf16"].replace(bias="zero")
    r = routing_inputs(cfg, seed=0)
    x = r["x"].float().double().numpy()
    gw = r["gate_w"].float().double().numpy()
    s = oracle.score(oracle.router_logits(x, gw), cfg.scoring)
    T, k, E = cfg.tokens, cfg.top_k, cfg.n_experts
    rank = np.random.default_rng(stream_seed(0, "zipf_rank")).permutation(E) + 1   # rank of expert e
    zipf = rank.astype(np.float64) ** -ZIPF_S
    target = np.round(np.minimum(T, T * k * zipf / (np.arange(1, E + 1) ** -ZIPF_S).sum()))
    b = np.zeros(E)
    for _ in range(ROUNDS):
        ids = oracle.select_experts(s, b, k, cfg.n_group, cfg.topk_group)
        load = np.bincount(ids.reshape(-1), minlength=E)
        b = oracle.bias_update(b, load, target, GAMMA)
    b32 = b.astype(np.float32)
    ids = oracle.select_experts(s, b32.astype(np.float64), k, cfg.n_group, cfg.topk_group)
    st = oracle.load_stats(ids, E)
    out = {
        "source": "bias rule of the DeepSeek V3/R1 overview (xxqk.cn/news/389306 §2.2) run in reverse "
                  "toward Zipf(1.1) targets on the seeded V3 decode batch; written by make_decode_bias.py",
        "zipf_s": ZIPF_S, "gamma": GAMMA, "rounds": ROUNDS, "seed": 0,
        "rank": rank.tolist(), "target": target.astype(int).tolist(),
        "realised_counts": st["counts"].tolist(), "non_empty": int(E - st["empty"]),
        "cv": st["cv"], "max": st["max"],
        "bias": [float(v) for v in b32],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "v3_decode_bias_seed0.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(f"wrote {path}: non-empty experts {out['non_empty']}, max load {st['max']}, cv {st['cv']:.3f}")


if __name__ == "__main__":
    main()
