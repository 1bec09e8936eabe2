"""Calibrate beta of the Zipf-skewed router bias (workload zipf_1t).

Finds beta >= 0 by bisection so that, routing the seeded tokens with the
oracle (float64 logits + bias, top-k), the busiest expert receives 10x the
mean per-expert load.  Calls only oracle/ and synth; writes zipf_beta.json
next to this file.  Run:  python tests/golden/calibrate_zipf.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402


def load_ratio(cfg, base_logits, beta):
    bias = synth.zipf_bias(synth.scaled(cfg, zipf_beta=beta)).astype(np.float64)
    idx, _ = oracle.topk_route(base_logits + bias[None, :], cfg.k)
    counts, _ = oracle.count_tokens(idx, cfg.E, 0, cfg.E)
    return counts.max() / (cfg.T * cfg.k / cfg.E)


def main():
    cfg = synth.CONFIGS["zipf_1t"]
    inp = synth.make_inputs(cfg, want=("wr", "x"))
    L = oracle.router_logits(synth.as_f32(inp["x"], cfg.dtype), synth.as_f32(inp["wr"], cfg.dtype))
    lo, hi = 0.0, 8.0
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        if load_ratio(cfg, L, mid) < 10.0:
            lo = mid
        else:
            hi = mid
    # round to a short binary fraction so the constant is exact in source
    beta = float(np.round(hi * 1024) / 1024)
    ratio = load_ratio(cfg, L, beta)
    out = {"workload": cfg.name, "beta": beta, "max_over_mean": float(ratio),
           "target": "max/mean per-expert load = 10 +- 0.25"}
    with open(os.path.join(os.path.dirname(__file__), "zipf_beta.json"), "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
