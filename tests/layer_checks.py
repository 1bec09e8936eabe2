"""Shared pieces of the GPU layer tests: tolerances, descriptors, the
whole-layer runner and the routing near-tie check (no layer arithmetic)."""
import numpy as np
import torch

import mixture_experts_layer_02_amd as moe
import synth
from gpu_util import to_dev

TOL = {"bf16": 2e-2, "f32": 1e-5}
LOGIT_TOL = 1e-5
W_ATOL, W_RTOL = 1e-6, 2e-6


def _desc(T, d, f, E, k, e0, NL, dtype, renorm=1):
    return moe.make_desc(T, d, f, E, k, e0, NL, moe.MOE_BF16 if dtype == "bf16" else moe.MOE_F32, renorm)


def _routing_agreement(idx_g, L_ref, idx_ref):
    """Tokens whose selection (set and slot order) equals the oracle's.

    Where they differ, the difference must be a near-tie of the oracle's own
    float64 logits: either the same set in another order, or the lowest logit
    the GPU kept is within the logit tolerance of the highest one it left out.
    """
    same = (idx_g == idx_ref).all(axis=1)
    for t in np.nonzero(~same)[0]:
        row = L_ref[t]
        if set(idx_g[t].tolist()) == set(idx_ref[t].tolist()):
            continue
        tol = 10 * LOGIT_TOL * max(1.0, np.abs(row).max())
        kept = row[idx_g[t]].min()
        left_out = row[sorted(set(idx_ref[t].tolist()) - set(idx_g[t].tolist()))].max()
        assert left_out - kept <= tol, (t, kept, left_out)
    return same


def _run_layer(cfg, backward, gpu, n_groups=1):
    inp = synth.make_inputs(cfg)
    dt = cfg.dtype
    D = _desc(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.expert_begin, cfg.num_local, dt, cfg.renormalize)
    b = moe.Buffers(D, backward=backward)
    dev = {n: to_dev(inp[n]) for n in ("x", "wr", "w1", "w3", "w2", "dy")}
    bias = to_dev(inp["bias"]) if "bias" in inp else None
    routing = (to_dev(inp["idx"]), to_dev(inp["w"])) if cfg.routing == "roundrobin" else None
    moe.forward(b, dev["x"], dev["wr"], dev["w1"], dev["w3"], dev["w2"], bias=bias, routing=routing,
                n_groups=n_groups)
    if backward:
        moe.backward(b, dev["x"], dev["wr"], dev["w1"], dev["w3"], dev["w2"], dev["dy"], routing=routing)
    torch.cuda.synchronize()
    return inp, b
