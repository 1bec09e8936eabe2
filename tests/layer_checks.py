"""Shared pieces of the GPU layer tests: tolerances, descriptors, the
whole-layer runner, the routing near-tie check and the whole-layer comparison
with the oracle (no layer arithmetic of their own)."""
import numpy as np
import torch

import mixture_experts_layer_02_amd as moe
import oracle
import synth
from gpu_util import f64, to_dev, to_host
from metrics import max_row_rel_err, whole_rel_err

TOL = {"bf16": 2e-2, "f32": 1e-5}
LOGIT_TOL = 1e-5
W_ATOL, W_RTOL = 1e-6, 2e-6


def random_routing(rng, T, E, k, skew=0.0):
    """Distinct experts per token; skew > 0 draws experts with Zipf-like popularity."""
    keys = rng.random((T, E))
    if skew > 0:
        pop = (np.arange(E) + 1.0) ** -skew
        keys = keys ** (1.0 / pop[rng.permutation(E)])
    return np.argsort(-keys, axis=1)[:, :k].astype(np.int32)


def _desc(T, d, f, E, k, e0, NL, dtype, renorm=1, wgrad="f32", tile_counters=None):
    return moe.make_desc(T, d, f, E, k, e0, NL, moe.MOE_BF16 if dtype == "bf16" else moe.MOE_F32, renorm,
                         tile_counters=tile_counters, wgrad_dtype=wgrad)


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


def _run_layer(cfg, backward, gpu, n_groups=1, gather=False, inp=None, gather_dy=None, wgrad="f32",
               tile_counters=None):
    inp = synth.make_inputs(cfg) if inp is None else inp
    dt = cfg.dtype
    D = _desc(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.expert_begin, cfg.num_local, dt, cfg.renormalize, wgrad,
              tile_counters)
    b = moe.Buffers(D, backward=backward, gather=gather, gather_dy=gather_dy)
    dev = {n: to_dev(inp[n]) for n in ("x", "wr", "w1", "w3", "w2", "dy")}
    bias = to_dev(inp["bias"]) if "bias" in inp else None
    routing = (to_dev(inp["idx"]), to_dev(inp["w"])) if cfg.routing == "roundrobin" else None
    moe.forward(b, dev["x"], dev["wr"], dev["w1"], dev["w3"], dev["w2"], bias=bias, routing=routing,
                n_groups=n_groups)
    if backward:
        moe.backward(b, dev["x"], dev["wr"], dev["w1"], dev["w3"], dev["w2"], dev["dy"], routing=routing)
    torch.cuda.synchronize()
    return inp, b


def check_layer_backward(cfg, inp, b):
    """Every forward and backward output of a GPU layer pass (Buffers b, run
    on inputs inp) against the oracle's layer on the same inputs.  The GPU
    routes on its own logits and the oracle on its own float64 logits; the
    shapes used here have no near-tie, so the routings must agree exactly."""
    dt = cfg.dtype
    tol = TOL[dt]
    x, wr = f64(inp["x"], dt), f64(inp["wr"], dt)
    w1, w3, w2 = f64(inp["w1"], dt), f64(inp["w3"], dt), f64(inp["w2"], dt)
    dy = f64(inp["dy"], dt)
    ref = oracle.layer_forward(x, wr, w1, w3, w2, cfg.k, cfg.expert_begin, cfg.num_local, cfg.renormalize)
    same = _routing_agreement(to_host(b.topk_idx), ref["logits"], ref["idx"])
    assert same.all(), "a routing near-tie flipped; the weight gradients are not comparable"
    np.testing.assert_array_equal(to_host(b.offsets), ref["offsets"])
    np.testing.assert_array_equal(to_host(b.slot_row), ref["slot_row"])
    g = oracle.layer_backward(ref, x, wr, w1, w3, w2, dy, cfg.renormalize)
    R = int(ref["offsets"][-1])
    assert max_row_rel_err(to_host(b.y), ref["y"]) <= tol
    if b.dy_perm is not None:
        assert max_row_rel_err(to_host(b.dy_perm)[:R], g["dy_perm"]) <= tol
    # dw and dlogits are scored against the whole tensor's maximum:
    # dw[t][j] = <y_perm[row], dy[t]> is a dot product over d whose rounding
    # error scales with the norms of its operands, not with its (often
    # cancelling) value, so a per-token row of k values is ill-conditioned.
    assert whole_rel_err(to_host(b.dtopk_w), g["dw"]) <= tol
    dgu = to_host(b.dgu)[:R]
    assert max_row_rel_err(dgu[:, :cfg.f], g["dG"]) <= tol
    assert max_row_rel_err(dgu[:, cfg.f:], g["dU"]) <= tol
    assert max_row_rel_err(to_host(b.dx_perm)[:R], g["dx_perm"]) <= tol
    for n in range(cfg.num_local):
        assert whole_rel_err(to_host(b.dW1)[n], g["dW1"][n]) <= tol, n
        assert whole_rel_err(to_host(b.dW3)[n], g["dW3"][n]) <= tol, n
        assert whole_rel_err(to_host(b.dW2)[n], g["dW2"][n]) <= tol, n
    assert whole_rel_err(to_host(b.dlogits), g["dlogits"]) <= tol
    assert whole_rel_err(to_host(b.dWr), g["dWr"]) <= tol
    assert max_row_rel_err(to_host(b.dx), g["dx"]) <= tol
