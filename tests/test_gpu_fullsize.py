"""GPU parity at the full 1T-shape workloads, on sampled outputs.

The whole layer runs at full size (the kernels, tile counts and launch shapes
of the benchmark); the float64 oracle then recomputes what it can afford:

* router logits and top-k of every token (one matrix product and a sort);
* counts, offsets and both index maps of every token, bit-exact, whenever the
  two routings agree everywhere (else the GPU's maps are checked for validity
  against its own selection, and every disagreement must be a near-tie);
* for a seeded sample of tokens (plus the first and the last), every per-row
  quantity: x_perm, gate/up, h, y_perm, y and, with the backward, dy_perm,
  dtopk_w, dG/dU, dx_perm, dlogits and dx (expert rows plus the router term).  Each of these depends on its own
  token only, so the oracle computes them by running the layer on the sample;
* the weight gradients dW1, dW3, dW2 of two whole experts (the least and the
  most loaded local expert that no near-tie touches), from the oracle's own
  routing of every token;
* the forward again with the gather fused into the GEMMs, whose every output
  must equal the x_perm path's bit for bit; and the forward + backward with
  x and dy read in place (the configuration the benchmark times), checked
  like the x_perm path above, plus its per-row weights and hw = w silu(G) U.

dWr sums dlogits over all tokens, and dlogits needs every token's expert
outputs, which is beyond what the oracle finishes in seconds at this size.
It is checked by the property that defines it, dWr = dlogits^T x, on sampled
entries with the GPU's dlogits (dlogits itself is checked on the sample
above), and against the oracle on the sampled tokens: the router backward
runs again at the full shape, with the split and launches of the layer's
own call, on a dlogits that holds the oracle's sampled rows and zeros
elsewhere; its dWr must equal the oracle's dWr of the sampled tokens alone,
and its input gradient the oracle's on those tokens.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import f64, to_host
from layer_checks import LOGIT_TOL, TOL, _routing_agreement, _run_layer
from metrics import max_row_rel_err, whole_rel_err

pytestmark = pytest.mark.gpu

N_SAMPLE = 62


def _sample_tokens(T, seed):
    rng = np.random.default_rng(seed)
    s = rng.choice(np.arange(1, T - 1), size=min(N_SAMPLE, T - 2), replace=False)
    return np.unique(np.concatenate([[0, T - 1], s])).astype(np.int64)


def _rows_t(t, rows):
    return to_host(t[torch.as_tensor(rows, device=t.device)])


def _dev_bf16(inp, name, dev):
    return torch.from_numpy(inp[name].view(np.int16)).to(dev).view(torch.bfloat16)


def _rows(b, name, rows):
    """Rows of a GPU buffer, fetched without copying the whole tensor."""
    return to_host(getattr(b, name)[torch.as_tensor(rows, device=getattr(b, name).device)])


def _check_index_maps(cfg, idx, counts, offsets, row_token, slot_row):
    """The GPU's counts and index maps are a valid stable counting sort of idx."""
    E, e0, NL = cfg.E, cfg.expert_begin, cfg.num_local
    assert (counts == np.bincount(idx.reshape(-1), minlength=E)).all()
    assert offsets[0] == 0 and (np.diff(offsets) == counts[e0:e0 + NL]).all()
    local = (idx >= e0) & (idx < e0 + NL)
    assert ((slot_row >= 0) == local).all()
    t_of, j_of = np.nonzero(local)
    r = slot_row[t_of, j_of]
    assert (row_token[r] == t_of).all()
    n = idx[t_of, j_of] - e0
    assert ((r >= offsets[n]) & (r < offsets[n + 1])).all()
    order = np.lexsort((t_of, n))                 # by expert, then ascending token
    assert (r[order] == np.arange(len(r))).all()


@pytest.mark.parametrize("name,gather,gather_dy,wgrad", [
    ("share_1t", False, False, "f32"), ("zipf_1t", False, False, "f32"), ("uniform_1t", False, False, "f32"),
    ("fwdbwd_1t", False, False, "f32"),
    ("fwdbwd_1t", False, True, "f32"),
    ("fwdbwd_1t", False, True, "bf16"),  # the benchmark's configuration: x_perm, dy read in place, bf16 dW
    ("fwdbwd_1t", True, True, "f32")])
def test_full_size_layer_sampled(gpu, name, gather, gather_dy, wgrad):
    cfg = synth.CONFIGS[name]
    back = cfg.backward
    print(f"[fullsize] {name}: T={cfg.T} d={cfg.d} f={cfg.f} E={cfg.E} NL={cfg.num_local} k={cfg.k} "
          f"backward={back} gather={gather} gather_dy={gather_dy} wgrad={wgrad}", flush=True)
    inp, b = _run_layer(cfg, back, gpu, gather=gather, gather_dy=gather_dy, wgrad=wgrad)
    dt, tol = cfg.dtype, TOL[cfg.dtype]
    T, E, k, e0, NL, f = cfg.T, cfg.E, cfg.k, cfg.expert_begin, cfg.num_local, cfg.f
    x32 = synth.as_f32(inp["x"], dt)
    wr = f64(inp["wr"], dt)
    bias = inp.get("bias")

    # --- routing of every token -------------------------------------------
    idx_g = to_host(b.topk_idx) if cfg.routing != "roundrobin" else inp["idx"]
    if cfg.routing == "roundrobin":
        idx_o, w_o = inp["idx"], inp["w"].astype(np.float64)
        same = np.ones(T, bool)
    else:
        L_o = oracle.router_logits(x32, wr, bias)
        L_g = to_host(b.logits)
        assert max_row_rel_err(L_g, L_o) <= LOGIT_TOL
        idx_o, w_o = oracle.topk_route(L_o, k, cfg.renormalize)
        same = _routing_agreement(idx_g, L_o, idx_o)
        assert same.mean() > 0.999
        w_g = to_host(b.topk_w)
        np.testing.assert_allclose(w_g[same], w_o[same], rtol=1e-4, atol=1e-6)

    counts_g, offsets_g = to_host(b.counts), to_host(b.offsets)
    slot_g = to_host(b.slot_row)
    R = int(offsets_g[-1])
    row_token_g = to_host(b.row_token)[:R]
    if same.all():
        counts_o, offsets_o = oracle.count_tokens(idx_o, E, e0, NL)
        row_token_o, slot_o = oracle.generate_indices(idx_o, e0, NL, offsets_o)
        np.testing.assert_array_equal(counts_g, counts_o)
        np.testing.assert_array_equal(offsets_g, offsets_o)
        np.testing.assert_array_equal(row_token_g, row_token_o)
        np.testing.assert_array_equal(slot_g, slot_o)
    else:
        _check_index_maps(cfg, idx_g, counts_g, offsets_g, to_host(b.row_token), slot_g)

    if not gather:
        # x_perm: every row bit-exact (a copy)
        xp = b.x_perm[:R]
        xs = torch.as_tensor(row_token_g.astype(np.int64), device=xp.device)
        x_dev = torch.from_numpy(inp["x"].view(np.int16)).to(xp.device)
        assert torch.equal(xp.view(torch.int16), x_dev[xs]), "x_perm rows differ from x[row_token]"
        del x_dev, xs

    if not gather and not gather_dy:
        # the gather-fused forward (no x_perm) gives bitwise the same outputs
        _, bg = _run_layer(cfg, False, gpu, gather=True, inp=inp)
        names = (["topk_idx"] if cfg.routing != "roundrobin" else []) + ["offsets", "slot_row", "row_token",
                                                                           "h", "y_perm", "y"]
        for n in names:
            a, c = getattr(b, n), getattr(bg, n)
            if a.shape[0] == b.desc.R_cap and n not in ("topk_idx", "slot_row"):
                a, c = a[:R], c[:R]
            assert torch.equal(a.view(torch.uint8) if a.dtype != torch.int32 else a,
                               c.view(torch.uint8) if c.dtype != torch.int32 else c), n
        del bg
        torch.cuda.empty_cache()

    # --- per-token quantities on a sample --------------------------------
    toks = _sample_tokens(T, cfg.seed)
    toks = toks[same[toks]]
    W = {n: synth.as_f32(inp[n], dt) for n in ("w1", "w3", "w2")}
    xs = x32[toks].astype(np.float64)
    routing = (inp["idx"][toks], inp["w"][toks]) if cfg.routing == "roundrobin" else None
    ref = oracle.layer_forward(xs, wr, W["w1"], W["w3"], W["w2"], k, e0, NL, cfg.renormalize,
                               bias=bias, routing=routing)
    sl_o = ref["slot_row"]
    ti, tj = np.nonzero(sl_o >= 0)
    r_o = sl_o[ti, tj]
    r_g = slot_g[toks[ti], tj]
    assert (r_g >= 0).all()
    gu = _rows(b, "gu", r_g) if back else None
    if gu is not None:
        assert max_row_rel_err(gu[:, :f], ref["G"][r_o]) <= tol
        assert max_row_rel_err(gu[:, f:], ref["U"][r_o]) <= tol
    assert max_row_rel_err(_rows(b, "h", r_g), ref["H"][r_o]) <= tol
    assert max_row_rel_err(_rows(b, "y_perm", r_g), ref["y_perm"][r_o]) <= tol
    assert max_row_rel_err(_rows(b, "y", toks), ref["y"]) <= tol
    if not back:
        return

    dy_s = f64(inp["dy"][toks], dt)
    g = oracle.layer_backward(ref, xs, wr, W["w1"], W["w3"], W["w2"], dy_s, cfg.renormalize)
    if gather_dy:
        # the weight each row carries, and hw = w silu(G) U (dW2's operand)
        w_rows = ref["w"][ti, tj]
        assert np.allclose(_rows(b, "row_w", r_g), w_rows, rtol=1e-4, atol=1e-6)
        assert max_row_rel_err(_rows(b, "hw", r_g), w_rows[:, None] * ref["H"][r_o]) <= tol
    else:
        assert max_row_rel_err(_rows(b, "dy_perm", r_g), g["dy_perm"][r_o]) <= tol
    assert whole_rel_err(_rows(b, "dtopk_w", toks), g["dw"]) <= tol
    dgu = _rows(b, "dgu", r_g)
    assert max_row_rel_err(dgu[:, :f], g["dG"][r_o]) <= tol
    assert max_row_rel_err(dgu[:, f:], g["dU"][r_o]) <= tol
    assert max_row_rel_err(_rows(b, "dx_perm", r_g), g["dx_perm"][r_o]) <= tol
    assert whole_rel_err(_rows(b, "dlogits", toks), g["dlogits"]) <= tol
    assert max_row_rel_err(_rows(b, "dx", toks), g["dx"]) <= tol

    # --- weight gradients of two whole experts ---------------------------
    flipped = np.unique(np.concatenate([idx_g[~same].ravel(), idx_o[~same].ravel()]))
    cnt = np.array([(idx_o == e0 + n).sum() for n in range(NL)])
    ok = [n for n in range(NL) if cnt[n] > 0 and (e0 + n) not in flipped]
    assert ok
    picks = sorted({min(ok, key=lambda n: cnt[n]), max(ok, key=lambda n: cnt[n])})
    dy32 = synth.as_f32(inp["dy"], dt)
    for n in picks:
        t_n, j_n = np.nonzero(idx_o == e0 + n)        # ascending tokens
        xr = x32[t_n].astype(np.float64)
        dyr = w_o[t_n, j_n][:, None] * dy32[t_n].astype(np.float64)
        _, _, _, dW1, dW3, dW2 = oracle.expert_ffn_bwd_rows(xr, W["w1"][n], W["w3"][n], W["w2"][n], dyr)
        assert whole_rel_err(to_host(b.dW1[n]), dW1) <= tol, n
        assert whole_rel_err(to_host(b.dW3[n]), dW3) <= tol, n
        assert whole_rel_err(to_host(b.dW2[n]), dW2) <= tol, n

    # --- router backward at full shape on the oracle's sampled dlogits ---------
    import mixture_experts_layer_02_amd as moe
    from layer_checks import _desc
    D = _desc(T, cfg.d, f, E, k, e0, NL, dt, cfg.renormalize)
    dl_full = torch.zeros(T, E, dtype=torch.float32, device=b.dlogits.device)
    dl_full[torch.as_tensor(toks, device=dl_full.device)] = torch.from_numpy(
        g["dlogits"].astype(np.float32)).to(dl_full.device)
    dwr_sub = torch.empty(E, cfg.d, dtype=torch.float32, device=dl_full.device)
    dx_r = torch.empty(T, cfg.d, dtype=torch.float32, device=dl_full.device)
    moe.router_bwd(D, _dev_bf16(inp, "x", dl_full.device), _dev_bf16(inp, "wr", dl_full.device), dl_full, dx_r,
                   dwr_sub, b.ws_router_bwd)
    torch.cuda.synchronize()
    assert whole_rel_err(to_host(dwr_sub), g["dWr"]) <= tol
    assert max_row_rel_err(_rows_t(dx_r, toks), g["dx_router"]) <= tol
    del dl_full, dx_r, dwr_sub

    # --- dWr = dlogits^T x on sampled entries (property) ------------------
    rng = np.random.default_rng(cfg.seed + 1)
    es = rng.choice(E, size=8, replace=False)
    js = rng.choice(cfg.d, size=16, replace=False)
    dl = to_host(b.dlogits[:, torch.as_tensor(es, device=b.dlogits.device)]).astype(np.float64)
    want = dl.T @ x32[:, js].astype(np.float64)
    got = to_host(b.dWr)[np.ix_(es, js)]
    assert np.abs(got - want).max() <= tol * np.abs(want).max()
