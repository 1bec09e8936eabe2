"""The gather fused into the grouped GEMMs (Domyn page, section "Dynamic tile
scheduling in SonicMoE": SonicMoE's expert GEMMs run on the token-dispatch
layout with no permuted copies).

Forward: gate/up reads x through row_token instead of the materialised
x_perm.  The operand values, the tiles and the order of every sum are the
same, so each forward output must equal the x_perm path's bit for bit; so
must dW1|dW3 read through row_token, given the same dG|dU.

Backward: dy is read through row_token too (dH and dW2), with the routing
weight applied inside the products instead of in a stored dy_perm, so the
rounding differs from the x_perm path; the whole gathered layer, forward and
backward, and its new intermediates (the per-row weights and hw = w silu(G) U)
are checked against the oracle.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_02_amd as moe
import oracle
import synth
from gpu_util import f64, to_dev, to_host
from layer_checks import TOL, _desc, check_layer_backward
from metrics import max_row_rel_err, whole_rel_err

pytestmark = pytest.mark.gpu

SHAPES = [
    dict(T=2048, d=512, f=256, E=32, num_local=16, expert_begin=8),
    dict(T=4096, d=1024, f=512, E=16, num_local=16, expert_begin=0, k=4),     # several tiles per CU
    dict(T=1500, d=320, f=192, E=64, num_local=24, expert_begin=40, k=6),     # ragged, empty experts
    dict(T=300, d=128, f=64, E=8, num_local=8, expert_begin=0, k=2),          # K of 2 k-tiles: no hand-over
    dict(T=777, d=256, f=128, E=64, num_local=3, expert_begin=61, k=8),       # few local experts
]


def _pair(cfg, dyn, gpu):
    inp = synth.make_inputs(cfg)
    dev = {n: to_dev(inp[n]) for n in ("x", "wr", "w1", "w3", "w2", "dy")}
    args = (cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.expert_begin, cfg.num_local, cfg.dtype, cfg.renormalize)
    out = []
    for gather in (False, True):
        D = moe.make_desc(*args, tile_counters=moe.new_tile_counters(gpu) if dyn else None)
        b = moe.Buffers(D, backward=True, gather=gather)
        moe.forward(b, dev["x"], dev["wr"], dev["w1"], dev["w3"], dev["w2"])
        moe.backward(b, dev["x"], dev["wr"], dev["w1"], dev["w3"], dev["w2"], dev["dy"])
        out.append(b)
    torch.cuda.synchronize()
    return inp, out


def _same(a, b):
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8))


@pytest.mark.parametrize("dyn", [False, True])
@pytest.mark.parametrize("scale", SHAPES)
def test_gather_fused_forward_is_bitwise_the_permuted_path(gpu, scale, dyn):
    cfg = synth.scaled(synth.CONFIGS["fwdbwd_1t"], **scale)
    print(f"[gather] {scale} dynamic={dyn}", flush=True)
    inp, (ref, got) = _pair(cfg, dyn, gpu)
    assert got.x_perm is None and got.dy_perm is None
    R = int(ref.offsets[-1].item())
    assert torch.equal(ref.row_token[:R], got.row_token[:R])
    for n in ("gu", "h", "y_perm"):
        assert _same(getattr(ref, n)[:R], getattr(got, n)[:R]), n
    assert _same(ref.y, got.y)
    # dW1 | dW3 with x read through row_token, on the permuted path's dG | dU
    D = got.desc
    dw1, dw3 = torch.empty_like(ref.dW1), torch.empty_like(ref.dW3)
    moe.expert_bwd_dw_gate_up(D, got.offsets, got.row_token, to_dev(inp["x"]), ref.dgu, dw1, dw3)
    torch.cuda.synchronize()
    assert _same(ref.dW1, dw1) and _same(ref.dW3, dw3)


@pytest.mark.parametrize("gather_x", [True, False])
@pytest.mark.parametrize("dyn", [False, True])
@pytest.mark.parametrize("scale", [
    dict(T=512, d=256, f=128, E=32, num_local=8, expert_begin=8),
    dict(T=700, d=192, f=192, E=16, num_local=16, expert_begin=0),
    dict(T=1500, d=320, f=192, E=64, num_local=24, expert_begin=40, k=6),     # ragged, empty experts
    dict(T=777, d=256, f=128, E=64, num_local=3, expert_begin=61, k=8),       # few local experts
])
def test_gather_layer_against_oracle(gpu, scale, dyn, gather_x):
    # gather_x False: x through x_perm, dy read in place (the benchmark's configuration)
    cfg = synth.scaled(synth.CONFIGS["fwdbwd_1t"], **scale)
    print(f"[gather vs oracle] {scale} dynamic={dyn} gather_x={gather_x}", flush=True)
    inp = synth.make_inputs(cfg)
    dev = {n: to_dev(inp[n]) for n in ("x", "wr", "w1", "w3", "w2", "dy")}
    args = (cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.expert_begin, cfg.num_local, cfg.dtype, cfg.renormalize)
    D = moe.make_desc(*args, tile_counters=moe.new_tile_counters(gpu) if dyn else None)
    b = moe.Buffers(D, backward=True, gather=gather_x, gather_dy=True)
    moe.forward(b, dev["x"], dev["wr"], dev["w1"], dev["w3"], dev["w2"])
    moe.backward(b, dev["x"], dev["wr"], dev["w1"], dev["w3"], dev["w2"], dev["dy"])
    torch.cuda.synchronize()
    assert b.dy_perm is None and (b.x_perm is None) == gather_x
    check_layer_backward(cfg, inp, b)
    # the per-row routing weights and hw = w silu(G) U
    dt, tol = cfg.dtype, TOL[cfg.dtype]
    x, wr = f64(inp["x"], dt), f64(inp["wr"], dt)
    w1, w3, w2 = f64(inp["w1"], dt), f64(inp["w3"], dt), f64(inp["w2"], dt)
    ref = oracle.layer_forward(x, wr, w1, w3, w2, cfg.k, cfg.expert_begin, cfg.num_local, cfg.renormalize)
    R = int(ref["offsets"][-1])
    t_of, j_of = np.nonzero(ref["slot_row"] >= 0)
    rows = ref["slot_row"][t_of, j_of]
    w_row = np.zeros(R)
    w_row[rows] = ref["w"][t_of, j_of]
    rw = to_host(b.row_w)[:R]
    np.testing.assert_array_equal(rw[rows], to_host(b.topk_w)[t_of, j_of])    # a copy of the GPU's weights
    np.testing.assert_allclose(rw, w_row, rtol=1e-4, atol=1e-6)
    assert max_row_rel_err(to_host(b.hw)[:R], w_row[:, None] * ref["H"]) <= tol


def test_gather_rejects_fp32_and_oversized_x(gpu):
    D = _desc(64, 128, 64, 8, 2, 0, 8, "f32")
    z = torch.zeros(1 << 16, dtype=torch.float32, device=gpu)
    with pytest.raises(moe.MoeError):
        moe.expert_gate_up_gather(D, z, z, z, z, z, z, z)
    with pytest.raises(moe.MoeError):
        moe.expert_bwd_dh_gather(D, z, z, z, z, z, z, z, z)
    with pytest.raises(moe.MoeError):
        moe.expert_bwd_dw_down_gather(D, z, z, z, z, z)
    D = _desc(1 << 20, 1024, 64, 8, 2, 0, 8, "bf16")          # x (and dy) of 2 GiB
    with pytest.raises(moe.MoeError):
        moe.grouped_ffn_bwd_dw_gather(D, z, z, z, z, z, z, z, z, z)
    with pytest.raises(moe.MoeError):
        moe.expert_bwd_dh_gather(D, z, z, z, z, z, z, z, z)
    with pytest.raises(moe.MoeError):
        moe.expert_bwd_dw_down_gather(D, z, z, z, z, z)


@pytest.mark.parametrize("scale", [
    dict(T=512, d=256, f=128, E=32, num_local=8, expert_begin=8),
    dict(T=1500, d=320, f=192, E=64, num_local=24, expert_begin=40, k=6),     # ragged, empty experts
])
def test_dtopk_w_two_ways_against_oracle(gpu, scale):
    # dtopk_w[t][j] = <dy[t], y_perm[row]> (the stage-5 backward) from the
    # combine backward's dot products, and = <dy[t] W2, h[row]> from the dH
    # product's partial sums (the layer's default); both against the oracle
    # on the layer's own forward, and row_weights against the weights.
    cfg = synth.scaled(synth.CONFIGS["fwdbwd_1t"], **scale)
    print(f"[dtopk_w] {scale}", flush=True)
    inp = synth.make_inputs(cfg)
    dev = {n: to_dev(inp[n]) for n in ("x", "wr", "w1", "w3", "w2", "dy")}
    args = (cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.expert_begin, cfg.num_local, cfg.dtype, cfg.renormalize)
    D = moe.make_desc(*args)
    b = moe.Buffers(D, backward=True, gather=False, gather_dy=True)
    moe.forward(b, dev["x"], dev["wr"], dev["w1"], dev["w3"], dev["w2"])
    moe.backward(b, dev["x"], dev["wr"], dev["w1"], dev["w3"], dev["w2"], dev["dy"])
    dw_parts = b.dtopk_w.clone()
    rw_parts = b.row_w.clone()
    dw_dot = torch.empty_like(b.dtopk_w)
    rw_dot = torch.empty_like(b.row_w)
    moe.combine_bwd_gather(D, b.slot_row, b.topk_w, b.y_perm, dev["dy"], rw_dot, dw_dot)
    torch.cuda.synchronize()
    R = int(b.offsets[-1].item())
    assert torch.equal(rw_parts[:R], rw_dot[:R])
    dt = cfg.dtype
    ref = oracle.layer_forward(f64(inp["x"], dt), f64(inp["wr"], dt), f64(inp["w1"], dt), f64(inp["w3"], dt),
                               f64(inp["w2"], dt), cfg.k, cfg.expert_begin, cfg.num_local, cfg.renormalize)
    idx_g = to_host(b.topk_idx)
    agree = (idx_g == ref["idx"]).all(axis=1)      # tokens routed alike (near-ties aside)
    _, dw_ref = oracle.combine_bwd(f64(inp["dy"], dt), ref["y_perm"], ref["slot_row"], ref["w"])
    for got in (dw_parts, dw_dot):
        g = to_host(got)[agree]
        assert whole_rel_err(g, dw_ref[agree]) <= TOL[dt]
    # non-local slots are exactly zero
    sl = to_host(b.slot_row)
    assert (to_host(dw_parts)[sl < 0] == 0).all()
