"""The gather fused into the grouped GEMMs (Domyn page, section "Dynamic tile
scheduling in SonicMoE": SonicMoE's expert GEMMs run on the token-dispatch
layout with no permuted copy of the tokens).

gate/up and dW1|dW3 read x through row_token instead of the materialised
x_perm.  The operand values, the tiles and the order of every sum are the
same, so each output must equal the x_perm path's bit for bit; the x_perm path
is itself checked against the oracle in the other GPU tests, and the whole
layer in gather mode is checked against the oracle here too.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_02_amd as moe
import oracle
import synth
from gpu_util import f64, to_dev, to_host
from layer_checks import TOL, _desc
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
def test_gather_fused_is_bitwise_the_permuted_path(gpu, scale, dyn):
    cfg = synth.scaled(synth.CONFIGS["fwdbwd_1t"], **scale)
    print(f"[gather] {scale} dynamic={dyn}", flush=True)
    inp, (ref, got) = _pair(cfg, dyn, gpu)
    assert got.x_perm is None
    R = int(ref.offsets[-1].item())
    assert torch.equal(ref.row_token[:R], got.row_token[:R])
    for n in ("gu", "h", "y_perm", "dgu", "dx_perm"):
        assert _same(getattr(ref, n)[:R], getattr(got, n)[:R]), n
    for n in ("y", "dW1", "dW3", "dW2", "dx", "dWr"):
        assert _same(getattr(ref, n), getattr(got, n)), n


def test_gather_layer_against_oracle(gpu):
    cfg = synth.scaled(synth.CONFIGS["fwdbwd_1t"], T=512, d=256, f=128, E=32, num_local=8, expert_begin=8)
    inp = synth.make_inputs(cfg)
    dev = {n: to_dev(inp[n]) for n in ("x", "wr", "w1", "w3", "w2", "dy")}
    D = _desc(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.expert_begin, cfg.num_local, cfg.dtype, cfg.renormalize)
    b = moe.Buffers(D, backward=True, gather=True)
    moe.forward(b, dev["x"], dev["wr"], dev["w1"], dev["w3"], dev["w2"])
    moe.backward(b, dev["x"], dev["wr"], dev["w1"], dev["w3"], dev["w2"], dev["dy"])
    torch.cuda.synchronize()
    dt, tol = cfg.dtype, TOL[cfg.dtype]
    x, wr = f64(inp["x"], dt), f64(inp["wr"], dt)
    w1, w3, w2 = f64(inp["w1"], dt), f64(inp["w3"], dt), f64(inp["w2"], dt)
    ref = oracle.layer_forward(x, wr, w1, w3, w2, cfg.k, cfg.expert_begin, cfg.num_local, cfg.renormalize)
    assert (to_host(b.topk_idx) == ref["idx"]).all(), "a routing near-tie flipped"
    g = oracle.layer_backward(ref, x, wr, w1, w3, w2, f64(inp["dy"], dt), cfg.renormalize)
    R = int(ref["offsets"][-1])
    assert max_row_rel_err(to_host(b.h)[:R], ref["H"]) <= tol
    assert max_row_rel_err(to_host(b.y), ref["y"]) <= tol
    assert max_row_rel_err(to_host(b.dx), g["dx"]) <= tol
    for n in range(cfg.num_local):
        assert whole_rel_err(to_host(b.dW1)[n], g["dW1"][n]) <= tol, n
        assert whole_rel_err(to_host(b.dW3)[n], g["dW3"][n]) <= tol, n


def test_gather_rejects_fp32_and_oversized_x(gpu):
    D = _desc(64, 128, 64, 8, 2, 0, 8, "f32")
    z = torch.zeros(1 << 16, dtype=torch.float32, device=gpu)
    with pytest.raises(moe.MoeError):
        moe.expert_gate_up_gather(D, z, z, z, z, z, z, z)
    D = _desc(1 << 20, 1024, 64, 8, 2, 0, 8, "bf16")          # x of 2 GiB
    with pytest.raises(moe.MoeError):
        moe.grouped_ffn_bwd_dw_gather(D, z, z, z, z, z, z, z, z, z)
