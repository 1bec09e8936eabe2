"""The row-grouped GEMMs on experts whose last m-tile is partial.

An expert's rows end in an m-tile of 1..256 valid rows; a tile with at most
128 runs with half of each wave's row blocks.  The segment sizes below give
tails of 1, 2, 44, 64, 65, 100, 127, 128 (half tiles), 129, 200, 255
(full-form tiles with padding), exact multiples of 256 and an empty expert,
in an order where half and full tiles follow each other in both directions.
With d = 1024 a tile has 16 k-tiles, so each one's successor is loaded ahead
of its epilogue.  Every product is compared with the oracle, in the static
and the dynamic tile order.
"""
import numpy as np
import pytest

import mixture_experts_layer_02_amd as moe
import oracle
import synth
from gpu_util import to_dev, to_host
from metrics import max_row_rel_err

pytestmark = pytest.mark.gpu

COUNTS = [300, 100, 256, 129, 128, 1, 0, 384, 513, 64, 65, 200, 127, 255, 257, 2]
D, F = 1024, 256
TOL = 2e-2


def _bf16(seed, idx, shape, std):
    return synth.f32_to_bf16_bits(synth.normal_f32(seed, idx, shape, std))


def _f64(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


@pytest.fixture(scope="module")
def case():
    NL = len(COUNTS)
    off = np.concatenate([[0], np.cumsum(COUNTS)]).astype(np.int32)
    R = int(off[-1])
    rng = np.random.default_rng(31)
    row_token = rng.permutation(R).astype(np.int32)  # T = R tokens, one row each
    c = {
        "NL": NL, "off": off, "R": R, "row_token": row_token,
        "x": _bf16(71, 0, (R, D), 1.0),
        "w1": _bf16(71, 1, (NL, F, D), 0.03), "w3": _bf16(71, 2, (NL, F, D), 0.03),
        "w2": _bf16(71, 3, (NL, D, F), 0.03), "dy": _bf16(71, 4, (R, D), 1.0),
        "row_w": rng.uniform(0.1, 1.0, R).astype(np.float32),
    }
    c["x_perm"] = c["x"][row_token]
    dy_perm = _f64(c["dy"])[row_token] * c["row_w"][:, None]
    c["ref_fwd"] = oracle.expert_ffn(_f64(c["x_perm"]), off, _f64(c["w1"]), _f64(c["w3"]), _f64(c["w2"]))
    c["dy_perm_f"] = dy_perm
    c["ref_bwd"] = oracle.expert_ffn_bwd(_f64(c["x_perm"]), off, _f64(c["w1"]), _f64(c["w3"]), _f64(c["w2"]),
                                         dy_perm)
    return c


def _desc(c, gpu, dyn):
    kw = {"tile_counters": moe.new_tile_counters(gpu)} if dyn else {}
    return moe.make_desc(c["R"], D, F, c["NL"], 1, 0, c["NL"], "bf16", **kw)


@pytest.mark.parametrize("dyn", [False, True])
def test_partial_tiles_forward(gpu, case, dyn):
    import torch
    c, R = case, case["R"]
    Dd = _desc(c, gpu, dyn)
    off = to_dev(c["off"])
    w1, w3, w2 = to_dev(c["w1"]), to_dev(c["w3"]), to_dev(c["w2"])
    gu = torch.empty(R, 2 * F, dtype=torch.bfloat16, device=gpu)
    h = torch.empty(R, F, dtype=torch.bfloat16, device=gpu)
    y = torch.empty(R, D, dtype=torch.bfloat16, device=gpu)
    moe.expert_gate_up(Dd, off, to_dev(c["x_perm"]), w1, w3, gu, h)
    moe.expert_down(Dd, off, h, w2, y)
    torch.cuda.synchronize()
    G, U, H, Y = c["ref_fwd"]
    g = to_host(gu)
    assert max_row_rel_err(g[:, :F], G) <= TOL
    assert max_row_rel_err(g[:, F:], U) <= TOL
    assert max_row_rel_err(to_host(h), H) <= TOL
    assert max_row_rel_err(to_host(y), Y) <= TOL
    # x read through row_token: the same tiles and sums, so the same bits
    gu2 = torch.empty_like(gu)
    h2 = torch.empty_like(h)
    moe.expert_gate_up_gather(Dd, off, to_dev(c["row_token"]), to_dev(c["x"]), w1, w3, gu2, h2)
    torch.cuda.synchronize()
    assert torch.equal(gu2.view(torch.int16), gu.view(torch.int16))
    assert torch.equal(h2.view(torch.int16), h.view(torch.int16))


@pytest.mark.parametrize("dyn", [False, True])
def test_partial_tiles_backward(gpu, case, dyn):
    import torch
    c, R = case, case["R"]
    Dd = _desc(c, gpu, dyn)
    off = to_dev(c["off"])
    w1, w3, w2 = to_dev(c["w1"]), to_dev(c["w3"]), to_dev(c["w2"])
    # G | U from the oracle's forward, rounded to bf16 as the forward stores them
    G, U, _, _ = c["ref_fwd"]
    gu = to_dev(np.concatenate([G, U], axis=1).astype(np.float32), "bf16")
    dgu = torch.empty(R, 2 * F, dtype=torch.bfloat16, device=gpu)
    hw = torch.empty(R, F, dtype=torch.bfloat16, device=gpu)
    moe.expert_bwd_dh_gather(Dd, off, to_dev(c["row_token"]), to_dev(c["row_w"]), to_dev(c["dy"]), w2, gu, dgu, hw)
    dx_perm = torch.empty(R, D, dtype=torch.bfloat16, device=gpu)
    moe.expert_bwd_dx(Dd, off, w1, w3, dgu, dx_perm)
    torch.cuda.synchronize()
    gub = to_host(gu).astype(np.float64)
    dG, dU, dX, _, _, _ = c["ref_bwd"]
    d = to_host(dgu)
    assert max_row_rel_err(d[:, :F], dG) <= TOL
    assert max_row_rel_err(d[:, F:], dU) <= TOL
    assert max_row_rel_err(to_host(dx_perm), dX) <= TOL
    # hw = row_w silu(G) U, from the stored G | U
    want_hw = c["row_w"][:, None] * oracle.silu(gub[:, :F]) * gub[:, F:]
    assert max_row_rel_err(to_host(hw), want_hw) <= TOL
    # dy_perm materialised: dH on it gives dG | dU again
    dy_perm = to_dev(c["dy_perm_f"].astype(np.float32), "bf16")
    dgu2 = torch.empty_like(dgu)
    moe.expert_bwd_dh(Dd, off, w2, gu, dy_perm, dgu2)
    torch.cuda.synchronize()
    d2 = to_host(dgu2)
    assert max_row_rel_err(d2[:, :F], dG) <= TOL
    assert max_row_rel_err(d2[:, F:], dU) <= TOL
