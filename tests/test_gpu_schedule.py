"""The dynamic tile order of the grouped GEMMs (Domyn page, section "Dynamic
tile scheduling in SonicMoE": free workgroups take the next tile from a shared
atomic counter instead of a list fixed at launch; the outputs are bitwise
identical to the static order's).

Every bf16 product of the layer (router, gate/up + SwiGLU, down, dH + SwiGLU
backward, dX, dW1|dW3, dW2, router backward and dW_r) runs once under each
order on the same inputs, alone and with another kernel holding a third of
the compute units for part of the run, and every output must match bit for
bit.  The counters must be zero again after each call.  The dynamic-order
layer is also compared with the oracle directly, alone and under contention.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_02_amd as moe
import synth
from gpu_util import to_dev
from layer_checks import _desc, check_layer_backward

pytestmark = pytest.mark.gpu

OUTS = ["logits", "topk_idx", "topk_w", "gu", "h", "y_perm", "y", "dy_perm", "dtopk_w", "dgu", "dx_perm",
        "dW1", "dW3", "dW2", "dlogits", "dx", "dWr"]


def _layer(cfg, desc, dev, bias):
    b = moe.Buffers(desc, backward=True)
    moe.forward(b, dev["x"], dev["wr"], dev["w1"], dev["w3"], dev["w2"], bias=bias)
    moe.backward(b, dev["x"], dev["wr"], dev["w1"], dev["w3"], dev["w2"], dev["dy"])
    return b


@pytest.mark.parametrize("scale,hold", [
    (dict(T=2048, d=512, f=256, E=32, num_local=16, expert_begin=8), False),
    (dict(T=2048, d=512, f=256, E=32, num_local=16, expert_begin=8), True),
    (dict(T=4096, d=1024, f=512, E=16, num_local=16, expert_begin=0, k=4), True),   # several tiles per CU
    (dict(T=64, d=128, f=64, E=8, num_local=8, expert_begin=0, k=2), False),        # fewer tiles than 8 CUs
    (dict(T=1500, d=320, f=192, E=64, num_local=24, expert_begin=40, k=6), True),   # ragged, empty experts
])
def test_dynamic_order_is_bitwise_identical(gpu, scale, hold):
    cfg = synth.scaled(synth.CONFIGS["fwdbwd_1t"], **scale)
    print(f"[schedule] {scale} hold={hold}", flush=True)
    inp = synth.make_inputs(cfg)
    dev = {n: to_dev(inp[n]) for n in ("x", "wr", "w1", "w3", "w2", "dy")}
    bias = None
    ds = _desc(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.expert_begin, cfg.num_local, cfg.dtype, cfg.renormalize)
    counters = moe.new_tile_counters(gpu)
    dd = moe.make_desc(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.expert_begin, cfg.num_local, cfg.dtype,
                       cfg.renormalize, tile_counters=counters)
    ref = _layer(cfg, ds, dev, bias)
    torch.cuda.synchronize()
    for rep in range(2):
        if hold:
            side = torch.cuda.Stream(device=gpu)
            side.wait_stream(torch.cuda.current_stream())
            moe.hold_cus(max(1, torch.cuda.get_device_properties(gpu).multi_processor_count // 3), 3000, stream=side)
        got = _layer(cfg, dd, dev, bias)
        torch.cuda.synchronize()
        for n in OUTS:
            a, b = getattr(ref, n), getattr(got, n)
            if n in ("gu", "h", "y_perm", "dy_perm", "dgu", "dx_perm"):
                R = int(ref.offsets[-1].item())
                a, b = a[:R], b[:R]
            assert torch.equal(a.view(torch.uint8) if a.dtype != torch.int32 else a,
                               b.view(torch.uint8) if b.dtype != torch.int32 else b), (n, rep)
        assert int(counters.abs().sum().item()) == 0, counters.tolist()


@pytest.mark.parametrize("scale,hold", [
    (dict(T=512, d=256, f=128, E=32, num_local=8, expert_begin=8), False),
    (dict(T=512, d=256, f=128, E=32, num_local=8, expert_begin=8), True),
    (dict(T=700, d=192, f=192, E=16, num_local=16, expert_begin=0), True),
])
def test_dynamic_order_matches_the_oracle(gpu, scale, hold):
    cfg = synth.scaled(synth.CONFIGS["fwdbwd_1t"], **scale)
    print(f"[schedule vs oracle] {scale} hold={hold}", flush=True)
    inp = synth.make_inputs(cfg)
    dev = {n: to_dev(inp[n]) for n in ("x", "wr", "w1", "w3", "w2", "dy")}
    counters = moe.new_tile_counters(gpu)
    dd = moe.make_desc(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.expert_begin, cfg.num_local, cfg.dtype,
                       cfg.renormalize, tile_counters=counters)
    if hold:
        side = torch.cuda.Stream(device=gpu)
        side.wait_stream(torch.cuda.current_stream())
        moe.hold_cus(max(1, torch.cuda.get_device_properties(gpu).multi_processor_count // 3), 3000, stream=side)
    b = _layer(cfg, dd, dev, None)
    torch.cuda.synchronize()
    assert int(counters.abs().sum().item()) == 0, counters.tolist()
    check_layer_backward(cfg, inp, b)
