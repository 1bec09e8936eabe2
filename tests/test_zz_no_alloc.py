"""moe_permute_noalloc (fixed device scratch, no allocation) against
moe_permute (caller workspace) through the C ABI: every output bit for bit,
on two calls in a row, the second with a smaller input, so that the second
call runs over the first call's scratch contents."""
import ctypes

import numpy as np
import pytest
import torch

import mixture_experts_layer_02_amd as moe
import synth
from gpu_util import to_dev
from layer_checks import random_routing

pytestmark = pytest.mark.gpu


def _outputs(D, dev, with_x):
    T, k, E, NL, d = D.T, D.k, D.E, D.num_local, D.d
    i32 = torch.int32
    o = dict(counts=torch.full((E,), -7, dtype=i32, device=dev),
             offsets=torch.full((NL + 1,), -7, dtype=i32, device=dev),
             row_token=torch.full((D.R_cap,), -7, dtype=i32, device=dev),
             slot_row=torch.full((T, k), -7, dtype=i32, device=dev))
    o["x_perm"] = torch.zeros(D.R_cap, d, dtype=torch.bfloat16, device=dev) if with_x else None
    return o


def _call(name, D, idx, x, o, *extra):
    l = moe.lib()
    args = [idx.data_ptr(), x.data_ptr() if x is not None else None, o["counts"].data_ptr(),
            o["offsets"].data_ptr(), o["row_token"].data_ptr(), o["slot_row"].data_ptr(),
            o["x_perm"].data_ptr() if o["x_perm"] is not None else None]
    rc = getattr(l, name)(ctypes.byref(D), *args, *extra, torch.cuda.current_stream().cuda_stream)
    assert rc == moe.MOE_OK, (name, rc, l.moe_last_error())


@pytest.mark.parametrize("with_x", [True, False])
def test_noalloc_permute_equals_the_workspace_permute(gpu, with_x):
    shapes = [(20000, 384, 8, 0, 96, 256),     # several hundred token blocks, 1T router width
              (1500, 64, 6, 40, 24, 128)]      # smaller, ragged, non-zero first local expert
    for i, (T, E, k, e0, NL, d) in enumerate(shapes):
        print(f"[noalloc] call {i}: T={T} E={E} k={k} e0={e0} NL={NL} d={d} x={with_x}", flush=True)
        cfg = synth.Config("t", 31 + i, T, d, E, k, 64, e0, NL, "bf16", 1.0, "router", False)
        x = to_dev(synth.make_inputs(cfg, want=("x",))["x"]) if with_x else None
        idx = to_dev(random_routing(np.random.default_rng(T), T, E, k, skew=1.0))
        D = moe.make_desc(T, d, 64, E, k, e0, NL, "bf16")
        ws = torch.empty(moe.workspace_size(D, moe.OP_PERMUTE), dtype=torch.uint8, device=gpu)
        ref, got = _outputs(D, gpu, with_x), _outputs(D, gpu, with_x)
        _call("moe_permute", D, idx, x, ref, ws.data_ptr(), ws.numel())
        _call("moe_permute_noalloc", D, idx, x, got)
        torch.cuda.synchronize()
        for n in ("counts", "offsets", "row_token", "slot_row"):
            assert torch.equal(ref[n], got[n]), (i, n)
        if with_x:
            assert torch.equal(ref["x_perm"].view(torch.int16), got["x_perm"].view(torch.int16)), i
