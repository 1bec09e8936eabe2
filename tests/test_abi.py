"""The C ABI without a GPU: the library loads, exports every declared entry
point, and rejects invalid arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

import mixture_experts_layer_02_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "moe.h")) as fh:
        txt = fh.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\*|int)\s+(moe_\w+)\s*\(", txt, re.M)))


def test_library_exports_every_declared_symbol():
    l = moe.lib()
    names = _declared()
    assert len(names) == 40
    assert names == moe.EXPORTS
    for n in names:
        assert hasattr(l, n), n


def test_desc_struct_matches_header_size():
    # 11 x 4-byte fields, 4 bytes of padding, one 8-byte pointer, one 4-byte
    # field and 4 bytes of tail padding
    assert ctypes.sizeof(moe.MoeDesc) == 64
    assert moe.MoeDesc.tile_counters.offset == 48
    assert moe.MoeDesc.wgrad_dtype.offset == 56


def _d(**kw):
    base = dict(T=64, d=128, f=64, E=8, k=2, expert_begin=0, num_local=8, dtype=moe.MOE_BF16)
    extra = {n: kw.pop(n) for n in ("tile_schedule", "tile_counters", "wgrad_dtype") if n in kw}
    base.update(kw)
    d = moe.make_desc(**base)
    for n, v in extra.items():
        setattr(d, n, v)
    return d


@pytest.mark.parametrize("kw,rc", [
    (dict(T=0), moe.MOE_ERR_INVALID_ARG),
    (dict(k=0), moe.MOE_ERR_INVALID_ARG),
    (dict(k=9), moe.MOE_ERR_INVALID_ARG),             # k > E
    (dict(expert_begin=4, num_local=5), moe.MOE_ERR_INVALID_ARG),
    (dict(num_local=0), moe.MOE_ERR_INVALID_ARG),
    (dict(d=96), moe.MOE_ERR_UNSUPPORTED),
    (dict(f=32), moe.MOE_ERR_UNSUPPORTED),
    (dict(E=12, num_local=12), moe.MOE_ERR_UNSUPPORTED),
    (dict(E=2048, num_local=8), moe.MOE_ERR_UNSUPPORTED),
    (dict(E=64, k=33, num_local=64), moe.MOE_ERR_UNSUPPORTED),
    (dict(dtype=7), moe.MOE_ERR_UNSUPPORTED),
    (dict(tile_schedule=2), moe.MOE_ERR_INVALID_ARG),
    (dict(tile_schedule=1), moe.MOE_ERR_INVALID_ARG),    # dynamic order without counters
    (dict(tile_schedule=1, tile_counters=8), moe.MOE_ERR_INVALID_ARG),  # misaligned counters
    (dict(wgrad_dtype=2), moe.MOE_ERR_INVALID_ARG),
    (dict(wgrad_dtype=moe.MOE_BF16, dtype=moe.MOE_F32), moe.MOE_ERR_UNSUPPORTED),  # bf16 gradients of fp32 weights
])
def test_invalid_descriptors_are_rejected(kw, rc):
    n = ctypes.c_size_t(0)
    assert moe.lib().moe_workspace_size(ctypes.byref(_d(**kw)), moe.OP_PERMUTE, ctypes.byref(n)) == rc


def test_wrong_struct_size_and_null_desc():
    d = _d()
    d.struct_size = 56                                  # the descriptor before the gradient type
    n = ctypes.c_size_t(0)
    assert moe.lib().moe_workspace_size(ctypes.byref(d), 0, ctypes.byref(n)) == moe.MOE_ERR_INVALID_ARG
    assert moe.lib().moe_route(None, None, None, None, None) == moe.MOE_ERR_INVALID_ARG


def test_null_and_misaligned_pointers_are_rejected():
    l = moe.lib()
    d = _d()
    good = 1 << 20
    assert l.moe_route(ctypes.byref(d), None, good, good, None) == moe.MOE_ERR_INVALID_ARG
    assert l.moe_route(ctypes.byref(d), good + 4, good, good, None) == moe.MOE_ERR_INVALID_ARG
    assert l.moe_combine(ctypes.byref(d), good, good, good, None, None) == moe.MOE_ERR_INVALID_ARG
    # renormalize = 0 needs logits in the route backward
    d0 = _d(renormalize=0)
    assert l.moe_route_bwd(ctypes.byref(d0), None, good, good, good, good, None) == moe.MOE_ERR_INVALID_ARG


def test_workspace_too_small_is_reported():
    l = moe.lib()
    d = _d()
    need = moe.workspace_size(d, moe.OP_PERMUTE)
    assert need > 0
    g = 1 << 20
    rc = l.moe_permute(ctypes.byref(d), g, g, g, g, g, g, g, g, need - 16, None)
    assert rc == moe.MOE_ERR_WORKSPACE
    rb = moe.workspace_size(d, moe.OP_ROUTER_BWD)
    assert rb >= d.E * d.d * 4
    rc = l.moe_router_bwd(ctypes.byref(d), g, g, g, g, g, g, rb - 16, None)
    assert rc == moe.MOE_ERR_WORKSPACE


def _router_splits(T, d, E, dtype):
    # bf16 products with fewer than 256 output tiles of 256 x 256 are split
    # over d into whole 64-wide chunks (at most 16), one per 256 / tiles
    if dtype != "bf16" or d % 64:
        return 1
    tiles = -(-T // 256) * -(-E // 256)
    s = min(-(-256 // tiles), d // 64, 16)
    if s <= 1:
        return 1
    chunk = -(-(d // 64) // s) * 64
    return -(-d // chunk)


def test_workspace_sizes():
    d = _d()
    assert moe.workspace_size(d, moe.OP_GROUPED_FFN) == 0
    with pytest.raises(moe.MoeError):
        moe.workspace_size(d, 99)
    for T, dd, E, dt in [(d.T, d.d, d.E, "bf16"), (65536, 6144, 384, "bf16"), (8192, 6144, 384, "bf16"),
                         (16384, 6144, 96, "bf16"), (300, 256, 72, "bf16"), (256, 128, 8, "f32")]:
        D = moe.make_desc(T, dd, 64, E, 2, 0, E, dt)
        s = _router_splits(T, dd, E, dt)
        assert moe.workspace_size(D, moe.OP_ROUTER_LOGITS) == (s * T * E * 4 if s > 1 else 0), (T, dd, E, dt)
    # the 1T fwd+bwd shape needs none; the 1T share splits in 4
    assert _router_splits(65536, 6144, 384, "bf16") == 1 and _router_splits(8192, 6144, 384, "bf16") == 4


def test_router_logits_rejects_short_workspace():
    l = moe.lib()
    D = moe.make_desc(300, 256, 64, 72, 2, 0, 72, "bf16")
    need = moe.workspace_size(D, moe.OP_ROUTER_LOGITS)
    assert need > 0
    g = 1 << 20
    rc = l.moe_router_logits(ctypes.byref(D), g, g, None, g, g, need - 16, None)
    assert rc == moe.MOE_ERR_WORKSPACE
    rc = l.moe_router_logits(ctypes.byref(D), g, g, None, g, None, 0, None)
    assert rc == moe.MOE_ERR_INVALID_ARG


def test_status_strings():
    l = moe.lib()
    for rc in (0, -1, -2, -3, -4, 5):
        assert isinstance(l.moe_status_str(rc), bytes)


def test_hold_cus_rejects_bad_arguments():
    l = moe.lib()
    for wg, lds, us in [(0, 1024, 10), (5000, 1024, 10), (4, 2, 10), (4, 200 * 1024, 10), (4, 1024, -1),
                        (4, 1024, 2000000)]:
        assert l.moe_hold_cus(wg, lds, us, None) == moe.MOE_ERR_INVALID_ARG


def test_fp8_entry_points_reject_bad_arguments():
    l = moe.lib()
    good = 1 << 20
    assert l.moe_fp8_quantize(good, moe.MOE_BF16, 100, good, good, None) == moe.MOE_ERR_INVALID_ARG   # not 128k
    assert l.moe_fp8_quantize(None, moe.MOE_BF16, 128, good, good, None) == moe.MOE_ERR_INVALID_ARG
    assert l.moe_fp8_quantize(good, 7, 128, good, good, None) == moe.MOE_ERR_UNSUPPORTED
    assert l.moe_fp8_dequantize(good, good + 4, 128, good, None) == moe.MOE_ERR_INVALID_ARG     # misaligned


def test_missing_library_raises(monkeypatch, tmp_path):
    # no fallback path: without libmoe.so every entry point fails loudly
    monkeypatch.setattr(moe, "LIB_PATH", str(tmp_path / "libmoe.so"))
    monkeypatch.setattr(moe, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        moe.lib()
    with pytest.raises(RuntimeError, match="missing"):
        moe.workspace_size(_d(), moe.OP_PERMUTE)


def test_permute_noalloc_rejects_shapes_beyond_its_scratch():
    # (E + NL) * ceil(T/256) * 4 bytes must fit the fixed 4 MiB scratch; the
    # check is on the host, before any launch.
    l = moe.lib()
    g = 1 << 20
    d = moe.make_desc(600_000, 6144, 1792, 384, 8, 0, 96)         # 480 * 2344 * 4 > 4 MiB
    assert l.moe_permute_noalloc(ctypes.byref(d), g, None, g, g, g, g, None, None) == moe.MOE_ERR_UNSUPPORTED
    assert b"scratch" in l.moe_last_error()
    d = _d()
    assert l.moe_permute_noalloc(ctypes.byref(d), None, None, g, g, g, g, None, None) == moe.MOE_ERR_INVALID_ARG
    assert l.moe_permute_noalloc(ctypes.byref(d), g, g, g, g, g, g, None, None) == moe.MOE_ERR_INVALID_ARG


def test_unpermute_router_bwd_rejects_dense_dlogits_and_nulls():
    # The router rows are summed over the selection only, which is dlogits'
    # support when the weights are renormalised; renormalize = 0 is refused.
    l = moe.lib()
    g = 1 << 20
    d0 = _d(renormalize=0)
    assert l.moe_unpermute_router_bwd(ctypes.byref(d0), g, g, g, g, g, g, None) == moe.MOE_ERR_UNSUPPORTED
    d = _d()
    assert l.moe_unpermute_router_bwd(ctypes.byref(d), g, g, None, g, g, g, None) == moe.MOE_ERR_INVALID_ARG
    assert l.moe_unpermute_router_bwd(ctypes.byref(d), g, g, g, g, None, g, None) == moe.MOE_ERR_INVALID_ARG


def test_fp8_row_quantise_and_down_reject_bad_arguments():
    l = moe.lib()
    g = 1 << 20
    # cols not a multiple of 128; a scale pitch below cols/128 or above it + 15; nrows misaligned
    assert l.moe_fp8_quantize_pow2_rows(g, moe.MOE_BF16, 4, 200, None, g, g, 2, None) == moe.MOE_ERR_INVALID_ARG
    assert l.moe_fp8_quantize_pow2_rows(g, moe.MOE_BF16, 4, 256, None, g, g, 1, None) == moe.MOE_ERR_INVALID_ARG
    assert l.moe_fp8_quantize_pow2_rows(g, moe.MOE_BF16, 4, 256, None, g, g, 18, None) == moe.MOE_ERR_INVALID_ARG
    assert l.moe_fp8_quantize_pow2_rows(g, moe.MOE_BF16, 4, 256, g + 2, g, g, 2, None) == moe.MOE_ERR_INVALID_ARG
    assert l.moe_fp8_quantize_pow2_rows(g, 7, 4, 256, None, g, g, 2, None) == moe.MOE_ERR_UNSUPPORTED
    # the down product: bf16 only, f in whole 128-code blocks
    assert l.moe_expert_down_fp8mm(ctypes.byref(_d(f=192)), g, g, g, g, g, g, None) == moe.MOE_ERR_UNSUPPORTED
    assert l.moe_expert_down_fp8mm(ctypes.byref(_d(f=128, dtype=moe.MOE_F32)), g, g, g, g, g, g,
                                   None) == moe.MOE_ERR_UNSUPPORTED
    assert l.moe_expert_down_fp8mm(ctypes.byref(_d(f=128)), g, None, g, g, g, g, None) == moe.MOE_ERR_INVALID_ARG


def test_row_weights_and_dtopk_parts_reject_nulls():
    l = moe.lib()
    g = 1 << 20
    d = _d()
    assert l.moe_row_weights(ctypes.byref(d), None, g, g, None) == moe.MOE_ERR_INVALID_ARG
    assert l.moe_row_weights(ctypes.byref(d), g, g, g + 4, None) == moe.MOE_ERR_INVALID_ARG
    assert l.moe_dtopk_w_from_parts(ctypes.byref(d), g, None, g, None) == moe.MOE_ERR_INVALID_ARG
    # the dH product's partial sums are optional, but aligned when given
    assert l.moe_expert_bwd_dh_gather(ctypes.byref(d), g, g, g, g, g, g, g, None, g + 4, None) == \
        moe.MOE_ERR_INVALID_ARG
