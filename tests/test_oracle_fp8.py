"""Pins of the oracle's FP8 (E4M3) blockwise weight quantisation (CPU only).

Domyn page, section "FP8 expert weight all-gather": blocks of 128 values are
scaled to the E4M3 range and cast, with one float32 scale per block, and
dequantised to bf16 before the expert GEMMs; the error is up to about 6% of
the block maximum per value.  The checks use another route than the
oracle's code: torch's float8_e4m3fn type (a library cast with round to
nearest even) for every code's value and for the rounding of many values,
including constructed ties and subnormals; the page's error bound (half a
step of a 3-bit mantissa is 1/16 of the value's binade, at most 448/16 of
the scaled block maximum); exactness where no rounding occurs; and
invariants of the block scaling.
"""
import numpy as np
import pytest
import torch

import oracle


def _torch_e4m3(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_of_every_code_matches_the_library():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.fp8_e4m3_decode(codes)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.nanmax(got) == 448.0 and oracle.fp8_e4m3_decode([1])[0] == 2.0 ** -9


def test_encode_matches_the_library_on_random_ties_and_subnormals():
    rng = np.random.default_rng(0)
    vals = [rng.uniform(-448, 448, 50000), rng.uniform(-0.05, 0.05, 20000), rng.normal(0, 3, 20000)]
    finite = oracle.fp8_e4m3_decode(np.arange(256))
    grid = np.unique(finite[np.isfinite(finite)])
    mids = (grid[1:] + grid[:-1]) / 2                      # exact ties (all representable in float32)
    vals += [mids, -mids, grid, -grid, [0.0, -0.0, 448.0, -448.0, 2.0 ** -10, -(2.0 ** -10)]]
    x = np.concatenate([np.asarray(v, np.float64) for v in vals]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    assert np.array_equal(oracle.fp8_e4m3_encode(x), _torch_e4m3(x))


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        oracle.fp8_e4m3_encode([449.0])


def _blocks(rng, nblk):
    w = rng.normal(0, 0.02, (nblk, 128)).astype(np.float32)
    w[0] = 0.0                                             # an all-zero block
    w[1] = 0.0
    w[1, 17] = -0.25                                       # a single value
    w[2] *= 1e-6                                           # tiny values
    w[3] = np.round(w[3] * 1000) / 1000
    return w


def test_quantise_error_is_within_the_pages_bound():
    rng = np.random.default_rng(1)
    w = _blocks(rng, 64)
    codes, scales = oracle.fp8_quantize_blocks(w)
    dq = (oracle.fp8_e4m3_decode(codes).reshape(64, 128) * scales[:, None].astype(np.float64))
    amax = np.abs(w).max(axis=1)
    err = np.abs(dq - w).max(axis=1)
    assert (err <= amax / 16 * (1 + 1e-6)).all()           # half a mantissa step of the block's top binade
    assert (err[amax > 0] / amax[amax > 0]).max() > 0.01   # not trivially exact
    assert (codes.reshape(64, 128)[0] == 0).all() and scales[0] == 0
    # the block maximum maps to +-448 and comes back to within one float32 rounding
    i = np.argmax(np.abs(w[1]))
    assert oracle.fp8_e4m3_decode(codes.reshape(64, 128)[1, i]) == -448.0
    assert abs(dq[1, i] - w[1, i]) <= 1e-7 * abs(w[1, i])


def test_quantise_uses_float32_scaling_and_clamps():
    rng = np.random.default_rng(2)
    w = _blocks(rng, 16)
    codes, scales = oracle.fp8_quantize_blocks(w)
    amax = np.abs(w).max(axis=1).astype(np.float32)
    for b in range(16):
        if amax[b] == 0:
            continue
        assert scales[b] == np.float32(amax[b] / np.float32(448))
        xs = np.clip((w[b] * (np.float32(448) / amax[b])).astype(np.float32), -448, 448)
        assert np.array_equal(codes.reshape(16, 128)[b], _torch_e4m3(xs))


def test_dequantise_is_decode_times_scale_rounded_to_bf16():
    rng = np.random.default_rng(3)
    w = _blocks(rng, 32)
    codes, scales = oracle.fp8_quantize_blocks(w)
    got = oracle.fp8_dequantize_blocks(codes, scales)
    v = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).reshape(32, 128) * \
        torch.from_numpy(scales)[:, None]
    want = v.to(torch.bfloat16).to(torch.float32).numpy().reshape(-1)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_values_on_the_grid_survive_a_round_trip():
    grid = oracle.fp8_e4m3_decode(np.arange(0, 127))      # every finite non-negative code
    w = np.zeros(256, np.float32)
    w[:127] = grid * 2.0 ** -8                             # exact in float32; block max 448 * 2^-8
    w[128:255] = -grid * 2.0 ** -8
    codes, scales = oracle.fp8_quantize_blocks(w)
    assert (scales == np.float32(448 * 2.0 ** -8 / 448)).all()
    assert np.array_equal(oracle.fp8_e4m3_decode(codes[:127]), grid)
    assert np.array_equal(oracle.fp8_dequantize_blocks(codes, scales)[:127], w[:127])


# ---------------------------------------------------------------------------
# The power-of-two block scales (the scale a block-scaled FP8 matrix
# instruction applies): scale = the least 2^e with amax <= 448 * 2^e.
# ---------------------------------------------------------------------------
def test_pow2_scale_puts_the_block_maximum_in_the_top_binade():
    rng = np.random.default_rng(11)
    w = (rng.normal(0, 1, (400, 128)) * 10.0 ** rng.uniform(-6, 4, (400, 1))).astype(np.float32)
    codes, e8 = oracle.fp8_quantize_blocks_pow2(w)
    e = e8.astype(np.int64) - 127
    amax = np.abs(w.astype(np.float64)).max(axis=1)
    scaled = amax * 2.0 ** -e
    assert (scaled > 224).all() and (scaled <= 448).all()      # so e is the least such exponent


@pytest.mark.parametrize("amax,e", [(448.0, 0), (449.0, 1), (224.0, -1), (224.5, 0), (1.0, -8), (0.875, -9),
                                    (2.0 ** -20, -28), (3.5, -7)])
def test_pow2_scale_of_hand_chosen_maxima(amax, e):
    # 448 = 1.75 * 2^8: amax <= 448 * 2^e  <=>  e >= log2(amax / 448), and the least integer is taken.
    w = np.zeros(128, np.float32)
    w[3] = -amax
    _, e8 = oracle.fp8_quantize_blocks_pow2(w)
    assert int(e8[0]) - 127 == e


def test_pow2_codes_match_the_library_cast_of_the_scaled_values():
    rng = np.random.default_rng(12)
    w = (rng.normal(0, 0.02, (300, 128))).astype(np.float32)
    w[0] = 0.0
    w[1, ::3] = -0.0
    w[2] = rng.normal(0, 1e-30, 128).astype(np.float32)          # tiny values: subnormal codes
    codes, e8 = oracle.fp8_quantize_blocks_pow2(w)
    scaled = w.astype(np.float64) * 2.0 ** -(e8.astype(np.int64) - 127)[:, None]
    assert np.array_equal(codes, _torch_e4m3(scaled.astype(np.float32)).reshape(-1))
    assert (codes.reshape(300, 128)[0] == 0).all() and e8[0] == 127


def test_pow2_round_trip_is_exact_on_the_grid_and_bounded_elsewhere():
    finite = oracle.fp8_e4m3_decode(np.arange(127))               # non-negative codes, finite
    rng = np.random.default_rng(13)
    for e in (-10, 0, 5):
        vals = rng.choice(finite, (50, 128)) * np.where(rng.random((50, 128)) < 0.5, -1, 1)
        vals[:, 0] = 448.0                                         # the block maximum, already in range
        w = (vals * 2.0 ** e).astype(np.float32)
        codes, e8 = oracle.fp8_quantize_blocks_pow2(w)
        assert (e8 == 127 + e).all()
        assert np.array_equal(oracle.fp8_dequantize_blocks_pow2(codes, e8), w.reshape(-1).astype(np.float64))
    w = rng.normal(0, 0.02, (500, 128)).astype(np.float32)
    codes, e8 = oracle.fp8_quantize_blocks_pow2(w)
    back = oracle.fp8_dequantize_blocks_pow2(codes, e8).reshape(500, 128)
    amax = np.abs(w).max(axis=1, keepdims=True)
    # half a step of a 3-bit mantissa is 1/16 of the value's binade; the largest binade reaches 448 * 2^e,
    # and 448 * 2^e < 2 * amax, so every error is under amax / 8 and a relative 2^-4 in the normal range
    err = np.abs(back - w)
    assert (err <= amax / 8).all()
    normal = np.abs(w) * 2.0 ** -(e8.astype(np.int64) - 127)[:, None] >= 2.0 ** -6
    assert (err[normal] <= np.abs(w[normal]) * 2.0 ** -4).all()
