"""Checks of the seeded input recipes (CPU only)."""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_draws_are_deterministic_and_chunk_independent(monkeypatch):
    a = synth.normal_f32(9, 3, (3, synth.CHUNK // 2 + 7), 0.5)
    monkeypatch.setattr(synth, "_threads", lambda: 1)
    b = synth.normal_f32(9, 3, (3, synth.CHUNK // 2 + 7), 0.5)
    assert a.dtype == np.float32 and (a.view(np.uint32) == b.view(np.uint32)).all()
    c = synth.normal_f32(9, 4, (3, synth.CHUNK // 2 + 7), 0.5)
    assert not np.array_equal(a, c)
    assert abs(a.std() - 0.5) < 0.01 and abs(a.mean()) < 0.01


def test_bf16_rounding_is_nearest_even():
    a = synth.normal_f32(1, 0, (1000, 257), 3.0)
    special = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -0.0, 0.0, 65504.0, 1e-30], np.float32)
    for arr in (a, special):
        assert (synth.f32_to_bf16_bits(arr) == synth.f32_to_bf16_bits_reference(arr)).all()
    # ties go to even: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7
    assert synth.f32_to_bf16_bits(np.array([1.0 + 2**-8], np.float32))[0] == 0x3F80
    assert synth.f32_to_bf16_bits(np.array([1.0 + 3 * 2**-8], np.float32))[0] == 0x3F82
    back = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(a))
    assert np.abs(back - a).max() <= np.abs(a).max() * 2**-8


def test_config_shapes():
    c = synth.CONFIGS
    assert (c["fwdbwd_1t"].T, c["fwdbwd_1t"].d, c["fwdbwd_1t"].E, c["fwdbwd_1t"].k, c["fwdbwd_1t"].f,
            c["fwdbwd_1t"].num_local) == (65536, 6144, 384, 8, 1792, 96)
    assert c["share_1t"].R_cap == 8192 * 8
    inp = synth.make_inputs(c["tiny_f32"])
    assert inp["w1"].shape == (8, 64, 128) and inp["w2"].shape == (8, 128, 64)
    assert inp["wr"].shape == (8, 128) and inp["x"].dtype == np.float32


def test_zipf_beta_matches_calibration_record():
    with open(os.path.join(GOLDEN, "zipf_beta.json")) as fh:
        rec = json.load(fh)
    assert synth.CONFIGS["zipf_1t"].zipf_beta == rec["beta"]
    assert abs(rec["max_over_mean"] - 10.0) <= 0.25


@pytest.mark.slow
def test_zipf_bias_gives_tenfold_hot_expert():
    cfg = synth.CONFIGS["zipf_1t"]
    inp = synth.make_inputs(cfg, want=("wr", "x"))
    L = oracle.router_logits(synth.as_f32(inp["x"], cfg.dtype), synth.as_f32(inp["wr"], cfg.dtype), inp["bias"])
    idx, _ = oracle.topk_route(L, cfg.k)
    counts, _ = oracle.count_tokens(idx, cfg.E, 0, cfg.E)
    ratio = counts.max() / (cfg.T * cfg.k / cfg.E)
    assert abs(ratio - 10.0) <= 0.25
