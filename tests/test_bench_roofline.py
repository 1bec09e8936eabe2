"""bench.py's choice of the kernel it grades against a roofline (CPU only):
the longest single launch of the step, and the bound by arithmetic intensity."""
import pytest

import bench


def test_longest_single_launch_is_chosen():
    avg = {"B3_dx": 4.9, "B4_dw13": 5.6, "B4_dw2": 2.9, "A5_gate_up": 4.8, "B5_router_bwd": 0.8}
    launches = {"B3_dx": 1, "B4_dw13": 1, "B4_dw2": 1, "A5_gate_up": 1, "B5_router_bwd": 4}
    assert bench.pick_dominant(avg, launches) == "B4_dw13"


def test_a_multi_launch_row_longer_than_the_choice_is_refused():
    # A row timed as a whole (here two launches of 8.5 ms together) could hide
    # a launch longer than the longest single-launch row.
    avg = {"B3_dx": 4.9, "B4_dw": 8.5}
    with pytest.raises(ValueError, match="B4_dw"):
        bench.pick_dominant(avg, {"B3_dx": 1, "B4_dw": 2})
    with pytest.raises(ValueError):
        bench.pick_dominant({"A34_permute": 0.4}, {"A34_permute": 4})


def test_bound_follows_the_arithmetic_intensity():
    R, d, f, NL = 130626, 6144, 1792, 96
    dw13 = bench.Row("B4_dw13", None, 1, 4.0 * R * d * f, R * d * 2 + R * 2 * f * 2 + 2 * NL * f * d * 4)
    g = bench.grade(dw13, 5.624)
    assert g["bound"] == "mfma" and g["unit"] == "TFLOP/s"
    assert g["frac"] == pytest.approx(4.0 * R * d * f / 5.624e-3 / 2.5e15, rel=1e-3)
    # the 1T share's gate/up: ~171 rows per expert, under the ridge -> HBM
    R3 = 16384
    gu = bench.Row("A5_gate_up", None, 1, 4.0 * R3 * d * f, R3 * d * 2 + 2 * NL * f * d * 2 + R3 * f * 2)
    g = bench.grade(gu, 1.2)
    assert g["bound"] == "hbm" and g["unit"] == "GB/s"
    assert g["achieved"] == pytest.approx(gu.nbytes / 1.2e-3 / 1e9, rel=1e-3)
