"""The build-time LDS-DMA wait-state check (mixture_experts_layer_02_amd/hazard_check.py) on
small hand-written gfx950 assembly: it must flag a VALU write of a DMA's SGPR operand within
five wait states on any path, and pass code whose waits are long enough or whose SGPRs come
from scalar instructions. Also the build's fallback when the check finds something."""
import io
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "mixture_experts_layer_02_amd"))
import hazard_check  # noqa: E402


def _check(tmp_path, body):
    p = tmp_path / "k.s"
    p.write_text("_Z6kernelv:\n" + "\n".join("\t" + l if not l.startswith(".L") else l for l in body) + "\n")
    return hazard_check.check(str(p), io.StringIO())


DMA = "buffer_load_dwordx4 v4, s[0:3], s8 offen lds"


def test_flags_readlane_into_soffset(tmp_path):
    assert _check(tmp_path, ["v_readlane_b32 s8, v10, 3", "s_nop 0", DMA]) == (1, 1)


def test_flags_readfirstlane_into_resource(tmp_path):
    assert _check(tmp_path, ["v_readfirstlane_b32 s2, v1", "s_mov_b32 m0, s9", "s_nop 0", DMA]) == (1, 1)


def test_flags_carry_out_into_resource(tmp_path):
    assert _check(tmp_path, ["v_add_co_u32_e64 v1, s[2:3], v2, v3", "s_nop 0", DMA]) == (1, 1)


def test_five_wait_states_clear_it(tmp_path):
    assert _check(tmp_path, ["v_readlane_b32 s8, v10, 3", "s_nop 4", DMA]) == (1, 0)
    assert _check(tmp_path, ["v_readlane_b32 s8, v10, 3", "s_nop 1", "s_mov_b32 m0, s9", "s_nop 1", DMA]) == (1, 0)


def test_scalar_writes_and_unrelated_sgprs_pass(tmp_path):
    assert _check(tmp_path, ["s_add_u32 s8, s8, 64", "v_readlane_b32 s20, v10, 3", "s_nop 0", DMA]) == (1, 0)
    # a VALU source SGPR is not a write
    assert _check(tmp_path, ["v_add_u32_e32 v1, s8, v2", "s_nop 0", DMA]) == (1, 0)


def test_follows_branches_into_the_dma_block(tmp_path):
    body = ["s_cbranch_scc1 .LBB0_2", "v_readlane_b32 s8, v10, 3", "s_branch .LBB0_3",
            ".LBB0_2:", "s_nop 7", ".LBB0_3:", "s_nop 0", DMA]
    assert _check(tmp_path, body) == (1, 1)   # the path through the readlane
    body[1] = "s_mov_b32 s8, 0"
    assert _check(tmp_path, body) == (1, 0)


# The build's response to a finding: compile again with five wait states before
# every DMA (MOE_LIGHT_DMA=0), and fail only if that build has a finding too.
# Compilation, the check and the link are stubbed; only the control flow runs.
import mixture_experts_layer_02_amd.build as moe_build  # noqa: E402
import pytest  # noqa: E402


def _stub_build(monkeypatch, findings):
    calls = []

    def compile_(light, verbose):
        calls.append(light)
        return ["a.o"], ["a.s"]

    results = iter(findings)
    monkeypatch.setattr(moe_build, "_compile", compile_)
    monkeypatch.setattr(moe_build, "_check", lambda asms: next(results))
    monkeypatch.setattr(moe_build, "_run", lambda cmd: "")
    monkeypatch.setattr(moe_build.os, "replace", lambda a, b: None)
    monkeypatch.setattr(moe_build.os, "makedirs", lambda *a, **k: None)
    return calls


def test_build_keeps_light_dmas_without_findings(monkeypatch):
    calls = _stub_build(monkeypatch, [(10, 0, "")])
    moe_build.build()
    assert calls == [True]


def test_build_falls_back_to_five_wait_states(monkeypatch, capsys):
    calls = _stub_build(monkeypatch, [(10, 2, "hazard in k"), (10, 0, "")])
    moe_build.build()
    assert calls == [True, False]
    assert "compiling again with five wait states" in capsys.readouterr().err


def test_build_fails_if_the_five_wait_state_build_has_findings(monkeypatch):
    calls = _stub_build(monkeypatch, [(10, 2, "hazard in k"), (10, 1, "hazard in k")])
    with pytest.raises(RuntimeError, match="hazards"):
        moe_build.build()
    assert calls == [True, False]
    calls = _stub_build(monkeypatch, [(10, 1, "hazard in k")])
    with pytest.raises(RuntimeError, match="hazards"):
        moe_build.build(light=False)
    assert calls == [False]


def test_flags_valu_write_of_m0(tmp_path):
    # the DMA reads M0 without naming it
    assert _check(tmp_path, ["v_readfirstlane_b32 m0, v1", "s_nop 0", DMA]) == (1, 1)
    assert _check(tmp_path, ["v_readfirstlane_b32 m0, v1", "s_nop 4", DMA]) == (1, 0)
    assert _check(tmp_path, ["s_mov_b32 m0, s9", "s_nop 0", DMA]) == (1, 0)


def test_follows_long_branches(tmp_path):
    body = ["v_readlane_b32 s8, v10, 3", "s_getpc_b64 s[20:21]", ".Lpost_getpc0:",
            "s_add_u32 s20, s20, (.LBB0_4-.Lpost_getpc0)&4294967295",
            "s_addc_u32 s21, s21, (.LBB0_4-.Lpost_getpc0)>>32", "s_setpc_b64 s[20:21]",
            ".LBB0_9:", "s_nop 7", "s_nop 7", ".LBB0_4:", DMA]
    assert _check(tmp_path, body) == (1, 1)   # reached from the readlane through the jump


def test_unknown_long_branch_target_fails(tmp_path):
    assert _check(tmp_path, ["s_setpc_b64 s[20:21]", "s_nop 7", DMA])[1] == 1
