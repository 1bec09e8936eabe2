"""Pins of the oracle's expert MLP and weighted combine (CPU only).

Routes other than the oracle's own: a textbook triple-loop SwiGLU MLP, the
identical-experts invariant (any routing reduces to the dense MLP because the
renormalised weights sum to one), the expert-parallel partition identity
(Algorithm 1 stage 5: the partial outputs of the ranks sum to the full
output), zero down-projection, and closed forms of silu.  The down
projection alone (expert_down) is pinned to the MLP's own output and to
explicit loops.
"""
import math

import numpy as np
import scipy.special

import oracle


def _loop_swiglu(x, w1, w3, w2):
    """Dense SwiGLU MLP with explicit loops (weights out x in)."""
    T, d = len(x), len(x[0])
    f = len(w1)
    y = [[0.0] * d for _ in range(T)]
    for t in range(T):
        h = []
        for c in range(f):
            g = sum(x[t][i] * w1[c][i] for i in range(d))
            u = sum(x[t][i] * w3[c][i] for i in range(d))
            h.append(g / (1.0 + math.exp(-g)) * u)
        for o in range(d):
            y[t][o] = sum(h[c] * w2[o][c] for c in range(f))
    return np.array(y)


def _layer(x, wr, w1, w3, w2, k, e0, NL, **kw):
    return oracle.layer_forward(x, wr, w1, w3, w2, k, e0, NL, **kw)


def test_single_expert_top1_is_dense_mlp():
    rng = np.random.default_rng(1)
    T, d, f = 5, 4, 3
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((1, d))
    w1, w3 = rng.standard_normal((1, f, d)), rng.standard_normal((1, f, d))
    w2 = rng.standard_normal((1, d, f))
    out = _layer(x, wr, w1, w3, w2, 1, 0, 1)
    ref = _loop_swiglu(x.tolist(), w1[0].tolist(), w3[0].tolist(), w2[0].tolist())
    np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-12)


def test_identical_experts_reduce_to_dense_mlp():
    rng = np.random.default_rng(2)
    T, d, f, E, k = 40, 6, 5, 6, 3
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((E, d))
    a1, a3, a2 = rng.standard_normal((f, d)), rng.standard_normal((f, d)), rng.standard_normal((d, f))
    w1 = np.repeat(a1[None], E, 0)
    w3 = np.repeat(a3[None], E, 0)
    w2 = np.repeat(a2[None], E, 0)
    out = _layer(x, wr, w1, w3, w2, k, 0, E)
    ref = _loop_swiglu(x.tolist(), a1.tolist(), a3.tolist(), a2.tolist())
    np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-12)


def test_expert_parallel_partial_outputs_sum_to_full_output():
    rng = np.random.default_rng(3)
    T, d, f, E, k, EP = 32, 8, 4, 8, 3, 4
    NR = E // EP
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((E, d))
    w1, w3 = rng.standard_normal((E, f, d)), rng.standard_normal((E, f, d))
    w2 = rng.standard_normal((E, d, f))
    full = _layer(x, wr, w1, w3, w2, k, 0, E)["y"]
    parts = [
        _layer(x, wr, w1[r * NR:(r + 1) * NR], w3[r * NR:(r + 1) * NR], w2[r * NR:(r + 1) * NR],
               k, r * NR, NR)["y"] for r in range(EP)]
    np.testing.assert_allclose(sum(parts), full, rtol=1e-12, atol=1e-12)


def test_zero_down_projection_gives_zero_output():
    rng = np.random.default_rng(4)
    T, d, f, E, k = 16, 4, 3, 4, 2
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((E, d))
    w1, w3 = rng.standard_normal((E, f, d)), rng.standard_normal((E, f, d))
    out = _layer(x, wr, w1, w3, np.zeros((E, d, f)), k, 0, E)
    assert (out["y"] == 0).all()


def test_token_without_local_expert_gets_zero():
    x = np.ones((2, 3))
    wr = np.array([[1.0, 0, 0], [0, 1.0, 0], [0, 0, 1.0], [-5.0, -5, -5]])
    x[1] = [-1.0, -1.0, 3.0]        # token 1 selects experts 2 then 0/1 (non-local)
    w1 = np.ones((2, 2, 3))
    w3 = np.ones((2, 2, 3))
    w2 = np.ones((2, 3, 2))
    out = _layer(x, wr, w1, w3, w2, 1, 0, 2)
    assert out["idx"][1, 0] == 2
    assert (out["y"][1] == 0).all()
    assert (out["slot_row"][1] == -1).all()


def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    np.testing.assert_allclose(oracle.silu(40.0), 40.0, rtol=1e-15)
    np.testing.assert_allclose(oracle.silu(-40.0), -40.0 * math.exp(-40.0), rtol=1e-12)
    g = np.linspace(-8, 8, 101)
    np.testing.assert_allclose(oracle.silu(g), g * scipy.special.expit(g), rtol=1e-14, atol=1e-300)
    assert oracle.silu_grad(0.0) == 0.5
    eps = 1e-6
    np.testing.assert_allclose(oracle.silu_grad(g), (oracle.silu(g + eps) - oracle.silu(g - eps)) / (2 * eps),
                               rtol=1e-7, atol=1e-9)


def test_expert_down_alone_is_the_mlps_last_product():
    # expert_down on the MLP's own H gives the MLP's y_perm; on tiny inputs it
    # equals an explicit loop over rows, outputs and the inner dimension, with
    # the right expert's weights for every segment (one empty).
    rng = np.random.default_rng(21)
    NL, d, f = 4, 6, 5
    off = np.array([0, 3, 3, 7, 9])
    x = rng.standard_normal((9, d))
    w1, w3, w2 = (rng.standard_normal((NL, f, d)), rng.standard_normal((NL, f, d)),
                  rng.standard_normal((NL, d, f)))
    _, _, H, Y = oracle.expert_ffn(x, off, w1, w3, w2)
    np.testing.assert_array_equal(oracle.expert_down(H, off, w2), Y)
    h = rng.standard_normal((9, f))
    got = oracle.expert_down(h, off, w2)
    for n in range(NL):
        for r in range(off[n], off[n + 1]):
            for o in range(d):
                want = sum(h[r][c] * w2[n][o][c] for c in range(f))
                assert abs(got[r][o] - want) <= 1e-12 * (1 + abs(want))
