"""Pins of the oracle's router, top-k and routing weights (CPU only).

Each check reaches the answer by a route other than the oracle's own code:
brute force over all k-subsets, numpy's argmax, scipy's softmax, closed
forms of the renormalised weights, and linearity of the router.
"""
import itertools

import numpy as np
import pytest
import scipy.special

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def _brute_topk_set(L, k):
    """The unique k-subset S with: for i in S, m not in S, L_i > L_m or (L_i == L_m and i < m)."""
    E = len(L)
    found = []
    for S in itertools.combinations(range(E), k):
        Sset = set(S)
        ok = all((L[i] > L[m]) or (L[i] == L[m] and i < m)
                 for i in S for m in range(E) if m not in Sset)
        if ok:
            found.append(S)
    assert len(found) == 1
    return set(found[0])


def _tied_logits(rng, T, E):
    # quantised to 1/8 so that ties are frequent; mix in signed zeros
    L = np.round(rng.standard_normal((T, E)) * 2) / 8.0
    z = rng.random((T, E)) < 0.15
    L[z] = np.where(rng.random(z.sum()) < 0.5, 0.0, -0.0)
    return L


@pytest.mark.parametrize("E,k", [(4, 1), (4, 2), (6, 3), (8, 2), (8, 5), (5, 5)])
def test_topk_set_matches_brute_force(E, k):
    L = _tied_logits(_rng(E * 10 + k), 64, E)
    idx, _ = oracle.topk_route(L, k)
    for t in range(L.shape[0]):
        assert set(idx[t].tolist()) == _brute_topk_set(L[t], k)
        # slot order: non-increasing logit, ties in ascending expert index
        for j in range(k - 1):
            a, b = idx[t, j], idx[t, j + 1]
            assert L[t, a] > L[t, b] or (L[t, a] == L[t, b] and a < b)


def test_signed_zero_tie_goes_to_lower_index():
    L = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]])
    idx, w = oracle.topk_route(L, 1)
    assert idx[:, 0].tolist() == [0, 0]
    assert (w == 1.0).all()


def test_k1_equals_first_argmax():
    L = _tied_logits(_rng(7), 200, 10)
    idx, w = oracle.topk_route(L, 1)
    assert (idx[:, 0] == np.argmax(L, axis=1)).all()
    assert (w == 1.0).all()


def test_k_equals_E_selects_all():
    L = _rng(8).standard_normal((50, 6))
    idx, w = oracle.topk_route(L, 6)
    assert (np.sort(idx, axis=1) == np.arange(6)).all()
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-15)


@pytest.mark.parametrize("E,k", [(8, 2), (16, 8), (384, 8)])
def test_renormalised_weights_closed_form(E, k):
    L = _rng(E + k).standard_normal((40, E)) * 3
    idx, w = oracle.topk_route(L, k, renormalize=1)
    sel = np.take_along_axis(L, idx.astype(np.int64), axis=1)
    # w_j = exp(L_j - L_0) / sum_i exp(L_i - L_0): softmax restricted to the selection
    ref = np.exp(sel - sel[:, :1])
    ref /= ref.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(w, ref, rtol=1e-13, atol=0)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)


def test_raw_softmax_weights_match_scipy():
    L = _rng(3).standard_normal((30, 12)) * 4
    idx, w = oracle.topk_route(L, 3, renormalize=0)
    p = scipy.special.softmax(L, axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(p, idx.astype(np.int64), axis=1), rtol=1e-13)


@pytest.mark.parametrize("k", [2, 8])
def test_equal_selected_logits_give_uniform_weights(k):
    E = 16
    L = np.full((4, E), -5.0)
    L[:, :k] = 1.25
    idx, w = oracle.topk_route(L, k)
    assert (idx == np.arange(k)).all()
    np.testing.assert_allclose(w, 1.0 / k, rtol=1e-15)


def test_large_logits_stay_finite():
    L = np.array([[80.0, -80.0, 79.5, 0.0], [-80.0, -80.0, -79.0, -80.0]])
    idx, w = oracle.topk_route(L, 2)
    assert np.isfinite(w).all()
    assert idx.tolist() == [[0, 2], [2, 0]]
    np.testing.assert_allclose(w[0], [1 / (1 + np.exp(-0.5)), np.exp(-0.5) / (1 + np.exp(-0.5))], rtol=1e-14)


def test_nan_logits_are_refused():
    with pytest.raises(ValueError):
        oracle.topk_route(np.array([[0.0, np.nan]]), 1)


def test_router_logits_linearity_and_one_hot():
    rng = _rng(11)
    d, E = 5, 7
    wr = rng.standard_normal((E, d))
    # one-hot tokens read out columns of W_r (i.e. W_r[:, i])
    L = oracle.router_logits(np.eye(d), wr)
    np.testing.assert_array_equal(L, wr.T)
    # bias is added per expert
    b = rng.standard_normal(E)
    np.testing.assert_allclose(oracle.router_logits(np.eye(d), wr, b), wr.T + b, rtol=0, atol=0)
    # linearity in x
    x1, x2 = rng.standard_normal((3, d)), rng.standard_normal((3, d))
    np.testing.assert_allclose(oracle.router_logits(2 * x1 - x2, wr),
                               2 * oracle.router_logits(x1, wr) - oracle.router_logits(x2, wr), atol=1e-12)
