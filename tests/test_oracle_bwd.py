"""Pins of the oracle's backward pass (CPU only).

The backward is not written out on the pages; it is derived by calculus.  It
is pinned here against central finite differences of the oracle's own
forward (a different computation: it never evaluates a derivative formula),
the adjoint identity of the gather/scatter pair, and the zero-sum property
of the renormalised router gradient.
"""
import numpy as np
import pytest

import oracle


def _setup(seed, T=12, d=6, f=4, E=4, k=2, NL=None):
    rng = np.random.default_rng(seed)
    NL = E if NL is None else NL
    p = dict(
        x=rng.standard_normal((T, d)),
        wr=rng.standard_normal((E, d)),
        w1=rng.standard_normal((NL, f, d)) * 0.7,
        w3=rng.standard_normal((NL, f, d)) * 0.7,
        w2=rng.standard_normal((NL, d, f)) * 0.7,
    )
    dy = rng.standard_normal((T, d))
    return p, dy, k, NL


def _loss(p, dy, k, e0, NL, renorm):
    out = oracle.layer_forward(p["x"], p["wr"], p["w1"], p["w3"], p["w2"], k, e0, NL, renormalize=renorm)
    return float((out["y"] * dy).sum()), out["idx"]


@pytest.mark.parametrize("renorm,e0,NL,E,k", [(1, 0, 4, 4, 2), (1, 1, 2, 4, 2), (0, 0, 4, 4, 2),
                                              (1, 0, 6, 6, 3), (0, 2, 3, 6, 3)])
def test_gradients_match_central_differences(renorm, e0, NL, E, k):
    p, dy, k, NL = _setup(renorm * 100 + e0 * 10 + NL + E, E=E, k=k, NL=NL)
    fwd = oracle.layer_forward(p["x"], p["wr"], p["w1"], p["w3"], p["w2"], k, e0, NL, renormalize=renorm)
    g = oracle.layer_backward(fwd, p["x"], p["wr"], p["w1"], p["w3"], p["w2"], dy, renormalize=renorm)
    grads = dict(x=g["dx"], wr=g["dWr"], w1=g["dW1"], w3=g["dW3"], w2=g["dW2"])
    eps = 1e-6
    rng = np.random.default_rng(0)
    for name, G in grads.items():
        for _ in range(12):
            pos = tuple(int(rng.integers(0, s)) for s in p[name].shape)
            q = {kk: v.copy() for kk, v in p.items()}
            q[name][pos] += eps
            lp, ip = _loss(q, dy, k, e0, NL, renorm)
            q[name][pos] -= 2 * eps
            lm, im = _loss(q, dy, k, e0, NL, renorm)
            assert (ip == fwd["idx"]).all() and (im == fwd["idx"]).all(), "routing flipped"
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - G[pos]) <= 1e-6 * max(1.0, abs(fd)), (name, pos, fd, G[pos])


def test_gather_scatter_adjoint():
    rng = np.random.default_rng(5)
    T, E, k, d = 30, 6, 3, 4
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets = oracle.count_tokens(idx, E, 1, 4)
    row_token, slot_row = oracle.generate_indices(idx, 1, 4, offsets)
    u = rng.standard_normal((T, d))
    v = rng.standard_normal((int(offsets[-1]), d))
    lhs = (oracle.permute(u, row_token) * v).sum()
    rhs = (u * oracle.unpermute_bwd(v, slot_row)).sum()
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12)


def test_renormalised_router_gradient_sums_to_zero_over_selection():
    rng = np.random.default_rng(6)
    T, E, k = 50, 16, 8
    L = rng.standard_normal((T, E))
    idx, w = oracle.topk_route(L, k)
    dw = rng.standard_normal((T, k))
    dw[:, 5:] = 0.0                      # slots whose expert is not local carry no dw
    dL = oracle.route_bwd(idx, w, dw, E)
    np.testing.assert_allclose(dL.sum(axis=1), 0.0, atol=1e-14)
    mask = np.zeros((T, E), bool)
    np.put_along_axis(mask, idx.astype(np.int64), True, axis=1)
    assert (dL[~mask] == 0).all()
    assert (dL[:, :][mask].reshape(T, -1) != 0).any()


def test_zero_row_expert_has_exact_zero_weight_grads():
    rng = np.random.default_rng(7)
    T, d, f, E, k = 10, 4, 3, 3, 1
    x = rng.standard_normal((T, d))
    wr = np.zeros((E, d))
    wr[0, 0] = 1.0
    x[:, 0] = np.abs(x[:, 0]) + 1.0        # every token picks expert 0
    w1, w3, w2 = rng.standard_normal((E, f, d)), rng.standard_normal((E, f, d)), rng.standard_normal((E, d, f))
    fwd = oracle.layer_forward(x, wr, w1, w3, w2, k, 0, E)
    g = oracle.layer_backward(fwd, x, wr, w1, w3, w2, rng.standard_normal((T, d)))
    assert (fwd["counts"][1:] == 0).all()
    assert (g["dW1"][1:] == 0).all() and (g["dW3"][1:] == 0).all() and (g["dW2"][1:] == 0).all()
