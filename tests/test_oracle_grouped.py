"""Pins of the oracle's group-limited routing (CPU only).

Domyn page, section "Group-limited expert routing": the experts are split
into groups of consecutive experts and the router takes the same number of
experts, k / groups, from every group.  The checks reach the answer by other
routes than the oracle's code: brute force over all admissible subsets, the
first maximum of numpy's argmax, the ungrouped top-k where it already meets
the quota, scipy's softmax for the weights, and the exact per-group balance
that the rule exists for.
"""
import itertools

import numpy as np
import pytest
import scipy.special

import oracle


def _tied_logits(rng, T, E):
    L = np.round(rng.standard_normal((T, E)) * 2) / 8.0
    z = rng.random((T, E)) < 0.15
    L[z] = np.where(rng.random(z.sum()) < 0.5, 0.0, -0.0)
    return L


def _beats(L, i, m):
    return L[i] > L[m] or (L[i] == L[m] and i < m)


def _brute_grouped_set(L, k, G):
    """The unique subset with k/G experts from each group in which every taken
    expert beats every untaken expert of its own group."""
    E = len(L)
    Eg, kg = E // G, k // G
    found = []
    for S in itertools.combinations(range(E), k):
        if any(sum(1 for e in S if e // Eg == g) != kg for g in range(G)):
            continue
        Sset = set(S)
        if all(_beats(L, i, m) for i in S for m in range(E) if m not in Sset and m // Eg == i // Eg):
            found.append(Sset)
    assert len(found) == 1
    return found[0]


@pytest.mark.parametrize("E,k,G", [(4, 2, 2), (6, 2, 2), (6, 4, 2), (8, 4, 4), (9, 3, 3), (8, 6, 2)])
def test_grouped_set_matches_brute_force(E, k, G):
    rng = np.random.default_rng(100 + E * 10 + k + G)
    L = _tied_logits(rng, 48, E)
    idx, _ = oracle.topk_route_grouped(L, k, G)
    for t in range(L.shape[0]):
        assert set(idx[t].tolist()) == _brute_grouped_set(L[t], k, G)
        for j in range(k - 1):
            assert _beats(L[t], idx[t, j], idx[t, j + 1])


def test_one_group_is_plain_topk():
    L = _tied_logits(np.random.default_rng(7), 200, 24)
    for k in (1, 3, 8):
        for renorm in (0, 1):
            i1, w1 = oracle.topk_route_grouped(L, k, 1, renorm)
            i0, w0 = oracle.topk_route(L, k, renorm)
            assert (i1 == i0).all()
            np.testing.assert_allclose(w1, w0, rtol=0, atol=1e-15)


def test_one_expert_per_group_is_argmax_of_each_group():
    rng = np.random.default_rng(8)
    L = _tied_logits(rng, 100, 32)
    G = 8
    idx, _ = oracle.topk_route_grouped(L, G, G)
    for t in range(100):
        firsts = [g * 4 + int(np.argmax(L[t, g * 4:(g + 1) * 4])) for g in range(G)]
        assert sorted(idx[t].tolist()) == sorted(firsts)


def test_quota_already_met_gives_plain_topk():
    rng = np.random.default_rng(9)
    L = rng.standard_normal((400, 16))
    i0, w0 = oracle.topk_route(L, 4, 1)
    ig, wg = oracle.topk_route_grouped(L, 4, 2, 1)
    met = np.array([(i0[t] < 8).sum() == 2 for t in range(400)])
    assert 50 < met.sum() < 400
    assert (ig[met] == i0[met]).all() and np.allclose(wg[met], w0[met], rtol=0, atol=1e-15)
    assert (ig[~met] != i0[~met]).any(axis=1).all()


def test_page_example_three_best_in_one_group():
    # 384 experts in 4 groups of 96, top-8 with 2 per group; the token's three
    # best experts all sit in group 1, so only the two best of them are taken.
    rng = np.random.default_rng(10)
    L = rng.standard_normal((1, 384)) * 0.1
    L[0, [100, 150, 170]] = [5.0, 4.0, 3.0]
    idx, _ = oracle.topk_route_grouped(L, 8, 4)
    sel = idx[0].tolist()
    assert sel[:2] == [100, 150] and 170 not in sel
    assert [sum(1 for e in sel if e // 96 == g) for g in range(4)] == [2, 2, 2, 2]


@pytest.mark.parametrize("renorm", [0, 1])
def test_weights_are_softmax_of_the_selection(renorm):
    rng = np.random.default_rng(11)
    L = rng.standard_normal((64, 24)) * 3
    idx, w = oracle.topk_route_grouped(L, 6, 3, renorm)
    sel = np.take_along_axis(L, idx.astype(np.int64), axis=1)
    if renorm:
        want = scipy.special.softmax(sel, axis=1)
        np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    else:
        want = np.take_along_axis(scipy.special.softmax(L, axis=1), idx.astype(np.int64), axis=1)
    np.testing.assert_allclose(w, want, rtol=1e-12, atol=0)


def test_every_group_gets_exactly_its_share():
    rng = np.random.default_rng(12)
    T, E, k, G = 500, 48, 8, 4
    L = rng.standard_normal((T, E)) + np.linspace(3, -3, E)[None, :]   # strongly skewed preference
    idx, _ = oracle.topk_route_grouped(L, k, G)
    Eg = E // G
    for g in range(G):
        counts, offsets = oracle.count_tokens(idx, E, g * Eg, Eg)
        assert offsets[-1] == T * k // G
    assert (np.sort(idx, axis=1)[:, 1:] != np.sort(idx, axis=1)[:, :-1]).all()   # no expert twice


def test_rejects_groups_not_dividing():
    L = np.zeros((2, 12))
    for k, G in [(4, 3), (6, 5)]:
        with pytest.raises(ValueError):
            oracle.topk_route_grouped(L, k, G)
