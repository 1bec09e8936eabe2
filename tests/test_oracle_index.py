"""Pins of the oracle's counting, prefix sums and index generation (CPU only).

The oracle writes stages 2-3 as a sequential stable counting sort.  Here the
same results are reached by other routes: the thread-blocked kernels of the
Aurora page's Algorithm 1 (stages 2 and 3) executed step by step, numpy's
stable argsort, a hand-derived fixture shaped like Figure 5, the
forced-uniform closed form, and the permutation invariants.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _random_routing(rng, T, E, k):
    return np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)


def _alg1_blocked(indices, n_start, NR, TBS=8):
    """Stages 2-3 of Algorithm 1 as the thread-blocked procedure on the page.

    TH threads each own a block of TBS tokens; per-(expert, thread) partial
    counts are laid out expert-major and prefix-summed, and a per-(expert,
    thread) counter places each selection at base + offset.  The garbled
    index names on the page are read as: t = tid*TBS + i defined before the
    slot loop, and partial counts indexed by (local expert, thread).
    """
    T, K = indices.shape
    assert T % TBS == 0
    TH = T // TBS
    n_end = n_start + NR - 1
    partial = [0] * (NR * TH)
    expert_counts = [0] * T
    for tid in range(TH):
        for i in range(TBS):
            t = tid * TBS + i
            for k in range(K):
                n = int(indices[t, k])
                if n_start <= n <= n_end:
                    partial[(n - n_start) * TH + tid] += 1
                    expert_counts[t] += 1
    partial_cum = [0] * (NR * TH + 1)
    for i in range(NR * TH):
        partial_cum[i + 1] = partial_cum[i] + partial[i]
    cum_expert = [0] * (T + 1)
    for t in range(T):
        cum_expert[t + 1] = cum_expert[t] + expert_counts[t]
    cum_token = [partial_cum[n * TH] for n in range(NR + 1)]
    RT = cum_token[-1]
    sel = [0] * RT
    inp = [0] * RT
    outp = [0] * RT
    counter = [[0] * TH for _ in range(NR)]
    for tid in range(TH):
        for i in range(TBS):
            t = tid * TBS + i
            o_ind = cum_expert[t]
            for k in range(K):
                n = int(indices[t, k])
                if n_start <= n <= n_end:
                    ln = n - n_start
                    i_ind = partial_cum[ln * TH + tid] + counter[ln][tid]
                    inp[i_ind] = t
                    outp[o_ind] = i_ind
                    sel[o_ind] = k
                    counter[ln][tid] += 1
                    o_ind += 1
    return dict(cum_token_counts=cum_token, input_indices=inp, output_indices=outp,
                selected_expert_indices=sel, cum_expert_counts=cum_expert)


def _alg1_view(slot_row):
    """Token-major (output_indices, selected_expert_indices, cum_expert_counts) of slot_row."""
    outp, sel, cum = [], [], [0]
    for t in range(slot_row.shape[0]):
        for j in range(slot_row.shape[1]):
            if slot_row[t, j] >= 0:
                outp.append(int(slot_row[t, j]))
                sel.append(j)
        cum.append(len(outp))
    return outp, sel, cum


def test_figure5_shaped_fixture():
    with open(os.path.join(GOLDEN, "fig5_index_generation.json")) as fh:
        g = json.load(fh)
    idx = np.array(g["indices"], np.int32)
    for case in g["cases"]:
        e0, NL = case["n_start"], case["NR"]
        counts, offsets = oracle.count_tokens(idx, g["N"], e0, NL)
        row_token, slot_row = oracle.generate_indices(idx, e0, NL, offsets)
        assert counts.tolist() == case["counts_all"], case["name"]
        assert offsets.tolist() == case["cum_token_counts"], case["name"]
        assert row_token.tolist() == case["input_indices"], case["name"]
        assert slot_row.tolist() == case["slot_row"], case["name"]
        outp, sel, cum = _alg1_view(slot_row)
        assert outp == case["output_indices"]
        assert sel == case["selected_expert_indices"]
        assert cum == case["cum_expert_counts"]


@pytest.mark.parametrize("T,E,k,e0,NL", [(64, 8, 2, 0, 8), (96, 16, 4, 4, 8), (256, 12, 3, 6, 6),
                                         (40, 4, 4, 0, 2), (32, 384, 8, 0, 96), (48, 10, 1, 3, 1)])
def test_matches_algorithm1_blocked_kernels(T, E, k, e0, NL):
    idx = _random_routing(np.random.default_rng(T + E + k), T, E, k)
    alg = _alg1_blocked(idx, e0, NL)
    counts, offsets = oracle.count_tokens(idx, E, e0, NL)
    row_token, slot_row = oracle.generate_indices(idx, e0, NL, offsets)
    assert offsets.tolist() == alg["cum_token_counts"]
    assert row_token.tolist() == alg["input_indices"]
    outp, sel, cum = _alg1_view(slot_row)
    assert outp == alg["output_indices"]
    assert sel == alg["selected_expert_indices"]
    assert cum == alg["cum_expert_counts"]


def test_blocked_result_does_not_depend_on_block_size():
    idx = _random_routing(np.random.default_rng(5), 64, 8, 3)
    a = _alg1_blocked(idx, 2, 4, TBS=8)
    b = _alg1_blocked(idx, 2, 4, TBS=16)
    c = _alg1_blocked(idx, 2, 4, TBS=64)
    assert a == b == c


def test_matches_stable_argsort_by_expert():
    rng = np.random.default_rng(9)
    T, E, k, e0, NL = 500, 20, 4, 5, 10
    idx = _random_routing(rng, T, E, k)
    counts, offsets = oracle.count_tokens(idx, E, e0, NL)
    row_token, slot_row = oracle.generate_indices(idx, e0, NL, offsets)
    flat_e = idx.reshape(-1).astype(np.int64)
    flat_t = np.repeat(np.arange(T), k)
    local = (flat_e >= e0) & (flat_e < e0 + NL)
    order = np.argsort(flat_e[local], kind="stable")
    assert (row_token == flat_t[local][order]).all()
    np.testing.assert_array_equal(counts, np.bincount(flat_e, minlength=E))


def test_permutation_invariants():
    rng = np.random.default_rng(21)
    T, E, k, e0, NL, d = 300, 24, 6, 8, 8, 5
    idx = _random_routing(rng, T, E, k)
    x = rng.standard_normal((T, d)).astype(np.float32)
    counts, offsets = oracle.count_tokens(idx, E, e0, NL)
    row_token, slot_row = oracle.generate_indices(idx, e0, NL, offsets)
    R = int(offsets[-1])
    assert counts.sum() == T * k
    assert R == counts[e0:e0 + NL].sum()
    rows = slot_row[slot_row >= 0]
    assert sorted(rows.tolist()) == list(range(R))           # bijection onto [0, R)
    tt, jj = np.nonzero(slot_row >= 0)
    assert (row_token[slot_row[tt, jj]] == tt).all()
    local = (idx >= e0) & (idx < e0 + NL)
    assert ((slot_row >= 0) == local).all()
    x_perm = oracle.permute(x, row_token)
    assert (x_perm[slot_row[tt, jj]].view(np.uint32) == x[tt].view(np.uint32)).all()
    # rows of a segment hold that segment's expert, tokens ascending
    for n in range(NL):
        seg = row_token[offsets[n]:offsets[n + 1]]
        assert (np.diff(seg) > 0).all()
        assert all(e0 + n in idx[t] for t in seg)


def test_forced_uniform_counts_closed_form():
    cfg = synth.CONFIGS["uniform_1t"]
    idx, w = synth.roundrobin_routing(cfg.T, cfg.E, cfg.k)
    counts, offsets = oracle.count_tokens(idx, cfg.E, 0, cfg.E)
    e = np.arange(cfg.E)
    closed = (cfg.T * cfg.k - 1 - e) // cfg.E + 1
    np.testing.assert_array_equal(counts, closed)
    assert (counts[:32] == 1366).all() and (counts[32:] == 1365).all()
    assert offsets[-1] == cfg.T * cfg.k


def test_empty_and_nonlocal_only():
    idx = np.array([[0, 1], [1, 0]], np.int32)
    counts, offsets = oracle.count_tokens(idx, 4, 2, 2)
    assert counts.tolist() == [2, 2, 0, 0]
    assert offsets.tolist() == [0, 0, 0]
    row_token, slot_row = oracle.generate_indices(idx, 2, 2, offsets)
    assert row_token.size == 0 and (slot_row == -1).all()


def test_repeated_expert_in_a_token_is_rejected():
    # The k selections of a token are k distinct experts (top-k over the
    # experts); a routing that lists one twice has no row layout and is
    # refused rather than silently counted.
    idx = np.array([[0, 1], [2, 2], [1, 3]], np.int64)
    with pytest.raises(ValueError):
        oracle.count_tokens(idx, 4, 0, 4)
    with pytest.raises(ValueError):
        oracle.generate_indices(idx, 0, 4, np.array([0, 1, 2, 4, 5]))
