"""Pins for the oracle's lightning-indexer score and top-k.

Source: page "CSA And HCA: Definition, State, And Cost Model", section 3.1: the
score is a per-head ReLU of q^I . K^I weighted by w^I and summed over heads, with
no scale term, over completed entries only; TopK then keeps k entries.
"""
import numpy as np
import pytest

import oracle


def test_scores_hand_constructed():
    # two heads, c^I = 4; head 0 reads coordinate 0, head 1 reads 2 * coordinate 1
    T, t0, m = 6, 10, 4
    qI = np.zeros((T, 2, 4))
    qI[:, 0, 0] = 1.0
    qI[:, 1, 1] = 2.0
    wI = np.tile([0.5, 3.0], (T, 1))
    E = 4
    KI = np.zeros((E, 4))
    s = np.arange(E)
    KI[:, 0] = s + 1.0       # head 0 dot = s+1 > 0
    KI[:, 1] = -(s + 1.0)    # head 1 dot = -2(s+1) < 0 -> ReLU 0
    sc = oracle.index_scores(qI, KI, wI, t0=t0, m=m, ld=E)
    for j in range(T):
        Et = (t0 + j + 1) // m
        assert np.allclose(sc[j, :Et], 0.5 * (s[:Et] + 1.0), rtol=0, atol=0)
        assert np.all(np.isnan(sc[j, Et:]))
    KI[:, 1] = s * 1.0       # head 1 now positive: 3 * 2s
    sc = oracle.index_scores(qI, KI, wI, t0=t0, m=m, ld=E)
    assert np.allclose(sc[-1], 0.5 * (s + 1.0) + 6.0 * s, rtol=0, atol=0)


def test_scores_are_linear_in_weights_and_ignore_negative_heads():
    rng = np.random.default_rng(0)
    T, nh, cI, E = 3, 5, 8, 7
    qI = rng.standard_normal((T, nh, cI))
    KI = rng.standard_normal((E, cI))
    w1, w2 = rng.random((T, nh)), rng.random((T, nh))
    t0 = 4 * E - 1 - (T - 1)  # the last query sees all E entries
    a = oracle.index_scores(qI, KI, w1, t0=t0, m=4, ld=E)
    b = oracle.index_scores(qI, KI, w2, t0=t0, m=4, ld=E)
    ab = oracle.index_scores(qI, KI, 2 * w1 + 3 * w2, t0=t0, m=4, ld=E)
    assert np.allclose(np.nan_to_num(ab), np.nan_to_num(2 * a + 3 * b), rtol=1e-13)
    # a head whose dot products are all negative contributes nothing
    q2 = qI.copy()
    q2[:, 0, :] = 0.0
    q2[:, 0, 0] = 1.0
    K2 = KI.copy()
    K2[:, 0] = -np.abs(K2[:, 0]) - 1.0
    base = oracle.index_scores(q2, K2, w1, t0=t0, m=4, ld=E)
    w3 = w1.copy()
    w3[:, 0] = 1e6
    big = oracle.index_scores(q2, K2, w3, t0=t0, m=4, ld=E)
    assert np.array_equal(np.nan_to_num(base), np.nan_to_num(big))


def _rank_select(scores_row, E, k):
    """Brute force: s is selected iff fewer than k entries precede it in (score desc, index asc)."""
    sel = []
    for s in range(E):
        ahead = sum(1 for u in range(E) if scores_row[u] > scores_row[s]
                    or (scores_row[u] == scores_row[s] and u < s))
        if ahead < k:
            sel.append(s)
    return sel


@pytest.mark.parametrize("k", [1, 3, 8, 40])
def test_topk_bruteforce_with_ties(k):
    rng = np.random.default_rng(k)
    T, m, t0 = 40, 4, 0
    ld = (t0 + T) // m
    scores = rng.integers(0, 5, size=(T, ld)).astype(np.float64)  # many ties
    idx, cnt = oracle.topk(scores, t0=t0, m=m, k=k)
    for j in range(T):
        E = (t0 + j + 1) // m
        want = _rank_select(scores[j], E, k)
        assert cnt[j] == min(k, E)
        assert idx[j, :cnt[j]].tolist() == want          # ascending indices
        assert np.all(idx[j, cnt[j]:] == -1)


def test_topk_only_sees_completed_entries():
    T, m, k = 12, 4, 2
    ld = 10
    scores = np.zeros((T, ld))
    scores[:, 5:] = 100.0  # large scores on entries no query here can see yet
    idx, cnt = oracle.topk(scores, t0=0, m=m, k=k)
    for j in range(T):
        E = (j + 1) // m
        assert np.all(idx[j, :cnt[j]] < E)
