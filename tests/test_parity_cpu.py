"""CPU checks of the parity judge itself (tests/parity.py ``valid_cut``): it
must accept the oracle's own cuts and the cuts rounding can legitimately
produce, and reject every plausible wrong selection. The mistakes are planted
in hand-made rows on the CPU."""
import numpy as np
import pytest

import oracle
from tests.parity import MASS_TOL, TIE_REL, valid_cut


def _mask(n, idx):
    m = np.zeros(n, dtype=bool)
    m[list(idx)] = True
    return m


def _rows(seed, n, count, sharp):
    rng = np.random.default_rng(seed)
    z = rng.normal(0, 2.0 if sharp else 0.03, size=(count, n))
    return oracle.block_probs(z)


@pytest.mark.parametrize("sharp", [False, True])
@pytest.mark.parametrize("thr", [0.2, 0.5, 0.79, 0.95])
def test_accepts_the_oracle_cut(sharp, thr):
    n = 97
    window = np.zeros(n, dtype=bool)
    window[10:13] = True
    for p in _rows(1, n, 20, sharp):
        kept, k, *_ = oracle.cdf_cut_details(p, thr)
        assert valid_cut(_mask(n, kept), p, np.zeros(n, bool), k, thr, "cdf")
        assert valid_cut(_mask(n, kept) | window, p, window, k, thr, "cdf")


N_ROW, K_ROW, THR_ROW = 50, 10, 0.6       # rows below: the cut falls at the 10th block


def _row(head_sum=None, s_k=None):
    """A descending row of 50 probabilities whose first 9 blocks sum to
    ``head_sum`` (or whose first 10 sum to ``s_k``)."""
    head = 0.0405 - 0.00005 * np.arange(1, K_ROW)
    if head_sum is not None:
        head = head * (head_sum / head.sum())
        pk = 0.95 * head[-1]
    else:
        pk = s_k - head.sum()
    rest = np.linspace(1.0, 0.9, N_ROW - K_ROW)
    rest *= (1.0 - head.sum() - pk) / rest.sum()
    p = np.concatenate([head, [pk], rest])
    assert np.all(np.diff(p) < 0) and p[-1] > 0 and abs(p.sum() - 1) < 1e-12
    return p


def test_accepts_one_block_more_or_less_only_inside_the_window():
    n, thr, target = N_ROW, THR_ROW, 1 - THR_ROW
    none = np.zeros(n, bool)
    first = lambda m: _mask(n, range(m))
    # S_k just above 1 - thr: keeping k + 1 blocks is a rounding-level difference
    p = _row(s_k=target + 0.3 * MASS_TOL)
    k = oracle.cdf_cut_details(p, thr)[1]
    assert k == K_ROW
    assert valid_cut(first(k), p, none, k, thr, "cdf")
    assert valid_cut(first(k + 1), p, none, k, thr, "cdf")
    assert not valid_cut(first(k + 2), p, none, k, thr, "cdf")
    assert not valid_cut(first(k - 1), p, none, k, thr, "cdf")
    # S_k well above the target: k + 1 is a wrong cut
    p = _row(s_k=target + 50 * MASS_TOL)
    assert not valid_cut(first(K_ROW + 1), p, none, K_ROW, thr, "cdf")
    # S_{k-1} just below the target: k - 1 blocks are a rounding-level difference
    p = _row(head_sum=target - 0.3 * MASS_TOL)
    k = oracle.cdf_cut_details(p, thr)[1]
    assert k == K_ROW
    assert valid_cut(first(k - 1), p, none, k, thr, "cdf")
    assert valid_cut(first(k), p, none, k, thr, "cdf")
    # ... but not when it is well below
    p = _row(head_sum=target - 50 * MASS_TOL)
    assert not valid_cut(first(K_ROW - 1), p, none, K_ROW, thr, "cdf")


def test_rejects_planted_mistakes():
    n, thr = 80, 0.5
    p = _rows(3, n, 1, True)[0]
    kept, k, *_ = oracle.cdf_cut_details(p, thr)
    order = np.lexsort((np.arange(n), -p))
    none = np.zeros(n, bool)
    good = _mask(n, kept)
    # a kept block exchanged for one well below the cut
    bad = good.copy()
    bad[order[k - 1]] = False
    bad[order[-1]] = True
    assert not valid_cut(bad, p, none, k, thr, "cdf")
    # the most probable block dropped
    bad = good.copy()
    bad[order[0]] = False
    assert not valid_cut(bad, p, none, k, thr, "cdf")
    # a window block missing
    window = _mask(n, [order[-1], order[-2]])
    assert not valid_cut(good | _mask(n, [order[-1]]), p, window, k, thr, "cdf")
    assert valid_cut(good | window, p, window, k, thr, "cdf")
    # every block kept
    assert not valid_cut(np.ones(n, bool), p, none, k, thr, "cdf")


def test_near_ties_at_the_cut_may_be_exchanged():
    n, thr = 40, 0.5
    p = np.linspace(3.0, 1.0, n)
    p /= p.sum()
    kept, k, *_ = oracle.cdf_cut_details(p, thr)
    order = np.lexsort((np.arange(n), -p))
    # make blocks k and k+1 (1-based) equal within a tenth of the tie tolerance
    a, b = order[k - 1], order[k]
    p = p.copy()
    p[b] = p[a] * (1 - 0.1 * TIE_REL)
    swapped = _mask(n, kept)
    swapped[a], swapped[b] = False, True
    none = np.zeros(n, bool)
    assert valid_cut(swapped, p, none, k, thr, "cdf")
    # a gap of ten times the tolerance is not a tie
    p[b] = p[a] * (1 - 10 * TIE_REL)
    assert not valid_cut(swapped, p, none, k, thr, "cdf")


def test_topk_count_is_fixed():
    n = 60
    p = _rows(5, n, 1, False)[0]
    order = np.lexsort((np.arange(n), -p))
    none = np.zeros(n, bool)
    for k in (1, 7, 59):
        assert valid_cut(_mask(n, order[:k]), p, none, k, 0.0, "topk")
        assert not valid_cut(_mask(n, order[:k + 1]), p, none, k, 0.0, "topk")
        if k > 1:
            assert not valid_cut(_mask(n, order[:k - 1]), p, none, k, 0.0, "topk")
