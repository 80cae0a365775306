"""Pins of the tie-avoidance rule (oracle/condition.py) on the CPU.

Every bit-exact index comparison rests on this rule: a seeded query landmark
is kept only if its k-th best relevance score (Eq. 1, paperhub.cn review page,
authors' reply "Cmt 1": score_scale * <lq, lk>) beats the (k+1)-th best by at
least min_gap.  The checks here never use kth_gap to judge itself: expected
values are literal numbers worked out by hand, or come from a plain Python
sort of the scores.  A partition on r instead of -r, a gap taken between the
wrong neighbours, a dropped score scale, or candidates past n_cand counted,
each fails one of them.
"""

import math

import numpy as np
import pytest

from oracle import condition


def _gap_by_sort(r, k):
    """k-th minus (k+1)-th largest of r with Python's sorted(); inf if len(r) <= k."""
    s = sorted((float(x) for x in r), reverse=True)
    return math.inf if len(s) <= k else s[k - 1] - s[k]


@pytest.mark.parametrize("r,k,gap", [
    ([3.0, 1.0, 2.0], 1, 1.0),             # sorted 3, 2, 1
    ([3.0, 1.0, 2.0], 2, 1.0),
    ([5.0, 5.0, 4.0], 1, 0.0),             # tie at the top
    ([5.0, 5.0, 4.0], 2, 1.0),
    ([4.0, 5.0, 5.0, 0.5], 3, 3.5),        # ties above the cut do not matter
    ([-1.0, -3.0, -2.0], 1, 1.0),          # negative scores: -1 > -2 > -3
    ([-1.0, -3.0, -2.0], 2, 1.0),
    ([0.25, -0.5, 0.75, 0.0, -2.0], 2, 0.25),  # 0.75, 0.25 | 0.0
    ([0.25, -0.5, 0.75, 0.0, -2.0], 4, 1.5),   # ..., -0.5 | -2.0
    ([7.0, 7.0, 7.0, 7.0], 2, 0.0),        # all equal
])
def test_kth_gap_literal_cases(r, k, gap):
    assert condition.kth_gap(np.array(r), k) == gap


@pytest.mark.parametrize("r,k", [([1.0, 2.0], 2), ([1.0, 2.0], 3), ([], 1), ([9.0], 1)])
def test_kth_gap_at_most_k_candidates_is_infinite(r, k):
    assert condition.kth_gap(np.array(r), k) == math.inf


def test_kth_gap_matches_a_full_sort_on_random_rows():
    rng = np.random.default_rng(123)
    for trial in range(300):
        n = int(rng.integers(1, 40))
        k = int(rng.integers(1, 17))
        # rounded to a coarse grid so that exact ties occur often
        r = np.round(rng.standard_normal(n) * 4) / 4
        assert condition.kth_gap(r, k) == _gap_by_sort(r, k), (trial, r, k)


def test_gap_ok_threshold_is_inclusive():
    # scores 1e-3 and 0 (one query, two candidates, unit scale): the gap is
    # exactly the minimum and passes; a hair less fails
    lq = np.array([[1.0]])
    lk = np.array([[1e-3], [0.0]])
    assert condition.gap_ok(lq, lk, [2], 1, 1.0, min_gap=1e-3).tolist() == [True]
    lk_close = np.array([[1e-3 - 1e-9], [0.0]])
    assert condition.gap_ok(lq, lk_close, [2], 1, 1.0, min_gap=1e-3).tolist() == [False]
    # 2^-9 and 2^-10 gaps on either side of 1e-3
    lk9 = np.array([[1.0], [1.0 - 2.0 ** -9]])
    lk10 = np.array([[1.0], [1.0 - 2.0 ** -10]])
    assert condition.gap_ok(lq, lk9, [2], 1, 1.0).tolist() == [True]
    assert condition.gap_ok(lq, lk10, [2], 1, 1.0).tolist() == [False]


def test_gap_ok_uses_the_scaled_dot_product():
    # lq = (1, 0); candidates score 0.5 * (2, 1, 0) = (1, 0.5, 0): gap 0.5 at k = 1
    lq = np.array([[1.0, 0.0]])
    lk = np.array([[2.0, 0.0], [1.0, 0.0], [0.0, 5.0]])
    assert condition.gap_ok(lq, lk, [3], 1, 0.5, min_gap=0.49).tolist() == [True]
    assert condition.gap_ok(lq, lk, [3], 1, 0.5, min_gap=0.51).tolist() == [False]
    # unscaled the gap would be 1.0: a dropped scale passes 0.51
    assert condition.gap_ok(lq, lk, [3], 1, 1.0, min_gap=0.51).tolist() == [True]


def test_gap_ok_counts_only_the_eligible_candidates():
    # scores (3, 2.9995, 1): with all three eligible the k=1 gap is 5e-4 and
    # fails; with n_cand = 1 there is a single candidate and the row passes;
    # with n_cand = 2 the near-tie is visible again
    lq = np.array([[1.0], [1.0], [1.0]])
    lk = np.array([[3.0], [2.9995], [1.0]])
    assert condition.gap_ok(lq, lk, [3, 1, 2], 1, 1.0).tolist() == [False, True, False]
    # per-row candidate sets (3-D lk): row 0 sees (3, 1), row 1 sees (3, 2.9995)
    lk3 = np.array([[[3.0], [1.0]], [[3.0], [2.9995]]])
    assert condition.gap_ok(lq[:2], lk3, [2, 2], 1, 1.0).tolist() == [True, False]


def test_gap_ok_matches_a_full_sort_on_random_rows():
    rng = np.random.default_rng(7)
    # a coarse grid of 3-dimensional landmarks: exact ties at the cut are common
    n, m, dl, k = 64, 30, 3, 4
    lq = np.round(rng.standard_normal((n, dl)) * 2) / 2
    lk = np.round(rng.standard_normal((m, dl)) * 2) / 2
    n_cand = rng.integers(0, m + 1, size=n)
    ok = condition.gap_ok(lq, lk, n_cand, k, 0.25, min_gap=1e-3)
    for i in range(n):
        r = [0.25 * sum(float(a) * float(b) for a, b in zip(lq[i], lk[j]))
             for j in range(n_cand[i])]
        assert ok[i] == (_gap_by_sort(r, k) >= 1e-3), i
    assert 0 < ok.sum() < n  # both outcomes occur
