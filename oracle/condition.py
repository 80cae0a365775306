"""Tie-avoidance rule for seeded GCA inputs (test infrastructure only).

Top-k indices are compared bit-exactly between the GPU library and the oracle,
so no query may have two candidates that tie, up to rounding, at the k-th place.
The rule keeps a draw only if, in float64 on the exact stored values, the k-th
best relevance score (Eq. 1: score_scale * <lq, lk>, paperhub.cn review page,
authors' reply "Cmt 1") beats the (k+1)-th best by at least `min_gap`.
Queries with at most k candidates always pass.

The input generator calls `gap_ok` through a callback; it never imports this
module itself.
"""

import numpy as np

__all__ = ["gap_ok", "kth_gap"]


def kth_gap(r, k):
    """r[k-1] - r[k] of the scores sorted descending (inf if len(r) <= k)."""
    r = np.asarray(r, dtype=np.float64)
    if r.shape[0] <= k:
        return np.inf
    top = -np.partition(-r, k)[: k + 1]
    top = np.sort(top)[::-1]
    return float(top[k - 1] - top[k])


def gap_ok(lq_rows, lk_rows, n_cand, k, score_scale, min_gap=1e-3):
    """Vector of booleans, one per query row.

    lq_rows : [n, Dl] query landmarks (any float dtype, upcast to float64)
    lk_rows : [n, m, Dl] candidate landmarks seen by each query, or [m, Dl]
              shared by all of them
    n_cand  : [n] number of eligible candidates (the first n_cand[i] rows)
    """
    lq_rows = np.asarray(lq_rows, dtype=np.float64)
    lk_rows = np.asarray(lk_rows, dtype=np.float64)
    n_cand = np.broadcast_to(np.asarray(n_cand, dtype=np.int64), (lq_rows.shape[0],))
    if lk_rows.ndim == 2:
        scores = float(score_scale) * (lq_rows @ lk_rows.T)
    else:
        scores = float(score_scale) * np.einsum("nd,nmd->nm", lq_rows, lk_rows)
    ok = np.ones(lq_rows.shape[0], dtype=bool)
    for i in range(lq_rows.shape[0]):
        ok[i] = kth_gap(scores[i, : n_cand[i]], k) >= min_gap
    return ok
