"""Sliding-window self-attention, float64 CPU oracle.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module; the GPU library never calls it and
shares no code with it.

What it computes:

* paperlayer.ai summary, section 1 and section 3.2: every DRT layer combines
  GCA over the top-k past chunks with fixed-size sliding-window
  self-attention, which keeps the cost of the sequence linear; section 4.1.2:
  the window is 512 tokens.

Readings of points the pages leave open:

* The window is causal and holds the token itself: token x attends to the
  keys y with x - W < y <= x (at most W keys), W = 512.
* Plain softmax attention inside the window, scale 1/sqrt(D) by default; the
  per-row log-sum-exp L is an output, as for GCA's attention, so the
  backward can recompute the probabilities.
* Backward: with P the window softmax and dO = dL/dO,
      dV = P^T dO,   dP = dO V^T,   dS = P * (dP - rowsum(dO * O)),
      dQ = scale * dS K,   dK = scale * dS^T Q.
Arrays: q, k, v, o, dout [B, H, T, D]; lse [B, H, T].
"""

import numpy as np

__all__ = ["window_mask", "swa_forward", "swa_backward", "swa_query_rows",
           "swa_key_rows"]


def window_mask(T, window):
    """Boolean [T, T]: True where query x may attend key y (x - W < y <= x)."""
    x = np.arange(T)[:, None]
    y = np.arange(T)[None, :]
    return (y <= x) & (y > x - int(window))


def _head_scores(q, k, window, scale):
    s = float(scale) * (q @ k.T)
    return np.where(window_mask(q.shape[0], window), s, -np.inf)


def swa_forward(q, k, v, window, scale):
    """(O [B, H, T, D], LSE [B, H, T]) of causal sliding-window attention."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, T, D = q.shape
    o = np.zeros((B, H, T, D))
    lse = np.zeros((B, H, T))
    for b in range(B):
        for h in range(H):
            s = _head_scores(q[b, h], k[b, h], window, scale)
            m = s.max(axis=1, keepdims=True)
            l = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
            p = np.exp(s - l[:, None])
            o[b, h] = p @ v[b, h]
            lse[b, h] = l
    return o, lse


def swa_backward(q, k, v, dout, window, scale):
    """(dQ, dK, dV), each [B, H, T, D], of causal sliding-window attention."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, H, T, D = q.shape
    dq = np.zeros((B, H, T, D))
    dk = np.zeros((B, H, T, D))
    dv = np.zeros((B, H, T, D))
    for b in range(B):
        for h in range(H):
            s = _head_scores(q[b, h], k[b, h], window, scale)
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            p /= p.sum(axis=1, keepdims=True)
            o = p @ v[b, h]
            dv[b, h] = p.T @ dout[b, h]
            dp = dout[b, h] @ v[b, h].T
            delta = (dout[b, h] * o).sum(axis=1, keepdims=True)
            ds = p * (dp - delta)
            dq[b, h] = float(scale) * (ds @ k[b, h])
            dk[b, h] = float(scale) * (ds.T @ q[b, h])
    return dq, dk, dv


def _row(q, k, v, x, window, scale):
    """P row, O row and LSE of query x of one head (keys max(0, x-W+1) .. x)."""
    lo = max(0, x - int(window) + 1)
    s = float(scale) * (k[lo:x + 1] @ q[x])
    m = s.max()
    l = m + np.log(np.exp(s - m).sum())
    p = np.exp(s - l)
    return lo, p, p @ v[lo:x + 1], l


def swa_query_rows(q, k, v, dout, window, scale, b, h, xs):
    """For the listed query rows x of head (b, h): O[x], LSE[x] and dQ[x],
    each computed from that row's own window alone (for spot checks of
    long sequences)."""
    q = np.asarray(q[b, h], dtype=np.float64)
    k = np.asarray(k[b, h], dtype=np.float64)
    v = np.asarray(v[b, h], dtype=np.float64)
    do = None if dout is None else np.asarray(dout[b, h], dtype=np.float64)
    o_rows, lse_rows, dq_rows = [], [], []
    for x in xs:
        lo, p, o_x, l = _row(q, k, v, x, window, scale)
        o_rows.append(o_x)
        lse_rows.append(l)
        if do is not None:
            dp = v[lo:x + 1] @ do[x]
            ds = p * (dp - do[x] @ o_x)
            dq_rows.append(float(scale) * (ds @ k[lo:x + 1]))
    return np.array(o_rows), np.array(lse_rows), (np.array(dq_rows) if do is not None else None)


def swa_key_rows(q, k, v, dout, window, scale, b, h, ys):
    """dK[y] and dV[y] of head (b, h) for the listed key rows y, summed over the
    queries x in [y, y + W - 1] that see them."""
    q = np.asarray(q[b, h], dtype=np.float64)
    k = np.asarray(k[b, h], dtype=np.float64)
    v = np.asarray(v[b, h], dtype=np.float64)
    do = np.asarray(dout[b, h], dtype=np.float64)
    T = q.shape[0]
    dk_rows, dv_rows = [], []
    for y in ys:
        dk_y = np.zeros(q.shape[1])
        dv_y = np.zeros(v.shape[1])
        for x in range(y, min(T, y + int(window))):
            lo, p, o_x, _ = _row(q, k, v, x, window, scale)
            p_xy = p[y - lo]
            dv_y += p_xy * do[x]
            ds_xy = p_xy * (v[y] @ do[x] - do[x] @ o_x)
            dk_y += float(scale) * ds_xy * q[x]
        dk_rows.append(dk_y)
        dv_rows.append(dv_y)
    return np.array(dk_rows), np.array(dv_rows)
