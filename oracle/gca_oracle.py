"""Plain float64 CPU oracle for Grouped Cross Attention (GCA).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module.  The GPU library never calls it and
shares no code with it.

What it computes follows "Efficient Length-Generalizable Attention via Causal
Retrieval for Long-Context Language Modeling" (Hu, Teng, Zhao, Wu, Tu; ICML 2025)
as stated on these pages:

* paperhub.cn review page, authors' reply "Cmt 1": with one group the causal
  relevance score of past chunk k for chunk t is the landmark inner product
  l_t . l_k / sqrt(d)  (Eq. 1).
* long-context-modeling README, "Model Architecture": the current chunk
  retrieves past chunks with the landmark of the chunk before it; after the
  top-k chunks are selected, every token attends to the tokens of each
  retrieved chunk separately (first stage, output O^i), and the softmax of the
  retrieval scores weights the sum of the O^i (second stage).
* paperlayer.ai summary, section 3.1: cross-attention is computed separately for
  the retrieved chunks and fused with softmax-normalised relevance scores.
* paperhub.cn review page, authors' replies to "Q4"/"Q1": an optional "softmax
  off-by-one" in Eq. 3 lets GCA down-weight every retrieved chunk.
* paperlayer.ai summary, appendix B: the hardware kernel returns the output and
  the log-sum-exp; its backward returns gradients for Q, K, V and the weights.

Readings of points the pages leave open (each also listed in the design notes):
* candidates of query chunk t are the past chunks j < q_pos[t] - 1 (the chunk
  right before t supplies the query landmark and is not a candidate);
* top-k picks by (score descending, chunk index ascending) and is stored in
  ascending chunk order; slots beyond the number of candidates are empty;
* the off-by-one form is w_i = e^{r_i} / (1 + sum_j e^{r_j}) over the selected
  chunks; it applies to the fusion weights only, never to the per-chunk token
  softmax;
* the attention scale is 1/sqrt(D); each retrieved chunk's S key rows are
  attended without a mask (they lie strictly in the past);
* the gradient to the scores treats the selection as fixed (top-k is piecewise
  constant in the scores).

Arrays follow the library's layout:
  q, o, dout : [G, B, H, Nq, S, D]      k, v : [G, B, H, Nk, S, D]
  lq : [G, B, H, Nq, Dl]                lk : [G, B, H, Nk, Dl]
  q_pos : [Nq]                           idx, score, w : [G, B, H, Nq, k]
  lse : [G, B, H, Nq, k, S]
Every floating input is converted to float64 first (exact for fp32 and bf16).
"""

import numpy as np

__all__ = [
    "candidate_count",
    "relevance_scores",
    "select_top_k",
    "fusion_weights",
    "retrieve",
    "retrieve_one",
    "chunk_attention",
    "forward",
    "forward_query_chunk",
    "backward",
    "backward_head",
]


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def candidate_count(q_pos, n_key):
    """Number of eligible past chunks of a query chunk at position q_pos.

    Chunk t scores with the landmark of chunk t-1 and may retrieve the chunks
    before that one (README "Model Architecture"; tiny-config reading j < t-1).
    """
    return int(max(0, min(int(q_pos) - 1, int(n_key))))


def relevance_scores(lq_row, lk_rows, score_scale):
    """Eq. 1: r_j = score_scale * <lq, lk_j> for every candidate row j."""
    return float(score_scale) * (_f64(lk_rows) @ _f64(lq_row))


def select_top_k(r, k):
    """Indices of the k best candidates, stored in ascending index order.

    "Best" orders by score descending, then index ascending.  Fewer than k
    candidates: all of them are kept.  The sort is numpy's stable lexsort.
    """
    r = _f64(r)
    n = r.shape[0]
    m = min(int(k), n)
    order = np.lexsort((np.arange(n), -r))
    return np.sort(order[:m])


def fusion_weights(r_sel, softmax_one):
    """Eq. 3 weights over the selected scores.

    vanilla:     w_i = e^{r_i} / sum_j e^{r_j}
    off-by-one:  w_i = e^{r_i} / (1 + sum_j e^{r_j})
    Both are evaluated after subtracting a shift M (max score; for the
    off-by-one form max(0, max score), so that the constant 1 becomes e^{-M}).
    """
    r_sel = _f64(r_sel)
    if r_sel.size == 0:
        return r_sel.copy()
    if softmax_one:
        shift = max(0.0, float(r_sel.max()))
        e = np.exp(r_sel - shift)
        return e / (np.exp(-shift) + e.sum())
    shift = float(r_sel.max())
    e = np.exp(r_sel - shift)
    return e / e.sum()


def retrieve_one(lq_row, lk_rows, q_pos, k, score_scale, softmax_one):
    """Retrieval for one (group, batch, head, query chunk).

    Returns (idx, score, w), each of length k; empty slots hold -1, 0, 0.
    """
    n = candidate_count(q_pos, lk_rows.shape[0])
    idx = np.full(k, -1, dtype=np.int64)
    score = np.zeros(k)
    w = np.zeros(k)
    if n == 0:
        return idx, score, w
    r = relevance_scores(lq_row, lk_rows[:n], score_scale)
    chosen = select_top_k(r, k)
    m = chosen.shape[0]
    idx[:m] = chosen
    score[:m] = r[chosen]
    w[:m] = fusion_weights(r[chosen], softmax_one)
    return idx, score, w


def retrieve(lq, lk, q_pos, k, score_scale, softmax_one, queries=None):
    """Top-k chunk retrieval and fusion weights for every query chunk.

    `queries` (optional) is a list of (g, b, h, q) tuples; only those rows are
    filled, the others keep their empty-slot values.
    """
    lq = _f64(lq)
    lk = _f64(lk)
    G, B, H, Nq, _ = lq.shape
    idx = np.full((G, B, H, Nq, k), -1, dtype=np.int64)
    score = np.zeros((G, B, H, Nq, k))
    w = np.zeros((G, B, H, Nq, k))
    if queries is None:
        queries = [(g, b, h, q) for g in range(G) for b in range(B)
                   for h in range(H) for q in range(Nq)]
    for (g, b, h, q) in queries:
        i_, s_, w_ = retrieve_one(lq[g, b, h, q], lk[g, b, h], q_pos[q], k,
                                  score_scale, softmax_one)
        idx[g, b, h, q] = i_
        score[g, b, h, q] = s_
        w[g, b, h, q] = w_
    return idx, score, w


def chunk_attention(q_tile, k_tile, v_tile, attn_scale):
    """Eq. 2 for one (query chunk, retrieved chunk) pair.

    Each query row attends to the S key rows of the retrieved chunk:
      s = attn_scale * Q K^T,  LSE = log sum_j exp(s_j),  O^i = softmax(s) V.
    Returns (O^i [S, D], LSE [S]).
    """
    s = float(attn_scale) * (_f64(q_tile) @ _f64(k_tile).T)
    m = s.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
    p = np.exp(s - lse[:, None])
    return p @ _f64(v_tile), lse


def _valid(c, n_key):
    return 0 <= int(c) < int(n_key)


def forward_query_chunk(q_tile, k_head, v_head, idx_row, w_row, attn_scale):
    """O for one query chunk: sum over valid slots of w_i * O^i (Eq. 3).

    Returns (O [S, D], LSE [k, S]); an empty slot has LSE = -inf and adds
    nothing, and a chunk with no valid slot has O = 0.
    """
    S, D = q_tile.shape
    kk = len(idx_row)
    o = np.zeros((S, D))
    lse = np.full((kk, S), -np.inf)
    for i in range(kk):
        c = int(idx_row[i])
        if not _valid(c, k_head.shape[0]):
            continue
        o_i, lse_i = chunk_attention(q_tile, k_head[c], v_head[c], attn_scale)
        o += float(w_row[i]) * o_i
        lse[i] = lse_i
    return o, lse


def forward(q, k, v, idx, w, attn_scale, queries=None):
    """GCA forward for every (or the listed) query chunk: (O, LSE)."""
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    G, B, H, Nq, S, D = q.shape
    kk = idx.shape[-1]
    o = np.zeros((G, B, H, Nq, S, D))
    lse = np.full((G, B, H, Nq, kk, S), -np.inf)
    if queries is None:
        queries = [(g, b, h, t) for g in range(G) for b in range(B)
                   for h in range(H) for t in range(Nq)]
    for (g, b, h, t) in queries:
        o[g, b, h, t], lse[g, b, h, t] = forward_query_chunk(
            q[g, b, h, t], k[g, b, h], v[g, b, h], idx[g, b, h, t],
            w[g, b, h, t], attn_scale)
    return o, lse


def backward_head(q, k, v, idx, w, dout, lq, lk, attn_scale, score_scale):
    """Gradients of one (group, batch, head) slice, written out directly.

    Inputs are the per-head slices: q, dout [Nq, S, D]; k, v [Nk, S, D];
    idx, w [Nq, k]; lq [Nq, Dl]; lk [Nk, Dl] (lq/lk may be None).

    With L a scalar loss and dO = dL/dO, for each query chunk t and valid slot i
    with retrieved chunk c (P = softmax of the pair's scores, O^i = P V_c):
      dw_i        = sum_x <dO[x], O^i[x]>                 (weight gradient)
      dV_c       += w_i P^T dO
      dP          = w_i dO V_c^T
      dS          = P * (dP - w_i * rowsum(dO * O^i))     (softmax backward)
      dQ_t       += attn_scale dS K_c
      dK_c       += attn_scale dS^T Q_t
    then through Eq. 3 (both weight forms share this Jacobian):
      dr_i        = w_i (dw_i - sum_l w_l dw_l)
    and through Eq. 1:
      dlq_t      += score_scale sum_i dr_i lk_c
      dlk_c      += score_scale dr_i lq_t
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    dout = _f64(dout)
    Nq, S, D = q.shape
    Nk = k.shape[0]
    kk = idx.shape[-1]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dw = np.zeros((Nq, kk))
    dr = np.zeros((Nq, kk))
    dlq = None if lq is None else np.zeros(np.shape(lq))
    dlk = None if lk is None else np.zeros(np.shape(lk))
    for t in range(Nq):
        valid = [i for i in range(kk) if _valid(idx[t, i], Nk)]
        for i in valid:
            c = int(idx[t, i])
            wi = float(w[t, i])
            s = attn_scale * (q[t] @ k[c].T)
            m = s.max(axis=1, keepdims=True)
            lse = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
            p = np.exp(s - lse[:, None])
            o_i = p @ v[c]
            dw[t, i] = float(np.sum(dout[t] * o_i))
            dv[c] += wi * (p.T @ dout[t])
            dp = wi * (dout[t] @ v[c].T)
            row = wi * np.sum(dout[t] * o_i, axis=1)
            ds = p * (dp - row[:, None])
            dq[t] += attn_scale * (ds @ k[c])
            dk[c] += attn_scale * (ds.T @ q[t])
        if valid:
            wv = np.array([float(w[t, i]) for i in valid])
            dwv = np.array([dw[t, i] for i in valid])
            drv = wv * (dwv - np.sum(wv * dwv))
            for n, i in enumerate(valid):
                dr[t, i] = drv[n]
                c = int(idx[t, i])
                if dlq is not None:
                    dlq[t] += score_scale * drv[n] * _f64(lk[c])
                if dlk is not None:
                    dlk[c] += score_scale * drv[n] * _f64(lq[t])
    return dict(dq=dq, dk=dk, dv=dv, dw=dw, dscore=dr, dlq=dlq, dlk=dlk)


def backward(q, k, v, idx, w, dout, lq, lk, attn_scale, score_scale, heads=None):
    """GCA backward for every (or the listed) (g, b, h) head.

    Returns a dict of float64 arrays dq, dk, dv [.., S, D], dw, dscore
    [.., k], dlq [.., Nq, Dl], dlk [.., Nk, Dl] in the full layout; heads not
    listed stay zero.
    """
    G, B, H, Nq, S, D = np.shape(q)
    Nk = np.shape(k)[3]
    kk = np.shape(idx)[-1]
    out = dict(
        dq=np.zeros((G, B, H, Nq, S, D)), dk=np.zeros((G, B, H, Nk, S, D)),
        dv=np.zeros((G, B, H, Nk, S, D)), dw=np.zeros((G, B, H, Nq, kk)),
        dscore=np.zeros((G, B, H, Nq, kk)),
        dlq=None if lq is None else np.zeros(np.shape(lq)),
        dlk=None if lk is None else np.zeros(np.shape(lk)))
    if heads is None:
        heads = [(g, b, h) for g in range(G) for b in range(B) for h in range(H)]
    for (g, b, h) in heads:
        r = backward_head(q[g, b, h], k[g, b, h], v[g, b, h], idx[g, b, h],
                          w[g, b, h], dout[g, b, h],
                          None if lq is None else lq[g, b, h],
                          None if lk is None else lk[g, b, h],
                          attn_scale, score_scale)
        for name in ("dq", "dk", "dv", "dw", "dscore"):
            out[name][g, b, h] = r[name]
        if lq is not None:
            out["dlq"][g, b, h] = r["dlq"]
        if lk is not None:
            out["dlk"][g, b, h] = r["dlk"]
    return out
