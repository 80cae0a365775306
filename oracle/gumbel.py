"""Gumbel top-k retrieval, float64 CPU oracle.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module; the GPU library never calls it and
shares no code with it.

What it computes:

* paperlayer.ai summary, section 3.2 (Training & Inference): while training,
  Gumbel noise is added to the relevance scores before the top-k selection, so
  that lower-scoring chunks are still retrieved now and then while higher
  scores stay more likely.  Section 5 of the same summary credits Gumbel top-k
  sampling for pre-training up to 64K tokens.
* The scores are Eq. 1's r_j (paperhub.cn review page, authors' reply "Cmt 1");
  the fusion weights are Eq. 3's softmax (or softmax off-by-one) over the
  selected chunks, exactly as in the noise-free retrieval.

Readings of points the pages leave open:

* The noise is standard Gumbel, G = -ln(-ln U) with U uniform on (0, 1), added
  at unit temperature to the scaled score r_j (so that, for k = 1, chunk j is
  picked with probability softmax(r)_j, and for larger k the selection is a
  draw without replacement from softmax(r)).
* The noise decides the selection only: the reported scores and the fusion
  weights use the clean r of the selected chunks, so the gradient of the
  weights reaches r as in the noise-free path.  Ties among perturbed scores go
  to the lower chunk index; the selection is stored in ascending chunk order.
* Noise values are reproducible from a 64-bit seed with the counter-based
  generator Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
  numbers: as easy as 1, 2, 3", SC 2011).  The candidate (head, q, j) uses
  counter (j >> 2, q, head, 0), key (seed mod 2^32, seed >> 32) and output word
  j mod 4, where head = (g * B + b) * H + h.  U is built from the word's top
  23 bits m as U = (m + 1/2) / 2^23: strictly inside (0, 1) and exactly
  representable in float32.
"""

import math

import numpy as np

from .gca_oracle import candidate_count, fusion_weights, relevance_scores

__all__ = ["philox4x32_10", "uniform_from_word", "gumbel_from_uniform",
           "gumbel_noise", "perturbed_scores", "retrieve_gumbel_one",
           "retrieve_gumbel"]

_MASK = np.uint64(0xFFFFFFFF)
# Philox4x32 round multipliers and Weyl key increments (Salmon et al. 2011).
_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = np.uint64(0x9E3779B9)
_W1 = np.uint64(0xBB67AE85)


def philox4x32_10(counter, key):
    """Philox4x32 with 10 rounds.

    counter : integer array [..., 4] (32-bit words); key : [..., 2].
    Each round multiplies words 0 and 2 by the two round constants, taking
    the 64-bit products apart into high and low halves; the new words are
    (hi(M1 x2) ^ x1 ^ k0, lo(M1 x2), hi(M0 x0) ^ x3 ^ k1, lo(M0 x0)).  The key
    advances by the Weyl increments between rounds.  Returns uint64 words
    holding 32-bit values, shape [..., 4].
    """
    c = np.asarray(counter, dtype=np.uint64) & _MASK
    k = np.asarray(key, dtype=np.uint64) & _MASK
    x0, x1, x2, x3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
    k0, k1 = k[..., 0], k[..., 1]
    for rnd in range(10):
        if rnd:
            k0 = (k0 + _W0) & _MASK
            k1 = (k1 + _W1) & _MASK
        p0 = _M0 * x0  # < 2^64: no wrap-around
        p1 = _M1 * x2
        x0, x1, x2, x3 = ((p1 >> np.uint64(32)) ^ x1 ^ k0, p1 & _MASK,
                          (p0 >> np.uint64(32)) ^ x3 ^ k1, p0 & _MASK)
    return np.stack([x0, x1, x2, x3], axis=-1)


def uniform_from_word(word):
    """U = (m + 1/2) / 2^23 with m the top 23 bits of a 32-bit word."""
    m = (np.asarray(word, dtype=np.uint64) >> np.uint64(9)).astype(np.float64)
    return (m + 0.5) / float(1 << 23)


def gumbel_from_uniform(u):
    """Standard Gumbel variate G = -ln(-ln U)."""
    u = np.asarray(u, dtype=np.float64)
    return -np.log(-np.log(u))


def gumbel_noise(seed, head, q, j):
    """Noise of candidates j (array) of query q of linear head `head`."""
    j = np.asarray(j, dtype=np.int64)
    seed = int(seed)
    ctr = np.zeros(j.shape + (4,), dtype=np.uint64)
    ctr[..., 0] = (j >> 2).astype(np.uint64)
    ctr[..., 1] = np.uint64(int(q))
    ctr[..., 2] = np.uint64(int(head))
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], dtype=np.uint64)
    words = philox4x32_10(ctr, np.broadcast_to(key, j.shape + (2,)))
    w = np.take_along_axis(words, (j & 3)[..., None].astype(np.int64), axis=-1)[..., 0]
    return gumbel_from_uniform(uniform_from_word(w))


def perturbed_scores(lq_row, lk_rows, q_pos, score_scale, seed, head, q):
    """(clean r, perturbed r + G) over the eligible candidates of one query."""
    n = candidate_count(q_pos, np.asarray(lk_rows).shape[0])
    if n == 0:
        return np.zeros(0), np.zeros(0)
    r = relevance_scores(lq_row, np.asarray(lk_rows)[:n], score_scale)
    return r, r + gumbel_noise(seed, head, q, np.arange(n))


def retrieve_gumbel_one(lq_row, lk_rows, q_pos, k, score_scale, softmax_one, seed,
                        head, q):
    """Gumbel top-k retrieval for one query: (idx, score, w), each of length k.

    Selection orders by perturbed score descending, then chunk index
    ascending; score and w use the clean r of the selected chunks.
    """
    idx = np.full(k, -1, dtype=np.int64)
    score = np.zeros(k)
    w = np.zeros(k)
    r, p = perturbed_scores(lq_row, lk_rows, q_pos, score_scale, seed, head, q)
    n = r.shape[0]
    if n == 0:
        return idx, score, w
    order = np.lexsort((np.arange(n), -p))
    chosen = np.sort(order[: min(int(k), n)])
    m = chosen.shape[0]
    idx[:m] = chosen
    score[:m] = r[chosen]
    w[:m] = fusion_weights(r[chosen], softmax_one)
    return idx, score, w


def retrieve_gumbel(lq, lk, q_pos, k, score_scale, softmax_one, seed, queries=None):
    """Gumbel top-k retrieval for every (or the listed (g, b, h, q)) query."""
    lq = np.asarray(lq, dtype=np.float64)
    lk = np.asarray(lk, dtype=np.float64)
    G, B, H, Nq, _ = lq.shape
    idx = np.full((G, B, H, Nq, k), -1, dtype=np.int64)
    score = np.zeros((G, B, H, Nq, k))
    w = np.zeros((G, B, H, Nq, k))
    if queries is None:
        queries = [(g, b, h, q) for g in range(G) for b in range(B)
                   for h in range(H) for q in range(Nq)]
    for (g, b, h, q) in queries:
        head = (g * B + b) * H + h
        i_, s_, w_ = retrieve_gumbel_one(lq[g, b, h, q], lk[g, b, h], q_pos[q], k,
                                         score_scale, softmax_one, seed, head, q)
        idx[g, b, h, q] = i_
        score[g, b, h, q] = s_
        w[g, b, h, q] = w_
    return idx, score, w


# Range of the noise on the lattice above: the extreme uniforms 2^-24 and
# 1 - 2^-24 bound G from both sides.
GUMBEL_MIN = -math.log(-math.log(0.5 / float(1 << 23)))
GUMBEL_MAX = -math.log(-math.log1p(-0.5 / float(1 << 23)))
