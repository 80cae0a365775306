"""Gather of the retrieved K/V tiles from offloaded memory, float64 CPU oracle.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module; the GPU library never calls it and
shares no code with it.

What it computes:

* paperlayer.ai summary, section 3.2 (Training & Inference): past chunk
  representations can be offloaded to CPU memory; the memory traffic this
  causes happens only when retrieval does (G times per S tokens).
* paperhub.cn review page, authors' reply "Q2": the offloaded GCA K/V is
  shared by the layers of a group, its size is set by batch, chunk count,
  chunk size, hidden size and groups, and a host link above 20 GB/s moves 8 GB
  in under 0.4 s.

Readings of points the pages leave open:

* Per retrieval, only the k selected chunks' K and V tiles of every query
  chunk travel to the GPU.  They are packed per query chunk: row t*k + i of the
  packed [G, B, H, Nq*k, S, D] arrays holds the tile of chunk idx[t, i]; an
  empty slot (idx outside [0, Nk)) gets a zero tile and packed index -1, else
  the packed index is t*k + i.
* Attention then runs on the packed arrays with the packed indices; it gives
  the same O and LSE as attention over the resident arrays with idx, because
  every slot sees the same tile and the same weight.
"""

import numpy as np

__all__ = ["gather_kv"]


def gather_kv(idx, k, v):
    """(k_packed, v_packed, idx_packed) of the retrieved tiles.

    idx : [G, B, H, Nq, kk] integer     k, v : [G, B, H, Nk, S, D]
    Returns k_packed, v_packed [G, B, H, Nq*kk, S, D] (dtype of k, v) and
    idx_packed [G, B, H, Nq, kk] int64.
    """
    idx = np.asarray(idx)
    k = np.asarray(k)
    v = np.asarray(v)
    G, B, H, Nq, kk = idx.shape
    Nk, S, D = k.shape[3], k.shape[4], k.shape[5]
    k_out = np.zeros((G, B, H, Nq * kk, S, D), dtype=k.dtype)
    v_out = np.zeros((G, B, H, Nq * kk, S, D), dtype=v.dtype)
    idx_out = np.full((G, B, H, Nq, kk), -1, dtype=np.int64)
    for g in range(G):
        for b in range(B):
            for h in range(H):
                for t in range(Nq):
                    for i in range(kk):
                        c = int(idx[g, b, h, t, i])
                        if 0 <= c < Nk:
                            row = t * kk + i
                            k_out[g, b, h, row] = k[g, b, h, c]
                            v_out[g, b, h, row] = v[g, b, h, c]
                            idx_out[g, b, h, t, i] = row
    return k_out, v_out, idx_out
