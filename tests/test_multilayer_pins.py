"""Multi-layer reuse of one retrieval within a group, on the oracle.

paperlayer.ai summary, section 3.1: the retrieved chunks' representations are
shared across the upper layers of a group, with shared key and value
transformations; paperhub.cn, authors' reply "Q2": the GCA K/V is shared
within a group.  Reading: one retrieval (idx, w from lq, lk) and one K/V serve
every upper layer l of the group, each with its own queries Q_l and output
O_l; the gradients of the shared tensors (K, V, the scores and the
landmarks) are the sums of the per-layer gradients.  Pinned here by central
finite differences of the composite loss sum_l <dO_l, O_l> through the whole
retrieval + L-layer forward.
"""

import numpy as np

from oracle import gca_oracle as orc


def _composite(q_layers, k, v, lq, lk, q_pos, kk, s_attn, s_score, soft1, douts):
    idx, _, w = orc.retrieve(lq, lk, q_pos, kk, s_score, soft1)
    total = 0.0
    for q, do in zip(q_layers, douts):
        o, _ = orc.forward(q, k, v, idx, w, s_attn)
        total += float((o * do).sum())
    return total


def test_group_gradients_are_sums_over_layers():
    rng = np.random.default_rng(12)
    G, B, H, Nq, Nk, S, D, Dl, kk, L = 1, 1, 1, 6, 6, 3, 4, 5, 2, 3
    q_layers = [rng.standard_normal((G, B, H, Nq, S, D)) for _ in range(L)]
    douts = [rng.standard_normal((G, B, H, Nq, S, D)) for _ in range(L)]
    k = rng.standard_normal((G, B, H, Nk, S, D))
    v = rng.standard_normal((G, B, H, Nk, S, D))
    lq = rng.standard_normal((G, B, H, Nq, Dl))
    lk = rng.standard_normal((G, B, H, Nk, Dl))
    q_pos = np.arange(Nq)
    s_attn, s_score = 0.5, 0.45
    for soft1 in (0, 1):
        idx, _, w = orc.retrieve(lq, lk, q_pos, kk, s_score, soft1)
        sums = {n: 0.0 for n in ("dk", "dv", "dlq", "dlk")}
        per_layer_dq = []
        for q, do in zip(q_layers, douts):
            g = orc.backward(q, k, v, idx, w, do, lq, lk, s_attn, s_score)
            for n in sums:
                sums[n] = sums[n] + g[n]
            per_layer_dq.append(g["dq"])
        f = lambda **over: _composite(over.get("q_layers", q_layers), over.get("k", k),
                                      over.get("v", v), over.get("lq", lq), over.get("lk", lk),
                                      q_pos, kk, s_attn, s_score, soft1, douts)
        h = 1e-6
        for name, arr, grad in (("k", k, sums["dk"]), ("v", v, sums["dv"]),
                                ("lq", lq, sums["dlq"]), ("lk", lk, sums["dlk"])):
            for pos in [tuple(rng.integers(0, n) for n in arr.shape) for _ in range(6)]:
                up, dn = arr.copy(), arr.copy()
                up[pos] += h
                dn[pos] -= h
                fd = (f(**{name: up}) - f(**{name: dn})) / (2 * h)
                assert abs(fd - grad[pos]) < 1e-6, (soft1, name, pos, fd, grad[pos])
        # each layer's queries get that layer's own dQ
        for l in range(L):
            pos = (0, 0, 0, 4, 1, 2)
            up = [q.copy() for q in q_layers]
            dn = [q.copy() for q in q_layers]
            up[l][pos] += h
            dn[l][pos] -= h
            fd = (f(q_layers=up) - f(q_layers=dn)) / (2 * h)
            assert abs(fd - per_layer_dq[l][pos]) < 1e-6
