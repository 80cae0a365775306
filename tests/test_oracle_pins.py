"""Pins of the float64 oracle to facts that do not come from the oracle itself.

* a worked example derived by hand from the pages' definitions
  (tests/golden/worked_example.json);
* brute force: the top-k set is the unique k-subset with the largest score sum;
* a textbook reduction: one candidate and k=1 is ordinary cross-attention,
  checked against torch's scaled_dot_product_attention (CPU, float64);
* closed forms (Q = 0, one key row, equal scores, off-by-one with equal scores);
* invariances (permutation of the retrieved set, linearity in V, shift of keys);
* central finite differences of the whole retrieve + forward composition;
* gradient identities of the softmax and of the fusion weights.
Shapes deliberately use S != D != Dl so that a transposed operand fails.
"""

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth
from oracle import condition
from oracle import gca_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")
LN3 = math.log(3.0)


def _val(s):
    s = str(s)
    if s.endswith("*L"):
        return float(Fraction(s[:-2])) * LN3
    return float(Fraction(s))


def _arr(x):
    if isinstance(x, list):
        return np.array([_arr(e) for e in x], dtype=np.float64)
    return _val(x)


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _golden_inputs(g):
    inp = g["inputs"]
    ex = lambda a: _arr(a)[None, None, None]  # add G, B, H axes
    return dict(q=ex(inp["q"]), k=ex(inp["k"]), v=ex(inp["v"]),
                lq=ex(inp["lq"]), lk=ex(inp["lk"]), dout=ex(inp["dout"]),
                q_pos=np.array(inp["q_pos"]), score_scale=_val(inp["score_scale"]),
                attn_scale=_val(inp["attn_scale"]))


@pytest.mark.parametrize("case", range(4))
def test_worked_example(case):
    g = _golden()
    x = _golden_inputs(g)
    c = g["cases"][case]
    idx, score, w = orc.retrieve(x["lq"], x["lk"], x["q_pos"], c["k"],
                                 x["score_scale"], c["softmax_one"])
    assert idx[0, 0, 0].tolist() == c["idx"]
    np.testing.assert_allclose(score[0, 0, 0], _arr(c["score"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(w[0, 0, 0], _arr(c["w"]), rtol=0, atol=1e-14)
    o, lse = orc.forward(x["q"], x["k"], x["v"], idx, w, x["attn_scale"])
    np.testing.assert_allclose(o[0, 0, 0], _arr(c["o"]), rtol=0, atol=1e-13)
    if "lse_ln" in c:
        np.testing.assert_allclose(lse[0, 0, 0], np.log(_arr(c["lse_ln"])), atol=1e-14)
    if "dw" in c:
        gr = orc.backward(x["q"], x["k"], x["v"], idx, w, x["dout"], x["lq"], x["lk"],
                          x["attn_scale"], x["score_scale"])
        for name in ("dw", "dscore", "dv", "dq", "dk", "dlq", "dlk"):
            if name in c:
                np.testing.assert_allclose(gr[name][0, 0, 0], _arr(c[name]),
                                           rtol=0, atol=1e-13, err_msg=name)


def _random_case(seed, G=1, B=1, H=2, Nc=7, S=3, D=5, Dl=4, k=2, softmax_one=0,
                 min_gap=1e-3):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((G, B, H, Nc, S, D))
    kk = rng.standard_normal((G, B, H, Nc, S, D))
    v = rng.standard_normal((G, B, H, Nc, S, D))
    lq = rng.standard_normal((G, B, H, Nc, Dl))
    lk = rng.standard_normal((G, B, H, Nc, Dl))
    dout = rng.standard_normal((G, B, H, Nc, S, D))
    q_pos = np.arange(Nc)
    sc = 1.0 / math.sqrt(Dl)
    # redraw query landmarks until every query has a clear k-th gap
    for idx in itertools.product(range(G), range(B), range(H), range(Nc)):
        n = orc.candidate_count(q_pos[idx[3]], Nc)
        while not condition.gap_ok(lq[idx][None], lk[idx[:3]][:n], [n], k, sc, min_gap)[0]:
            lq[idx] = rng.standard_normal(Dl)
    return dict(q=q, k=kk, v=v, lq=lq, lk=lk, dout=dout, q_pos=q_pos, k_top=k,
                softmax_one=softmax_one, attn_scale=1.0 / math.sqrt(D), score_scale=sc)


def _loss(c, **over):
    x = dict(c)
    x.update(over)
    idx, _, w = orc.retrieve(x["lq"], x["lk"], x["q_pos"], x["k_top"], x["score_scale"],
                             x["softmax_one"])
    o, _ = orc.forward(x["q"], x["k"], x["v"], idx, w, x["attn_scale"])
    return float(np.sum(o * x["dout"]))


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_top_k_is_max_sum_subset(seed):
    rng = np.random.default_rng(100 + seed)
    Dl, Nk, k = 3, 9, 3
    lk = rng.standard_normal((Nk, Dl))
    for q_pos in range(0, Nk + 3):
        lq = rng.standard_normal(Dl)
        idx, score, w = orc.retrieve_one(lq, lk, q_pos, k, 0.5, 0)
        n = max(0, min(q_pos - 1, Nk))
        r = [0.5 * float(np.dot(lq, lk[j])) for j in range(n)]
        m = min(k, n)
        best = max(itertools.combinations(range(n), m), key=lambda s: sum(r[j] for j in s))
        assert idx[:m].tolist() == sorted(best)
        assert (idx[m:] == -1).all() and (w[m:] == 0).all() and (score[m:] == 0).all()
        assert all(j < q_pos - 1 for j in idx[:m])
        sel = set(best)
        if sel and len(sel) < n:
            assert min(r[j] for j in sel) >= max(r[j] for j in range(n) if j not in sel)


def test_tie_break_prefers_lower_index():
    lk = np.ones((6, 2))
    idx, score, w = orc.retrieve_one(np.array([1.0, 2.0]), lk, 10, 3, 1.0, 0)
    assert idx.tolist() == [0, 1, 2]
    np.testing.assert_allclose(w, [1 / 3] * 3, atol=1e-15)


def test_tiny_config_candidate_rule():
    # tiny fp32 workload text: chunk t >= 2 retrieves top-min(2, t-1) among j < t-1
    x = synth.training_inputs("tiny_fp32")
    cfg = x["cfg"]
    idx, _, w = orc.retrieve(x["lq"].double().numpy(), x["lk"].double().numpy(),
                             x["q_pos"].numpy(), cfg["k"], cfg["score_scale"], 0)
    for t in range(cfg["n_query"]):
        n_valid = (idx[..., t, :] >= 0).sum(axis=-1)
        assert (n_valid == (min(2, t - 1) if t >= 2 else 0)).all()
        assert (idx[..., t, :][idx[..., t, :] >= 0] < t - 1).all()
        np.testing.assert_allclose(w[..., t, :].sum(-1), 1.0 if t >= 2 else 0.0, atol=1e-14)


def test_planted_needle_is_ranked_first():
    lk = synth.context_landmarks("infer1m_step", n_key=2048, H=3)
    qb = synth.query_batch("infer1m_step", lk, step=3, n_key=2048, H=3, n_query=4,
                           q_pos=2049)
    cfg = qb["cfg"]
    idx, score, _ = orc.retrieve(qb["lq"].double().numpy(), lk.double().numpy(),
                                 qb["q_pos"].numpy(), cfg["k"], cfg["score_scale"], 0)
    for h in range(3):
        for n in range(4):
            best = idx[0, 0, h, n][np.argmax(score[0, 0, h, n])]
            assert best == int(qb["needle"][n])


@pytest.mark.parametrize("kk", [1, 4])
@pytest.mark.parametrize("softmax_one", [0, 1])
def test_single_candidate_is_cross_attention(kk, softmax_one):
    rng = np.random.default_rng(7)
    S, D, Dl = 5, 6, 3
    q = rng.standard_normal((1, 1, 1, 1, S, D))
    k = rng.standard_normal((1, 1, 1, 1, S, D))
    v = rng.standard_normal((1, 1, 1, 1, S, D))
    lq = rng.standard_normal((1, 1, 1, 1, Dl))
    lk = rng.standard_normal((1, 1, 1, 1, Dl))
    scale = 0.37
    idx, score, w = orc.retrieve(lq, lk, np.array([2]), kk, 0.5, softmax_one)
    o, lse = orc.forward(q, k, v, idx, w, scale)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q[0, 0, 0, 0])[None], torch.from_numpy(k[0, 0, 0, 0])[None],
        torch.from_numpy(v[0, 0, 0, 0])[None], scale=scale)[0].numpy()
    r = 0.5 * float(lq[0, 0, 0, 0] @ lk[0, 0, 0, 0])
    factor = math.exp(r) / (1.0 + math.exp(r)) if softmax_one else 1.0
    np.testing.assert_allclose(o[0, 0, 0, 0], factor * ref, rtol=1e-13, atol=1e-13)
    s = scale * q[0, 0, 0, 0] @ k[0, 0, 0, 0].T
    np.testing.assert_allclose(lse[0, 0, 0, 0, 0],
                               np.log(np.sum(np.exp(s), axis=1)), rtol=1e-13)


def test_closed_forms():
    rng = np.random.default_rng(11)
    S, D = 4, 3
    k = rng.standard_normal((S, D))
    v = rng.standard_normal((S, D))
    o, lse = orc.chunk_attention(np.zeros((S, D)), k, v, 0.9)
    np.testing.assert_allclose(o, np.tile(v.mean(axis=0), (S, 1)), atol=1e-15)
    np.testing.assert_allclose(lse, math.log(S), atol=1e-15)
    o1, _ = orc.chunk_attention(rng.standard_normal((2, D)), k[:1], v[:1], 0.9)
    np.testing.assert_allclose(o1, np.tile(v[0], (2, 1)), atol=1e-15)
    # a constant vector added to every key row of a chunk changes nothing
    qt = rng.standard_normal((S, D))
    oa, _ = orc.chunk_attention(qt, k, v, 0.9)
    ob, _ = orc.chunk_attention(qt, k + rng.standard_normal(D), v, 0.9)
    np.testing.assert_allclose(oa, ob, atol=1e-13)


@pytest.mark.parametrize("softmax_one", [0, 1])
def test_equal_scores_give_mean(softmax_one):
    rng = np.random.default_rng(5)
    S, D, Nk, kk = 3, 4, 6, 4
    q = rng.standard_normal((1, 1, 1, 1, S, D))
    k = rng.standard_normal((1, 1, 1, Nk, S, D))
    v = rng.standard_normal((1, 1, 1, Nk, S, D))
    lq = np.array([[[[[0.3, -0.2]]]]])
    lk = np.tile(np.array([0.5, 1.5]), (1, 1, 1, Nk, 1))
    idx, score, w = orc.retrieve(lq, lk, np.array([Nk + 1]), kk, 1.0, softmax_one)
    assert idx[0, 0, 0, 0].tolist() == [0, 1, 2, 3]
    r = 0.3 * 0.5 - 0.2 * 1.5
    o, _ = orc.forward(q, k, v, idx, w, 0.5)
    per = [orc.chunk_attention(q[0, 0, 0, 0], k[0, 0, 0, c], v[0, 0, 0, c], 0.5)[0]
           for c in range(kk)]
    if softmax_one:
        expect = math.exp(r) / (1.0 + kk * math.exp(r)) * np.sum(per, axis=0)
        assert w[0, 0, 0, 0].sum() < 1.0
    else:
        expect = np.mean(per, axis=0)
        np.testing.assert_allclose(w.sum(), 1.0, atol=1e-15)
    np.testing.assert_allclose(o[0, 0, 0, 0], expect, atol=1e-13)


def test_off_by_one_vanishes_for_very_negative_scores():
    w = orc.fusion_weights(np.array([-60.0, -61.0, -59.5]), 1)
    assert w.sum() < 1e-25
    w0 = orc.fusion_weights(np.array([-60.0, -61.0, -59.5]), 0)
    np.testing.assert_allclose(w0.sum(), 1.0, atol=1e-15)


def test_permutation_invariance_and_linearity():
    c = _random_case(3, Nc=8, k=3)
    idx, _, w = orc.retrieve(c["lq"], c["lk"], c["q_pos"], 3, c["score_scale"], 0)
    o, lse = orc.forward(c["q"], c["k"], c["v"], idx, w, c["attn_scale"])
    perm = np.array([2, 0, 1])
    op, lsep = orc.forward(c["q"], c["k"], c["v"], idx[..., perm], w[..., perm],
                           c["attn_scale"])
    np.testing.assert_allclose(o, op, atol=1e-13)
    np.testing.assert_allclose(lse[..., perm, :], lsep, atol=1e-13)
    o2, _ = orc.forward(c["q"], c["k"], 2.0 * c["v"] - 1.0, idx, w, c["attn_scale"])
    o1, _ = orc.forward(c["q"], c["k"], np.ones_like(c["v"]), idx, w, c["attn_scale"])
    np.testing.assert_allclose(o2, 2.0 * o - o1, atol=1e-12)


@pytest.mark.parametrize("softmax_one", [0, 1])
def test_finite_differences(softmax_one):
    c = _random_case(17 + softmax_one, k=2, softmax_one=softmax_one)
    idx, score, w = orc.retrieve(c["lq"], c["lk"], c["q_pos"], 2, c["score_scale"],
                                 softmax_one)
    gr = orc.backward(c["q"], c["k"], c["v"], idx, w, c["dout"], c["lq"], c["lk"],
                      c["attn_scale"], c["score_scale"])
    h = 1e-6
    for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("lq", "dlq"),
                        ("lk", "dlk")):
        base = c[name]
        fd = np.zeros_like(base)
        for pos in itertools.product(*[range(n) for n in base.shape]):
            xp = base.copy()
            xp[pos] += h
            xm = base.copy()
            xm[pos] -= h
            fd[pos] = (_loss(c, **{name: xp}) - _loss(c, **{name: xm})) / (2 * h)
        np.testing.assert_allclose(gr[gname], fd, rtol=0, atol=2e-8, err_msg=gname)
    # weights as an input of the forward: dL/dw_i
    fdw = np.zeros_like(w)
    for pos in zip(*np.nonzero(idx >= 0)):
        wp = w.copy()
        wp[pos] += h
        wm = w.copy()
        wm[pos] -= h
        fp = np.sum(orc.forward(c["q"], c["k"], c["v"], idx, wp, c["attn_scale"])[0] * c["dout"])
        fm = np.sum(orc.forward(c["q"], c["k"], c["v"], idx, wm, c["attn_scale"])[0] * c["dout"])
        fdw[pos] = (fp - fm) / (2 * h)
    np.testing.assert_allclose(gr["dw"], fdw, rtol=0, atol=2e-8)
    # selected scores through the fusion weights: dL/dr_i
    fdr = np.zeros_like(w)
    for pos in zip(*np.nonzero(idx >= 0)):
        g, b, hh, t, _ = pos
        m = int((idx[g, b, hh, t] >= 0).sum())
        for sgn in (1, -1):
            r = score[g, b, hh, t, :m].copy()
            r[pos[4]] += sgn * h
            wn = w.copy()
            wn[g, b, hh, t, :m] = orc.fusion_weights(r, softmax_one)
            val = np.sum(orc.forward(c["q"], c["k"], c["v"], idx, wn, c["attn_scale"])[0]
                         * c["dout"])
            fdr[pos] += sgn * val / (2 * h)
    np.testing.assert_allclose(gr["dscore"], fdr, rtol=0, atol=2e-8)


@pytest.mark.parametrize("softmax_one", [0, 1])
def test_gradient_identities(softmax_one):
    c = _random_case(29, Nc=9, k=3, softmax_one=softmax_one)
    idx, _, w = orc.retrieve(c["lq"], c["lk"], c["q_pos"], 3, c["score_scale"], softmax_one)
    gr = orc.backward(c["q"], c["k"], c["v"], idx, w, c["dout"], c["lq"], c["lk"],
                      c["attn_scale"], c["score_scale"])
    dr_sum = gr["dscore"].sum(-1)
    if softmax_one:
        expect = (1.0 - w.sum(-1)) * (w * gr["dw"]).sum(-1)
        np.testing.assert_allclose(dr_sum, expect, atol=1e-12)
    else:
        np.testing.assert_allclose(dr_sum, 0.0, atol=1e-12)
    # per key chunk the key-row gradients sum to zero (softmax shift invariance)
    np.testing.assert_allclose(gr["dk"].sum(axis=-2), 0.0, atol=1e-12)
    # value-row gradients sum to the weighted upstream gradients that reach the chunk
    G, B, H, Nc, S, D = c["q"].shape
    expect = np.zeros((G, B, H, Nc, D))
    for g, b, h, t, i in itertools.product(range(G), range(B), range(H), range(Nc), range(3)):
        cc = idx[g, b, h, t, i]
        if cc >= 0:
            expect[g, b, h, cc] += w[g, b, h, t, i] * c["dout"][g, b, h, t].sum(axis=0)
    np.testing.assert_allclose(gr["dv"].sum(axis=-2), expect, atol=1e-12)


def test_one_slot_vanilla_has_no_score_gradient():
    c = _random_case(31, Nc=6, k=1)
    idx, _, w = orc.retrieve(c["lq"], c["lk"], c["q_pos"], 1, c["score_scale"], 0)
    gr = orc.backward(c["q"], c["k"], c["v"], idx, w, c["dout"], c["lq"], c["lk"],
                      c["attn_scale"], c["score_scale"])
    assert np.abs(gr["dscore"]).max() == 0.0
    assert np.abs(gr["dlq"]).max() == 0.0 and np.abs(gr["dlk"]).max() == 0.0


def test_out_of_range_slots_are_empty():
    c = _random_case(37, Nc=6, k=2)
    idx, _, w = orc.retrieve(c["lq"], c["lk"], c["q_pos"], 2, c["score_scale"], 0)
    bad = idx.copy()
    bad[..., 1] = np.where(bad[..., 1] >= 0, 99, -1)
    o, lse = orc.forward(c["q"], c["k"], c["v"], bad, w, c["attn_scale"])
    o1, _ = orc.forward(c["q"], c["k"], c["v"], np.where(bad == 99, -1, bad), w,
                        c["attn_scale"])
    np.testing.assert_allclose(o, o1, atol=0)
    assert np.isneginf(lse[..., 1, :][bad[..., 1] == 99]).all()
