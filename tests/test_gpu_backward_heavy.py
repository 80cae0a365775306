"""GPU parity of the backward where one key chunk is retrieved by (almost) every
query chunk, at more than 512 chunks per head.

Training at 64K tokens (paperlayer.ai summary, section 5: Gumbel top-k
pre-training up to 64K tokens) gives 1024 chunks per head, and a chunk that
every later query chunk finds relevant (a needle) collects up to n_query
retrievals.  Here 640 query and key chunks per head, off-by-one weights, and in
each head one planted chunk c* whose landmark lies along a direction every
query landmark shares: it is in the top-8 of every query chunk t >= c* + 2, so
its reverse list holds over 600 entries (the key-side kernel walks it in three
blocks of at most 256), and the reverse index counts 640 key chunks in two
passes of 512.  Every output is compared element by element with the float64
oracle, and a second backward must repeat the first bit for bit.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import condition
from oracle import gca_oracle as orc
from gpu_common import (close, compare_lse, dev, f64, require_gpu, run_backward, run_forward,
                        run_retrieve, shape_of)

pytestmark = pytest.mark.gpu

NEEDLE = 3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def heavy_inputs(n, H, seed):
    """bf16 inputs of a 2-head, n-chunk training problem with a planted chunk that
    every query chunk t >= NEEDLE + 2 retrieves, and a >= 1e-3 gap at the k-th
    score of every query (rejected query landmarks are redrawn)."""
    cfg = synth.workload("train16k_fwdbwd_g2", G=1, B=1, H=H, n_query=n, n_key=n)
    x = synth.training_inputs("train16k_fwdbwd_g2", G=1, B=1, H=H, n_query=n, n_key=n,
                              seed=seed)
    rng = np.random.default_rng(seed + 1)
    dl, k = cfg["Dl"], cfg["k"]
    lq = x["lq"].float().numpy()
    lk = x["lk"].float().numpy()
    for h in range(H):
        u = rng.standard_normal(dl)
        u /= np.linalg.norm(u)
        lk[0, 0, h, NEEDLE] = 8.0 * u
        lq[0, 0, h] += 0.5 * u  # every query landmark leans towards the needle
    lq_t = torch.from_numpy(lq.astype(np.float32)).bfloat16()
    lk_t = torch.from_numpy(lk.astype(np.float32)).bfloat16()
    lk64 = f64(lk_t)
    for h in range(H):
        u = lk64[0, 0, h, NEEDLE] / np.linalg.norm(lk64[0, 0, h, NEEDLE])
        todo = np.arange(k + 2, n)
        while todo.size:
            ok = condition.gap_ok(f64(lq_t)[0, 0, h, todo], lk64[0, 0, h], todo - 1, k,
                                  cfg["score_scale"], 1e-3)
            for t in todo[~ok]:
                new = rng.standard_normal(dl).astype(np.float32) / 8 + 0.5 * u
                lq_t[0, 0, h, t] = torch.from_numpy(new.astype(np.float32)).bfloat16()
            todo = todo[~ok]
    x["lq"], x["lk"] = lq_t, lk_t
    return cfg, x


def test_backward_needle_retrieved_by_every_query_chunk():
    n, H = 640, 2
    cfg, x = heavy_inputs(n, H, seed=31)
    shape = shape_of(cfg)
    d = {key: dev(x[key]) for key in ("q", "k", "v", "lq", "lk", "dout", "q_pos")}
    idx, score, w = run_retrieve(shape, d["lq"], d["lk"], d["q_pos"])
    lq64, lk64 = f64(x["lq"]), f64(x["lk"])
    r_idx, r_score, r_w = orc.retrieve(lq64, lk64, x["q_pos"].numpy(), cfg["k"],
                                       cfg["score_scale"], cfg["softmax_one"])
    assert np.array_equal(idx.cpu().numpy(), r_idx), "top-k indices differ"
    # the planted chunk is retrieved by every query chunk that may see it
    retrievers = (r_idx[0, 0] == NEEDLE).any(-1).sum(-1)
    assert (retrievers == n - NEEDLE - 2).all(), retrievers
    close("score", f64(score), r_score, True)
    close("w", f64(w), r_w, True)
    o, lse = run_forward(shape, d["q"], d["k"], d["v"], idx, w)
    q64, k64, v64, do64 = f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["dout"])
    r_o, r_lse = orc.forward(q64, k64, v64, r_idx, r_w, cfg["attn_scale"])
    close("o", f64(o), r_o, True)
    compare_lse(lse, r_lse, True)
    g = run_backward(shape, d["q"], d["k"], d["v"], idx, w, lse, d["dout"], d["lq"], d["lk"])
    r = orc.backward(q64, k64, v64, r_idx, r_w, do64, lq64, lk64, cfg["attn_scale"],
                     cfg["score_scale"])
    for key in ("dq", "dk", "dv", "dw", "dscore", "dlq", "dlk"):
        close(key, f64(g[key]), r[key], True)
    # the planted chunk's own gradients, on their own (they sum 635 pairs)
    for key in ("dk", "dv", "dlk"):
        close(f"{key}[needle]", f64(g[key])[0, 0, :, NEEDLE], r[key][0, 0, :, NEEDLE], True)
    g2 = run_backward(shape, d["q"], d["k"], d["v"], idx, w, lse, d["dout"], d["lq"], d["lk"])
    for key in g:
        assert torch.equal(g[key], g2[key]), f"{key} differs between two runs"
