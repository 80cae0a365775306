"""GPU checks of the backward's reverse index (the list of (query chunk, slot)
pairs that retrieved each key chunk), fed with chosen idx instead of a
retrieval: empty slots (-1), indices past n_key, repeated chunks within a row,
a chunk that every query chunk retrieves, and key counts that take the index
two and three passes of 512 chunks.

The backward returns gradients for Q, K, V and the weights (paperlayer.ai
summary, appendix B); the key-side gradients of chunk c sum over exactly the
pairs that retrieved c.  Two checks per case:
  - the lists in the workspace equal a stable sort of the valid entries by
    chunk (entry e = t * k + i, ascending within each chunk), bit for bit;
  - every gradient matches the float64 oracle at the bf16 tolerances.
"""

import numpy as np
import pytest
import torch

import retrieval_sparse_attention_amd as gca
import synth
from oracle import gca_oracle as orc
from gpu_common import close, compare_lse, dev, f64, require_gpu, run_forward, shape_of

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _idx_pattern(rng, H, n_query, n_key, k, heavy):
    """Random chunks with about 10% empty slots, 5% past n_key and repeats
    within rows; `heavy`: chunk 5 sits in slot 0 of every row."""
    idx = rng.integers(0, n_key, size=(1, 1, H, n_query, k)).astype(np.int32)
    u = rng.random(idx.shape)
    idx[u < 0.10] = -1
    idx[(u >= 0.10) & (u < 0.15)] = n_key + rng.integers(0, 50, size=idx[(u >= 0.10) & (u < 0.15)].shape)
    rep = rng.random(idx.shape[:-1]) < 0.2           # a repeated chunk in 20% of rows
    idx[..., 1][rep] = idx[..., 2][rep]
    if heavy:
        idx[..., 0] = 5
    return idx


def _expected_lists(idx_head, n_key):
    """rev_off [n_key + 1] and rev_ent of one head by a stable sort."""
    flat = idx_head.reshape(-1).astype(np.int64)
    ent = np.flatnonzero((flat >= 0) & (flat < n_key))
    order = np.argsort(flat[ent], kind="stable")
    rev_ent = ent[order]
    rev_off = np.searchsorted(flat[ent][order], np.arange(n_key + 1), side="left")
    return rev_off.astype(np.int32), rev_ent.astype(np.int32)


@pytest.mark.parametrize("n_query,n_key,S,D,heavy", [
    (40, 700, 64, 64, False),      # index segments held in registers, two passes
    (520, 1100, 64, 64, True),     # segments re-read, three passes, a 520-entry list
    (24, 600, 16, 32, True),       # the 16-token key-side kernel, two passes
    (24, 600, 5, 7, True),         # the generic key-side kernel, two passes
], ids=["two_passes", "three_passes_heavy", "s16_d32", "generic_s5_d7"])
def test_reverse_lists_and_gradients(n_query, n_key, S, D, heavy):
    H, k = 2, 8
    over = dict(G=1, B=1, H=H, n_query=n_query, n_key=n_key, S=S, D=D)
    cfg = synth.workload("train16k_fwdbwd_g2", **over)
    rng = np.random.default_rng(n_query * 7 + n_key)
    sc = cfg["value_scale"]

    def normal(*shape):
        return torch.from_numpy((rng.standard_normal(shape) * sc).astype(np.float32)).bfloat16()

    q, kk, v = normal(1, 1, H, n_query, S, D), normal(1, 1, H, n_key, S, D), normal(1, 1, H, n_key, S, D)
    dout = normal(1, 1, H, n_query, S, D)
    lq, lk = normal(1, 1, H, n_query, 64), normal(1, 1, H, n_key, 64)
    idx = _idx_pattern(rng, H, n_query, n_key, k, heavy)
    w = rng.random((1, 1, H, n_query, k)).astype(np.float32) / k
    shape = shape_of(cfg)
    d = dict(q=dev(q), k=dev(kk), v=dev(v), dout=dev(dout), lq=dev(lq), lk=dev(lk),
             idx=dev(torch.from_numpy(idx)), w=dev(torch.from_numpy(w)))
    o, lse = run_forward(shape, d["q"], d["k"], d["v"], d["idx"], d["w"])
    ws_bytes = gca.gca_workspace_size(shape, gca.OP_BACKWARD)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    nan = float("nan")
    g = dict(dq=torch.full_like(d["q"], nan), dk=torch.full_like(d["k"], nan),
             dv=torch.full_like(d["v"], nan),
             dw=torch.full((1, 1, H, n_query, k), nan, device="cuda"),
             dscore=torch.full((1, 1, H, n_query, k), nan, device="cuda"),
             dlq=torch.full((1, 1, H, n_query, 64), nan, device="cuda"),
             dlk=torch.full((1, 1, H, n_key, 64), nan, device="cuda"))
    gca.gca_backward(shape, d["q"], d["k"], d["v"], d["idx"], d["w"], lse, d["dout"], d["lq"],
                     d["lk"], g["dq"], g["dk"], g["dv"], g["dw"], g["dscore"], g["dlq"], g["dlk"],
                     ws=ws)
    torch.cuda.synchronize()
    # workspace layout: delta [H * Nq * k * S] floats, rev_off [H * (Nk + 1)] ints,
    # rev_ent [H * Nq * k] ints, each starting on a 256-byte boundary
    n_ent = n_query * k
    up = lambda n: (n + 255) // 256 * 256
    o_off = up(H * n_ent * S * 4)
    o_ent = o_off + up(H * (n_key + 1) * 4)
    raw = ws.cpu().numpy()
    rev_off = raw[o_off:o_off + H * (n_key + 1) * 4].view(np.int32).reshape(H, n_key + 1)
    rev_ent = raw[o_ent:o_ent + H * n_ent * 4].view(np.int32).reshape(H, n_ent)
    for h in range(H):
        e_off, e_ent = _expected_lists(idx[0, 0, h], n_key)
        assert np.array_equal(rev_off[h], e_off), f"head {h}: list offsets differ"
        assert np.array_equal(rev_ent[h, :len(e_ent)], e_ent), f"head {h}: list entries differ"
    if heavy:
        assert (e_off[6] - e_off[5]) >= n_query  # chunk 5's list holds every row
    r_o, r_lse = orc.forward(f64(q), f64(kk), f64(v), idx, w.astype(np.float64), cfg["attn_scale"])
    close("o", f64(o), r_o, True)
    compare_lse(lse, r_lse, True)
    r = orc.backward(f64(q), f64(kk), f64(v), idx, w.astype(np.float64), f64(dout), f64(lq),
                     f64(lk), cfg["attn_scale"], cfg["score_scale"])
    for key in ("dq", "dk", "dv", "dw", "dscore", "dlq", "dlk"):
        close(key, f64(g[key]), r[key], True)
