"""GPU parity of the GCA library against the float64 oracle (needs an MI355X).

Every test feeds the same seeded inputs to both sides.  Top-k indices must be
bit-identical; values must meet the tolerances: float32 workloads 1e-5
max-abs; bf16 workloads 2e-2 max-abs and 1e-2 mean-relative (mean |gpu - ref| /
mean |ref| per tensor), with float32 accumulation on the GPU.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import gca_oracle as orc
from gpu_common import (accept_for, close, compare_lse, dev, f64, require_gpu, run_backward,
                        run_forward, run_retrieve, shape_of)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _full_path(name, heads=None, **over):
    """retrieve -> forward -> backward on the GPU and in the oracle; all compared."""
    cfg = synth.workload(name, **over)
    x = synth.training_inputs(name, accept=accept_for(cfg), **over)
    bf = cfg["dtype"] == "bf16"
    shape = shape_of(cfg)
    d = {key: dev(x[key]) for key in ("q", "k", "v", "lq", "lk", "dout", "q_pos")}
    idx, score, w = run_retrieve(shape, d["lq"], d["lk"], d["q_pos"])
    lq64, lk64 = f64(x["lq"]), f64(x["lk"])
    r_idx, r_score, r_w = orc.retrieve(lq64, lk64, x["q_pos"].numpy(), cfg["k"],
                                       cfg["score_scale"], cfg["softmax_one"])
    assert np.array_equal(idx.cpu().numpy(), r_idx), "top-k indices differ"
    close("score", f64(score), r_score, bf)
    close("w", f64(w), r_w, bf)
    o, lse = run_forward(shape, d["q"], d["k"], d["v"], idx, w)
    q64, k64, v64, do64 = f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["dout"])
    r_o, r_lse = orc.forward(q64, k64, v64, r_idx, r_w, cfg["attn_scale"])
    close("o", f64(o), r_o, bf)
    compare_lse(lse, r_lse, bf)
    g = run_backward(shape, d["q"], d["k"], d["v"], idx, w, lse, d["dout"], d["lq"], d["lk"])
    r = orc.backward(q64, k64, v64, r_idx, r_w, do64, lq64, lk64, cfg["attn_scale"],
                     cfg["score_scale"], heads=heads)
    if heads is None:
        for key in ("dq", "dk", "dv", "dw", "dscore", "dlq", "dlk"):
            close(key, f64(g[key]), r[key], bf)
    else:
        for (gg, b, h) in heads:
            for key in ("dq", "dk", "dv", "dw", "dscore", "dlq", "dlk"):
                close(f"{key}[{gg},{b},{h}]", f64(g[key][gg, b, h]), r[key][gg, b, h], bf)
    return g


def test_tiny_fp32_full_path():
    _full_path("tiny_fp32")


def test_tiny_fp32_ragged_and_k3():
    # 21 chunks of 5 tokens, D=7, Dl=9, top-3: nothing is a power of two
    _full_path("tiny_fp32", n_query=21, n_key=21, S=5, D=7, Dl=9, k=3, H=3, softmax_one=1)


def test_bf16_small_vanilla_aliased():
    # 40 query chunks: one full 32-query tile plus a ragged tail of 8
    _full_path("train16k_fwd", B=1, H=3, n_query=40, n_key=40)


def test_bf16_small_off_by_one_two_groups():
    _full_path("train16k_fwdbwd_g2", B=2, H=2, n_query=72, n_key=72)


@pytest.mark.parametrize("k", [1, 5, 16])
def test_bf16_top_k_sizes(k):
    _full_path("train16k_fwdbwd_g2", G=1, B=1, H=2, n_query=48, n_key=48, k=k)


@pytest.mark.parametrize("S,D", [(16, 32), (16, 64), (64, 32), (5, 7)])
def test_bf16_chunk_and_head_sizes(S, D):
    # bf16 attention at other sizes (64 x 32: the MFMA kernels with half-width
    # rows; 16 x 64 and 16 x 32: the one-wave-per-chunk MFMA kernels; 5 x 7:
    # the float32 VALU path): every output of retrieve -> forward -> backward
    # against the oracle, two groups
    _full_path("train16k_fwdbwd_g2", B=1, H=2, n_query=40, n_key=40, S=S, D=D)


@pytest.mark.parametrize("D", [64, 32])
def test_bf16_chunk_16_ragged_workgroups(D):
    # the 16-token kernels run four chunks per workgroup: 3 heads x 161 chunks
    # leave the last workgroup with one busy wave on each side, and reverse
    # lists run past one 64-entry block
    _full_path("train16k_fwdbwd_g2", G=1, B=1, H=3, n_query=161, n_key=161, S=16, D=D)


def test_bf16_head_dim_32_mfma_multiple_tiles():
    # the 64 x 32 MFMA kernels over enough query and key chunks for several
    # tiles per XCD and reverse lists past one block: a 3-head training shape
    _full_path("train16k_fwdbwd_g2", G=1, B=1, H=3, n_query=160, n_key=160, D=32)


def test_bf16_landmark_dim_32():
    _full_path("train16k_fwdbwd_g2", G=1, B=1, H=2, n_query=40, n_key=40, Dl=32)


@pytest.mark.parametrize("over", [
    dict(n_key=5000, n_query=37, H=2, q_pos=5001),
    # 96 heads x 2 query tiles: four slices of 2304 candidates (18 rounds each)
    dict(n_key=9000, n_query=40, B=8, H=12, q_pos=9001),
    # one head: 512 slices of one round; the merge takes 4096 partial keys per query
    dict(n_key=65536, n_query=20, H=1, q_pos=65537),
    dict(n_key=65536, n_query=20, H=1, q_pos=65537, k=16),
    # merge widths: 101 slices x 8 = 808 keys (registers, ragged last slice),
    # 64 x 16 = 1024 (registers, full), 200 x 8 = 1600 (streamed, ragged)
    dict(n_key=12900, n_query=20, H=1, q_pos=12901),
    dict(n_key=8192, n_query=20, H=1, q_pos=8193, k=16),
    dict(n_key=25500, n_query=20, H=1, q_pos=25501),
], ids=["short_slices", "long_slices", "many_slices", "many_slices_k16", "merge_808",
        "merge_1024_k16", "merge_1600"])
def test_bf16_sliced_scan_with_needles(over):
    """n_key > 1024 takes the sliced scan + merge path; planted needles rank 1."""
    cfg = synth.workload("retrieve16m", **over)
    lk = synth.context_landmarks("retrieve16m", **over)
    qb = synth.query_batch("retrieve16m", lk, accept=accept_for(cfg), **over)
    shape = shape_of(cfg)
    idx, score, w = run_retrieve(shape, dev(qb["lq"]), dev(lk), dev(qb["q_pos"]))
    r_idx, r_score, r_w = orc.retrieve(f64(qb["lq"]), f64(lk), qb["q_pos"].numpy(), cfg["k"],
                                       cfg["score_scale"], cfg["softmax_one"])
    assert np.array_equal(idx.cpu().numpy(), r_idx)
    close("score", f64(score), r_score, True)
    close("w", f64(w), r_w, True)
    best = np.take_along_axis(r_idx, np.argmax(r_score, axis=-1)[..., None], -1)[..., 0]
    assert (best == qb["needle"].numpy()[None, None, None, :]).all()


@pytest.mark.parametrize("k,dl", [(8, 64), (16, 64), (4, 32)], ids=["k8", "k16", "k4_dl32"])
def test_bf16_long_slices_mixed_positions(k, dl):
    """Sliced scan + merge where the queries of a tile end at different
    positions: none, one, fewer than k, inside the first slice, at and past
    slice edges, all.  48 heads x 2 query tiles: 8 slices of 2560 candidates."""
    from oracle import condition
    B, H, nq, nk = 4, 12, 50, 20000
    cfg = synth.workload("retrieve16m", B=B, H=H, n_query=nq, n_key=nk, k=k, Dl=dl)
    rng = np.random.default_rng(40 + k + dl)
    lq = torch.from_numpy((rng.standard_normal((1, B, H, nq, dl)) / 8).astype(np.float32))
    lk = torch.from_numpy((rng.standard_normal((1, B, H, nk, dl)) / 8).astype(np.float32))
    lq, lk = lq.bfloat16(), lk.bfloat16()
    q_pos = rng.integers(0, nk + 2, size=nq).astype(np.int32)
    q_pos[:8] = [0, 1, 2 + k // 2, 1000, 1300, 5121, nk, nk + 1]
    q_pos[40:44] = [3, 700, 2600, 19000]
    shape = shape_of(cfg)
    idx, score, w = run_retrieve(shape, dev(lq), dev(lk), dev(torch.from_numpy(q_pos)))
    lq64, lk64 = f64(lq), f64(lk)
    r_idx, r_score, r_w = orc.retrieve(lq64, lk64, q_pos, k, cfg["score_scale"],
                                       cfg["softmax_one"])
    # rows whose k-th and (k+1)-th scores lie within float32 rounding of each
    # other may order either way; 1e-5 is far above that (|score| < 2 here)
    n_cand = np.clip(q_pos.astype(np.int64) - 1, 0, nk)
    sep = np.stack([condition.gap_ok(lq64[0, b, h], lk64[0, b, h], n_cand, k,
                                     cfg["score_scale"], 1e-5)
                    for b in range(B) for h in range(H)]).reshape(1, B, H, nq)
    assert sep.mean() > 0.95
    assert np.array_equal(idx.cpu().numpy()[sep], r_idx[sep])
    close("score", f64(score), r_score, True, mask=sep)
    close("w", f64(w), r_w, True, mask=sep)


@pytest.mark.parametrize("nq,nk,k,dl,pos", [
    (1, 1025, 8, 64, [1026]),                     # 5 slices, the last holds one candidate
    (4, 5000, 8, 64, [0, 6, 257, 5001]),          # none, fewer than k, one slice + 1, all
    (3, 20000, 16, 64, [1, 12801, 19999]),        # 79 slices, k = 16
    (4, 65536, 16, 64, [513, 30000, 65536, 65537]),  # 256 slices x 16 = the merge's 4096
    (2, 3000, 4, 32, [2000, 3001]),               # 32-dimensional landmarks
    (4, 65537, 16, 64, [65538, 2, 40000, 257]),   # 257 slices would pass 4096: 32-query path
], ids=["one_query", "edges", "k16", "merge_max", "dl32", "past_merge_max"])
def test_bf16_few_query_scan(nq, nk, k, dl, pos):
    """Retrieval for up to 4 query chunks per head (decoding steps) takes one
    workgroup per (head, query, 256-candidate slice) before the merge; indices
    bit-exact where the k-th score is separated, scores and weights within bf16
    tolerance, on 12 heads."""
    from oracle import condition
    B, H = 2, 6
    cfg = synth.workload("retrieve16m", B=B, H=H, n_query=nq, n_key=nk, k=k, Dl=dl)
    rng = np.random.default_rng(nq * 1000 + k + dl)
    lq = torch.from_numpy((rng.standard_normal((1, B, H, nq, dl)) / 8).astype(np.float32))
    lk = torch.from_numpy((rng.standard_normal((1, B, H, nk, dl)) / 8).astype(np.float32))
    lq, lk = lq.bfloat16(), lk.bfloat16()
    q_pos = np.array(pos, np.int32)
    shape = shape_of(cfg)
    idx, score, w = run_retrieve(shape, dev(lq), dev(lk), dev(torch.from_numpy(q_pos)))
    lq64, lk64 = f64(lq), f64(lk)
    r_idx, r_score, r_w = orc.retrieve(lq64, lk64, q_pos, k, cfg["score_scale"],
                                       cfg["softmax_one"])
    n_cand = np.clip(q_pos.astype(np.int64) - 1, 0, nk)
    sep = np.stack([condition.gap_ok(lq64[0, b, h], lk64[0, b, h], n_cand, k,
                                     cfg["score_scale"], 1e-5)
                    for b in range(B) for h in range(H)]).reshape(1, B, H, nq)
    assert sep.mean() > 0.9
    assert np.array_equal(idx.cpu().numpy()[sep], r_idx[sep])
    close("score", f64(score), r_score, True, mask=sep)
    close("w", f64(w), r_w, True, mask=sep)


def test_bf16_few_query_scan_ties():
    """Every landmark equal: all scores tie, so the k chunks of lowest index are
    taken, in ascending order, with equal weights (score desc, index asc)."""
    B, H, nq, nk, k = 1, 3, 2, 4000, 8
    cfg = synth.workload("retrieve16m", B=B, H=H, n_query=nq, n_key=nk, k=k)
    rng = np.random.default_rng(77)
    row = torch.from_numpy((rng.standard_normal(64) / 8).astype(np.float32)).bfloat16()
    lq = torch.from_numpy((rng.standard_normal((1, B, H, nq, 64)) / 8).astype(np.float32))
    lq = lq.bfloat16()
    lk = row.expand(1, B, H, nk, 64).contiguous()
    q_pos = np.array([4001, 1500], np.int32)
    idx, score, w = run_retrieve(shape_of(cfg), dev(lq), dev(lk), dev(torch.from_numpy(q_pos)))
    r_idx, r_score, r_w = orc.retrieve(f64(lq), f64(lk), q_pos, k, cfg["score_scale"],
                                       cfg["softmax_one"])
    assert np.array_equal(idx.cpu().numpy(), r_idx)
    assert (r_idx == np.arange(k)).all()
    close("score", f64(score), r_score, True)
    close("w", f64(w), r_w, True)


def test_bf16_edge_positions():
    """q_pos giving 0, fewer than k, exactly k and all candidates; n_key not a multiple of 32."""
    cfg = synth.workload("train16k_fwdbwd_g2", G=1, B=1, H=2, n_query=6, n_key=45)
    rng = np.random.default_rng(4)
    lq = torch.from_numpy(rng.standard_normal((1, 1, 2, 6, 64)).astype(np.float32) / 8).bfloat16()
    lk = torch.from_numpy(rng.standard_normal((1, 1, 2, 45, 64)).astype(np.float32) / 8).bfloat16()
    q_pos = torch.tensor([0, 1, 4, 9, 46, 1000], dtype=torch.int32)
    shape = shape_of(cfg)
    idx, score, w = run_retrieve(shape, dev(lq), dev(lk), dev(q_pos))
    r_idx, r_score, r_w = orc.retrieve(f64(lq), f64(lk), q_pos.numpy(), cfg["k"],
                                       cfg["score_scale"], cfg["softmax_one"])
    # no near-ties here: the k-th gaps of these draws exceed the float32 score error
    assert np.array_equal(idx.cpu().numpy(), r_idx)
    close("score", f64(score), r_score, True)
    close("w", f64(w), r_w, True)


def test_bf16_forward_invalid_and_duplicate_slots():
    """Slots with idx -1 or >= n_key are empty; a duplicated chunk counts twice."""
    cfg = synth.workload("train16k_fwd", B=1, H=1, n_query=4, n_key=9)
    x = synth.training_inputs("train16k_fwd", B=1, H=1, n_query=4, n_key=4)
    rng = np.random.default_rng(8)
    k = torch.from_numpy(rng.standard_normal((1, 1, 1, 9, 64, 64)).astype(np.float32) / 8).bfloat16()
    v = torch.from_numpy(rng.standard_normal((1, 1, 1, 9, 64, 64)).astype(np.float32) / 8).bfloat16()
    idx = torch.tensor([[[[[3, -1, 7, 9, 2, 2, 100, 0],
                          [-1] * 8,
                          [0, 1, 2, 3, 4, 5, 6, 8],
                          [8, 7, 6, 5, 4, 3, 2, 1]]]]], dtype=torch.int32)
    w = torch.from_numpy(rng.random((1, 1, 1, 4, 8)).astype(np.float32))
    shape = shape_of(cfg)
    o, lse = run_forward(shape, dev(x["q"]), dev(k), dev(v), dev(idx), dev(w))
    r_o, r_lse = orc.forward(f64(x["q"]), f64(k), f64(v), idx.numpy(), w.numpy().astype(np.float64),
                             cfg["attn_scale"])
    close("o", f64(o), r_o, True)
    compare_lse(lse, r_lse, True)
    assert (f64(o)[0, 0, 0, 1] == 0).all()


@pytest.mark.parametrize("H,n_query,k,D", [
    (1, 4, 8, 64), (3, 100, 8, 64), (4, 250, 8, 64),
    (1, 4, 16, 64), (2, 100, 16, 64), (3, 100, 16, 32), (1, 200, 12, 32), (2, 128, 3, 32)],
    ids=["4_chunks", "300_chunks", "1000_chunks", "4_chunks_k16", "200_chunks_k16",
         "300_chunks_k16_d32", "200_chunks_k12_d32", "256_chunks_k3_d32"])
def test_bf16_forward_valid_slot_counts(H, n_query, k, D):
    """Rows with every count of valid slots from 0 to k, the others empty (-1)
    or out of range, and repeated chunks, at several query-chunk counts, k and
    head_dim: O and LSE must match the oracle and repeat bit for bit."""
    n_key = 40
    cfg = synth.workload("train16k_fwd", B=1, H=H, n_query=n_query, n_key=n_key, k=k, D=D)
    rng = np.random.default_rng(H * 1000 + n_query + 100000 * k + D)
    sc = cfg["value_scale"]
    mk = lambda *shape: torch.from_numpy(
        (rng.standard_normal(shape) * sc).astype(np.float32)).bfloat16()
    q, kk, v = mk(1, 1, H, n_query, 64, D), mk(1, 1, H, n_key, 64, D), mk(1, 1, H, n_key, 64, D)
    idx = rng.integers(0, n_key, size=(1, 1, H, n_query, k)).astype(np.int32)
    n_valid = rng.integers(0, k + 1, size=(1, 1, H, n_query))
    m = min(k + 1, n_valid.size)
    n_valid.reshape(-1)[:m] = np.arange(m)
    for pos in np.ndindex(n_valid.shape):
        slots = rng.permutation(k)[n_valid[pos]:]
        idx[pos][slots] = np.where(rng.random(len(slots)) < 0.5, -1, n_key + 3)
    if k >= 2:
        rep = rng.random(idx.shape[:-1]) < 0.2
        idx[..., k - 2][rep] = idx[..., k - 1][rep]
    w = rng.random((1, 1, H, n_query, k)).astype(np.float32)
    shape = shape_of(cfg)
    d = [dev(t) for t in (q, kk, v, torch.from_numpy(idx), torch.from_numpy(w))]
    o, lse = run_forward(shape, *d)
    r_o, r_lse = orc.forward(f64(q), f64(kk), f64(v), idx, w.astype(np.float64),
                             cfg["attn_scale"])
    close("o", f64(o), r_o, True)
    compare_lse(lse, r_lse, True)
    o2, lse2 = run_forward(shape, *d)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_bf16_backward_is_deterministic():
    cfg = synth.workload("train16k_fwdbwd_g2", G=1, B=1, H=2, n_query=64, n_key=64)
    x = synth.training_inputs("train16k_fwdbwd_g2", accept=accept_for(cfg), G=1, B=1, H=2,
                              n_query=64, n_key=64)
    shape = shape_of(cfg)
    d = {key: dev(x[key]) for key in ("q", "k", "v", "lq", "lk", "dout", "q_pos")}
    idx, score, w = run_retrieve(shape, d["lq"], d["lk"], d["q_pos"])
    o, lse = run_forward(shape, d["q"], d["k"], d["v"], idx, w)
    g1 = run_backward(shape, d["q"], d["k"], d["v"], idx, w, lse, d["dout"], d["lq"], d["lk"])
    g2 = run_backward(shape, d["q"], d["k"], d["v"], idx, w, lse, d["dout"], d["lq"], d["lk"])
    for key in g1:
        assert torch.equal(g1[key], g2[key]), key
    o2, lse2 = run_forward(shape, d["q"], d["k"], d["v"], idx, w)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def _ordered_landmarks(order, B, H, n_key, n_query, seed):
    """Landmarks whose scores follow `order` along the chunk axis: lk_j = c_j * u and
    lq = u for one direction u per head, so score_j = c_j <u, u> / sqrt(Dl).
    'equal': c_j = 1 (every candidate ties); 'rising' / 'falling': c_j steps up / down
    with j over 128 levels (runs of equal c_j, so ties appear too).  Components of u
    are +-2^e / 8 with e in {0, -1, -2} and c_j has at most 8 significant bits, so every
    product and partial sum is exact in bfloat16 inputs and float32 accumulation:
    float32 and float64 scores agree bit for bit and ties are exact."""
    rng = np.random.default_rng(seed)
    sign = rng.choice([-1.0, 1.0], size=(1, B, H, 1, 64))
    u = (sign * 2.0 ** -rng.integers(0, 3, size=(1, B, H, 1, 64)) / 8).astype(np.float32)
    step = np.floor(np.arange(n_key) * 128 / n_key).astype(np.float32) / 128
    c = {"equal": np.ones(n_key, np.float32), "rising": 1.0 + step, "falling": 2.0 - step}[order]
    lk = torch.from_numpy((c[None, None, None, :, None] * u).astype(np.float32))
    lq = torch.from_numpy(np.broadcast_to(u, (1, B, H, n_query, 64)).copy())
    assert torch.equal(lk.bfloat16().float(), lk) and torch.equal(lq.bfloat16().float(), lq)
    return lq.bfloat16(), lk.bfloat16()


@pytest.mark.parametrize("order", ["equal", "rising", "falling"])
@pytest.mark.parametrize("k", [8, 16])
@pytest.mark.parametrize("sliced", [False, True])
def test_bf16_scan_adversarial_orders(order, k, sliced):
    """Score orders that defeat the running threshold (every candidate ties, or each
    one beats all before it) or make it trivial; one slice and long slices."""
    if sliced:  # 192 heads: 6000 candidates cut into a few slices of 12 rounds each
        B, H, n_key, n_query = 16, 12, 6000, 3
        q_pos = torch.tensor([6001, 6001, 3500], dtype=torch.int32)
    else:
        B, H, n_key, n_query = 1, 3, 700, 40
        q_pos = torch.arange(n_query, dtype=torch.int32) * 18
    cfg = synth.workload("retrieve16m", B=B, H=H, n_key=n_key, n_query=n_query, k=k)
    lq, lk = _ordered_landmarks(order, B, H, n_key, n_query, seed=11 + k)
    shape = shape_of(cfg)
    idx, score, w = run_retrieve(shape, dev(lq), dev(lk), dev(q_pos))
    r_idx, r_score, r_w = orc.retrieve(f64(lq), f64(lk), q_pos.numpy(), k, cfg["score_scale"],
                                       cfg["softmax_one"])
    assert np.array_equal(idx.cpu().numpy(), r_idx)
    close("score", f64(score), r_score, True)
    close("w", f64(w), r_w, True)


def test_bf16_no_resident_chunks():
    """n_key = 0: every slot is empty; O = 0, lse = -inf and all gradients 0, with
    NULL K/V/lk (zero-size tensors) and dlq still requested."""
    cfg = synth.workload("train16k_fwdbwd_g2", G=1, B=1, H=2, n_query=5, n_key=0)
    shape = shape_of(cfg)
    rng = np.random.default_rng(7)
    lq = dev(torch.from_numpy(rng.standard_normal((1, 1, 2, 5, 64)).astype(np.float32) / 8)
             .bfloat16())
    q = dev(torch.from_numpy(rng.standard_normal((1, 1, 2, 5, 64, 64)).astype(np.float32) / 8)
            .bfloat16())
    dout = dev(torch.from_numpy(rng.standard_normal((1, 1, 2, 5, 64, 64)).astype(np.float32))
               .bfloat16())
    lk = torch.empty((1, 1, 2, 0, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((1, 1, 2, 0, 64, 64), dtype=torch.bfloat16, device="cuda")
    v = torch.empty_like(k)
    q_pos = dev(torch.tensor([0, 1, 2, 3, 100], dtype=torch.int32))
    idx, score, w = run_retrieve(shape, lq, lk, q_pos)
    assert (idx.cpu() == -1).all() and (score.cpu() == 0).all() and (w.cpu() == 0).all()
    o, lse = run_forward(shape, q, k, v, idx, w)
    assert (o.float().cpu() == 0).all() and torch.isneginf(lse.cpu()).all()
    g = run_backward(shape, q, k, v, idx, w, lse, dout, lq, lk)
    for key in ("dq", "dw", "dscore", "dlq"):
        assert (g[key].float().cpu() == 0).all(), key
