"""The retrieval-plus-forward call (gca_retrieve_forward) against the two calls
made in turn and against the float64 oracle.

Definition: long-context-modeling README, "Model Architecture" (a chunk
retrieves its top-k past chunks with the landmark of the chunk before it, then
attends to each and fuses the O^i with the softmax of the scores); paperhub.cn,
authors' reply "Cmt 1" (Eq. 1 scores).  Where the retrieval is sliced and the
tiles are 64-token bf16, the slice lists are merged inside the forward's kernel;
the outputs must still equal those of gca_retrieve then gca_forward bit for bit
(the same merge and the same attention arithmetic), and meet the oracle: indices
bit-exact where the k-th score is separated by 1e-5, O and L within the bf16
bounds.  Shapes: decoding steps (1-3 query chunks over 1000-20000 candidates,
the few-query scan), 32-query tiles over long lists, an unsliced training shape
(no merge: the call runs the two launches) and rows with fewer than k or no
candidates.
"""

import numpy as np
import pytest
import torch

import retrieval_sparse_attention_amd as gca
import synth
from oracle import condition
from oracle import gca_oracle as orc
from gpu_common import close, compare_lse, dev, f64, require_gpu, shape_of

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


CASES = [
    # (H, n_query, n_key, k, D, softmax_one, q_pos rule, expect_fused)
    (3, 1, 5000, 8, 64, 0, "fresh", True),       # few-query scan: 20 slices of 256
    (2, 3, 10000, 16, 32, 1, "fresh", True),     # 40 slices x 16 keys = 640 per row
    (2, 2, 1500, 1, 64, 0, "fresh", True),
    (1, 2, 20000, 16, 64, 0, "fresh", False),    # 79 x 16 = 1264 keys: the separate merge
    (4, 40, 3000, 8, 64, 0, "causal_tail", True),  # 32-query tiles, 24 slices
    (2, 33, 9000, 4, 32, 1, "mixed", True),      # 71 slices
    (2, 64, 64, 8, 64, 1, "causal", False),      # unsliced: the scan finalises itself
]
IDS = ["decode_h3", "decode_k16_d32", "decode_k1", "decode_k16_unfused", "tiles40",
       "tiles33_k4_d32", "unsliced"]


def _q_pos(rule, nq, nk, rng):
    if rule == "fresh":
        return np.full(nq, nk + 1, dtype=np.int32)
    if rule == "causal":
        return np.arange(nq, dtype=np.int32)
    if rule == "causal_tail":  # the last nq chunks of an nk-chunk context
        return np.arange(nk - nq + 1, nk + 1, dtype=np.int32)
    # mixed: no candidates, fewer than k, and long lists
    return rng.integers(0, nk + 2, size=nq).astype(np.int32)


@pytest.mark.parametrize("H,nq,nk,k,D,s1,rule,expect_fused", CASES, ids=IDS)
def test_retrieve_forward_matches_two_calls_and_oracle(H, nq, nk, k, D, s1, rule, expect_fused):
    print(f"[retrieve_forward] H={H} nq={nq} nk={nk} k={k} D={D} softmax_one={s1} {rule}",
          flush=True)
    rng = np.random.default_rng(nq * 7919 + nk + 31 * k + D)
    cfg = synth.workload("infer1m_step", H=H, n_query=nq, n_key=nk, k=k, D=D,
                         softmax_one=s1)
    sc = cfg["value_scale"]

    def bf(*shape, scale=1.0):
        x = rng.standard_normal(shape, dtype=np.float32)
        x *= np.float32(scale)
        return torch.from_numpy(x).bfloat16()

    lq, lk = bf(1, 1, H, nq, 64, scale=1 / 8), bf(1, 1, H, nk, 64, scale=1 / 8)
    q, kk, v = bf(1, 1, H, nq, 64, D, scale=sc), bf(1, 1, H, nk, 64, D, scale=sc), \
        bf(1, 1, H, nk, 64, D, scale=sc)
    q_pos = _q_pos(rule, nq, nk, rng)
    shape = shape_of(cfg)
    d = {name: dev(t) for name, t in dict(lq=lq, lk=lk, q=q, k=kk, v=v,
                                          q_pos=torch.from_numpy(q_pos)).items()}
    slots = (1, 1, H, nq, k)

    def outputs():
        return (torch.full(slots, -7, dtype=torch.int32, device="cuda"),
                torch.full(slots, float("nan"), device="cuda"),
                torch.full(slots, float("nan"), device="cuda"),
                torch.full(tuple(q.shape), float("nan"), dtype=torch.bfloat16, device="cuda"),
                torch.full((1, 1, H, nq, k, 64), float("nan"), device="cuda"))

    # the two calls in turn
    i1, s1_, w1, o1, l1 = outputs()
    gca.gca_retrieve(shape, d["lq"], d["lk"], d["q_pos"], i1, s1_, w1)
    gca.gca_forward(shape, d["q"], d["k"], d["v"], i1, w1, o1, l1)
    # one call, with the library's kernel timing on to see which kernels ran
    i2, s2, w2, o2, l2 = outputs()
    torch.cuda.synchronize()
    gca.gca_timing_enable(True)
    gca.gca_timing_collect()
    gca.gca_retrieve_forward(shape, d["lq"], d["lk"], d["q_pos"], d["q"], d["k"], d["v"], i2, s2,
                             w2, o2, l2)
    torch.cuda.synchronize()
    gca.gca_timing_enable(False)
    ran = {name: n for name, (_, n) in gca.gca_timing_collect().items() if n}
    assert (ran.get("topk_merge_forward", 0) > 0) == expect_fused, ran
    if expect_fused:
        assert "topk_merge" not in ran and "forward" not in ran, ran
    for name, a, b in (("idx", i1, i2), ("score", s1_, s2), ("w", w1, w2), ("o", o1, o2),
                       ("lse", l1, l2)):
        assert torch.equal(a, b) or (name in ("score", "w", "lse") and
                                     torch.equal(torch.nan_to_num(a), torch.nan_to_num(b))), name

    # the oracle: indices where the k-th score is separated, O and L from them
    lq64, lk64 = f64(lq), f64(lk)
    r_idx, r_score, r_w = orc.retrieve(lq64, lk64, q_pos, k, cfg["score_scale"], s1)
    n_cand = np.clip(q_pos.astype(np.int64) - 1, 0, nk)
    sep = np.stack([condition.gap_ok(lq64[0, 0, h], lk64[0, 0, h], n_cand, k,
                                     cfg["score_scale"], 1e-5)
                    for h in range(H)]).reshape(1, 1, H, nq)
    # with k up to 16 among thousands of random candidates a few rows have a k-th gap
    # below 1e-5; the indices are compared on the others
    assert sep.mean() >= 0.5
    assert np.array_equal(i2.cpu().numpy()[sep], r_idx[sep])
    close("score", f64(s2), r_score, True, mask=sep)
    close("w", f64(w2), r_w, True, mask=sep)
    r_o, r_lse = orc.forward(f64(q), f64(kk), f64(v), i2.cpu().numpy(), f64(w2),
                             cfg["attn_scale"])
    close("o", f64(o2), r_o, True)
    compare_lse(l2, r_lse, True)
    if rule == "mixed":  # rows with no candidate: empty slots and O = 0
        none = np.nonzero(n_cand == 0)[0]
        for t in none:
            assert (i2.cpu().numpy()[0, 0, :, t] == -1).all()
            assert (f64(o2)[0, 0, :, t] == 0).all()


def test_retrieve_forward_rejects_before_launching():
    """A bad forward argument fails the call before the retrieval runs."""
    cfg = synth.workload("infer1m_step", H=1, n_query=1, n_key=2000)
    shape = shape_of(cfg)
    lq = torch.zeros((1, 1, 1, 1, 64), dtype=torch.bfloat16, device="cuda")
    lk = torch.zeros((1, 1, 1, 2000, 64), dtype=torch.bfloat16, device="cuda")
    q_pos = torch.full((1,), 2001, dtype=torch.int32, device="cuda")
    idx = torch.full((1, 1, 1, 1, 8), -7, dtype=torch.int32, device="cuda")
    score = torch.zeros((1, 1, 1, 1, 8), device="cuda")
    w = torch.zeros_like(score)
    q = torch.zeros((1, 1, 1, 1, 64, 64), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, 1, 1, 2000, 64, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gca.GcaError, match="o is NULL"):
        gca.gca_retrieve_forward(shape, lq, lk, q_pos, q, kv, kv, idx, score, w, None)
    torch.cuda.synchronize()
    assert (idx == -7).all()  # the retrieval did not run


@pytest.mark.parametrize("dtype_name", ["tiny_fp32", "bf16_no_lse"])
def test_retrieve_forward_other_paths(dtype_name):
    """float32 (the VALU kernels: two launches) and a fused bf16 call without L
    (lse = NULL): the same outputs as the two calls."""
    if dtype_name == "tiny_fp32":
        cfg = synth.workload("tiny_fp32")
        x = synth.training_inputs("tiny_fp32", accept=None)
    else:
        cfg = synth.workload("infer1m_step", H=2, n_query=2, n_key=3000)
        x = None
    rng = np.random.default_rng(5)
    G, B, H, nq, nk, S, D, Dl, k = (cfg[n] for n in ("G", "B", "H", "n_query", "n_key", "S",
                                                     "D", "Dl", "k"))
    bf = cfg["dtype"] == "bf16"
    tdt = torch.bfloat16 if bf else torch.float32

    def mk(*shape, scale):
        return torch.from_numpy(rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)).to(tdt)

    if x is not None:
        lq, lk, q, kk, v = x["lq"], x["lk"], x["q"], x["k"], x["v"]
        q_pos = x["q_pos"].numpy()
    else:
        lq, lk = mk(G, B, H, nq, Dl, scale=1 / 8), mk(G, B, H, nk, Dl, scale=1 / 8)
        q, kk, v = (mk(G, B, H, n, S, D, scale=cfg["value_scale"]) for n in (nq, nk, nk))
        q_pos = np.full(nq, nk + 1, dtype=np.int32)
    shape = shape_of(cfg)
    d = {name: dev(t) for name, t in dict(lq=lq, lk=lk, q=q, k=kk, v=v,
                                          q_pos=torch.from_numpy(q_pos)).items()}
    slots = (G, B, H, nq, k)
    i1 = torch.empty(slots, dtype=torch.int32, device="cuda")
    s1, w1 = torch.empty(slots, device="cuda"), torch.empty(slots, device="cuda")
    o1 = torch.empty(tuple(q.shape), dtype=tdt, device="cuda")
    l1 = torch.empty(slots + (S,), device="cuda")
    gca.gca_retrieve(shape, d["lq"], d["lk"], d["q_pos"], i1, s1, w1)
    gca.gca_forward(shape, d["q"], d["k"], d["v"], i1, w1, o1, l1)
    i2, s2, w2 = torch.full_like(i1, -7), torch.zeros_like(s1), torch.zeros_like(w1)
    o2 = torch.zeros_like(o1)
    lse2 = None if dtype_name == "bf16_no_lse" else torch.zeros_like(l1)
    gca.gca_retrieve_forward(shape, d["lq"], d["lk"], d["q_pos"], d["q"], d["k"], d["v"], i2, s2,
                             w2, o2, lse2)
    torch.cuda.synchronize()
    for name, a, b in (("idx", i1, i2), ("score", s1, s2), ("w", w1, w2), ("o", o1, o2)):
        assert torch.equal(a, b), name
    if lse2 is not None:
        assert torch.equal(l1, lse2)
    r_o, _ = orc.forward(f64(q), f64(kk), f64(v), i2.cpu().numpy(), f64(w2), cfg["attn_scale"])
    close("o", f64(o2), r_o, bf)


@pytest.mark.parametrize("seed", range(24))
def test_retrieve_forward_random_long_lists(seed):
    """Random decoding and tile shapes (1..64 query chunks, 257..30000 candidates,
    k 1..16, head_dim and landmark width 32 or 64, both weight variants, query
    positions anywhere from no candidate to past the end): the one call equals
    the two calls bit for bit, fused or not."""
    rng = np.random.default_rng(4000 + seed)
    H = int(rng.integers(1, 5))
    nq = int(rng.choice([1, 2, 3, 4, 5, 9, 17, 33, 40, 64]))
    nk, k = int(rng.integers(257, 30000)), int(rng.integers(1, 17))
    D, dl, s1 = int(rng.choice([32, 64])), int(rng.choice([32, 64])), int(rng.integers(2))
    print(f"[retrieve_forward random] seed {seed}: H={H} nq={nq} nk={nk} k={k} D={D} dl={dl} "
          f"softmax_one={s1}", flush=True)
    cfg = synth.workload("infer1m_step", H=H, n_query=nq, n_key=nk, k=k, D=D, Dl=dl,
                         softmax_one=s1)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)

    def draw(*shape, scale):
        return (torch.randn(shape, generator=gen, device="cuda") * scale).bfloat16()

    lq, lk = draw(1, 1, H, nq, dl, scale=1 / 8), draw(1, 1, H, nk, dl, scale=1 / 8)
    q, kk, v = (draw(1, 1, H, n, 64, D, scale=cfg["value_scale"]) for n in (nq, nk, nk))
    q_pos = torch.from_numpy(rng.integers(0, nk + 2, size=nq).astype(np.int32)).cuda()
    shape = shape_of(cfg)
    slots = (1, 1, H, nq, k)

    def outputs():
        return (torch.full(slots, -7, dtype=torch.int32, device="cuda"),
                torch.full(slots, 7.0, device="cuda"), torch.full(slots, 7.0, device="cuda"),
                torch.full(tuple(q.shape), 7.0, dtype=torch.bfloat16, device="cuda"),
                torch.full(slots + (64,), 7.0, device="cuda"))

    a = outputs()
    gca.gca_retrieve(shape, lq, lk, q_pos, a[0], a[1], a[2])
    gca.gca_forward(shape, q, kk, v, a[0], a[2], a[3], a[4])
    b = outputs()
    gca.gca_retrieve_forward(shape, lq, lk, q_pos, q, kk, v, *b)
    torch.cuda.synchronize()
    for name, x, y in zip(("idx", "score", "w", "o", "lse"), a, b):
        assert torch.equal(torch.nan_to_num(x.float()), torch.nan_to_num(y.float())), name
