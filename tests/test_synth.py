"""Input generator: determinism, the tie-avoidance rule and planted needles."""

import numpy as np
import torch

import synth
from oracle import condition
from oracle import gca_oracle as orc


def _accept(cfg):
    return lambda rows, cands, n: condition.gap_ok(rows, cands, n, cfg["k"],
                                                   cfg["score_scale"], 1e-3)


def test_deterministic_per_seed():
    a = synth.training_inputs("tiny_fp32")
    b = synth.training_inputs("tiny_fp32")
    for key in ("q", "k", "v", "lq", "lk", "dout"):
        assert torch.equal(a[key], b[key])
    c = synth.training_inputs("tiny_fp32", seed=99)
    assert not torch.equal(a["q"], c["q"])


def test_aliased_landmarks_layout():
    x = synth.training_inputs("tiny_fp32")
    assert torch.equal(x["lq"][..., 1:, :], x["lk"][..., :-1, :])
    assert x["q_pos"].tolist() == list(range(16))


def test_bf16_values_are_rounded_once():
    x = synth.training_inputs("train16k_fwd", H=1, B=1, n_query=32, n_key=32)
    assert x["q"].dtype == torch.bfloat16
    assert abs(float(x["q"].float().std()) - 0.125) < 0.01


def _check_gaps(x):
    cfg = x["cfg"]
    lq = x["lq"].double().numpy()
    lk = x["lk"].double().numpy()
    G, B, H, Nq, _ = lq.shape
    for g in range(G):
        for b in range(B):
            for h in range(H):
                for t in range(Nq):
                    n = orc.candidate_count(int(x["q_pos"][t]), lk.shape[3])
                    r = orc.relevance_scores(lq[g, b, h, t], lk[g, b, h, :n],
                                             cfg["score_scale"])
                    assert condition.kth_gap(r, cfg["k"]) >= 1e-3


def test_gap_rule_aliased():
    cfg = synth.workload("train16k_fwd", B=1, H=2, n_query=64, n_key=64)
    x = synth.training_inputs("train16k_fwd", accept=_accept(cfg), B=1, H=2,
                              n_query=64, n_key=64)
    _check_gaps(x)


def test_gap_rule_separate():
    cfg = synth.workload("train16k_fwdbwd_g2", B=1, H=2, n_query=48, n_key=48)
    x = synth.training_inputs("train16k_fwdbwd_g2", accept=_accept(cfg), B=1, H=2,
                              n_query=48, n_key=48)
    _check_gaps(x)


def test_needles_distinct_and_gap():
    over = dict(n_key=4096, H=2, n_query=8, q_pos=4097)
    cfg = synth.workload("retrieve16m", **over)
    lk = synth.context_landmarks("retrieve16m", **over)
    qb = synth.query_batch("retrieve16m", lk, accept=_accept(cfg), **over)
    assert len(set(qb["needle"].tolist())) == 8
    x = dict(lq=qb["lq"], lk=lk, q_pos=qb["q_pos"], cfg=cfg)
    _check_gaps(x)
    lq = qb["lq"].double().numpy()
    lk64 = lk.double().numpy()
    for h in range(2):
        for n in range(8):
            a = lq[0, 0, h, n]
            b = lk64[0, 0, h, int(qb["needle"][n])]
            cos = a @ b / np.linalg.norm(a) / np.linalg.norm(b)
            assert abs(cos - 0.9) < 0.02
