"""GPU check of multi-layer reuse within a group: one gca_retrieve feeds the
gca_forward / gca_backward_accumulate calls of L = 3 upper layers that share
K, V and the landmarks (paperlayer.ai summary, section 3.1; paperhub.cn reply
"Q2").  The library adds every layer's dK, dV, dw, dscore, dlq and dlk into
float32 accumulators; they must match the oracle's sums over the layers,
which tests/test_multilayer_pins.py pins to finite differences of the
composite loss.  Per-layer outputs (O, dQ) must match the oracle layer by
layer.  A second case runs the three layers over tiles packed once by
gca_gather_kv.
"""

import numpy as np
import pytest
import torch

import retrieval_sparse_attention_amd as gca
import synth
from oracle import gca_oracle as orc
from gpu_common import (accept_for, close, dev, f64, require_gpu, run_backward, run_forward,
                        run_retrieve, shape_of)

pytestmark = pytest.mark.gpu

SHARED = ("dk", "dv", "dw", "dscore", "dlq", "dlk")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _accumulators(shape, lq, lk):
    G, B, H, Nq, Nk, k = shape.G, shape.B, shape.H, shape.n_query, shape.n_key, shape.top_k
    S, D = shape.chunk_size, shape.head_dim
    z = lambda *dims: torch.zeros(dims, dtype=torch.float32, device="cuda")
    return dict(dk=z(G, B, H, Nk, S, D), dv=z(G, B, H, Nk, S, D), dw=z(G, B, H, Nq, k),
                dscore=z(G, B, H, Nq, k), dlq=z(*lq.shape), dlk=z(*lk.shape))


def _layers(name, L, **over):
    cfg = synth.workload(name, **over)
    base = synth.training_inputs(name, accept=accept_for(cfg), **over)
    layers = [base] + [synth.training_inputs(name, seed=100 + l, **over) for l in range(1, L)]
    return cfg, base, layers


def _group_step(shape, d, layers, idx, w, acc, k=None, v=None):
    """forward + backward_accumulate of every layer; returns per-layer (o, dq)."""
    k = d["k"] if k is None else k
    v = d["v"] if v is None else v
    outs = []
    for x in layers:
        q, do = dev(x["q"]), dev(x["dout"])
        o, lse = run_forward(shape, q, k, v, idx, w)
        dq = torch.full_like(q, float("nan"))
        gca.gca_backward_accumulate(shape, q, k, v, idx, w, lse, do, d["lq"], d["lk"], dq,
                                    acc["dk"], acc["dv"], acc["dw"], acc["dscore"], acc["dlq"],
                                    acc["dlk"])
        outs.append((o, dq))
    torch.cuda.synchronize()
    return outs


def _oracle_group(cfg, base, layers, r_idx, r_w):
    k64, v64, lq64, lk64 = f64(base["k"]), f64(base["v"]), f64(base["lq"]), f64(base["lk"])
    refs = {n: 0.0 for n in SHARED}
    per = []
    for x in layers:
        q64, do64 = f64(x["q"]), f64(x["dout"])
        r_o, _ = orc.forward(q64, k64, v64, r_idx, r_w, cfg["attn_scale"])
        r = orc.backward(q64, k64, v64, r_idx, r_w, do64, lq64, lk64, cfg["attn_scale"],
                         cfg["score_scale"])
        per.append((r_o, r["dq"]))
        for n in SHARED:
            refs[n] = refs[n] + r[n]
    return per, refs


@pytest.mark.parametrize("name,over", [
    ("train16k_fwdbwd_g2", dict(B=1, H=2, n_query=72, n_key=72)),
    ("train16k_fwdbwd_g2", dict(B=1, H=2, n_query=72, n_key=72, D=32)),
    ("train16k_fwdbwd_g2", dict(B=1, H=2, n_query=40, n_key=40, S=16, D=32)),
    ("train16k_fwdbwd_g2", dict(B=1, H=3, n_query=70, n_key=70, S=16, D=64)),
    ("tiny_fp32", dict(H=3)),
], ids=["bf16", "bf16_d32", "bf16_s16_d32", "bf16_s16_d64", "fp32"])
def test_one_retrieval_three_layers_accumulate(name, over):
    L = 3
    cfg, base, layers = _layers(name, L, **over)
    bf = cfg["dtype"] == "bf16"
    shape = shape_of(cfg)
    d = {key: dev(base[key]) for key in ("k", "v", "lq", "lk", "q_pos")}
    idx, _, w = run_retrieve(shape, d["lq"], d["lk"], d["q_pos"])
    r_idx, _, r_w = orc.retrieve(f64(base["lq"]), f64(base["lk"]), base["q_pos"].numpy(),
                                 cfg["k"], cfg["score_scale"], cfg["softmax_one"])
    assert np.array_equal(idx.cpu().numpy(), r_idx)
    acc = _accumulators(shape, d["lq"], d["lk"])
    # after the first layer the accumulators hold exactly what gca_backward writes
    x0 = layers[0]
    q0, do0 = dev(x0["q"]), dev(x0["dout"])
    o0, lse0 = run_forward(shape, q0, d["k"], d["v"], idx, w)
    single = run_backward(shape, q0, d["k"], d["v"], idx, w, lse0, do0, d["lq"], d["lk"])
    outs = _group_step(shape, d, layers[:1], idx, w, acc)
    for n in SHARED:
        got = acc[n].to(single[n].dtype) if n in ("dk", "dv") else acc[n]
        assert torch.equal(got, single[n]), f"{n}: one accumulated layer differs from gca_backward"
    assert torch.equal(outs[0][1], single["dq"])
    outs += _group_step(shape, d, layers[1:], idx, w, acc)
    per, refs = _oracle_group(cfg, base, layers, r_idx, r_w)
    for l, ((o, dq), (r_o, r_dq)) in enumerate(zip(outs, per)):
        close(f"o[layer {l}]", f64(o), r_o, bf)
        close(f"dq[layer {l}]", f64(dq), r_dq, bf)
    # each layer's gradient is held to the per-result bound (single layer: bit
    # for bit gca_backward's, checked above); their sum to L times it
    for n in SHARED:
        close(f"{n} accumulated over {L} layers", f64(acc[n]), refs[n], bf, terms=L)
    # the whole group again from zeroed accumulators: the same bits
    acc2 = _accumulators(shape, d["lq"], d["lk"])
    _group_step(shape, d, layers, idx, w, acc2)
    for n in SHARED:
        assert torch.equal(acc[n], acc2[n]), n


def test_one_gather_feeds_three_layers():
    """One retrieval and one gca_gather_kv (the packed tiles of the retrieved
    chunks) serve three layers' forward and backward.  Over the packed tiles,
    slot (t, i) owns packed row t*k + i, so a layer's dK/dV rows are per slot;
    the rows of the slots that retrieved chunk c add up to dK/dV of c."""
    L = 3
    cfg, base, layers = _layers("train16k_fwdbwd_g2", L, B=1, H=2, n_query=40, n_key=40)
    shape = shape_of(cfg)
    G, B, H, Nq, k = shape.G, shape.B, shape.H, shape.n_query, shape.top_k
    d = {key: dev(base[key]) for key in ("k", "v", "lq", "lk", "q_pos")}
    idx, _, w = run_retrieve(shape, d["lq"], d["lk"], d["q_pos"])
    r_idx, _, r_w = orc.retrieve(f64(base["lq"]), f64(base["lk"]), base["q_pos"].numpy(),
                                 cfg["k"], cfg["score_scale"], cfg["softmax_one"])
    assert np.array_equal(idx.cpu().numpy(), r_idx)
    kp = torch.empty((G, B, H, Nq * k, 64, 64), dtype=torch.bfloat16, device="cuda")
    vp = torch.empty_like(kp)
    ip = torch.empty_like(idx)
    gca.gca_gather_kv(shape, idx, d["k"], d["v"], kp, vp, ip)
    packed = gca.make_shape(G, B, H, Nq, Nq * k, 64, 64, cfg["Dl"], k, gca.GCA_BF16,
                            cfg["softmax_one"], cfg["attn_scale"], cfg["score_scale"])
    # dlk is per packed row here (its landmark is not gathered): not requested
    acc = _accumulators(packed, d["lq"], d["lk"][:, :, :, :0])
    outs = []
    for x in layers:
        q, do = dev(x["q"]), dev(x["dout"])
        o, lse = run_forward(packed, q, kp, vp, ip, w)
        dq = torch.empty_like(q)
        gca.gca_backward_accumulate(packed, q, kp, vp, ip, w, lse, do, None, None, dq,
                                    acc["dk"], acc["dv"], acc["dw"], acc["dscore"], None, None)
        outs.append((o, dq))
    torch.cuda.synchronize()
    per, refs = _oracle_group(cfg, base, layers, r_idx, r_w)
    for l, ((o, dq), (r_o, r_dq)) in enumerate(zip(outs, per)):
        close(f"o[layer {l}] (packed)", f64(o), r_o, True)
        close(f"dq[layer {l}] (packed)", f64(dq), r_dq, True)
    close("dw (packed)", f64(acc["dw"]), refs["dw"], True, terms=L)
    close("dscore (packed)", f64(acc["dscore"]), refs["dscore"], True, terms=L)
    # per-chunk dK/dV: the packed rows of the slots that hold each chunk
    ip_h = ip.cpu().numpy()
    dkp, dvp = f64(acc["dk"]), f64(acc["dv"])
    for name, rows, ref in (("dk", dkp, refs["dk"]), ("dv", dvp, refs["dv"])):
        per_chunk = np.zeros_like(ref)
        for g in range(G):
            for b in range(B):
                for h in range(H):
                    for t in range(Nq):
                        for i in range(k):
                            c = r_idx[g, b, h, t, i]
                            if c >= 0:
                                assert ip_h[g, b, h, t, i] == t * k + i
                                per_chunk[g, b, h, c] += rows[g, b, h, t * k + i]
        close(f"{name} over packed rows and layers", per_chunk, ref, True, terms=L)
