"""HIP-graph capture of the GCA step (torch.cuda.CUDAGraph on torch's stream):
the library's calls enqueue only kernels, so one training step (retrieve +
forward + backward) can be captured and replayed.  Every replay, with eager
work and synchronisations between replays, must reproduce the eager step's
outputs bit for bit (same kernels, same fixed summation order)."""

import threading

import pytest
import torch

import retrieval_sparse_attention_amd as gca
import synth
from gpu_common import accept_for, dev, require_gpu, shape_of

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def test_training_step_replays_match_eager():
    name, over = "train16k_fwdbwd_g2", dict(B=1, H=2, n_query=72, n_key=72)
    cfg = synth.workload(name, **over)
    x = synth.training_inputs(name, accept=accept_for(cfg), **over)
    shape = shape_of(cfg)
    d = {key: dev(x[key]) for key in ("q", "k", "v", "lq", "lk", "dout", "q_pos")}
    G, B, H, Nq, k = shape.G, shape.B, shape.H, shape.n_query, shape.top_k
    out = dict(idx=torch.empty((G, B, H, Nq, k), dtype=torch.int32, device="cuda"),
               score=torch.empty((G, B, H, Nq, k), device="cuda"),
               w=torch.empty((G, B, H, Nq, k), device="cuda"),
               o=torch.empty_like(d["q"]),
               lse=torch.empty((G, B, H, Nq, k, 64), device="cuda"),
               dq=torch.empty_like(d["q"]), dk=torch.empty_like(d["k"]),
               dv=torch.empty_like(d["v"]),
               dw=torch.empty((G, B, H, Nq, k), device="cuda"),
               dscore=torch.empty((G, B, H, Nq, k), device="cuda"),
               dlq=torch.empty(tuple(d["lq"].shape), device="cuda"),
               dlk=torch.empty(tuple(d["lk"].shape), device="cuda"))
    wsr = torch.empty(max(256, gca.gca_workspace_size(shape, gca.OP_RETRIEVE)),
                      dtype=torch.uint8, device="cuda")
    wsb = torch.empty(gca.gca_workspace_size(shape, gca.OP_BACKWARD), dtype=torch.uint8,
                      device="cuda")

    def step():
        gca.gca_retrieve(shape, d["lq"], d["lk"], d["q_pos"], out["idx"], out["score"],
                         out["w"], ws=wsr)
        gca.gca_forward(shape, d["q"], d["k"], d["v"], out["idx"], out["w"], out["o"],
                        out["lse"])
        gca.gca_backward(shape, d["q"], d["k"], d["v"], out["idx"], out["w"], out["lse"],
                         d["dout"], d["lq"], d["lk"], out["dq"], out["dk"], out["dv"],
                         out["dw"], out["dscore"], out["dlq"], out["dlk"], ws=wsb)

    step()
    torch.cuda.synchronize()
    eager = {key: val.clone() for key, val in out.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        for val in out.values():
            val.fill_(7)  # eager work between replays; every output must be rewritten
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for key, val in out.items():
            assert torch.equal(val, eager[key]), (r, key)


def test_decoding_steps_replay_through_the_one_call():
    """Three decoding steps (one query chunk per head over a 3000-chunk context,
    so that the retrieval is sliced and its merge runs inside the forward's
    kernel) through gca_retrieve_forward, captured in one graph: every replay,
    with eager work between replays, reproduces the eager steps' bits."""
    cfg = synth.workload("infer1m_step", H=3, n_query=1, n_key=3000)
    shape = shape_of(cfg)
    gen = torch.Generator().manual_seed(11)
    H, nk, steps = 3, 3000, 3

    def mk(*shp, scale):
        return (torch.randn(*shp, generator=gen) * scale).bfloat16().cuda()

    lk = mk(1, 1, H, nk, 64, scale=1 / 8)
    kk, v = mk(1, 1, H, nk, 64, 64, scale=0.125), mk(1, 1, H, nk, 64, 64, scale=0.125)
    lqs = [mk(1, 1, H, 1, 64, scale=1 / 8) for _ in range(steps)]
    qs = [mk(1, 1, H, 1, 64, 64, scale=0.125) for _ in range(steps)]
    q_pos = torch.full((1,), nk + 1, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(256, gca.gca_workspace_size(shape, gca.OP_RETRIEVE)), dtype=torch.uint8,
                     device="cuda")
    out = [dict(idx=torch.empty((1, 1, H, 1, 8), dtype=torch.int32, device="cuda"),
                score=torch.empty((1, 1, H, 1, 8), device="cuda"),
                w=torch.empty((1, 1, H, 1, 8), device="cuda"),
                o=torch.empty_like(qs[0]), lse=torch.empty((1, 1, H, 1, 8, 64), device="cuda"))
           for _ in range(steps)]

    def body():
        for s in range(steps):
            b = out[s]
            gca.gca_retrieve_forward(shape, lqs[s], lk, q_pos, qs[s], kk, v, b["idx"], b["score"],
                                     b["w"], b["o"], b["lse"], ws=ws)

    body()
    torch.cuda.synchronize()
    eager = [{key: val.clone() for key, val in b.items()} for b in out]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        body()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    torch.cuda.synchronize()
    for r in range(4):
        for b in out:
            for val in b.values():
                val.fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for s in range(steps):
            for key, val in out[s].items():
                assert torch.equal(val, eager[s][key]), (r, s, key)


def test_eager_backward_in_another_thread_during_a_capture():
    """A backward being captured on one thread and an eager backward on another
    thread's stream at the same time: each call enqueues on its own stream only,
    so the capture holds none of the eager call's work.  Replays and the eager
    call reproduce the reference bits."""
    name, over = "train16k_fwdbwd_g2", dict(B=1, H=2, n_query=72, n_key=72)
    cfg = synth.workload(name, **over)
    x = synth.training_inputs(name, accept=accept_for(cfg), **over)
    shape = shape_of(cfg)
    d = {key: dev(x[key]) for key in ("q", "k", "v", "lq", "lk", "dout", "q_pos")}
    G, B, H, Nq, k = shape.G, shape.B, shape.H, shape.n_query, shape.top_k
    idx = torch.empty((G, B, H, Nq, k), dtype=torch.int32, device="cuda")
    score = torch.empty((G, B, H, Nq, k), device="cuda")
    w = torch.empty_like(score)
    lse = torch.empty((G, B, H, Nq, k, 64), device="cuda")
    o = torch.empty_like(d["q"])
    gca.gca_retrieve(shape, d["lq"], d["lk"], d["q_pos"], idx, score, w)
    gca.gca_forward(shape, d["q"], d["k"], d["v"], idx, w, o, lse)
    torch.cuda.synchronize()

    def buffers():
        return dict(dq=torch.empty_like(d["q"]), dk=torch.empty_like(d["k"]),
                    dv=torch.empty_like(d["v"]), dw=torch.empty_like(w),
                    dscore=torch.empty_like(w), dlq=torch.empty(tuple(d["lq"].shape), device="cuda"),
                    dlk=torch.empty(tuple(d["lk"].shape), device="cuda"),
                    ws=torch.empty(gca.gca_workspace_size(shape, gca.OP_BACKWARD),
                                   dtype=torch.uint8, device="cuda"))

    def backward(b):
        gca.gca_backward(shape, d["q"], d["k"], d["v"], idx, w, lse, d["dout"], d["lq"], d["lk"],
                         b["dq"], b["dk"], b["dv"], b["dw"], b["dscore"], b["dlq"], b["dlk"],
                         ws=b["ws"])

    ref = buffers()
    backward(ref)
    torch.cuda.synchronize()
    cap, eager = buffers(), buffers()
    eager_stream = torch.cuda.Stream()
    errors = []

    def eager_call():
        try:
            with torch.cuda.stream(eager_stream):
                backward(eager)
            eager_stream.synchronize()
        except Exception as e:  # reported below, on the main thread
            errors.append(e)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        backward(cap)  # warm-up of the capture's buffers, as torch recommends
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="thread_local"):
        backward(cap)
        t = threading.Thread(target=eager_call)
        t.start()
        t.join()
    assert not errors, errors
    torch.cuda.synchronize()
    for key in ("dq", "dk", "dv", "dw", "dscore", "dlq", "dlk"):
        assert torch.equal(eager[key], ref[key]), ("eager", key)
    for r in range(3):
        for key in ("dq", "dk", "dv", "dw", "dscore", "dlq", "dlk"):
            cap[key].fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for key in ("dq", "dk", "dv", "dw", "dscore", "dlq", "dlk"):
            assert torch.equal(cap[key], ref[key]), (r, key)
