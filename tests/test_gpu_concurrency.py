"""Concurrent callers: the library keeps no stream, event or lock of its own for
gca_backward, so two host threads that call the backward at the same time on
their own streams (ctypes drops the GIL during each call) must each get exactly
the bits a lone call gives."""

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


def _problem(seed):
    name, over = "train16k_fwdbwd_g2", dict(B=1, H=2, n_query=72, n_key=72)
    cfg = synth.workload(name, **over)
    x = synth.training_inputs(name, seed=seed, accept=accept_for(cfg), **over)
    shape = shape_of(cfg)
    d = {key: dev(x[key]) for key in ("q", "k", "v", "lq", "lk", "dout", "q_pos")}
    G, B, H, Nq, k = shape.G, shape.B, shape.H, shape.n_query, shape.top_k
    d["idx"] = torch.empty((G, B, H, Nq, k), dtype=torch.int32, device="cuda")
    d["score"] = torch.empty((G, B, H, Nq, k), device="cuda")
    d["w"] = torch.empty((G, B, H, Nq, k), device="cuda")
    d["o"] = torch.empty_like(d["q"])
    d["lse"] = torch.empty((G, B, H, Nq, k, 64), device="cuda")
    gca.gca_retrieve(shape, d["lq"], d["lk"], d["q_pos"], d["idx"], d["score"], d["w"])
    gca.gca_forward(shape, d["q"], d["k"], d["v"], d["idx"], d["w"], d["o"], d["lse"])
    torch.cuda.synchronize()
    return shape, d


def _outputs(d):
    return dict(dq=torch.empty_like(d["q"]), dk=torch.empty_like(d["k"]),
                dv=torch.empty_like(d["v"]), dw=torch.empty_like(d["w"]),
                dscore=torch.empty_like(d["w"]),
                dlq=torch.empty(tuple(d["lq"].shape), device="cuda"),
                dlk=torch.empty(tuple(d["lk"].shape), device="cuda"))


def _backward(shape, d, out, ws):
    gca.gca_backward(shape, d["q"], d["k"], d["v"], d["idx"], d["w"], d["lse"], d["dout"],
                     d["lq"], d["lk"], out["dq"], out["dk"], out["dv"], out["dw"],
                     out["dscore"], out["dlq"], out["dlk"], ws=ws)


def test_two_threads_two_streams():
    probs = [_problem(3), _problem(4)]
    ref = []
    for shape, d in probs:
        out = _outputs(d)
        ws = torch.empty(gca.gca_workspace_size(shape, gca.OP_BACKWARD), dtype=torch.uint8,
                         device="cuda")
        _backward(shape, d, out, ws)
        torch.cuda.synchronize()
        ref.append(out)
    errors = []

    def worker(i):
        try:
            shape, d = probs[i]
            stream = torch.cuda.Stream()
            out = _outputs(d)
            ws = torch.empty(gca.gca_workspace_size(shape, gca.OP_BACKWARD),
                             dtype=torch.uint8, device="cuda")
            torch.cuda.synchronize()
            with torch.cuda.stream(stream):
                for _ in range(20):
                    for val in out.values():
                        val.fill_(7)
                    _backward(shape, d, out, ws)
            stream.synchronize()
            for key, val in out.items():
                if not torch.equal(val, ref[i][key]):
                    errors.append((i, key))
        except Exception as e:  # reported below, on the main thread
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads)
    assert not errors, errors
