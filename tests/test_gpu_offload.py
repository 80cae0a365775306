"""GPU parity of gca_gather_kv (retrieved K/V tiles from offloaded memory).

The gather is byte movement, so the packed tiles and indices must equal the
oracle's (oracle/offload.py) bit for bit, with K/V in device memory and in
pinned host memory alike.  Attention over the packed tiles must then give
exactly the bits of attention over the resident tiles: every slot sees the
same tile bytes and weight, in the same order.
"""

import ctypes

import numpy as np
import pytest
import torch

import retrieval_sparse_attention_amd as gca
import synth
from oracle import offload
from gpu_common import dev, require_gpu, run_forward, run_retrieve, shape_of

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _bits(t):
    """Integer view of a tensor's bytes (bf16 -> int16, f32 -> int32) on the host."""
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).numpy()


def run_gather(shape, idx, k, v):
    G, B, H, Nq, kk = shape.G, shape.B, shape.H, shape.n_query, shape.top_k
    S, D = shape.chunk_size, shape.head_dim
    dt = torch.bfloat16 if shape.dtype == gca.GCA_BF16 else torch.float32
    kp = torch.full((G, B, H, Nq * kk, S, D), 7.0, dtype=dt, device="cuda")
    vp = torch.full_like(kp, 7.0)
    ip = torch.full((G, B, H, Nq, kk), -7, dtype=torch.int32, device="cuda")
    gca.gca_gather_kv(shape, idx, k, v, kp, vp, ip)
    torch.cuda.synchronize()
    return kp, vp, ip


def packed_shape(shape):
    return gca.make_shape(shape.G, shape.B, shape.H, shape.n_query,
                          shape.n_query * shape.top_k, shape.chunk_size, shape.head_dim,
                          shape.landmark_dim, shape.top_k, shape.dtype, shape.softmax_one,
                          shape.attn_scale, shape.score_scale)


def _case(name, **over):
    cfg = synth.workload(name, **over)
    x = synth.training_inputs(name, with_dout=False, **over)
    shape = shape_of(cfg)
    d = {key: dev(x[key]) for key in ("q", "k", "v", "lq", "lk", "q_pos")}
    idx, _, w = run_retrieve(shape, d["lq"], d["lk"], d["q_pos"])
    # plant slots the gather must treat as empty: -1, past n_key, negative
    idx = idx.clone()
    idx[..., 0, :] = -1
    flat = idx.view(-1, shape.top_k)
    flat[1::7, 0] = shape.n_key
    flat[2::9, -1] = -5
    return cfg, x, shape, d, idx, w


def _check_gather(shape, x, idx, got):
    kp, vp, ip = got
    rk, rv, ri = offload.gather_kv(idx.cpu().numpy(), _bits(x["k"]), _bits(x["v"]))
    assert np.array_equal(ip.cpu().numpy(), ri)
    assert np.array_equal(_bits(kp), rk)
    assert np.array_equal(_bits(vp), rv)


@pytest.mark.parametrize("name,over", [
    ("train16k_fwdbwd_g2", dict(B=1, H=2, n_query=72, n_key=72)),
    ("tiny_fp32", dict(n_query=21, n_key=21, S=5, D=7, Dl=9, k=3, H=3)),
    ("tiny_fp32", {}),
])
def test_gather_from_device_memory(name, over):
    cfg, x, shape, d, idx, w = _case(name, **over)
    got = run_gather(shape, idx, d["k"], d["v"])
    _check_gather(shape, x, idx, got)
    # attention over the packed tiles == attention over the resident tiles, bit for bit
    o_ref, lse_ref = run_forward(shape, d["q"], d["k"], d["v"], idx, w)
    o_pk, lse_pk = run_forward(packed_shape(shape), d["q"], got[0], got[1], got[2], w)
    assert np.array_equal(_bits(o_pk), _bits(o_ref))
    assert np.array_equal(_bits(lse_pk), _bits(lse_ref))


def test_gather_from_pinned_host_memory():
    cfg, x, shape, d, idx, w = _case("train16k_fwdbwd_g2", B=2, H=3, n_query=64, n_key=64)
    kh = torch.empty(tuple(x["k"].shape), dtype=x["k"].dtype, pin_memory=True)
    vh = torch.empty(tuple(x["v"].shape), dtype=x["v"].dtype, pin_memory=True)
    kh.copy_(x["k"])
    vh.copy_(x["v"])
    assert kh.is_pinned() and vh.is_pinned()
    got_host = run_gather(shape, idx, kh, vh)
    _check_gather(shape, x, idx, got_host)
    got_dev = run_gather(shape, idx, d["k"], d["v"])
    for a, b in zip(got_host, got_dev):
        assert torch.equal(a, b)


def test_unregistered_host_memory_is_refused():
    cfg, x, shape, d, idx, w = _case("train16k_fwdbwd_g2", B=1, H=1, n_query=8, n_key=8)
    plain = np.zeros(x["k"].numel() + 64, dtype=np.uint16)  # ordinary (unpinned) host memory
    addr = plain.ctypes.data
    addr += (-addr) % 16
    kp = torch.zeros((1, 1, 1, 8 * shape.top_k, 64, 64), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    ip = torch.zeros((1, 1, 1, 8, shape.top_k), dtype=torch.int32, device="cuda")
    lib = gca.load()
    P = ctypes.c_void_p
    st = lib.gca_gather_kv(ctypes.byref(shape), P(idx.data_ptr()), P(addr), P(d["v"].data_ptr()),
                           P(kp.data_ptr()), P(vp.data_ptr()), P(ip.data_ptr()), None)
    assert st == 1, gca.gca_last_error()
    assert "pinned" in gca.gca_last_error()
    torch.cuda.synchronize()
    assert int(ip.abs().sum()) == 0  # nothing was launched


def test_gather_full_size_infer1m_from_host():
    """The 1M-token inference step's shape: 16384 resident chunks per head in pinned
    host memory (3.2 GB), 8 retrieved tiles for each of 12 heads."""
    name = "infer1m_step"
    cfg = synth.workload(name)
    lk = synth.context_landmarks(name)
    kd, vd = synth.device_kv(name, "cuda")
    kh = torch.empty(tuple(kd.shape), dtype=kd.dtype, pin_memory=True)
    vh = torch.empty(tuple(vd.shape), dtype=vd.dtype, pin_memory=True)
    kh.copy_(kd)
    vh.copy_(vd)
    del kd, vd
    torch.cuda.empty_cache()
    shape = gca.make_shape(1, 1, cfg["H"], 1, cfg["n_key"], 64, 64, 64, cfg["k"], gca.GCA_BF16, 0)
    for step in (0, 1):
        qb = synth.query_batch(name, lk, step=step)
        idx, _, _ = run_retrieve(shape, dev(qb["lq"]), dev(lk), dev(qb["q_pos"]))
        kp, vp, ip = run_gather(shape, idx, kh, vh)
        rk, rv, ri = offload.gather_kv(idx.cpu().numpy(), kh.view(torch.int16).numpy(),
                                       vh.view(torch.int16).numpy())
        assert np.array_equal(ip.cpu().numpy(), ri)
        assert np.array_equal(_bits(kp), rk)
        assert np.array_equal(_bits(vp), rv)


def test_gather_with_no_resident_chunks():
    # n_key = 0: every slot is empty, k and v may be NULL
    shape = gca.make_shape(1, 2, 2, 3, 0, 64, 64, 64, 4, gca.GCA_BF16, 0)
    idx = torch.full((1, 2, 2, 3, 4), 5, dtype=torch.int32, device="cuda")
    kp = torch.full((1, 2, 2, 12, 64, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    vp = torch.full_like(kp, 7.0)
    ip = torch.zeros((1, 2, 2, 3, 4), dtype=torch.int32, device="cuda")
    gca.gca_gather_kv(shape, idx, None, None, kp, vp, ip)
    torch.cuda.synchronize()
    assert torch.all(ip == -1)
    assert torch.all(kp == 0) and torch.all(vp == 0)
