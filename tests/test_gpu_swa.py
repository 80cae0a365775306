"""GPU parity of the sliding-window self-attention (gca_swa_*) against the
float64 oracle (oracle/swa.py).

bf16 inputs, float32 accumulation: O, dQ, dK, dV and lse must meet the bf16
tolerances (2e-2 max-abs, 1e-2 mean-relative).  Small sequences are compared
element by element; the 16K-token training shape is compared on sampled rows
that the oracle computes one by one from their own windows.
"""

import numpy as np
import pytest
import torch

import retrieval_sparse_attention_amd as gca
import synth
from oracle import swa
from gpu_common import close, f64, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def run_swa(shape, x, backward=True):
    d = {key: val.contiguous().cuda() for key, val in x.items()}
    nan = float("nan")
    o = torch.full_like(d["q"], nan)
    lse = torch.full((shape.B, shape.H, shape.T), nan, dtype=torch.float32, device="cuda")
    gca.gca_swa_forward(shape, d["q"], d["k"], d["v"], o, lse)
    out = dict(o=o, lse=lse)
    if backward:
        dq, dk, dv = (torch.full_like(d["q"], nan) for _ in range(3))
        gca.gca_swa_backward(shape, d["q"], d["k"], d["v"], o, lse, d["dout"], dq, dk, dv)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {key: f64(val) for key, val in out.items()}


@pytest.mark.parametrize("B,H,T,W", [
    (1, 2, 64, 512),     # one block, window past the start
    (1, 2, 320, 512),    # window covers the sequence: causal attention
    (2, 3, 1024, 512),   # the pages' window, several full windows
    (1, 2, 640, 100),    # window not a multiple of 64
    (1, 2, 512, 64),     # window of exactly one block
    (1, 1, 384, 65),
    (1, 2, 256, 1),      # degenerate: every token sees itself only
    (1, 1, 192, 2 ** 31 - 1),  # the largest window: clamped to T, causal attention
])
def test_swa_parity(B, H, T, W):
    x = synth.swa_inputs(B, H, T, 64, seed=T + W)
    shape = gca.make_swa_shape(B, H, T, 64, W)
    got = run_swa(shape, x)
    q, k, v, do = (f64(x[n]) for n in ("q", "k", "v", "dout"))
    o, lse = swa.swa_forward(q, k, v, W, shape.scale)
    dq, dk, dv = swa.swa_backward(q, k, v, do, W, shape.scale)
    for name, ref in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        close(name, got[name], ref, True)


@pytest.mark.parametrize("seed", range(16))
def test_swa_random_shapes(seed):
    """Random B (1..2), H (1..3), T (64..1536 in blocks of 64) and window (1..1600,
    mostly not a multiple of 64): O, L and every gradient against the oracle.  With
    unit-variance inputs a window of a few tokens gives gradients up to ~6, where
    the output's own bf16 rounding (half an ulp, up to 2^-9 |x|) nearly fills the
    2e-2 max-abs bound; each element may then also differ by 2^-8 |x| (the
    output's rounding plus one rounding of a bf16 operand, P or dS)."""
    rng = np.random.default_rng(5000 + seed)
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    T, W = 64 * int(rng.integers(1, 25)), int(rng.integers(1, 1601))
    print(f"[swa random] seed {seed}: B={B} H={H} T={T} window={W}", flush=True)
    x = synth.swa_inputs(B, H, T, 64, seed=6000 + seed)
    shape = gca.make_swa_shape(B, H, T, 64, W)
    got = run_swa(shape, x)
    q, k, v, do = (f64(x[n]) for n in ("q", "k", "v", "dout"))
    o, lse = swa.swa_forward(q, k, v, W, shape.scale)
    dq, dk, dv = swa.swa_backward(q, k, v, do, W, shape.scale)
    for name, ref in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        close(name, got[name], ref, True, rel=2.0 ** -8)


def test_swa_empty_sequence_is_a_no_op():
    shape = gca.make_swa_shape(2, 2, 0, 64, 512)
    z = torch.empty((2, 2, 0, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((2, 2, 0), dtype=torch.float32, device="cuda")
    gca.gca_swa_forward(shape, z, z, z, z, lse)
    torch.cuda.synchronize()


def test_swa_rejects_unsupported_shapes():
    for bad in (gca.make_swa_shape(1, 1, 100, 64, 512), gca.make_swa_shape(1, 1, 128, 32, 512),
                gca.make_swa_shape(1, 1, 128, 64, 512, dtype=gca.GCA_F32)):
        with pytest.raises(gca.GcaError):
            gca.gca_swa_workspace_size(bad)
    with pytest.raises(gca.GcaError):
        gca.gca_swa_workspace_size(gca.make_swa_shape(1, 1, 128, 64, 0))


def test_swa_full_size_sampled_rows():
    """The 16K-token training shape (B=4, H=12, T=16384, W=512), in the launch
    configuration the benchmark times; rows sampled across heads, the first
    window, block edges and the end of the sequence."""
    cfg = synth.SWA_WORKLOADS["train16k_swa"]
    B, H, T, D, W = cfg["B"], cfg["H"], cfg["T"], cfg["D"], cfg["window"]
    x = synth.swa_inputs(B, H, T, D, cfg["seed"], device="cuda")
    shape = gca.make_swa_shape(B, H, T, D, W)
    o = torch.empty_like(x["q"])
    lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    gca.gca_swa_forward(shape, x["q"], x["k"], x["v"], o, lse)
    dq, dk, dv = (torch.empty_like(x["q"]) for _ in range(3))
    gca.gca_swa_backward(shape, x["q"], x["k"], x["v"], o, lse, x["dout"], dq, dk, dv)
    torch.cuda.synchronize()
    rows = [0, 1, 63, 64, 511, 512, 513, 4095, 8191, 12345, 16320, 16383]
    for (b, h) in [(0, 0), (1, 7), (3, 11)]:
        sl = lambda t: f64(t[b:b + 1, h:h + 1])
        q, k, v, do = sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["dout"])
        o_r, l_r, dq_r = swa.swa_query_rows(q, k, v, do, W, shape.scale, 0, 0, rows)
        dk_r, dv_r = swa.swa_key_rows(q, k, v, do, W, shape.scale, 0, 0, rows)
        close(f"o[{b},{h}]", f64(o[b, h, rows]), o_r, True)
        close(f"lse[{b},{h}]", f64(lse[b, h, rows]), l_r, True)
        close(f"dq[{b},{h}]", f64(dq[b, h, rows]), dq_r, True)
        close(f"dk[{b},{h}]", f64(dk[b, h, rows]), dk_r, True)
        close(f"dv[{b},{h}]", f64(dv[b, h, rows]), dv_r, True)
    for t in (o, lse, dq, dk, dv):
        assert torch.isfinite(t).all()
