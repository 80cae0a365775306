"""NaN propagation through the attention path: a NaN planted in one element of
Q, K, V (forward) or dO (backward) must reach exactly the outputs that depend
on it, as in the float64 oracle, so that a diverging training step shows up in
O, LSE and the gradients instead of being masked.  Every other element still
meets the bf16 tolerance.

Where each NaN goes (per-chunk attention and fusion, long-context-modeling
README, "Model Architecture"; backward, paperlayer.ai summary, appendix B):
  Q[t][x][d]  -> row x of O[t] and of L for every slot of t;
  K[c][j][d]  -> every row of O and L of the slots that retrieved c;
  V[c][j][d]  -> column d of O[t] for every t that retrieved c;
  dO[t][x][d] -> dQ, dw, dscore and dlq of t, and dK, dV, dlk of the
                 chunks t retrieved (in the oracle's pattern).
"""

import numpy as np
import pytest
import torch

import retrieval_sparse_attention_amd as gca
import synth
from oracle import gca_oracle as orc
from gpu_common import close, dev, f64, require_gpu, run_backward, run_forward, shape_of

pytestmark = pytest.mark.gpu

NQ, NK = 6, 10


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _inputs(seed, S=64, D=64):
    cfg = synth.workload("train16k_fwdbwd_g2", G=1, B=1, H=1, n_query=NQ, n_key=NK, S=S, D=D)
    rng = np.random.default_rng(seed)
    sc = cfg["value_scale"]
    mk = lambda *s: (rng.standard_normal(s) * sc).astype(np.float32)
    x = dict(q=mk(1, 1, 1, NQ, S, D), k=mk(1, 1, 1, NK, S, D), v=mk(1, 1, 1, NK, S, D),
             dout=mk(1, 1, 1, NQ, S, D), lq=mk(1, 1, 1, NQ, 64), lk=mk(1, 1, 1, NK, 64))
    # query chunk t retrieves chunks t, t+1, t+2, t+3 (chunk 2 by t = 0, 1, 2)
    idx = np.full((1, 1, 1, NQ, 8), -1, np.int32)
    for t in range(NQ):
        idx[0, 0, 0, t, :4] = [t, t + 1, t + 2, t + 3]
    w = (rng.random((1, 1, 1, NQ, 8)) / 4).astype(np.float32)
    return cfg, x, idx, w


def _bf16(a):
    return torch.from_numpy(a).bfloat16()


def _same_nan_pattern(name, got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert np.isnan(ref).any(), f"{name}: the oracle shows no NaN (test setup)"
    assert np.array_equal(np.isnan(got), np.isnan(ref)), (
        f"{name}: NaN pattern differs ({int(np.isnan(got).sum())} vs {int(np.isnan(ref).sum())})")
    # infinities (LSE of empty slots) must coincide too
    num = ~np.isnan(ref)
    assert np.array_equal(got[num & np.isinf(ref)], ref[num & np.isinf(ref)]), f"{name}: inf differs"
    assert np.isfinite(got[num & np.isfinite(ref)]).all(), f"{name}: inf where the oracle is finite"
    close(name, got, ref, True, mask=np.isfinite(ref))


# the 64-token MFMA kernels, the 16-token ones and the half-width rows
SIZES = [(64, 64), (16, 64), (16, 32)]


@pytest.mark.parametrize("S,D", SIZES, ids=["s64_d64", "s16_d64", "s16_d32"])
@pytest.mark.parametrize("where", ["q", "k", "v"])
def test_forward_nan_reaches_its_outputs(where, S, D):
    cfg, x, idx, w = _inputs(5, S, D)
    pos = {"q": (0, 0, 0, 1, 7, 3), "k": (0, 0, 0, 2, 11, 20), "v": (0, 0, 0, 2, 11, 20)}[where]
    x[where][pos] = np.nan
    t = {key: _bf16(x[key]) for key in ("q", "k", "v")}
    shape = shape_of(cfg)
    o, lse = run_forward(shape, dev(t["q"]), dev(t["k"]), dev(t["v"]), dev(torch.from_numpy(idx)),
                         dev(torch.from_numpy(w)))
    r_o, r_lse = orc.forward(f64(t["q"]), f64(t["k"]), f64(t["v"]), idx, w.astype(np.float64),
                             cfg["attn_scale"])
    _same_nan_pattern("o", f64(o), r_o)
    if where != "v":
        _same_nan_pattern("lse", f64(lse), r_lse)


@pytest.mark.parametrize("S,D", SIZES, ids=["s64_d64", "s16_d64", "s16_d32"])
def test_backward_nan_in_dout_reaches_its_gradients(S, D):
    cfg, x, idx, w = _inputs(6, S, D)
    x["dout"][0, 0, 0, 3, 12, 5] = np.nan
    t = {key: _bf16(x[key]) for key in ("q", "k", "v", "dout", "lq", "lk")}
    shape = shape_of(cfg)
    d = {key: dev(val) for key, val in t.items()}
    di, dw = dev(torch.from_numpy(idx)), dev(torch.from_numpy(w))
    o, lse = run_forward(shape, d["q"], d["k"], d["v"], di, dw)
    g = run_backward(shape, d["q"], d["k"], d["v"], di, dw, lse, d["dout"], d["lq"], d["lk"])
    r = orc.backward(f64(t["q"]), f64(t["k"]), f64(t["v"]), idx, w.astype(np.float64),
                     f64(t["dout"]), f64(t["lq"]), f64(t["lk"]), cfg["attn_scale"],
                     cfg["score_scale"])
    for key in ("dq", "dk", "dv", "dw", "dscore", "dlq", "dlk"):
        _same_nan_pattern(key, f64(g[key]), r[key])
