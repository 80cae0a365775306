"""Helpers shared by the GPU parity tests: run the library, compare with the oracle."""

import numpy as np
import torch

import retrieval_sparse_attention_amd as gca
from oracle import condition

BF16_MAX_ABS = 2e-2   # bf16 tolerances: max-abs and mean-relative
BF16_MEAN_REL = 1e-2
F32_MAX_ABS = 1e-5    # float32 tolerance: max-abs


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm device")
    gca.load()


def accept_for(cfg):
    return lambda rows, cands, n: condition.gap_ok(rows, cands, n, cfg["k"],
                                                   cfg["score_scale"], 1e-3)


def shape_of(cfg, n_query=None, n_key=None):
    return gca.make_shape(cfg["G"], cfg["B"], cfg["H"],
                          cfg["n_query"] if n_query is None else n_query,
                          cfg["n_key"] if n_key is None else n_key,
                          cfg["S"], cfg["D"], cfg["Dl"], cfg["k"],
                          gca.GCA_BF16 if cfg["dtype"] == "bf16" else gca.GCA_F32,
                          cfg["softmax_one"], cfg["attn_scale"], cfg["score_scale"])


def dev(t):
    return t.contiguous().to("cuda")


def f64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def run_retrieve(shape, lq, lk, q_pos):
    G, B, H, Nq, k = shape.G, shape.B, shape.H, shape.n_query, shape.top_k
    idx = torch.full((G, B, H, Nq, k), -7, dtype=torch.int32, device="cuda")
    score = torch.full((G, B, H, Nq, k), float("nan"), dtype=torch.float32, device="cuda")
    w = torch.full((G, B, H, Nq, k), float("nan"), dtype=torch.float32, device="cuda")
    gca.gca_retrieve(shape, lq, lk, q_pos, idx, score, w)
    return idx, score, w


def run_forward(shape, q, k, v, idx, w):
    o = torch.full_like(q, float("nan"))
    lse = torch.full((shape.G, shape.B, shape.H, shape.n_query, shape.top_k, shape.chunk_size),
                     float("nan"), dtype=torch.float32, device="cuda")
    gca.gca_forward(shape, q, k, v, idx, w, o, lse)
    return o, lse


def run_backward(shape, q, k, v, idx, w, lse, dout, lq, lk):
    G, B, H, Nq, Nk, k_ = shape.G, shape.B, shape.H, shape.n_query, shape.n_key, shape.top_k
    nan = float("nan")
    dq = torch.full_like(q, nan)
    dk = torch.full_like(k, nan)
    dv = torch.full_like(v, nan)
    dw = torch.full((G, B, H, Nq, k_), nan, dtype=torch.float32, device="cuda")
    dscore = torch.full_like(dw, nan)
    dlq = torch.full(tuple(lq.shape), nan, dtype=torch.float32, device="cuda")
    dlk = torch.full(tuple(lk.shape), nan, dtype=torch.float32, device="cuda")
    gca.gca_backward(shape, q, k, v, idx, w, lse, dout, lq, lk, dq, dk, dv, dw, dscore, dlq, dlk)
    return dict(dq=dq, dk=dk, dv=dv, dw=dw, dscore=dscore, dlq=dlq, dlk=dlk)


def close(name, got, ref, is_bf16_out, mask=None, terms=1, rel=0.0):
    """Asserts the tolerance for one tensor; returns (max_abs, mean_rel).

    terms > 1: `got` is a sum of that many results each held to the bound (a
    group's layers), so the max-abs bound is terms times the per-result one.
    rel > 0 (bf16 outputs): each element may also differ by rel * |ref|, the
    relative rounding of bf16 results and operands for elements well above 1,
    where the fixed max-abs bound (sized for values of order 1) is less than
    the output's own half ulp plus one operand rounding."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    if mask is not None:
        got, ref = got[mask], ref[mask]
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    if got.size == 0:
        return 0.0, 0.0
    err = np.abs(got - ref)
    max_abs = float(err.max())
    denom = float(np.abs(ref).mean())
    mean_rel = float(err.mean() / denom) if denom > 0 else float(err.mean())
    if is_bf16_out:
        bound = terms * BF16_MAX_ABS
        excess = float((err - rel * np.abs(ref)).max())
        assert excess <= bound, f"{name}: max-abs {max_abs:.3g} (beyond {rel:g}|ref|: {excess:.3g}) > {bound}"
        assert mean_rel <= BF16_MEAN_REL, f"{name}: mean-rel {mean_rel:.3g} > {BF16_MEAN_REL}"
    else:
        bound = terms * F32_MAX_ABS
        assert max_abs <= bound, f"{name}: max-abs {max_abs:.3g} > {bound}"
    return max_abs, mean_rel


def compare_lse(got, ref, is_bf16):
    got = f64(got)
    inf_g, inf_r = np.isneginf(got), np.isneginf(ref)
    assert (inf_g == inf_r).all(), "lse: empty-slot pattern differs"
    return close("lse", got, ref, is_bf16, mask=~inf_r)
