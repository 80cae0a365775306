"""Host-side logic of bench.py (no GPU): the one-GPU guard and the algorithmic
work model the roofline fractions are computed from."""

import os
import subprocess
import sys

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""


def test_swa_pairs_brute_force():
    for T, W in [(1, 1), (7, 3), (64, 64), (100, 17), (300, 512)]:
        brute = sum(1 for x in range(T) for y in range(T) if x - W < y <= x)
        assert bench.swa_pairs(T, W) == brute


def test_training_step_work_model():
    """The G=2 16K step: 192384 (query chunk, slot) pairs; each kernel's bytes and flops
    counted here independently from the tensor shapes."""
    cfg = synth.workload("train16k_fwdbwd_g2")
    G, B, H, Nq, Nk = cfg["G"], cfg["B"], cfg["H"], cfg["n_query"], cfg["n_key"]
    S, D, Dl, k = cfg["S"], cfg["D"], cfg["Dl"], cfg["k"]
    heads = G * B * H
    pairs = heads * sum(min(k, max(0, t - 1)) for t in range(Nq))
    assert pairs == 192384
    work = bench.kernel_work(cfg, pairs)
    tile = S * D * 2                      # bf16 bytes of one chunk tile
    q_bytes = heads * Nq * tile           # Q, dO, O, dQ alike
    kv_bytes = heads * Nk * tile          # K, V, dK, dV alike
    slots = heads * Nq * k
    lse = slots * S * 4
    # forward: read Q, K, V; write O and LSE; idx and w
    assert work["forward"]["bytes"] == 2 * q_bytes + 2 * kv_bytes + lse + slots * 8
    assert work["forward"]["flops"] == pairs * 2 * (2 * S * S * D)
    assert work["backward_q"]["flops"] == pairs * 3 * (2 * S * S * D)
    assert work["backward_kv"]["flops"] == pairs * 4 * (2 * S * S * D)
    # the committed HBM-traffic summary was scaled against the same model
    import json
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        rec = json.load(f)
    for name in ("scan_topk", "forward", "reverse_index", "backward_q", "backward_kv"):
        assert rec[f"{name}@train16k_fwdbwd_g2"]["algorithmic_bytes"] == work[name]["bytes"]


def test_fraction_of_measured_peak():
    """A roofline entry gains its achieved rate over the measured peak of its own bound."""
    peaks = {"hbm_read_GBps": 6000.0, "mfma_bf16_dense_TFLOPs": 2000.0}
    hbm = bench.with_measured(dict(bound="hbm", achieved=3000.0), peaks)
    assert hbm["measured_peak"] == 6000.0 and hbm["frac_of_measured_peak"] == 0.5
    mf = bench.with_measured(dict(bound="mfma", achieved=500.0), peaks)
    assert mf["measured_peak"] == 2000.0 and mf["frac_of_measured_peak"] == 0.25
    assert bench.with_measured(dict(bound="hbm", achieved=1.0), None) == dict(bound="hbm",
                                                                            achieved=1.0)
