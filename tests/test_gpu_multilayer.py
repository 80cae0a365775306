"""GPU check of multi-layer reuse within a group: one gca_retrieve feeds the
gca_forward / gca_backward of L = 3 upper layers that share K, V and the
landmarks (paperlayer.ai summary, section 3.1; paperhub.cn reply "Q2").  The
per-layer outputs must match the oracle layer by layer, and the shared
tensors' gradients summed over the layers (in float64 on the host) must match
the oracle's sums, which tests/test_multilayer_pins.py pins to finite
differences of the composite loss.
"""

import numpy as np
import pytest

import synth
from oracle import gca_oracle as orc
from gpu_common import (accept_for, close, dev, f64, require_gpu, run_backward, run_forward,
                        run_retrieve, shape_of)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def test_one_retrieval_three_layers():
    name, over, L = "train16k_fwdbwd_g2", dict(B=1, H=2, n_query=72, n_key=72), 3
    cfg = synth.workload(name, **over)
    base = synth.training_inputs(name, accept=accept_for(cfg), **over)
    layers = [base] + [synth.training_inputs(name, seed=100 + l, **over) for l in range(1, L)]
    shape = shape_of(cfg)
    d = {key: dev(base[key]) for key in ("k", "v", "lq", "lk", "q_pos")}
    idx, _, w = run_retrieve(shape, d["lq"], d["lk"], d["q_pos"])
    k64, v64, lq64, lk64 = f64(base["k"]), f64(base["v"]), f64(base["lq"]), f64(base["lk"])
    r_idx, _, r_w = orc.retrieve(lq64, lk64, base["q_pos"].numpy(), cfg["k"],
                                 cfg["score_scale"], cfg["softmax_one"])
    assert np.array_equal(idx.cpu().numpy(), r_idx)
    sums = {n: 0.0 for n in ("dk", "dv", "dscore", "dlq", "dlk")}
    refs = {n: 0.0 for n in sums}
    for l, x in enumerate(layers):
        q, do = dev(x["q"]), dev(x["dout"])
        o, lse = run_forward(shape, q, d["k"], d["v"], idx, w)
        g = run_backward(shape, q, d["k"], d["v"], idx, w, lse, do, d["lq"], d["lk"])
        q64, do64 = f64(x["q"]), f64(x["dout"])
        r_o, _ = orc.forward(q64, k64, v64, r_idx, r_w, cfg["attn_scale"])
        r = orc.backward(q64, k64, v64, r_idx, r_w, do64, lq64, lk64, cfg["attn_scale"],
                         cfg["score_scale"])
        close(f"o[layer {l}]", f64(o), r_o, True)
        close(f"dq[layer {l}]", f64(g["dq"]), r["dq"], True)
        for n in sums:
            sums[n] = sums[n] + f64(g[n])
            refs[n] = refs[n] + r[n]
    for n in sums:
        close(f"{n} summed over {L} layers", sums[n], refs[n], True)
