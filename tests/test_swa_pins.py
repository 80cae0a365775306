"""Pins of the sliding-window attention oracle (oracle/swa.py) to facts outside it.

* library reductions: with a window covering the sequence it is causal
  attention, torch.nn.functional.scaled_dot_product_attention(is_causal=True)
  in float64 on the CPU; with any window it equals that routine under a band
  mask built independently (tril/triu), forward and, through torch autograd,
  backward;
* closed forms: a window of 1 gives O = V, LSE = scale <q_x, k_x>, dQ = dK = 0
  and dV = dO;
* locality: O[x] ignores every key and value outside x's window and depends on
  the ones inside;
* central finite differences of a scalar loss through the forward.
Shapes use T != D so that a transposed operand fails.
"""

import numpy as np
import pytest
import torch

from oracle import swa

F = torch.nn.functional


def _inputs(B, H, T, D, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, H, T, D)) for _ in range(4)]


def _band(T, W):
    ones = torch.ones(T, T, dtype=torch.bool)
    return torch.tril(ones) & torch.triu(ones, diagonal=-(W - 1))


def test_full_window_is_causal_attention():
    q, k, v, _ = _inputs(2, 2, 37, 5, 0)
    o, _ = swa.swa_forward(q, k, v, window=37, scale=0.3)
    ref = F.scaled_dot_product_attention(*(torch.from_numpy(a) for a in (q, k, v)),
                                         is_causal=True, scale=0.3)
    assert np.allclose(o, ref.numpy(), rtol=0, atol=1e-12)
    o2, _ = swa.swa_forward(q, k, v, window=1000, scale=0.3)
    assert np.array_equal(o, o2)


@pytest.mark.parametrize("W", [2, 7, 16, 64])
def test_band_mask_forward_and_backward_match_torch(W):
    q, k, v, do = _inputs(1, 3, 50, 6, W)
    o, _ = swa.swa_forward(q, k, v, window=W, scale=0.25)
    dq, dk, dv = swa.swa_backward(q, k, v, do, window=W, scale=0.25)
    tq, tk, tv = (torch.from_numpy(a).requires_grad_() for a in (q, k, v))
    ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=_band(50, W), scale=0.25)
    ref.backward(torch.from_numpy(do))
    assert np.allclose(o, ref.detach().numpy(), rtol=0, atol=1e-12)
    for got, t in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.allclose(got, t.grad.numpy(), rtol=0, atol=1e-11)


def test_window_of_one():
    q, k, v, do = _inputs(1, 2, 9, 4, 3)
    o, lse = swa.swa_forward(q, k, v, window=1, scale=0.5)
    assert np.allclose(o, v, rtol=0, atol=1e-15)
    assert np.allclose(lse, 0.5 * (q * k).sum(-1), rtol=0, atol=1e-14)
    dq, dk, dv = swa.swa_backward(q, k, v, do, window=1, scale=0.5)
    assert np.allclose(dq, 0, atol=1e-14) and np.allclose(dk, 0, atol=1e-14)
    assert np.allclose(dv, do, rtol=0, atol=1e-14)


def test_locality():
    T, W = 40, 8
    q, k, v, _ = _inputs(1, 1, T, 3, 4)
    o, _ = swa.swa_forward(q, k, v, W, 0.5)
    x = 25
    for y in list(range(0, x - W + 1)) + list(range(x + 1, T)):
        k2, v2 = k.copy(), v.copy()
        k2[0, 0, y] += 3.0
        v2[0, 0, y] -= 2.0
        o2, _ = swa.swa_forward(q, k2, v2, W, 0.5)
        assert np.array_equal(o2[0, 0, x], o[0, 0, x]), y
    for y in range(x - W + 1, x + 1):
        v2 = v.copy()
        v2[0, 0, y] += 1.0
        o2, _ = swa.swa_forward(q, k, v2, W, 0.5)
        assert not np.allclose(o2[0, 0, x], o[0, 0, x]), y


def test_finite_differences():
    q, k, v, do = _inputs(1, 1, 12, 3, 5)
    W, sc, h = 5, 0.7, 1e-6
    dq, dk, dv = swa.swa_backward(q, k, v, do, W, sc)
    loss = lambda q_, k_, v_: float((swa.swa_forward(q_, k_, v_, W, sc)[0] * do).sum())
    for arr, grad, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        for pos in [(0, 0, 0, 0), (0, 0, 4, 2), (0, 0, 11, 1), (0, 0, 7, 0)]:
            args = [q.copy(), k.copy(), v.copy()]
            args[which][pos] += h
            up = loss(*args)
            args[which][pos] -= 2 * h
            dn = loss(*args)
            assert abs((up - dn) / (2 * h) - grad[pos]) < 1e-7, (which, pos)


def test_row_helpers_match_the_full_computation():
    q, k, v, do = _inputs(2, 2, 30, 4, 6)
    W, sc = 7, 0.4
    o, lse = swa.swa_forward(q, k, v, W, sc)
    dq, dk, dv = swa.swa_backward(q, k, v, do, W, sc)
    xs = [0, 1, 6, 7, 29]
    o_r, l_r, dq_r = swa.swa_query_rows(q, k, v, do, W, sc, 1, 0, xs)
    assert np.allclose(o_r, o[1, 0, xs], rtol=0, atol=1e-13)
    assert np.allclose(l_r, lse[1, 0, xs], rtol=0, atol=1e-13)
    assert np.allclose(dq_r, dq[1, 0, xs], rtol=0, atol=1e-13)
    dk_r, dv_r = swa.swa_key_rows(q, k, v, do, W, sc, 0, 1, xs)
    assert np.allclose(dk_r, dk[0, 1, xs], rtol=0, atol=1e-13)
    assert np.allclose(dv_r, dv[0, 1, xs], rtol=0, atol=1e-13)
