"""Pins of the packed K/V gather (oracle/offload.py) to facts outside it.

* a hand-built case whose packed rows are written out literally;
* the reduction that defines the packing's purpose: attention over the packed
  tiles with the packed indices equals attention over the resident tiles
  (Eq. 2 and Eq. 3 of the oracle, themselves pinned elsewhere), for random
  inputs with empty, repeated and out-of-range slots, in both weight forms;
* the packed layout moves only k tiles per query chunk (the transfer volume the
  offloading reading rests on).
"""

import numpy as np

from oracle import gca_oracle as orc
from oracle import offload


def test_hand_built_rows():
    # 3 resident chunks, tile value = 10 * chunk + row-major position
    k = (10.0 * np.arange(3)[:, None, None] + np.arange(4).reshape(1, 2, 2))[None, None, None]
    v = -k
    idx = np.array([[[[[2, -1], [0, 2], [5, 1]]]]])
    kp, vp, ip = offload.gather_kv(idx, k, v)
    assert kp.shape == (1, 1, 1, 6, 2, 2)
    expect_rows = [2, None, 0, 2, None, 1]
    for row, c in enumerate(expect_rows):
        want = np.zeros((2, 2)) if c is None else k[0, 0, 0, c]
        assert np.array_equal(kp[0, 0, 0, row], want)
        assert np.array_equal(vp[0, 0, 0, row], -want + 0.0)
    assert ip[0, 0, 0].tolist() == [[0, -1], [2, 3], [-1, 5]]


def test_attention_on_packed_tiles_equals_resident():
    rng = np.random.default_rng(8)
    G, B, H, Nq, Nk, S, D, kk = 2, 1, 2, 5, 7, 4, 3, 3
    q = rng.standard_normal((G, B, H, Nq, S, D))
    k = rng.standard_normal((G, B, H, Nk, S, D))
    v = rng.standard_normal((G, B, H, Nk, S, D))
    idx = rng.integers(-2, Nk + 2, size=(G, B, H, Nq, kk))
    idx[0, 0, 0, 1] = [4, 4, 4]            # repeated chunk
    idx[1, 0, 1, 2] = [-1, -1, -1]         # nothing retrieved
    w = rng.random((G, B, H, Nq, kk))
    kp, vp, ip = offload.gather_kv(idx, k, v)
    o_ref, lse_ref = orc.forward(q, k, v, idx, w, 0.5)
    o_pk, lse_pk = orc.forward(q, kp, vp, ip, w, 0.5)
    assert np.array_equal(o_pk, o_ref)
    assert np.array_equal(lse_pk, lse_ref)
    assert np.all(o_pk[1, 0, 1, 2] == 0.0)


def test_packed_volume_is_k_tiles_per_query():
    rng = np.random.default_rng(9)
    idx = rng.integers(0, 50, size=(1, 1, 1, 4, 2))
    k = rng.standard_normal((1, 1, 1, 50, 2, 2))
    kp, _, ip = offload.gather_kv(idx, k, k)
    assert kp.shape[3] == 4 * 2
    assert np.array_equal(ip[0, 0, 0].ravel(), np.arange(8))
