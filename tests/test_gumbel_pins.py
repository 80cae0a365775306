"""Pins of the Gumbel top-k oracle (oracle/gumbel.py) to facts outside it.

* Philox4x32-10 known-answer vectors published with the generator (Salmon et
  al., "Parallel random numbers: as easy as 1, 2, 3", SC 2011, and the test
  vectors distributed with its reference implementation);
* the uniform lattice: every U is an odd multiple of 2^-24 inside (0, 1);
* the Gumbel law: mean = Euler-Mascheroni constant, variance = pi^2 / 6, and a
  Kolmogorov-Smirnov test against exp(-exp(-x));
* the Gumbel-max identity: with k = 1, chunk j is selected with probability
  softmax(r)_j (paperlayer.ai summary, section 3.2: noise added to the
  relevance scores before top-k);
* Gumbel top-k as sampling without replacement: the probability of a selected
  pair {a, b} is p_a p_b / (1 - p_a) + p_b p_a / (1 - p_b);
* a closed-form bound: the noise lies in [GUMBEL_MIN, GUMBEL_MAX], so score gaps
  wider than that range make the selection equal the noise-free top-k;
* the outputs: score and w come from the clean scores of the selected chunks.
Frequencies use 5-sigma binomial bounds: a fixed seed makes each test
deterministic, and a wrong formula misses by far more.
"""

import math

import numpy as np
import pytest
from scipy import stats

from oracle import gca_oracle as orc
from oracle import gumbel as gb

KAT = [
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF), (0xFFFFFFFF, 0xFFFFFFFF),
     (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,expect", KAT)
def test_philox_known_answers(ctr, key, expect):
    out = gb.philox4x32_10(np.array(ctr), np.array(key))
    assert [int(x) for x in out] == list(expect)


def test_philox_vectorised_matches_scalar():
    rng = np.random.default_rng(0)
    ctr = rng.integers(0, 2**32, size=(50, 4), dtype=np.uint64)
    key = rng.integers(0, 2**32, size=(50, 2), dtype=np.uint64)
    batch = gb.philox4x32_10(ctr, key)
    for i in range(50):
        assert np.array_equal(batch[i], gb.philox4x32_10(ctr[i], key[i]))


def _noise(n, seed=7, head=3, q=11):
    return gb.gumbel_noise(seed, head, q, np.arange(n))


def test_uniform_lattice():
    words = np.array([0, 1, 511, 512, 2**31, 2**32 - 1], dtype=np.uint64)
    u = gb.uniform_from_word(words)
    scaled = u * float(1 << 24)
    assert np.all(scaled == np.round(scaled))
    assert np.all(np.round(scaled).astype(np.int64) % 2 == 1)
    assert u.min() == 0.5 / 2**23 and u.max() == 1.0 - 0.5 / 2**23
    # float32 holds every lattice point exactly
    assert np.all(u.astype(np.float32).astype(np.float64) == u)


def test_gumbel_moments_and_law():
    n = 200_000
    g = _noise(n)
    sd = math.pi / math.sqrt(6.0)
    assert abs(g.mean() - 0.5772156649015329) < 5 * sd / math.sqrt(n)
    # variance of the sample variance: (mu4 - sigma^4) / n, excess kurtosis 12/5
    assert abs(g.var() - math.pi**2 / 6) < 5 * sd**2 * math.sqrt(4.4 / n)
    assert stats.kstest(g, lambda x: np.exp(-np.exp(-x))).pvalue > 1e-3
    assert g.min() >= gb.GUMBEL_MIN and g.max() <= gb.GUMBEL_MAX


def test_noise_depends_on_every_key_part():
    base = gb.gumbel_noise(5, 2, 9, np.arange(64))
    for args in [(6, 2, 9), (5, 3, 9), (5, 2, 10), (5 + (1 << 32), 2, 9)]:
        other = gb.gumbel_noise(*args, np.arange(64))
        assert np.mean(other == base) < 0.05
    # words within one counter feed four consecutive candidates
    assert len(set(np.round(base, 12))) == 64


SCALE = 0.25  # score_scale of the hand-built cases: a power of two, so r is exact


def _single_head_lm(r, n_query):
    """lq = e_0, lk_j = (r_j / SCALE) e_0: Eq. 1 with score_scale SCALE gives r_j."""
    n, dl = len(r), 4
    lq = np.zeros((1, 1, 1, n_query, dl))
    lq[..., 0] = 1.0
    lk = np.zeros((1, 1, 1, n, dl))
    lk[0, 0, 0, :, 0] = np.asarray(r) / SCALE
    q_pos = np.full(n_query, n + 1)
    return lq, lk, q_pos


def _freq_bound(p, n):
    return 5.0 * np.sqrt(p * (1.0 - p) / n) + 1e-12


def test_gumbel_max_is_softmax_sampling():
    r = np.array([0.3, -0.5, 1.2, 0.0, -1.0, 0.7])
    n = 20_000
    lq, lk, q_pos = _single_head_lm(r, n)
    idx, score, w = gb.retrieve_gumbel(lq, lk, q_pos, 1, SCALE, 0, seed=1234)
    picks = idx[0, 0, 0, :, 0]
    p = np.exp(r) / np.exp(r).sum()
    freq = np.bincount(picks, minlength=len(r)) / n
    assert np.all(np.abs(freq - p) < _freq_bound(p, n)), (freq, p)
    # the selected chunk's clean score and its (single-slot) weight
    assert np.array_equal(score[0, 0, 0, :, 0], r[picks])
    assert np.all(w[0, 0, 0, :, 0] == 1.0)


def test_gumbel_top2_is_sampling_without_replacement():
    r = np.array([0.9, 0.1, -0.4, 0.5])
    n = 20_000
    lq, lk, q_pos = _single_head_lm(r, n)
    idx, _, _ = gb.retrieve_gumbel(lq, lk, q_pos, 2, SCALE, 0, seed=99)
    p = np.exp(r) / np.exp(r).sum()
    pairs = idx[0, 0, 0]
    for a in range(4):
        for b in range(a + 1, 4):
            expect = p[a] * p[b] / (1 - p[a]) + p[b] * p[a] / (1 - p[b])
            got = np.mean((pairs[:, 0] == a) & (pairs[:, 1] == b))
            assert abs(got - expect) < _freq_bound(expect, n), (a, b, got, expect)


def test_wide_gaps_reduce_to_noise_free_top_k():
    span = gb.GUMBEL_MAX - gb.GUMBEL_MIN
    rng = np.random.default_rng(3)
    r = rng.permutation(np.arange(12)) * (span + 1.0)
    n_query = 40
    lq, lk, q_pos = _single_head_lm(r, n_query)
    for k in (1, 3, 5):
        noisy = gb.retrieve_gumbel(lq, lk, q_pos, k, SCALE, 1, seed=5)
        clean = orc.retrieve(lq, lk, q_pos, k, SCALE, 1)
        for a, b in zip(noisy, clean):
            assert np.array_equal(a, b)


def test_outputs_use_clean_scores():
    rng = np.random.default_rng(4)
    G, B, H, Nq, Nk, Dl, k = 1, 2, 2, 24, 24, 16, 4
    lq = rng.standard_normal((G, B, H, Nq, Dl))
    lk = rng.standard_normal((G, B, H, Nk, Dl))
    q_pos = np.arange(Nq)
    scale = 1.0 / math.sqrt(Dl)
    for softmax_one in (0, 1):
        idx, score, w = gb.retrieve_gumbel(lq, lk, q_pos, k, scale, softmax_one, seed=77)
        clean_idx, _, _ = orc.retrieve(lq, lk, q_pos, k, scale, softmax_one)
        assert not np.array_equal(idx, clean_idx)  # the noise changes some selections
        for b in range(B):
            for h in range(H):
                for q in range(Nq):
                    sel = idx[0, b, h, q]
                    m = int((sel >= 0).sum())
                    assert m == min(k, max(0, q - 1))
                    assert np.all(np.diff(sel[:m]) > 0) and np.all(sel[m:] == -1)
                    r = scale * (lk[0, b, h, sel[:m]] @ lq[0, b, h, q])
                    assert np.allclose(score[0, b, h, q, :m], r, rtol=0, atol=1e-14)
                    assert np.allclose(w[0, b, h, q, :m], orc.fusion_weights(r, softmax_one),
                                       rtol=0, atol=1e-14)
                    # the selection is the top k of r + G, ties to the lower index
                    _, p = gb.perturbed_scores(lq[0, b, h, q], lk[0, b, h], q, scale, 77,
                                               b * H + h, q)
                    if m:
                        order = np.lexsort((np.arange(p.size), -p))
                        assert set(order[:m]) == set(sel[:m])
        # same seed: same result; another seed: another selection
        again = gb.retrieve_gumbel(lq, lk, q_pos, k, scale, softmax_one, seed=77)
        assert all(np.array_equal(a, b) for a, b in zip(again, (idx, score, w)))
        other = gb.retrieve_gumbel(lq, lk, q_pos, k, scale, softmax_one, seed=78)
        assert not np.array_equal(other[0], idx)
