"""The peak microbenchmarks (include/gca_peaks.h) read what they claim to read:
the streaming read's per-thread XOR folds and the tile gather's last words are
recomputed on the host from a known buffer; the MFMA loop reports its flop count
and repeats bit for bit.  They only calibrate the measured peaks that bench.py
quotes beside the published ones."""

import numpy as np
import pytest
import torch

import retrieval_sparse_attention_amd as gca
from gpu_common import require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _words(n):
    rng = np.random.default_rng(7)
    return rng.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32)


def test_peak_read_folds():
    n = 16 * 2048 * 256 + 4 * 1000  # a partial range for the last workgroups
    host = _words(n)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    out = torch.empty(gca.PEAK_OUT_BYTES, dtype=torch.uint8, device="cuda")
    gca.gca_peak_read(src, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    # workgroup b covers 16-byte units [b * per, min((b + 1) * per, n16)); thread t
    # takes units beg + t, beg + t + 256, ...
    n16 = n // 4
    per = -(-n16 // 2048)
    u = host.reshape(n16, 4)
    fold = u[:, 0] ^ u[:, 1] ^ u[:, 2] ^ u[:, 3]
    want = np.zeros(2048 * 256, dtype=np.uint32)
    for b in range(2048):
        beg, end = b * per, min((b + 1) * per, n16)
        if beg >= end:
            continue
        seg = fold[beg:end]
        pad = np.zeros(-(-len(seg) // 256) * 256, dtype=np.uint32)
        pad[:len(seg)] = seg
        want[b * 256:(b + 1) * 256] = np.bitwise_xor.reduce(pad.reshape(-1, 256), axis=0)
    assert np.array_equal(got, want)


def test_peak_gather_reads_the_chosen_tiles():
    n_tiles, iters = 37, 5
    host = np.arange(n_tiles * 4096, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    out = torch.empty(gca.PEAK_GATHER_OUT_BYTES, dtype=torch.uint8, device="cuda")
    moved = gca.gca_peak_gather(src, out, iters)
    torch.cuda.synchronize()
    assert moved == 4096 * iters * 16384
    got = out.cpu().numpy().view(np.uint32)
    # per-workgroup linear congruential sequence: h0 = b * 2654435761 + 12345,
    # h <- h * 1664525 + 1013904223 (mod 2^32), tile (h >> 8) mod n_tiles; the
    # workgroup reports word h mod 4096 of its last tile
    b = np.arange(4096, dtype=np.uint64)
    m = np.uint64(0xFFFFFFFF)
    h = (b * np.uint64(2654435761) + np.uint64(12345)) & m
    for _ in range(iters):
        h = (h * np.uint64(1664525) + np.uint64(1013904223)) & m
    tile = (h >> np.uint64(8)) % np.uint64(n_tiles)
    want = host[(tile * np.uint64(4096) + (h & np.uint64(4095))).astype(np.int64)]
    assert np.array_equal(got, want)


def test_peak_mfma_repeats():
    out = torch.empty(1024 * 256, dtype=torch.float32, device="cuda")
    f1 = gca.gca_peak_mfma(out, 3)
    a = out.clone()
    f2 = gca.gca_peak_mfma(out, 3)
    torch.cuda.synchronize()
    assert f1 == f2 == 1024 * 4 * 3 * 8 * 16 * 16 * 32 * 2
    assert torch.isfinite(out).all() and torch.equal(a, out)
