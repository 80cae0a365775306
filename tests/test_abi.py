"""C-ABI boundary on the host: the library loads, exports what include/gca.h
declares, and rejects bad arguments before touching the device."""

import ctypes
import os
import re

import pytest

import retrieval_sparse_attention_amd as gca

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "gca.h")
PEAKS_HEADER = os.path.join(os.path.dirname(HEADER), "gca_peaks.h")
P = ctypes.c_void_p


def _declared(header=None):
    text = open(header or HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(gca_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    lib = gca.load()
    names = _declared()
    assert set(names) == set(gca.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n
    peaks = _declared(PEAKS_HEADER)
    assert set(peaks) == set(gca.PEAK_EXPORTED)
    for n in peaks:
        assert hasattr(lib, n), n


def test_peak_calls_reject_bad_arguments():
    # validated on the host before any launch (fake device addresses are never touched)
    st, msg = _status("gca_peak_read", None, ctypes.c_size_t(16), A, None)
    assert st == 1 and "src is NULL" in msg
    st, msg = _status("gca_peak_read", A, ctypes.c_size_t(24), A, None)
    assert st == 1 and "multiple of 16" in msg
    st, msg = _status("gca_peak_copy", A, A, ctypes.c_size_t(64), None)
    assert st == 1 and "overlap" in msg
    st, msg = _status("gca_peak_mfma", A, 0, None, None)
    assert st == 1 and "iters" in msg
    st, msg = _status("gca_peak_gather", A, ctypes.c_size_t(16384 + 16), A, 1, None, None)
    assert st == 1 and "multiple of 16384" in msg
    st, msg = _status("gca_peak_gather", A, ctypes.c_size_t(16384), A, 4097, None, None)
    assert st == 1 and "iters" in msg
    st, msg = _status("gca_peak_gather", A, ctypes.c_size_t(16384), None, 1, None, None)
    assert st == 1 and "out is NULL" in msg
    assert "4096 * 4" in open(PEAKS_HEADER).read()
    assert gca.PEAK_GATHER_OUT_BYTES == 4096 * 4
    assert "2048 * 256 * 4" in open(PEAKS_HEADER).read()
    assert gca.PEAK_OUT_BYTES == 2048 * 256 * 4


def test_version_and_strings():
    assert gca.gca_abi_version() == 2
    assert gca.gca_status_string(0) == "GCA_OK"
    assert gca.gca_status_string(3) == "GCA_ERR_WORKSPACE"
    assert gca.gca_status_string(99) == "GCA_UNKNOWN_STATUS"


def _bf16_shape(**over):
    s = dict(G=2, B=4, H=12, n_query=256, n_key=256, chunk_size=64, head_dim=64,
             landmark_dim=64, top_k=8, dtype=gca.GCA_BF16, softmax_one=1)
    s.update(over)
    return gca.make_shape(**s)


def _status(fn, *args):
    lib = gca.load()
    return getattr(lib, fn)(*args), gca.gca_last_error()


def test_workspace_sizes():
    s = _bf16_shape()
    assert gca.gca_workspace_size(s, gca.OP_FORWARD) == 0
    # delta: 96 heads * 256 * 8 * 64 floats; rev_off: 96 * 257 ints; rev_ent: 96 * 2048 ints;
    # one layer's dscore (accumulate mode): 96 * 2048 floats
    expect = (96 * 256 * 8 * 64 * 4 + ((96 * 257 * 4 + 255) // 256) * 256 + 96 * 2048 * 4
              + 96 * 2048 * 4)
    assert gca.gca_workspace_size(s, gca.OP_BACKWARD) == expect
    assert gca.gca_workspace_size(s, gca.OP_RETRIEVE) == 0  # 256 candidates: one slice
    big = _bf16_shape(G=1, B=1, n_query=32, n_key=262144, softmax_one=0)
    assert gca.gca_workspace_size(big, gca.OP_RETRIEVE) > 0


@pytest.mark.parametrize("over,code", [
    (dict(G=0), 1), (dict(n_key=-1), 1), (dict(top_k=0), 1), (dict(top_k=17), 2),
    (dict(dtype=7), 1), (dict(softmax_one=2), 1), (dict(chunk_size=65), 2),
    (dict(head_dim=128), 2), (dict(landmark_dim=48), 2), (dict(n_key=2 ** 31), 1),
    (dict(attn_scale=float("inf")), 1),
])
def test_bad_shapes(over, code):
    s = _bf16_shape(**over)
    n = ctypes.c_size_t(0)
    st, msg = _status("gca_workspace_size", ctypes.byref(s), 2, ctypes.byref(n))
    assert st == code and msg


def test_bf16_attention_sizes():
    # S in {16, 64} x D in {32, 64} and other sizes up to 64 are accepted;
    # beyond 64 they are not
    for S, D in ((16, 32), (16, 64), (64, 32), (64, 64), (5, 7)):
        s = _bf16_shape(chunk_size=S, head_dim=D)
        assert gca.gca_workspace_size(s, gca.OP_BACKWARD) > 0
        assert gca.gca_workspace_size(s, gca.OP_FORWARD) == 0
    n = ctypes.c_size_t(0)
    for S, D in ((128, 64), (64, 96)):
        bad = _bf16_shape(chunk_size=S, head_dim=D)
        st, msg = _status("gca_workspace_size", ctypes.byref(bad), 1, ctypes.byref(n))
        assert st == 2 and "<= 64" in msg
    # the non-negative scale condition holds only for the MFMA forwards
    # (chunk_size 64 or 16, head_dim 64 or 32)
    s = _bf16_shape(chunk_size=5, head_dim=7, attn_scale=-0.5)
    st, msg = _status("gca_forward", ctypes.byref(s), None, A, A, A, A, A, None, None)
    assert st == 1 and "q is NULL" in msg
    for S, D in ((64, 32), (16, 64), (16, 32)):
        s = _bf16_shape(chunk_size=S, head_dim=D, attn_scale=-0.5)
        st, msg = _status("gca_forward", ctypes.byref(s), A, A, A, A, A, A, None, None)
        assert st == 2 and "attn_scale >= 0" in msg


def test_f32_limits():
    ok = _bf16_shape(dtype=gca.GCA_F32, chunk_size=16, head_dim=32, landmark_dim=128)
    assert gca.gca_workspace_size(ok, gca.OP_BACKWARD) > 0
    bad = _bf16_shape(dtype=gca.GCA_F32, chunk_size=65)
    n = ctypes.c_size_t(0)
    assert _status("gca_workspace_size", ctypes.byref(bad), 1, ctypes.byref(n))[0] == 2


def test_null_shape_and_op():
    n = ctypes.c_size_t(0)
    assert _status("gca_workspace_size", None, 0, ctypes.byref(n))[0] == 1
    s = _bf16_shape()
    assert _status("gca_workspace_size", ctypes.byref(s), 5, ctypes.byref(n))[0] == 1
    assert _status("gca_workspace_size", ctypes.byref(s), 0, None)[0] == 1


# Fake device addresses: the calls below must fail in validation, before any
# HIP call, so these are never dereferenced.
A = P(0x7f0000000000)
MIS = P(0x7f0000000002)


def test_forward_rejects_null_and_misaligned():
    s = _bf16_shape()
    st, msg = _status("gca_forward", ctypes.byref(s), None, A, A, A, A, A, None, None)
    assert st == 1 and "q is NULL" in msg
    st, msg = _status("gca_forward", ctypes.byref(s), MIS, A, A, A, A, A, None, None)
    assert st == 1 and "aligned" in msg
    st, msg = _status("gca_forward", ctypes.byref(s), A, A, A, A, A, None, None, None)
    assert st == 1 and "o is NULL" in msg


def test_retrieve_forward_checks_both_parts_before_any_device_call():
    s = _bf16_shape(G=1, B=1, n_query=1, n_key=5000, softmax_one=0)
    ws = ctypes.c_size_t(1 << 20)
    # the forward's arguments are checked first, then the retrieval's
    st, msg = _status("gca_retrieve_forward", ctypes.byref(s), A, A, A, A, A, A, A, A, A, None,
                      None, A, ws, None)
    assert st == 1 and "o is NULL" in msg
    st, msg = _status("gca_retrieve_forward", ctypes.byref(s), A, A, None, A, A, A, A, A, A, A,
                      None, A, ws, None)
    assert st == 1 and "q_pos is NULL" in msg
    st, msg = _status("gca_retrieve_forward", ctypes.byref(s), A, A, A, A, A, A, A, A, A, A,
                      None, None, ctypes.c_size_t(0), None)
    assert st == 3 and "workspace" in msg
    neg = _bf16_shape(G=1, B=1, n_query=1, n_key=5000, attn_scale=-0.5)
    st, msg = _status("gca_retrieve_forward", ctypes.byref(neg), A, A, A, A, A, A, A, A, A, A,
                      None, A, ws, None)
    assert st == 2 and "attn_scale >= 0" in msg


def test_forwards_need_non_negative_attention_scale():
    # the bf16 forwards shift rows by the largest unscaled product
    s = _bf16_shape(attn_scale=-0.125)
    st, msg = _status("gca_forward", ctypes.byref(s), A, A, A, A, A, A, None, None)
    assert st == 2 and "attn_scale >= 0" in msg
    sw = gca.make_swa_shape(2, 3, 1024, 64, 512, scale=-0.125)
    st, msg = _status("gca_swa_forward", ctypes.byref(sw), A, A, A, A, None, None)
    assert st == 2 and "scale >= 0" in msg


def test_retrieve_needs_workspace_when_sliced():
    s = _bf16_shape(G=1, B=1, n_query=32, n_key=262144, softmax_one=0)
    st, msg = _status("gca_retrieve", ctypes.byref(s), A, A, A, A, A, A, None,
                      ctypes.c_size_t(0), None)
    assert st == 3 and "workspace" in msg


@pytest.mark.parametrize("scale", [-0.125, 0.0, float("-0.0")])
def test_bf16_retrieve_needs_positive_score_scale(scale):
    # the bf16 scan prunes on unscaled dot products: rejected before any device call
    s = _bf16_shape(score_scale=scale)
    st, msg = _status("gca_retrieve", ctypes.byref(s), A, A, A, A, A, A, A,
                      ctypes.c_size_t(1 << 30), None)
    assert st == 2 and "score_scale > 0" in msg


def test_backward_rejects_small_workspace_and_missing_landmarks():
    s = _bf16_shape()
    need = gca.gca_workspace_size(s, gca.OP_BACKWARD)
    args = [A] * 14
    st, msg = _status("gca_backward", ctypes.byref(s), *args, A, A, A, ctypes.c_size_t(need - 1),
                      None)
    assert st == 3
    # dlk requested without lq
    args = [A, A, A, A, A, A, A, None, A, A, A, A, A, A, A, A]
    st, msg = _status("gca_backward", ctypes.byref(s), *args, A, ctypes.c_size_t(need), None)
    assert st == 1 and "lq" in msg


def test_empty_problem_is_a_no_op():
    s = _bf16_shape(n_query=0, n_key=0)
    assert _status("gca_forward", ctypes.byref(s), None, None, None, None, None, None, None,
                   None)[0] == 0


def test_gather_rejects_before_any_device_call():
    s = _bf16_shape()
    st, msg = _status("gca_gather_kv", ctypes.byref(s), None, A, A, A, A, A, None)
    assert st == 1 and "idx is NULL" in msg
    st, msg = _status("gca_gather_kv", ctypes.byref(s), A, A, A, MIS, A, A, None)
    assert st == 1 and "k_packed" in msg and "aligned" in msg
    st, msg = _status("gca_gather_kv", ctypes.byref(s), A, None, A, A, A, A, None)
    assert st == 1 and "k is NULL" in msg
    bad = _bf16_shape(chunk_size=80)
    assert _status("gca_gather_kv", ctypes.byref(bad), A, A, A, A, A, A, None)[0] == 2
    empty = _bf16_shape(n_query=0)
    assert _status("gca_gather_kv", ctypes.byref(empty), None, None, None, None, None, None,
                   None)[0] == 0


def test_swa_checks_before_any_device_call():
    ok = gca.make_swa_shape(2, 3, 1024, 64, 512)
    assert gca.gca_swa_workspace_size(ok) == ((2 * 3 * 1024 * 4 + 255) // 256) * 256
    n = ctypes.c_size_t(0)
    for bad, code in ((gca.make_swa_shape(1, 1, 100, 64, 512), 2),
                      (gca.make_swa_shape(1, 1, 128, 32, 512), 2),
                      (gca.make_swa_shape(1, 1, 128, 64, 512, dtype=gca.GCA_F32), 2),
                      (gca.make_swa_shape(1, 1, 128, 64, 0), 1),
                      (gca.make_swa_shape(0, 1, 128, 64, 8), 1)):
        st, msg = _status("gca_swa_workspace_size", ctypes.byref(bad), ctypes.byref(n))
        assert st == code and msg
    st, msg = _status("gca_swa_forward", ctypes.byref(ok), A, A, None, A, None, None)
    assert st == 1 and "v is NULL" in msg
    st, msg = _status("gca_swa_backward", ctypes.byref(ok), A, A, A, A, A, A, A, A, A, A,
                      ctypes.c_size_t(16), None)
    assert st == 3 and "workspace" in msg


def test_swa_rejects_sequences_past_2_30():
    n = ctypes.c_size_t(0)
    big = gca.make_swa_shape(1, 1, 2 ** 30, 64, 512)
    st, msg = _status("gca_swa_workspace_size", ctypes.byref(big), ctypes.byref(n))
    assert st == 2 and "2^30" in msg
