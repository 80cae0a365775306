"""Python binding of libgca.so, the MI355X (gfx950) Grouped Cross Attention library.

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Functions take torch tensors that live in device memory (PyTorch is
used for device memory and streams) and enqueue work on torch's current
stream.  The entry points mirror the C ABI in include/gca.h:

  gca_retrieve(shape, lq, lk, q_pos, idx, score, w, ws=None)
  gca_retrieve_noalloc(shape, lq, lk, q_pos, idx, score, w)     no workspace, no allocation
  gca_retrieve_gumbel(shape, seed, lq, lk, q_pos, idx, score, w, ws=None)
  gca_gather_kv(shape, idx, k, v, k_packed, v_packed, idx_packed)   k, v may be pinned host
  gca_forward(shape, q, k, v, idx, w, o, lse=None)
  gca_retrieve_forward(shape, lq, lk, q_pos, q, k, v, idx, score, w, o, lse=None, ws=None)
  gca_backward(shape, q, k, v, idx, w, lse, dout, lq, lk, dq, dk, dv, dw, dscore,
               dlq=None, dlk=None, ws=None)
  gca_backward_accumulate(shape, q, k, v, idx, w, lse, dout, lq, lk, dq, dk_acc, dv_acc,
               dw_acc, dscore_acc, dlq_acc=None, dlk_acc=None, ws=None)   float32 sums
  gca_workspace_size(shape, op)          op: 0 retrieve, 1 forward, 2 backward
  gca_swa_forward(swa_shape, q, k, v, o, lse=None)      sliding-window self-attention
  gca_swa_backward(swa_shape, q, k, v, o, lse, dout, dq, dk, dv, ws=None)
  gca_swa_workspace_size(swa_shape)

A missing library raises; there is no fallback path.
"""

import ctypes
import math
import os

__all__ = ["GCA_F32", "GCA_BF16", "GcaShape", "GcaError", "make_shape", "library_path",
           "load", "gca_abi_version", "gca_status_string", "gca_last_error",
           "gca_workspace_size", "gca_retrieve", "gca_retrieve_noalloc", "gca_retrieve_gumbel",
           "gca_gather_kv",
           "gca_forward", "gca_retrieve_forward", "gca_backward", "gca_backward_accumulate",
           "GcaSwaShape",
           "make_swa_shape",
           "gca_swa_workspace_size", "gca_swa_forward", "gca_swa_backward",
           "OP_RETRIEVE", "OP_FORWARD", "OP_BACKWARD",
           "EXPORTED", "gca_num_kernels", "gca_kernel_name", "gca_timing_enable",
           "gca_timing_collect"]

GCA_F32 = 0
GCA_BF16 = 1
OP_RETRIEVE, OP_FORWARD, OP_BACKWARD = 0, 1, 2
EXPORTED = ("gca_abi_version", "gca_status_string", "gca_last_error", "gca_workspace_size",
            "gca_retrieve", "gca_retrieve_noalloc", "gca_retrieve_gumbel", "gca_gather_kv",
            "gca_forward", "gca_retrieve_forward", "gca_backward", "gca_backward_accumulate",
            "gca_num_kernels", "gca_kernel_name",
            "gca_timing_enable", "gca_timing_collect", "gca_swa_workspace_size",
            "gca_swa_forward", "gca_swa_backward")
# include/gca_peaks.h: microbenchmarks for the peaks measured on the GPU at hand
PEAK_EXPORTED = ("gca_peak_read", "gca_peak_copy", "gca_peak_gather", "gca_peak_mfma")
PEAK_OUT_BYTES = 2048 * 256 * 4
PEAK_GATHER_OUT_BYTES = 4096 * 4

_HERE = os.path.dirname(os.path.abspath(__file__))


class GcaShape(ctypes.Structure):
    _fields_ = [("G", ctypes.c_int64), ("B", ctypes.c_int64), ("H", ctypes.c_int64),
                ("n_query", ctypes.c_int64), ("n_key", ctypes.c_int64),
                ("chunk_size", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("landmark_dim", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("softmax_one", ctypes.c_int32),
                ("attn_scale", ctypes.c_float), ("score_scale", ctypes.c_float)]


class GcaSwaShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("H", ctypes.c_int64), ("T", ctypes.c_int64),
                ("head_dim", ctypes.c_int32), ("window", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("scale", ctypes.c_float)]


def make_swa_shape(B, H, T, head_dim, window, dtype=GCA_BF16, scale=None):
    return GcaSwaShape(B, H, T, head_dim, window, dtype,
                       1.0 / math.sqrt(head_dim) if scale is None else scale)


class GcaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{gca_status_string(status)}: {message}")
        self.status = status


def make_shape(G, B, H, n_query, n_key, chunk_size, head_dim, landmark_dim, top_k, dtype,
               softmax_one=0, attn_scale=None, score_scale=None):
    return GcaShape(G, B, H, n_query, n_key, chunk_size, head_dim, landmark_dim, top_k, dtype,
                    int(softmax_one),
                    1.0 / math.sqrt(head_dim) if attn_scale is None else attn_scale,
                    1.0 / math.sqrt(landmark_dim) if score_scale is None else score_scale)


def library_path():
    return os.environ.get("GCA_LIBRARY", os.path.join(_HERE, "libgca.so"))


_lib = None


def load():
    """Loads libgca.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with retrieval_sparse_attention_amd.build")
    lib = ctypes.CDLL(path)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    sp = ctypes.POINTER(GcaShape)
    lib.gca_abi_version.restype = ctypes.c_int
    lib.gca_abi_version.argtypes = []
    lib.gca_status_string.restype = ctypes.c_char_p
    lib.gca_status_string.argtypes = [ctypes.c_int]
    lib.gca_last_error.restype = ctypes.c_char_p
    lib.gca_last_error.argtypes = []
    lib.gca_workspace_size.restype = ctypes.c_int
    lib.gca_workspace_size.argtypes = [sp, ctypes.c_int, ctypes.POINTER(sz)]
    lib.gca_retrieve.restype = ctypes.c_int
    lib.gca_retrieve.argtypes = [sp] + [vp] * 6 + [vp, sz, vp]
    lib.gca_retrieve_noalloc.restype = ctypes.c_int
    lib.gca_retrieve_noalloc.argtypes = [sp] + [vp] * 6 + [vp]
    lib.gca_retrieve_gumbel.restype = ctypes.c_int
    lib.gca_retrieve_gumbel.argtypes = [sp, ctypes.c_uint64] + [vp] * 6 + [vp, sz, vp]
    lib.gca_gather_kv.restype = ctypes.c_int
    lib.gca_gather_kv.argtypes = [sp] + [vp] * 6 + [vp]
    lib.gca_forward.restype = ctypes.c_int
    lib.gca_forward.argtypes = [sp] + [vp] * 7 + [vp]
    lib.gca_retrieve_forward.restype = ctypes.c_int
    lib.gca_retrieve_forward.argtypes = [sp] + [vp] * 12 + [sz, vp]
    lib.gca_backward.restype = ctypes.c_int
    lib.gca_backward.argtypes = [sp] + [vp] * 16 + [vp, sz, vp]
    lib.gca_backward_accumulate.restype = ctypes.c_int
    lib.gca_backward_accumulate.argtypes = [sp] + [vp] * 16 + [vp, sz, vp]
    swp = ctypes.POINTER(GcaSwaShape)
    lib.gca_swa_workspace_size.restype = ctypes.c_int
    lib.gca_swa_workspace_size.argtypes = [swp, ctypes.POINTER(sz)]
    lib.gca_swa_forward.restype = ctypes.c_int
    lib.gca_swa_forward.argtypes = [swp] + [vp] * 5 + [vp]
    lib.gca_swa_backward.restype = ctypes.c_int
    lib.gca_swa_backward.argtypes = [swp] + [vp] * 10 + [sz, vp]
    lib.gca_num_kernels.restype = ctypes.c_int
    lib.gca_peak_read.argtypes = [vp, sz, vp, vp]
    lib.gca_peak_read.restype = ctypes.c_int
    lib.gca_peak_copy.argtypes = [vp, vp, sz, vp]
    lib.gca_peak_copy.restype = ctypes.c_int
    lib.gca_peak_gather.argtypes = [vp, sz, vp, ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                    vp]
    lib.gca_peak_gather.restype = ctypes.c_int
    lib.gca_peak_mfma.argtypes = [vp, ctypes.c_int, ctypes.POINTER(ctypes.c_double), vp]
    lib.gca_peak_mfma.restype = ctypes.c_int
    lib.gca_num_kernels.argtypes = []
    lib.gca_kernel_name.restype = ctypes.c_char_p
    lib.gca_kernel_name.argtypes = [ctypes.c_int]
    lib.gca_timing_enable.restype = ctypes.c_int
    lib.gca_timing_enable.argtypes = [ctypes.c_int]
    lib.gca_timing_collect.restype = ctypes.c_int
    lib.gca_timing_collect.argtypes = [ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_int64)]
    _lib = lib
    return lib


def gca_abi_version():
    return load().gca_abi_version()


def gca_status_string(status):
    return load().gca_status_string(int(status)).decode()


def gca_last_error():
    return load().gca_last_error().decode()


def _check(status):
    if status != 0:
        raise GcaError(status, gca_last_error())


def _ptr(t, name):
    """Device address of a contiguous CUDA tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    # torch's current stream of the current device, as a raw HIP stream handle
    # (the direct getter: a Stream object per call costs microseconds)
    import torch
    return ctypes.c_void_p(torch._C._cuda_getCurrentRawStream(torch.cuda.current_device()))


def gca_workspace_size(shape, op):
    n = ctypes.c_size_t(0)
    _check(load().gca_workspace_size(ctypes.byref(shape), int(op), ctypes.byref(n)))
    return int(n.value)


def _workspace(shape, op, ws, like):
    if ws is not None:
        return ws
    n = gca_workspace_size(shape, op)
    if n == 0:
        return None
    import torch
    return torch.empty(n, dtype=torch.uint8, device=like.device)


def gca_retrieve(shape, lq, lk, q_pos, idx, score, w, ws=None):
    ws = _workspace(shape, OP_RETRIEVE, ws, lq)
    _check(load().gca_retrieve(
        ctypes.byref(shape), _ptr(lq, "lq"), _ptr(lk, "lk"), _ptr(q_pos, "q_pos"),
        _ptr(idx, "idx"), _ptr(score, "score"), _ptr(w, "w"), _ptr(ws, "ws"),
        ctypes.c_size_t(0 if ws is None else ws.numel() * ws.element_size()), _stream()))


def gca_retrieve_noalloc(shape, lq, lk, q_pos, idx, score, w):
    _check(load().gca_retrieve_noalloc(
        ctypes.byref(shape), _ptr(lq, "lq"), _ptr(lk, "lk"), _ptr(q_pos, "q_pos"),
        _ptr(idx, "idx"), _ptr(score, "score"), _ptr(w, "w"), _stream()))


def gca_retrieve_gumbel(shape, seed, lq, lk, q_pos, idx, score, w, ws=None):
    ws = _workspace(shape, OP_RETRIEVE, ws, lq)
    _check(load().gca_retrieve_gumbel(
        ctypes.byref(shape), ctypes.c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF), _ptr(lq, "lq"),
        _ptr(lk, "lk"), _ptr(q_pos, "q_pos"), _ptr(idx, "idx"), _ptr(score, "score"),
        _ptr(w, "w"), _ptr(ws, "ws"),
        ctypes.c_size_t(0 if ws is None else ws.numel() * ws.element_size()), _stream()))


def _ptr_readable(t, name):
    """Address of a contiguous device tensor or pinned host tensor."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda and not t.is_pinned():
        raise ValueError(f"{name} must be a device tensor or pinned host memory")
    return ctypes.c_void_p(t.data_ptr())


def gca_gather_kv(shape, idx, k, v, k_packed, v_packed, idx_packed):
    _check(load().gca_gather_kv(
        ctypes.byref(shape), _ptr(idx, "idx"), _ptr_readable(k, "k"), _ptr_readable(v, "v"),
        _ptr(k_packed, "k_packed"), _ptr(v_packed, "v_packed"), _ptr(idx_packed, "idx_packed"),
        _stream()))


def gca_forward(shape, q, k, v, idx, w, o, lse=None):
    _check(load().gca_forward(
        ctypes.byref(shape), _ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"), _ptr(idx, "idx"),
        _ptr(w, "w"), _ptr(o, "o"), _ptr(lse, "lse"), _stream()))


def gca_retrieve_forward(shape, lq, lk, q_pos, q, k, v, idx, score, w, o, lse=None, ws=None):
    """gca_retrieve then gca_forward in one call (the slice merge fused into the forward
    where the retrieval is sliced); ws: the retrieval's workspace (op 0)."""
    ws = _workspace(shape, OP_RETRIEVE, ws, lq)
    _check(load().gca_retrieve_forward(
        ctypes.byref(shape), _ptr(lq, "lq"), _ptr(lk, "lk"), _ptr(q_pos, "q_pos"), _ptr(q, "q"),
        _ptr(k, "k"), _ptr(v, "v"), _ptr(idx, "idx"), _ptr(score, "score"), _ptr(w, "w"),
        _ptr(o, "o"), _ptr(lse, "lse"), _ptr(ws, "ws"),
        ctypes.c_size_t(0 if ws is None else ws.numel() * ws.element_size()), _stream()))


def gca_backward(shape, q, k, v, idx, w, lse, dout, lq, lk, dq, dk, dv, dw, dscore,
                 dlq=None, dlk=None, ws=None):
    ws = _workspace(shape, OP_BACKWARD, ws, q)
    _check(load().gca_backward(
        ctypes.byref(shape), _ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"), _ptr(idx, "idx"),
        _ptr(w, "w"), _ptr(lse, "lse"), _ptr(dout, "dout"), _ptr(lq, "lq"), _ptr(lk, "lk"),
        _ptr(dq, "dq"), _ptr(dk, "dk"), _ptr(dv, "dv"), _ptr(dw, "dw"), _ptr(dscore, "dscore"),
        _ptr(dlq, "dlq"), _ptr(dlk, "dlk"), _ptr(ws, "ws"),
        ctypes.c_size_t(0 if ws is None else ws.numel() * ws.element_size()), _stream()))


def gca_backward_accumulate(shape, q, k, v, idx, w, lse, dout, lq, lk, dq, dk_acc, dv_acc,
                            dw_acc, dscore_acc, dlq_acc=None, dlk_acc=None, ws=None):
    for name, t in (("dk_acc", dk_acc), ("dv_acc", dv_acc), ("dw_acc", dw_acc),
                    ("dscore_acc", dscore_acc), ("dlq_acc", dlq_acc), ("dlk_acc", dlk_acc)):
        if t is not None and t.dtype != __import__("torch").float32:
            raise ValueError(f"{name} must be float32")
    ws = _workspace(shape, OP_BACKWARD, ws, q)
    _check(load().gca_backward_accumulate(
        ctypes.byref(shape), _ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"), _ptr(idx, "idx"),
        _ptr(w, "w"), _ptr(lse, "lse"), _ptr(dout, "dout"), _ptr(lq, "lq"), _ptr(lk, "lk"),
        _ptr(dq, "dq"), _ptr(dk_acc, "dk_acc"), _ptr(dv_acc, "dv_acc"), _ptr(dw_acc, "dw_acc"),
        _ptr(dscore_acc, "dscore_acc"), _ptr(dlq_acc, "dlq_acc"), _ptr(dlk_acc, "dlk_acc"),
        _ptr(ws, "ws"), ctypes.c_size_t(0 if ws is None else ws.numel() * ws.element_size()),
        _stream()))


def gca_swa_workspace_size(shape):
    n = ctypes.c_size_t(0)
    _check(load().gca_swa_workspace_size(ctypes.byref(shape), ctypes.byref(n)))
    return int(n.value)


def gca_swa_forward(shape, q, k, v, o, lse=None):
    _check(load().gca_swa_forward(
        ctypes.byref(shape), _ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"), _ptr(o, "o"),
        _ptr(lse, "lse"), _stream()))


def gca_swa_backward(shape, q, k, v, o, lse, dout, dq, dk, dv, ws=None):
    if ws is None:
        n = gca_swa_workspace_size(shape)
        if n:
            import torch
            ws = torch.empty(n, dtype=torch.uint8, device=q.device)
    _check(load().gca_swa_backward(
        ctypes.byref(shape), _ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"), _ptr(o, "o"),
        _ptr(lse, "lse"), _ptr(dout, "dout"), _ptr(dq, "dq"), _ptr(dk, "dk"), _ptr(dv, "dv"),
        _ptr(ws, "ws"), ctypes.c_size_t(0 if ws is None else ws.numel() * ws.element_size()),
        _stream()))


def gca_num_kernels():
    return load().gca_num_kernels()


def gca_kernel_name(kernel_id):
    return load().gca_kernel_name(int(kernel_id)).decode()


def gca_timing_enable(on):
    _check(load().gca_timing_enable(1 if on else 0))


def gca_timing_collect():
    """{kernel name: (total_ms, launches)} since the previous collect."""
    n = gca_num_kernels()
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _check(load().gca_timing_collect(ms, cnt))
    return {gca_kernel_name(i): (float(ms[i]), int(cnt[i])) for i in range(n)}


def gca_peak_read(src, out):
    """Streaming read of the device tensor src (its bytes); out: >= PEAK_OUT_BYTES."""
    _check(load().gca_peak_read(_ptr(src, "src"), ctypes.c_size_t(src.numel() * src.element_size()),
                                _ptr(out, "out"), _stream()))


def gca_peak_copy(src, dst):
    """Streaming copy of src's bytes into dst (same size, device tensors)."""
    _check(load().gca_peak_copy(_ptr(src, "src"), _ptr(dst, "dst"),
                                ctypes.c_size_t(src.numel() * src.element_size()), _stream()))


def gca_peak_gather(src, out, iters):
    """Gather of 16 KB tiles picked among src's bytes into LDS; returns the bytes moved.
    out: >= PEAK_GATHER_OUT_BYTES."""
    moved = ctypes.c_double(0.0)
    _check(load().gca_peak_gather(_ptr(src, "src"),
                                  ctypes.c_size_t(src.numel() * src.element_size()),
                                  _ptr(out, "out"), int(iters), ctypes.byref(moved), _stream()))
    return moved.value


def gca_peak_mfma(out, iters):
    """Loop of independent 16x16x32 bf16 MFMAs; returns the launch's flop count."""
    flops = ctypes.c_double(0.0)
    _check(load().gca_peak_mfma(_ptr(out, "out"), int(iters), ctypes.byref(flops), _stream()))
    return flops.value
