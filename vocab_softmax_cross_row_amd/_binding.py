"""ctypes binding of libvocab_ce.so (include/vocab_ce.h).

Argument marshalling only: every step of the computation runs in the HIP
library.  torch supplies device memory and the current stream; tensors are
passed as raw device pointers.  The functions carry the C names and the C
argument order; tensors may be given where the C call takes a device
pointer, ``None`` where it takes NULL.  A nonzero status raises
:class:`CEError` with the library's message.

The library is loaded from this package's directory; if it is missing the
import of any function here raises (there is no fallback of any kind).
"""
import ctypes
import os

import numpy as np
import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libvocab_ce.so")

CE_F32, CE_BF16 = 0, 1
CE_RED_NONE, CE_RED_SUM, CE_RED_MEAN = 0, 1, 2
CE_OP_FORWARD, CE_OP_BACKWARD, CE_OP_FUSED, CE_OP_MERGE = 0, 1, 2, 3
CE_MAX_SHARDS = 64
REDUCTIONS = {"none": CE_RED_NONE, "sum": CE_RED_SUM, "mean": CE_RED_MEAN}

# symbols declared in include/vocab_ce.h
EXPORTS = ("ce_workspace_bytes", "ce_forward", "ce_merge_shard_stats", "ce_backward",
           "ce_fused_fwd_bwd", "ce_linear_workspace_bytes", "ce_linear_fwd_bwd",
           "ce_status_str", "ce_version", "ce_fused_fwd_bwd_timed", "ce_fused_fwd_bwd_noalloc")
CE_NOALLOC_SCRATCH_BYTES = 8 << 20
CE_ACC_FP32, CE_ACC_KAHAN = 0, 1
ACCUMS = {"fp32": CE_ACC_FP32, "kahan": CE_ACC_KAHAN}
CE_LINEAR_CHUNK = 16384

# device structs, as numpy dtypes for reading them back
ROW_STATS_DTYPE = np.dtype([("m", "<f4"), ("zt", "<f4"), ("own", "<i4"), ("reserved", "<i4"),
                            ("s", "<f8"), ("sz", "<f8")])
ROW_FINAL_DTYPE = np.dtype([("lse", "<f8"), ("gt", "<f8"), ("m", "<f4"), ("status", "<i4")])
ROW_STATS_BYTES = 32
ROW_FINAL_BYTES = 24


class CEProblem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("V_local", ctypes.c_int64), ("ld", ctypes.c_int64),
                ("vocab_start", ctypes.c_int64), ("V_total", ctypes.c_int64),
                ("ignore_index", ctypes.c_int64), ("label_smoothing", ctypes.c_float),
                ("reduction", ctypes.c_int32)]


class CELinearProblem(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int64), ("D", ctypes.c_int64), ("V", ctypes.c_int64),
                ("ignore_index", ctypes.c_int64), ("label_smoothing", ctypes.c_float),
                ("reduction", ctypes.c_int32), ("accum", ctypes.c_int32),
                ("filter_eps", ctypes.c_float)]


class CEError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m vocab_softmax_cross_row_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        P, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        prob = ctypes.POINTER(CEProblem)
        L.ce_workspace_bytes.argtypes = [prob, i32]
        L.ce_workspace_bytes.restype = sz
        L.ce_forward.argtypes = [prob, P, i32, P, P, P, P, P, P, P, P, sz, P]
        L.ce_forward.restype = i32
        L.ce_merge_shard_stats.argtypes = [prob, i32, P, P, P, P, P, P, P, P, sz, P]
        L.ce_merge_shard_stats.restype = i32
        L.ce_backward.argtypes = [prob, P, i32, P, P, P, P, P, i32, i64, P]
        L.ce_backward.restype = i32
        L.ce_fused_fwd_bwd.argtypes = [prob, P, i32, P, P, P, P, P, P, P, i32, i64, P, sz, P]
        L.ce_fused_fwd_bwd.restype = i32
        lprob = ctypes.POINTER(CELinearProblem)
        L.ce_linear_workspace_bytes.argtypes = [lprob, i32]
        L.ce_linear_workspace_bytes.restype = sz
        L.ce_linear_fwd_bwd.argtypes = [lprob, P, P, P, P, P, P, P, P, P, P, P, sz, P]
        L.ce_linear_fwd_bwd.restype = i32
        L.ce_status_str.argtypes = [i32]
        L.ce_status_str.restype = ctypes.c_char_p
        L.ce_version.argtypes = []
        L.ce_version.restype = i32
        L.ce_fused_fwd_bwd_timed.argtypes = [prob, P, i32, P, P, P, P, P, P, P, i32, i64, P, sz, P,
                                             P, P]
        L.ce_fused_fwd_bwd_timed.restype = i32
        L.ce_fused_fwd_bwd_noalloc.argtypes = [prob, P, i32, P, P, P, P, P, P, P, i32, i64, P]
        L.ce_fused_fwd_bwd_noalloc.restype = i32
        _lib = L
    return _lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return ctypes.c_void_p(x.data_ptr())
    return ctypes.c_void_p(int(x))


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check(fn, rc):
    if rc != 0:
        raise CEError(fn, rc, lib().ce_status_str(rc).decode())


def dtype_code(dt):
    if dt == torch.bfloat16:
        return CE_BF16
    if dt == torch.float32:
        return CE_F32
    raise TypeError(f"unsupported dtype {dt}: bf16 or fp32")


def make_problem(T, V_local, ld=None, *, vocab_start=0, V_total=None, ignore_index=-100,
                 label_smoothing=0.0, reduction="mean"):
    red = REDUCTIONS[reduction] if isinstance(reduction, str) else int(reduction)
    return CEProblem(int(T), int(V_local), int(V_local if ld is None else ld), int(vocab_start),
                     int(V_local if V_total is None else V_total), int(ignore_index),
                     float(label_smoothing), red)


def ce_workspace_bytes(prob, op):
    return int(lib().ce_workspace_bytes(ctypes.byref(prob), int(op)))


def ce_forward(prob, logits, logits_dtype, target, stats, fin, loss_rows, loss, n_valid,
               err_count, ws, ws_bytes, stream=None):
    _check("ce_forward", lib().ce_forward(
        ctypes.byref(prob), _ptr(logits), int(logits_dtype), _ptr(target), _ptr(stats),
        _ptr(fin), _ptr(loss_rows), _ptr(loss), _ptr(n_valid), _ptr(err_count), _ptr(ws),
        int(ws_bytes), _stream(stream)))


def ce_merge_shard_stats(prob, n_shards, shard_stats, target, fin, loss_rows, loss, n_valid,
                         err_count, ws, ws_bytes, stream=None):
    _check("ce_merge_shard_stats", lib().ce_merge_shard_stats(
        ctypes.byref(prob), int(n_shards), _ptr(shard_stats), _ptr(target), _ptr(fin),
        _ptr(loss_rows), _ptr(loss), _ptr(n_valid), _ptr(err_count), _ptr(ws), int(ws_bytes),
        _stream(stream)))


def ce_backward(prob, logits, logits_dtype, target, fin, n_valid, grad_output, grad, grad_dtype,
                ldg, stream=None):
    _check("ce_backward", lib().ce_backward(
        ctypes.byref(prob), _ptr(logits), int(logits_dtype), _ptr(target), _ptr(fin),
        _ptr(n_valid), _ptr(grad_output), _ptr(grad), int(grad_dtype), int(ldg),
        _stream(stream)))


def ce_fused_fwd_bwd(prob, logits, logits_dtype, target, grad_output, loss_rows, loss, n_valid,
                     err_count, grad, grad_dtype, ldg, ws, ws_bytes, stream=None):
    _check("ce_fused_fwd_bwd", lib().ce_fused_fwd_bwd(
        ctypes.byref(prob), _ptr(logits), int(logits_dtype), _ptr(target), _ptr(grad_output),
        _ptr(loss_rows), _ptr(loss), _ptr(n_valid), _ptr(err_count), _ptr(grad),
        int(grad_dtype), int(ldg), _ptr(ws), int(ws_bytes), _stream(stream)))


def make_linear_problem(N, D, V, *, ignore_index=-100, label_smoothing=0.0, reduction="mean",
                        accum="fp32", filter_eps=0.0):
    red = REDUCTIONS[reduction] if isinstance(reduction, str) else int(reduction)
    acc = ACCUMS[accum] if isinstance(accum, str) else int(accum)
    return CELinearProblem(int(N), int(D), int(V), int(ignore_index), float(label_smoothing),
                           red, acc, float(filter_eps))


def ce_linear_workspace_bytes(prob, backward):
    return int(lib().ce_linear_workspace_bytes(ctypes.byref(prob), int(backward)))


def ce_linear_fwd_bwd(prob, E, C, target, grad_output, loss_rows, loss, n_valid, err_count, dE,
                      dC, ws, ws_bytes, stream=None):
    _check("ce_linear_fwd_bwd", lib().ce_linear_fwd_bwd(
        ctypes.byref(prob), _ptr(E), _ptr(C), _ptr(target), _ptr(grad_output), _ptr(loss_rows),
        _ptr(loss), _ptr(n_valid), _ptr(err_count), _ptr(dE), _ptr(dC), _ptr(ws), int(ws_bytes),
        _stream(stream)))


def ce_status_str(status):
    return lib().ce_status_str(int(status)).decode()


def ce_version():
    return int(lib().ce_version())


def ce_fused_fwd_bwd_noalloc(prob, logits, logits_dtype, target, grad_output, loss_rows, loss,
                             n_valid, err_count, grad, grad_dtype, ldg, stream=None):
    """ce_fused_fwd_bwd without a workspace: the library's static per-device
    scratch array (calls overlapping on one GPU race)."""
    _check("ce_fused_fwd_bwd_noalloc", lib().ce_fused_fwd_bwd_noalloc(
        ctypes.byref(prob), _ptr(logits), int(logits_dtype), _ptr(target), _ptr(grad_output),
        _ptr(loss_rows), _ptr(loss), _ptr(n_valid), _ptr(err_count), _ptr(grad),
        int(grad_dtype), int(ldg), _stream(stream)))


def ce_fused_fwd_bwd_timed(prob, logits, logits_dtype, target, grad_output, loss_rows, loss,
                           n_valid, err_count, grad, grad_dtype, ldg, ws, ws_bytes, stream,
                           ev_start, ev_stop):
    """Measurement only: ce_fused_fwd_bwd plus two HIP events (raw hipEvent_t
    handles, or None) recorded around its main kernels."""
    _check("ce_fused_fwd_bwd_timed", lib().ce_fused_fwd_bwd_timed(
        ctypes.byref(prob), _ptr(logits), int(logits_dtype), _ptr(target), _ptr(grad_output),
        _ptr(loss_rows), _ptr(loss), _ptr(n_valid), _ptr(err_count), _ptr(grad),
        int(grad_dtype), int(ldg), _ptr(ws), int(ws_bytes), _stream(stream),
        ctypes.c_void_p(ev_start) if ev_start else None,
        ctypes.c_void_p(ev_stop) if ev_stop else None))


def read_stats(raw):
    """Host numpy structured array from a device ce_row_stats buffer."""
    b = raw.detach().to("cpu").contiguous().view(torch.uint8).numpy()
    return b.view(ROW_STATS_DTYPE).reshape(-1)


def read_final(raw):
    """Host numpy structured array from a device ce_row_final buffer."""
    b = raw.detach().to("cpu").contiguous().view(torch.uint8).numpy()
    return b.view(ROW_FINAL_DTYPE).reshape(-1)
