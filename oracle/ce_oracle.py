"""ctypes wrapper around the fp64 CPU oracle in ``ce_oracle.c``.

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg are the only callers.  It imports numpy and
nothing from the HIP package.  Arrays are numpy; bf16 logits are passed as
``uint16`` arrays holding the raw bit patterns, fp32 logits as ``float32``.

What each function computes is stated in ``ce_oracle.c``; in short
(torchtitan PR "[loss] fix softmax collapse with improved ce perf",
Numerics; Megatron-core core.tensor_parallel.cross_entropy,
VocabParallelCrossEntropy):

  loss_r = (1 - eps) softplus(lse_{j != t} z_j - z_t) + eps (lse - mean_j z_j)
  grad   = k_r (softmax(z) - q),  q = (1 - eps) onehot(t) + eps / V
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libce_oracle.so")

F32 = 0
BF16 = 1
F64 = 2
RED_NONE, RED_SUM, RED_MEAN = 0, 1, 2
_RED = {"none": RED_NONE, "sum": RED_SUM, "mean": RED_MEAN}

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        d = ctypes.c_double
        i = ctypes.c_int
        lib.oracle_forward.argtypes = [P, i, i64, i64, i64, P, i64, d, P, P, P, P, P, P, P, P]
        lib.oracle_forward.restype = None
        lib.oracle_grad.argtypes = [P, i, i64, i64, i64, P, P, P, P, d, P, P]
        lib.oracle_grad.restype = None
        lib.oracle_shard_stats.argtypes = [P, i, i64, i64, i64, i64, P, i64, P, P, P, P, P]
        lib.oracle_shard_stats.restype = None
        lib.oracle_merge.argtypes = [i64, i64, P, P, P, P, P, P, i64, i64, d,
                                     P, P, P, P, P, P, P, P]
        lib.oracle_merge.restype = None
        lib.oracle_reduce.argtypes = [P, P, i64, i, P, P]
        lib.oracle_reduce.restype = d
        lib.oracle_to_bf16.argtypes = [P, i64, P]
        lib.oracle_to_bf16.restype = None
        lib.oracle_linear_forward.argtypes = [P, P, i, i64, i64, i64, P, i64, d, P, P, P, P]
        lib.oracle_linear_forward.restype = None
        lib.oracle_linear_backward.argtypes = [P, P, i, i64, i64, i64, P, P, P, P, d, P, d,
                                               P, P, P, P, P, P, P]
        lib.oracle_linear_backward.restype = None
        lib.oracle_threads.argtypes = []
        lib.oracle_threads.restype = i
        lib.oracle_set_threads.argtypes = [i]
        lib.oracle_set_threads.restype = None
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _logits_args(z):
    """Validate a 2-D logits array; return (array, dtype code, n, V, ld)."""
    if z.ndim != 2:
        raise ValueError("logits must be 2-D [n, V]")
    if z.dtype == np.float32:
        code = F32
    elif z.dtype == np.uint16:
        code = BF16
    else:
        raise TypeError("logits must be float32 or uint16 (bf16 bits)")
    if z.strides[1] != z.itemsize or z.strides[0] % z.itemsize:
        raise ValueError("logits rows must be contiguous")
    n, V = z.shape
    ld = z.strides[0] // z.itemsize if n > 1 else V
    return z, code, n, V, ld


def _i64(a):
    return np.ascontiguousarray(a, dtype=np.int64)


def forward(z, target, *, ignore_index=-100, eps=0.0):
    """Per-row forward.  Returns a dict of [n] arrays: loss, status, m, s,
    zt, sz, x, lse (diagnostics are 0 on rows whose status is not 1)."""
    z, code, n, V, ld = _logits_args(z)
    target = _i64(target)
    assert target.shape == (n,)
    out = {k: np.zeros(n, np.float64) for k in ("loss", "m", "s", "zt", "sz", "x", "lse")}
    out["status"] = np.zeros(n, np.int32)
    _load().oracle_forward(_ptr(z), code, n, V, ld, _ptr(target), int(ignore_index),
                           float(eps), _ptr(out["loss"]), _ptr(out["status"]),
                           _ptr(out["m"]), _ptr(out["s"]), _ptr(out["zt"]),
                           _ptr(out["sz"]), _ptr(out["x"]), _ptr(out["lse"]))
    return out


def grad(z, target, fwd, k, *, eps=0.0):
    """Gradient rows [n, V] (float64) scaled by k ([n] or scalar), using the
    x, lse and status that :func:`forward` returned for the same rows."""
    z, code, n, V, ld = _logits_args(z)
    target = _i64(target)
    k = np.ascontiguousarray(np.broadcast_to(np.asarray(k, np.float64), (n,)))
    g = np.empty((n, V), np.float64)
    _load().oracle_grad(_ptr(z), code, n, V, ld, _ptr(target),
                        _ptr(np.ascontiguousarray(fwd["status"], np.int32)),
                        _ptr(np.ascontiguousarray(fwd["x"], np.float64)),
                        _ptr(np.ascontiguousarray(fwd["lse"], np.float64)),
                        float(eps), _ptr(k), _ptr(g))
    return g


def shard_stats(z, target, vocab_start, *, ignore_index=-100):
    """Statistics of one vocabulary shard: z is the [n, V_local] view of
    columns [vocab_start, vocab_start + V_local).  Returns m, s, zt, own, sz."""
    z, code, n, V, ld = _logits_args(z)
    target = _i64(target)
    out = {k: np.zeros(n, np.float64) for k in ("m", "s", "zt", "sz")}
    out["own"] = np.zeros(n, np.int32)
    _load().oracle_shard_stats(_ptr(z), code, n, V, ld, int(vocab_start), _ptr(target),
                               int(ignore_index), _ptr(out["m"]), _ptr(out["s"]),
                               _ptr(out["zt"]), _ptr(out["own"]), _ptr(out["sz"]))
    return out


def merge(shards, target, V_total, *, ignore_index=-100, eps=0.0):
    """Merge a list of per-shard stat dicts (from :func:`shard_stats`) in
    list order and finalize.  Returns the same dict as :func:`forward`."""
    target = _i64(target)
    n = target.shape[0]
    S = len(shards)
    cat = {k: np.ascontiguousarray(np.stack([sh[k] for sh in shards]))
           for k in ("m", "s", "zt", "sz")}
    own = np.ascontiguousarray(np.stack([sh["own"] for sh in shards]).astype(np.int32))
    out = {k: np.zeros(n, np.float64) for k in ("loss", "m", "s", "zt", "sz", "x", "lse")}
    out["status"] = np.zeros(n, np.int32)
    _load().oracle_merge(S, n, _ptr(cat["m"]), _ptr(cat["s"]), _ptr(cat["zt"]), _ptr(own),
                         _ptr(cat["sz"]), _ptr(target), int(ignore_index), int(V_total),
                         float(eps), _ptr(out["loss"]), _ptr(out["status"]),
                         _ptr(out["m"]), _ptr(out["s"]), _ptr(out["zt"]), _ptr(out["sz"]),
                         _ptr(out["x"]), _ptr(out["lse"]))
    return out


def reduce(loss, status, reduction):
    """Scalar loss and counts: returns (loss, n_valid, n_bad)."""
    loss = np.ascontiguousarray(loss, np.float64)
    status = np.ascontiguousarray(status, np.int32)
    nv = ctypes.c_int64()
    nb = ctypes.c_int64()
    val = _load().oracle_reduce(_ptr(loss), _ptr(status), loss.shape[0], _RED[reduction],
                                ctypes.byref(nv), ctypes.byref(nb))
    return val, nv.value, nb.value


def row_scale(status, reduction, grad_output, n_valid):
    """Per-row gradient scale k_r: grad_output (sum), grad_output / N_valid
    (mean), grad_output[r] (none); Megatron-core scale_gradients_inplace."""
    n = status.shape[0]
    if reduction == "none":
        return np.broadcast_to(np.asarray(grad_output, np.float64), (n,)).copy()
    g = float(np.asarray(grad_output, np.float64).reshape(-1)[0])
    if reduction == "sum":
        return np.full(n, g)
    return np.full(n, g / n_valid if n_valid else np.nan)


def fwd_bwd(z, target, *, ignore_index=-100, eps=0.0, reduction="mean", grad_output=1.0,
            n_valid=None):
    """Loss, per-row loss, counts and fp64 gradient of ``z``.  ``n_valid``
    overrides the mean's denominator when ``z`` is a sample of a larger batch."""
    f = forward(z, target, ignore_index=ignore_index, eps=eps)
    loss, nv, nb = reduce(f["loss"], f["status"], reduction)
    denom = nv if n_valid is None else n_valid
    k = row_scale(f["status"], reduction, grad_output, denom)
    g = grad(z, target, f, k, eps=eps)
    return {"loss": loss, "loss_rows": f["loss"], "status": f["status"], "n_valid": nv,
            "n_bad": nb, "grad": g, "fwd": f, "k": k}


def _matrix_args(a):
    if a.ndim != 2:
        raise ValueError("expected a 2-D matrix")
    a = np.ascontiguousarray(a)
    code = {np.dtype(np.uint16): BF16, np.dtype(np.float32): F32,
            np.dtype(np.float64): F64}.get(a.dtype)
    if code is None:
        raise TypeError("matrix must be uint16 (bf16 bits), float32 or float64")
    return a, code


def linear_fwd_bwd(E, C, target, *, ignore_index=-100, eps=0.0, reduction="mean",
                   grad_output=1.0, n_valid=None, grads=True, dC=True, scales=True,
                   filter_eps=0.0):
    """Cross-entropy of the logits E C^T (apple/ml-cross-entropy issue #14,
    linear_cross_entropy): E [n, D] and C [V, D] of one dtype (bf16 bits as
    uint16, float32 or float64).  Returns loss, loss_rows, status, n_valid,
    lse, and with ``grads`` the fp64 G [n, V], dE [n, D], dC [V, D] (unless
    ``dC`` is False) and the root-sum-square scales rsE, rsC (with
    ``scales``).  ``n_valid`` overrides the mean's denominator when E holds a
    sample of the rows of a larger batch.  ``filter_eps`` > 0 applies
    gradient filtering (256 x 256 blocks of the unscaled gradient whose
    entries are all below it in magnitude are dropped, see ce_oracle.c);
    then ``keep`` and ``block_max`` give the block decisions."""
    E, code = _matrix_args(E)
    C, code_c = _matrix_args(C)
    if code != code_c or E.shape[1] != C.shape[1]:
        raise ValueError("E and C must share dtype and hidden size")
    n, D = E.shape
    V = C.shape[0]
    target = _i64(target)
    assert target.shape == (n,)
    lib = _load()
    loss_rows = np.zeros(n, np.float64)
    status = np.zeros(n, np.int32)
    x = np.zeros(n, np.float64)
    lse = np.zeros(n, np.float64)
    lib.oracle_linear_forward(_ptr(E), _ptr(C), code, n, D, V, _ptr(target), int(ignore_index),
                              float(eps), _ptr(loss_rows), _ptr(status), _ptr(x), _ptr(lse))
    loss, nv, nb = reduce(loss_rows, status, reduction)
    out = {"loss": loss, "loss_rows": loss_rows, "status": status, "n_valid": nv, "n_bad": nb,
           "x": x, "lse": lse}
    if not grads:
        return out
    k = row_scale(status, reduction, grad_output, nv if n_valid is None else n_valid)
    G = np.empty((n, V), np.float64)
    dE = np.empty((n, D), np.float64)
    dCo = np.empty((V, D), np.float64) if dC else None
    rsE = np.empty((n, D), np.float64) if scales else None
    rsC = np.empty((V, D), np.float64) if (scales and dC) else None
    nb = ((n + 255) // 256, (V + 255) // 256)
    keep = np.empty(nb, np.int32)
    bmax = np.empty(nb, np.float64)
    lib.oracle_linear_backward(_ptr(E), _ptr(C), code, n, D, V, _ptr(target), _ptr(status),
                               _ptr(x), _ptr(lse), float(eps), _ptr(np.ascontiguousarray(k)),
                               float(filter_eps), _ptr(G), _ptr(dE), _ptr(dCo), _ptr(rsE),
                               _ptr(rsC), _ptr(keep), _ptr(bmax))
    out.update(G=G, dE=dE, dC=dCo, rsE=rsE, rsC=rsC, k=k, keep=keep, block_max=bmax)
    return out


def to_bf16(v):
    """fp64 -> bf16 bit patterns (uint16), round-to-nearest-even, one rounding."""
    v = np.ascontiguousarray(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    _load().oracle_to_bf16(_ptr(v), v.size, _ptr(out))
    return out


def bf16_to_f64(bits):
    """Exact widening of bf16 bit patterns to float64."""
    bits = np.asarray(bits, np.uint16)
    with np.errstate(invalid="ignore"):
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def threads():
    """OpenMP threads the oracle's row loops use."""
    return int(_load().oracle_threads())


def set_threads(n):
    """OpenMP threads for later calls (timing only; results do not change)."""
    _load().oracle_set_threads(int(n))
