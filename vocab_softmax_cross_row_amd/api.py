"""torch-facing helpers over the C ABI: allocate outputs with torch, call
the library, return tensors.  No arithmetic happens here; options are
keyword-only (Megatron-core unfused_cross_entropy passes the process group
by keyword because the third positional argument is label_smoothing).

``stream``: the torch stream (or raw hipStream_t handle) the call runs on;
None is torch's current stream.  Outputs and the workspace are allocated
with that stream current, so torch's caching allocator orders their reuse
after the call's kernels; inputs made on another stream must be ready on
this one (the caller's wait, as for any torch op).
"""
import contextlib
import functools

import torch

from . import _binding as B


def _logits2d(logits):
    if logits.dim() != 2:
        raise ValueError("logits must be 2-D [T, V] (flatten [seq, batch, V] first)")
    if logits.stride(1) != 1:
        raise ValueError("logits rows must be contiguous (stride(1) == 1)")
    if not logits.is_cuda:
        raise ValueError("logits must be on the GPU")
    return logits.shape[0], logits.shape[1], (logits.stride(0) if logits.shape[0] > 1
                                              else logits.shape[1])


def _target(target, T):
    if target.dtype != torch.int64 or target.dim() != 1 or target.shape[0] != T:
        raise ValueError("target must be int64 [T]")
    if not target.is_contiguous():
        raise ValueError("target must be contiguous")
    return target


def _grad_output(grad_output, reduction, T, device):
    if grad_output is None:
        return None
    if not isinstance(grad_output, torch.Tensor):
        grad_output = torch.tensor([float(grad_output)], device=device)
    go = grad_output.to(device=device, dtype=torch.float32).contiguous().reshape(-1)
    need = T if reduction == "none" else 1
    if go.numel() != need:
        raise ValueError(f"grad_output must have {need} element(s) for reduction={reduction}")
    return go


def _grad_dtype(grad, grad_dtype, logits):
    """The gradient dtype: that of a given buffer (which must agree with
    grad_dtype if both are given), else grad_dtype, else the logits'."""
    if grad is not None:
        if grad_dtype is not None and grad_dtype != grad.dtype:
            raise ValueError(f"grad is {grad.dtype} but grad_dtype={grad_dtype}")
        if grad.dim() != 2 or grad.stride(1) != 1 or tuple(grad.shape) != tuple(logits.shape):
            raise ValueError("grad must be a [T, V] view with contiguous rows")
        return grad.dtype
    return grad_dtype or logits.dtype


def _on(stream):
    """Context that makes `stream` current (allocations and the launch go on
    it), or does nothing for None."""
    if stream is None:
        return contextlib.nullcontext()
    if not isinstance(stream, torch.cuda.Stream):
        stream = torch.cuda.ExternalStream(int(stream))
    return torch.cuda.stream(stream)


def _on_stream(fn):
    """Runs `fn` with its `stream` keyword current (see the module notes)."""
    @functools.wraps(fn)
    def run(*args, stream=None, **kw):
        with _on(stream):
            return fn(*args, stream=stream, **kw)
    return run


def _workspace(prob, op, device):
    n = B.ce_workspace_bytes(prob, op)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device), n


@_on_stream
def fused_fwd_bwd(logits, target, *, ignore_index=-100, label_smoothing=0.0, reduction="mean",
                  grad_output=None, grad_dtype=None, grad=None, stream=None):
    """Loss, per-row loss, counts and d loss / d logits in one call."""
    T, V, ld = _logits2d(logits)
    target = _target(target, T)
    dev = logits.device
    gdt = _grad_dtype(grad, grad_dtype, logits)
    if grad is None:
        grad = torch.empty((T, V), dtype=gdt, device=dev)
    ldg = grad.stride(0) if T > 1 else V
    prob = B.make_problem(T, V, ld, ignore_index=ignore_index, label_smoothing=label_smoothing,
                          reduction=reduction)
    ws, nws = _workspace(prob, B.CE_OP_FUSED, dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    loss_rows = torch.empty(T, dtype=torch.float32, device=dev)
    n_valid = torch.empty(1, dtype=torch.int32, device=dev)
    err = torch.empty(1, dtype=torch.int32, device=dev)
    go = _grad_output(grad_output, reduction, T, dev)
    B.ce_fused_fwd_bwd(prob, logits, B.dtype_code(logits.dtype), target, go, loss_rows, loss,
                       n_valid, err, grad, B.dtype_code(gdt), ldg, ws, nws, stream)
    return {"loss": loss, "loss_rows": loss_rows, "grad": grad, "n_valid": n_valid,
            "err_count": err}


@_on_stream
def forward(logits, target, *, vocab_start=0, V_total=None, ignore_index=-100,
            label_smoothing=0.0, reduction="mean", stream=None):
    """Row statistics of this call's columns; when they are the whole
    vocabulary, also the finalize (fin, per-row and reduced loss, counts)."""
    T, V, ld = _logits2d(logits)
    target = _target(target, T)
    dev = logits.device
    V_total = V if V_total is None else V_total
    prob = B.make_problem(T, V, ld, vocab_start=vocab_start, V_total=V_total,
                          ignore_index=ignore_index, label_smoothing=label_smoothing,
                          reduction=reduction)
    ws, nws = _workspace(prob, B.CE_OP_FORWARD, dev)
    stats = torch.empty((T, B.ROW_STATS_BYTES), dtype=torch.uint8, device=dev)
    whole = vocab_start == 0 and V == V_total
    out = {"stats": stats}
    fin = loss_rows = loss = n_valid = err = None
    if whole:
        fin = torch.empty((T, B.ROW_FINAL_BYTES), dtype=torch.uint8, device=dev)
        loss_rows = torch.empty(T, dtype=torch.float32, device=dev)
        loss = torch.empty(1, dtype=torch.float32, device=dev)
        n_valid = torch.empty(1, dtype=torch.int32, device=dev)
        err = torch.empty(1, dtype=torch.int32, device=dev)
        out.update(fin=fin, loss_rows=loss_rows, loss=loss, n_valid=n_valid, err_count=err)
    B.ce_forward(prob, logits, B.dtype_code(logits.dtype), target, stats, fin, loss_rows, loss,
                 n_valid, err, ws, nws, stream)
    return out


@_on_stream
def merge_shard_stats(shard_stats, target, V_total, *, ignore_index=-100, label_smoothing=0.0,
                      reduction="mean", stream=None):
    """Merge per-shard statistics (a list of [T, 32] byte buffers in shard
    order, or one [S, T, 32] buffer) and finalize."""
    if isinstance(shard_stats, (list, tuple)):
        shard_stats = torch.stack(list(shard_stats))
    S, T = shard_stats.shape[0], shard_stats.shape[1]
    target = _target(target, T)
    dev = target.device
    prob = B.make_problem(T, 1, 1, V_total=V_total, ignore_index=ignore_index,
                          label_smoothing=label_smoothing, reduction=reduction)
    ws, nws = _workspace(prob, B.CE_OP_MERGE, dev)
    fin = torch.empty((T, B.ROW_FINAL_BYTES), dtype=torch.uint8, device=dev)
    loss_rows = torch.empty(T, dtype=torch.float32, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    n_valid = torch.empty(1, dtype=torch.int32, device=dev)
    err = torch.empty(1, dtype=torch.int32, device=dev)
    B.ce_merge_shard_stats(prob, S, shard_stats.contiguous(), target, fin, loss_rows, loss,
                           n_valid, err, ws, nws, stream)
    return {"fin": fin, "loss_rows": loss_rows, "loss": loss, "n_valid": n_valid,
            "err_count": err}


@_on_stream
def backward(logits, target, fin, n_valid, *, grad_output=None, vocab_start=0, V_total=None,
             ignore_index=-100, label_smoothing=0.0, reduction="mean", grad_dtype=None,
             grad=None, stream=None):
    """Gradient of this call's columns from the row constants `fin`."""
    T, V, ld = _logits2d(logits)
    target = _target(target, T)
    dev = logits.device
    V_total = V if V_total is None else V_total
    gdt = _grad_dtype(grad, grad_dtype, logits)
    if grad is None:
        grad = torch.empty((T, V), dtype=gdt, device=dev)
    ldg = grad.stride(0) if T > 1 else V
    prob = B.make_problem(T, V, ld, vocab_start=vocab_start, V_total=V_total,
                          ignore_index=ignore_index, label_smoothing=label_smoothing,
                          reduction=reduction)
    go = _grad_output(grad_output, reduction, T, dev)
    B.ce_backward(prob, logits, B.dtype_code(logits.dtype), target, fin, n_valid, go, grad,
                  B.dtype_code(gdt), ldg, stream)
    return grad


class CrossEntropy(torch.autograd.Function):
    """Autograd wrapper: the forward saves the logits (never copied or
    upcast), the targets and the 24-byte row constants; the backward runs
    the library's gradient pass."""

    @staticmethod
    def forward(ctx, logits, target, ignore_index, label_smoothing, reduction):
        out = forward(logits, target, ignore_index=ignore_index,
                      label_smoothing=label_smoothing, reduction=reduction)
        ctx.save_for_backward(logits, target, out["fin"], out["n_valid"])
        ctx.opts = (ignore_index, label_smoothing, reduction)
        return out["loss"][0] if reduction != "none" else out["loss_rows"]

    @staticmethod
    def backward(ctx, grad_out):
        logits, target, fin, n_valid = ctx.saved_tensors
        ignore_index, label_smoothing, reduction = ctx.opts
        g = backward(logits, target, fin, n_valid, grad_output=grad_out.reshape(-1),
                     ignore_index=ignore_index, label_smoothing=label_smoothing,
                     reduction=reduction)
        return g, None, None, None, None


def cross_entropy(logits, target, *, ignore_index=-100, label_smoothing=0.0, reduction="mean"):
    """Differentiable stable cross-entropy over [T, V] logits."""
    return CrossEntropy.apply(logits, target, ignore_index, label_smoothing, reduction)


@_on_stream
def linear_cross_entropy(E, C, target, *, ignore_index=-100, label_smoothing=0.0,
                         reduction="mean", grad_output=None, backward=True, accum="fp32",
                         filter_eps=0.0, stream=None):
    """Cross-entropy of the logits E C^T without forming them (the library's
    ce_linear_fwd_bwd): E [N, D] and C [V, D] bf16 with contiguous rows.
    Returns loss, loss_rows, n_valid, err_count and, with ``backward``, the
    fp32 gradients dE [N, D] and dC [V, D].  ``filter_eps`` > 0 turns on
    gradient filtering (256 x 256 blocks of softmax - q below it dropped
    from the backward products; 0, the default, is exact)."""
    if E.dtype != torch.bfloat16 or C.dtype != torch.bfloat16:
        raise ValueError("E and C must be bf16")
    if E.dim() != 2 or C.dim() != 2 or E.shape[1] != C.shape[1]:
        raise ValueError("E must be [N, D] and C [V, D]")
    if not (E.is_contiguous() and C.is_contiguous()):
        raise ValueError("E and C must be contiguous")
    N, D = E.shape
    V = C.shape[0]
    target = _target(target, N)
    dev = E.device
    prob = B.make_linear_problem(N, D, V, ignore_index=ignore_index,
                                 label_smoothing=label_smoothing, reduction=reduction,
                                 accum=accum, filter_eps=filter_eps)
    nws = B.ce_linear_workspace_bytes(prob, backward)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    loss_rows = torch.empty(N, dtype=torch.float32, device=dev)
    n_valid = torch.empty(1, dtype=torch.int32, device=dev)
    err = torch.empty(1, dtype=torch.int32, device=dev)
    dE = torch.empty((N, D), dtype=torch.float32, device=dev) if backward else None
    dC = torch.empty((V, D), dtype=torch.float32, device=dev) if backward else None
    go = _grad_output(grad_output, reduction, N, dev)
    B.ce_linear_fwd_bwd(prob, E, C, target, go, loss_rows, loss, n_valid, err, dE, dC, ws, nws,
                        stream)
    return {"loss": loss, "loss_rows": loss_rows, "n_valid": n_valid, "err_count": err,
            "dE": dE, "dC": dC}
