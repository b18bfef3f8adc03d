"""Comparison of the HIP path's outputs with the fp64 oracle (test helper).

Tolerances (stated with each check):
  loss and per-row loss  relative error <= 1e-5 on every valid row
  fp32 gradients         absolute error <= 1e-6
  bf16 gradients         <= 1 ulp from the oracle value rounded once to bf16
                         (ulps counted on the sign-magnitude -> ordered
                         integer map, +0 and -0 equal)
  collapse rows          loss_r and the target gradient nonzero; with fp32
                         gradients the target entry within 1e-5 relative
  ignored / bad rows     loss_r exactly +0 / NaN, gradient rows exactly 0
  counts                 exact
"""
import math

import numpy as np
import torch

from oracle import ce_oracle as O
from synth.ce_inputs import to_numpy_logits

LOSS_RTOL = 1e-5
F32_ATOL = 1e-6
BF16_ULPS = 1


def ordered_bf16(bits):
    b = np.asarray(bits).astype(np.int64) & 0xFFFF
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def bf16_bits(t):
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def grad_errors(gpu, ref):
    """(max error, kind) of a gradient block against the fp64 oracle."""
    if gpu.dtype == torch.bfloat16:
        g = ordered_bf16(bf16_bits(gpu))
        r = ordered_bf16(O.to_bf16(ref))
        return int(np.abs(g - r).max(initial=0)), "ulp"
    g = gpu.detach().to("cpu").double().numpy()
    return float(np.abs(g - ref).max(initial=0.0)), "abs"


def assert_grad_close(gpu, ref, what=""):
    err, kind = grad_errors(gpu, ref)
    if kind == "ulp":
        assert err <= BF16_ULPS, f"{what}: bf16 gradient off by {err} ulp"
    else:
        assert err <= F32_ATOL, f"{what}: fp32 gradient abs error {err:.3e}"


def assert_loss_rows(gpu_rows, ref, what=""):
    g = gpu_rows.detach().to("cpu").double().numpy()
    st = ref["status"]
    v = st == 1
    inf = v & ~np.isfinite(ref["loss_rows"])   # e.g. -inf logits with smoothing: +inf
    assert np.array_equal(g[inf], ref["loss_rows"][inf]), f"{what}: infinite per-row loss"
    v = v & ~inf
    rel = np.abs(g[v] - ref["loss_rows"][v]) / np.maximum(np.abs(ref["loss_rows"][v]), 1e-300)
    assert rel.max(initial=0.0) <= LOSS_RTOL, f"{what}: per-row loss rel err {rel.max():.3e}"
    ign = st == 0
    assert np.all(g[ign] == 0.0) and not np.any(np.signbit(g[ign])), f"{what}: ignored rows"
    assert np.all(np.isnan(g[st == -1])), f"{what}: bad-target rows must be NaN"


def assert_scalar_loss(gpu_loss, ref_loss, what=""):
    g = float(gpu_loss)
    if math.isnan(ref_loss):
        assert math.isnan(g), f"{what}: loss {g} should be NaN"
        return
    if math.isinf(ref_loss):
        # an infinite row loss (e.g. -inf logits with smoothing) carries over
        assert g == ref_loss, f"{what}: loss {g!r} should be {ref_loss!r}"
        return
    assert abs(g - ref_loss) <= LOSS_RTOL * abs(ref_loss) + 1e-30, \
        f"{what}: loss {g!r} vs {ref_loss!r}"


def assert_collapse_rows(gpu_rows, gpu_grad, target, ref, rows, what=""):
    """Rows whose target margin is large (where the cancelling form returns
    exactly 0): loss and target gradient stay nonzero, with the oracle's
    sign; fp32 target gradients within 1e-5 relative."""
    lr = gpu_rows.detach().to("cpu").double().numpy()
    for i in rows:
        t = int(target[i])
        assert lr[i] > 0.0, f"{what}: collapse row {i} has zero loss"
        gt = float(gpu_grad[i, t].double())
        ref_gt = ref["grad"][i, t]
        assert gt != 0.0 and (gt > 0) == (ref_gt > 0), \
            f"{what}: collapse row {i} target gradient {gt} vs {ref_gt}"
        if gpu_grad.dtype == torch.float32:
            assert abs(gt - ref_gt) <= 1e-5 * abs(ref_gt), f"{what}: row {i} g_t {gt} vs {ref_gt}"


def oracle_for(logits, target, *, ignore_index=-100, eps=0.0, reduction="mean",
               grad_output=1.0, n_valid=None):
    """The oracle on exactly what the GPU consumed: the same logits bytes and
    the label smoothing as the binary32 value the C ABI carries."""
    eps = float(np.float32(eps))
    z = to_numpy_logits(logits)
    t = target.detach().to("cpu").numpy()
    go = grad_output
    if isinstance(go, torch.Tensor):
        go = go.detach().to("cpu").double().numpy()
        if reduction != "none":
            go = float(go.reshape(-1)[0])
    return O.fwd_bwd(z, t, ignore_index=ignore_index, eps=eps, reduction=reduction,
                     grad_output=go, n_valid=n_valid)


def collapse_rows(logits, target, margin=15.0, ignore_index=-100):
    """Rows whose target beats every other logit by more than `margin`."""
    z = logits.detach().to("cpu").double()
    out = []
    for i in range(z.shape[0]):
        t = int(target[i])
        if t == ignore_index or t < 0 or t >= z.shape[1]:
            continue
        row = z[i].clone()
        zt = row[t].item()
        row[t] = -math.inf
        if zt - row.max().item() > margin:
            out.append(i)
    return out


# --------------------------------------------------------------------------
# linear classifier (logits E C^T)
# --------------------------------------------------------------------------
# The backward products take G = k (softmax - q) rounded once to bf16, as the
# matrix-core operand; each element's rounding error is at most 2^-8 of it
# (half a bf16 ulp) and about 2^-7.5 / sqrt(12) = 1.6e-3 of it in rms.  A
# gradient entry sum_v G_v C_v then carries an error of rms about
# 1.6e-3 * rs, rs = sqrt(sum_v (G_v C_v)^2) (the oracle's rsE / rsC).  The
# checks: every entry within 2^-6 rs (about 10 rms), and the whole matrix
# within 4e-3 in the rs-weighted Frobenius norm (2.5x the expected 1.6e-3,
# which a 1% scale or sign slip in any term exceeds).  fp32 accumulation and
# the fp32 logits add about 1e-5 of rs and are inside both bounds.
LIN_ELEM_TOL = 2.0 ** -6
LIN_FROB_TOL = 4e-3


def assert_linear_grad_close(gpu, ref, rs, what=""):
    g = gpu.detach().to("cpu").double().numpy()
    assert np.all(np.isfinite(g)), f"{what}: non-finite gradient"
    d = np.abs(g - ref)
    bad = d > LIN_ELEM_TOL * rs + 1e-30
    assert not bad.any(), (f"{what}: {int(bad.sum())} entries beyond 2^-6 rs; worst "
                           f"{float((d / np.maximum(rs, 1e-300)).max()):.3e} rs")
    den = float(np.sqrt((rs * rs).sum()))
    if den > 0:
        fro = float(np.sqrt((d * d).sum())) / den
        assert fro <= LIN_FROB_TOL, f"{what}: Frobenius error {fro:.3e} of rs"


def linear_oracle_for(E, C, target, *, ignore_index=-100, eps=0.0, reduction="mean",
                      grad_output=1.0, n_valid=None, dC=True):
    """The linear-classifier oracle on exactly the bytes the GPU consumed."""
    eps = float(np.float32(eps))
    Eb = E.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)
    Cb = C.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)
    t = target.detach().to("cpu").numpy()
    go = grad_output
    if isinstance(go, torch.Tensor):
        go = go.detach().to("cpu").double().numpy()
        if reduction != "none":
            go = float(go.reshape(-1)[0])
    return O.linear_fwd_bwd(Eb, Cb, t, ignore_index=ignore_index, eps=eps, reduction=reduction,
                            grad_output=go, n_valid=n_valid, dC=dC)
