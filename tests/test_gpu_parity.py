"""GPU parity: the HIP library through its C ABI against the fp64 oracle.

Sizes the oracle finishes in seconds but that span several vectors per
thread, several workgroup shapes, a scalar tail and the split-V grid; every
case is seeded (synth/ce_inputs.py).  Tolerances: tests/parity_util.py.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import vocab_softmax_cross_row_amd as vce
from oracle import ce_oracle as O
from synth import ce_inputs as S
from synth.ce_inputs import to_numpy_logits
from tests import parity_util as P

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _case(base, T, V, seed, **kw):
    c = S.scaled(base, T, V, seed, **kw)
    logits, target = S.generate(c)
    return c, logits.to(DEV), target.to(DEV)


def _say(*a):
    print(*a, flush=True)


def _fused_check(case, logits, target, *, grad_dtype=None, grad_output=None, what=""):
    _say(f"[fused] {what} T={case.T} V={case.V} {logits.dtype}->{grad_dtype or logits.dtype} "
         f"eps={case.eps} red={case.reduction}")
    before = logits.contiguous().view(torch.uint8).clone()
    out = vce.fused_fwd_bwd(logits, target, ignore_index=case.ignore_index,
                            label_smoothing=case.eps, reduction=case.reduction,
                            grad_output=grad_output, grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    assert torch.equal(before, logits.contiguous().view(torch.uint8)), "logits modified"
    ref = P.oracle_for(logits, target, ignore_index=case.ignore_index, eps=case.eps,
                       reduction=case.reduction,
                       grad_output=1.0 if grad_output is None else grad_output)
    assert int(out["n_valid"].item()) == ref["n_valid"]
    assert int(out["err_count"].item()) == ref["n_bad"]
    P.assert_loss_rows(out["loss_rows"], ref, what)
    if case.reduction != "none":
        P.assert_scalar_loss(out["loss"].item(), ref["loss"], what)
    P.assert_grad_close(out["grad"], ref["grad"], what)
    bad = ref["status"] != 1
    if bad.any():
        g = out["grad"].detach().cpu()[torch.from_numpy(bad)]
        assert torch.all(g == 0), f"{what}: non-valid rows must have zero gradient"
    coll = P.collapse_rows(logits, target)
    P.assert_collapse_rows(out["loss_rows"], out["grad"].cpu(), target.cpu(), ref, coll, what)
    return out, ref


# --------------------------------------------------------------------------
# the named workloads, at parity size
# --------------------------------------------------------------------------

def test_tiny_workload_fp32():
    """T=64, V=1000 fp32, 4 ignored rows, 8 rows at rowmax + 25, mean."""
    c = S.TINY
    logits, target = S.generate(c)
    out, ref = _fused_check(c, logits.to(DEV), target.to(DEV), what="tiny")
    assert len(P.collapse_rows(logits, target)) == 8


def test_mid_workload_scaled():
    _fused_check(*_case(S.MID, 192, 32000, 7), what="mid")


def test_page_workload_scaled():
    c, logits, target = _case(S.PAGE, 96, 128256, 8)
    _fused_check(c, logits, target, what="page")


@pytest.mark.parametrize("V", [300, 1000, 2000, 4000, 8192, 16000, 32000, 64128, 128256])
def test_every_resident_shape_bf16(V):
    c, logits, target = _case(S.PAGE, 520, V, 100 + V % 97)
    _fused_check(c, logits, target, what=f"resident V={V}")


@pytest.mark.parametrize("V", [200, 1000, 4000, 16000, 65536])
def test_resident_shapes_fp32(V):
    c, logits, target = _case(S.TINY, 520, V, 200 + V % 89)
    _fused_check(c, logits, target, what=f"resident fp32 V={V}")


@pytest.mark.parametrize("V", [1003, 32005, 128257])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_ragged_tail(V, dt):
    base = S.PAGE if dt == "bf16" else S.TINY
    c, logits, target = _case(base, 520, V, 300 + V % 31)
    # put targets into the scalar tail for some rows
    target[1] = V - 1
    target[2] = V - 2
    _fused_check(c, logits, target, what=f"ragged {dt} V={V}")


@pytest.mark.parametrize("dt,V", [("bf16", 151936), ("bf16", 171776), ("bf16", 171784),
                                  ("f32", 80000)])
def test_long_rows_one_workgroup_per_cu(dt, V):
    # beyond what two workgroups per CU hold, the register + LDS kernel runs
    # one workgroup per CU (up to 171776 bf16 / 85888 fp32 columns); past
    # that the rows stream
    base = S.PAGE if dt == "bf16" else S.TINY
    c, logits, target = _case(base, 520, V, 88 + V % 13)
    target[5] = V - 1
    _fused_check(c, logits, target, what=f"long rows {dt} V={V}")


@pytest.mark.parametrize("eps", [0.0, 0.1])
def test_rows_too_long_for_registers_bf16(eps):
    # bf16 rows longer than 131072 columns do not fit the resident kernels:
    # the fused entry point streams them (column-chunk statistics, on-device
    # merge, gradient pass)
    c, logits, target = _case(S.PAGE, 600, 150001, 77, eps=eps)
    target[3] = 150000
    _fused_check(c, logits, target, what=f"long rows eps={eps}")


@pytest.mark.parametrize("in_dt,out_dt", [("bf16", torch.float32), ("f32", torch.bfloat16)])
def test_mixed_dtypes(in_dt, out_dt):
    base = S.PAGE if in_dt == "bf16" else S.TINY
    c, logits, target = _case(base, 530, 5000, 41)
    _fused_check(c, logits, target, grad_dtype=out_dt, what=f"mixed {in_dt}->{out_dt}")


@pytest.mark.parametrize("reduction", ["none", "sum", "mean"])
def test_reductions_and_grad_output(reduction):
    c, logits, target = _case(S.PAGE, 520, 3000, 51, reduction=reduction)
    if reduction == "none":
        go = torch.randn(c.T, generator=torch.Generator().manual_seed(3)).to(DEV)
    else:
        go = torch.tensor([0.37], device=DEV)
    _fused_check(c, logits, target, grad_output=go, what=f"reduction {reduction}")


@pytest.mark.parametrize("eps", [0.1, 0.3])
@pytest.mark.parametrize("V", [300, 1000, 2000, 4000, 8000, 32000, 32768, 32769, 128256])
def test_label_smoothing_fused(eps, V):
    # bf16 rows up to 32768 columns stay resident; longer ones stream
    c, logits, target = _case(S.PAGE, 520, V, 61, eps=eps)
    _fused_check(c, logits, target, what=f"smoothing eps={eps} V={V}")


def test_label_smoothing_fp32_out():
    c, logits, target = _case(S.TINY, 520, 1500, 62, eps=0.2, reduction="sum")
    _fused_check(c, logits, target, what="smoothing fp32 sum")


@pytest.mark.parametrize("reduction", ["sum", "none"])
def test_label_smoothing_bf16_in_fp32_out_table(reduction):
    # bf16 rows of 16385 to 32768 columns with smoothing: the fused kernel
    # that sums e^z from the LDS table, writing an fp32 gradient
    c, logits, target = _case(S.PAGE, 300, 24000, 63, eps=0.2, reduction=reduction)
    go = None
    if reduction == "none":
        go = torch.linspace(-2.0, 2.0, c.T, device=DEV)
    _fused_check(c, logits, target, grad_dtype=torch.float32, grad_output=go,
                 what=f"smoothing bf16 -> fp32, {reduction}")


def test_split_v_grid_short_T():
    """Few rows, long rows: the fused entry point splits every row into
    column chunks (partial statistics merged on the device)."""
    c, logits, target = _case(S.PAGE, 24, 128256, 71)
    _fused_check(c, logits, target, what="split-V grid")
    c, logits, target = _case(S.PAGE, 24, 128256, 72, eps=0.1)
    _fused_check(c, logits, target, what="split-V grid smoothing")


def test_unaligned_rows_take_the_scalar_path():
    """ld not a multiple of 8 elements: rows are not 16-byte aligned."""
    c, full, target = _case(S.PAGE, 520, 2003, 81)
    view = full[:, :2001]        # ld = 2003, V = 2001
    _fused_check(c, view, target, what="unaligned ld")
    g = torch.empty((c.T, 2005), dtype=torch.bfloat16, device=DEV)[:, 1:2002]
    out = vce.fused_fwd_bwd(view, target, grad=g)
    torch.cuda.synchronize()
    ref = P.oracle_for(view, target)
    P.assert_grad_close(out["grad"], ref["grad"], "unaligned grad")


@pytest.mark.parametrize("dt,T,V,eps", [
    ("bf16", 520, 2001, 0.0),      # odd width: every row starts at a different 16-byte offset
    ("bf16", 520, 2001, 0.1),      # resident with smoothing
    ("bf16", 520, 100003, 0.0),    # beyond 65536: the resident kernel, not the LDS-split one
    ("bf16", 40, 50257, 0.0),      # short T: column chunks, each with its own head
    ("bf16", 600, 50257, 0.1),     # smoothing: the table statistics peel the head too
    ("f32", 520, 1001, 0.0),
])
def test_odd_width_rows_take_the_vector_path(dt, T, V, eps):
    """Contiguous rows of odd width are not 16-byte aligned, but a contiguous
    gradient has the same misalignment in every row: the streaming kernels
    peel each row's head up to the first 16-byte boundary and use vectors
    after it.  Fused, in place, and per-shard forward/backward on views that
    start at an odd column."""
    base = S.PAGE if dt == "bf16" else S.TINY
    c, logits, target = _case(base, T, V, 500 + V % 97, eps=eps)
    _fused_check(c, logits, target, what=f"odd width {dt} T={T} V={V} eps={eps}")
    ref = P.oracle_for(logits, target, eps=eps)
    buf = logits.clone()
    out = vce.fused_fwd_bwd(buf, target, grad=buf, label_smoothing=eps)
    torch.cuda.synchronize()
    P.assert_grad_close(out["grad"], ref["grad"], "odd width in place")
    # shards that start at odd columns of the same rows
    edges = [0, 3, V // 2 + 1, V]
    stats = [vce.forward(logits[:, a:b], target, vocab_start=a, V_total=V,
                         label_smoothing=eps)["stats"] for a, b in zip(edges[:-1], edges[1:])]
    m = vce.merge_shard_stats(stats, target, V, label_smoothing=eps)
    g = torch.empty_like(logits)
    for a, b in zip(edges[:-1], edges[1:]):
        vce.backward(logits[:, a:b], target, m["fin"], m["n_valid"], grad=g[:, a:b],
                     vocab_start=a, V_total=V, label_smoothing=eps)
    torch.cuda.synchronize()
    P.assert_loss_rows(m["loss_rows"], ref, "odd width shards")
    P.assert_grad_close(g, ref["grad"], "odd width shard grads")


# --------------------------------------------------------------------------
# unfused path: forward, split-vocabulary shards, merge, backward
# --------------------------------------------------------------------------

def _stats_check(gpu_stats, ref_stats, target, V_total, what, eps):
    """m, z_t and own exactly, s and the row sum to 1e-5 relative, on rows
    with a valid target; rows that are ignored or have a bad target are not
    read and carry m = -inf, s = 0, z_t = 0, own = 0, sum 0."""
    st = vce.read_stats(gpu_stats)
    t = np.asarray(target)
    read = (t != -100) & (t >= 0) & (t < V_total)
    assert np.array_equal(st["own"][read], ref_stats["own"][read]), what
    assert np.array_equal(st["m"][read].astype(np.float64), ref_stats["m"][read]), f"{what}: m"
    assert np.array_equal(st["zt"][read].astype(np.float64), ref_stats["zt"][read]), \
        f"{what}: zt"
    rs = ref_stats["s"][read]
    rel = np.abs(st["s"][read] - rs) / np.maximum(rs, 1e-300)
    assert rel.max(initial=0) <= 1e-5, f"{what}: s rel {rel.max():.2e}"
    if eps > 0:   # the row sum is only formed when smoothing needs it
        sz = ref_stats["sz"][read]
        gz = st["sz"][read]
        fin = np.isfinite(sz)
        assert np.array_equal(gz[~fin], sz[~fin]), f"{what}: infinite sum z"
        scale = np.maximum(np.abs(sz[fin]), 1.0)
        assert (np.abs(gz[fin] - sz[fin]) / scale).max(initial=0) <= 1e-5, f"{what}: sum z"
    skip = ~read
    assert np.all(st["m"][skip] == -np.inf) and np.all(st["s"][skip] == 0)
    assert np.all(st["own"][skip] == 0) and np.all(st["zt"][skip] == 0)


@pytest.mark.parametrize("V,eps", [(20000, 0.0), (20000, 0.1), (40003, 0.0), (64128, 0.0)])
def test_forward_backward_unsharded(V, eps):
    # 40003 and 64128 columns: rows long enough for the 128-thread
    # statistics shape (odd width: a peeled head)
    c, logits, target = _case(S.PAGE, 1100, V, 91, eps=eps)
    _say(f"[unfused] T={c.T} V={c.V} eps={eps}")
    f = vce.forward(logits, target, label_smoothing=eps)
    g = vce.backward(logits, target, f["fin"], f["n_valid"], label_smoothing=eps)
    torch.cuda.synchronize()
    ref = P.oracle_for(logits, target, eps=eps)
    assert int(f["n_valid"].item()) == ref["n_valid"]
    P.assert_loss_rows(f["loss_rows"], ref, "unfused")
    P.assert_scalar_loss(f["loss"].item(), ref["loss"], "unfused")
    P.assert_grad_close(g, ref["grad"], "unfused grad")
    # statistics of the whole row
    z = to_numpy_logits(logits)
    t = target.cpu().numpy()
    rs = O.shard_stats(z, t, 0)
    _stats_check(f["stats"], rs, t, c.V, "whole-row stats", eps)
    fin = vce.read_final(f["fin"])
    assert np.array_equal(fin["status"], ref["status"])


@pytest.mark.parametrize("cuts,eps,T", [([64128], 0.1, 700), ([64128], 0.0, 700),
                                        ([40000, 90000], 0.1, 650), ([64128], 0.1, 40)])
def test_split_vocabulary_shards(cuts, eps, T):
    """Shards of a 128256-column vocabulary: per-shard statistics (checked
    against the oracle's shard emulation), the on-device merge, and the
    per-shard backward."""
    c, logits, target = _case(S.PAGE, T, 128256, 95 + len(cuts), eps=eps)
    V = c.V
    edges = [0] + cuts + [V]
    _say(f"[shards] T={T} edges={edges} eps={eps}")
    z = to_numpy_logits(logits)
    t = target.cpu().numpy()
    stats = []
    for a, b in zip(edges[:-1], edges[1:]):
        f = vce.forward(logits[:, a:b], target, vocab_start=a, V_total=V,
                        label_smoothing=eps)
        stats.append(f["stats"])
        rs = O.shard_stats(np.ascontiguousarray(z[:, a:b]), t, a)
        torch.cuda.synchronize()
        _stats_check(f["stats"], rs, t, V, f"shard [{a},{b})", eps)
    m = vce.merge_shard_stats(stats, target, V, label_smoothing=eps)
    grads = []
    for a, b in zip(edges[:-1], edges[1:]):
        grads.append(vce.backward(logits[:, a:b], target, m["fin"], m["n_valid"],
                                  vocab_start=a, V_total=V, label_smoothing=eps))
    torch.cuda.synchronize()
    ref = P.oracle_for(logits, target, eps=eps)
    assert int(m["n_valid"].item()) == ref["n_valid"]
    P.assert_loss_rows(m["loss_rows"], ref, "merged")
    P.assert_scalar_loss(m["loss"].item(), ref["loss"], "merged")
    for (a, b), g in zip(zip(edges[:-1], edges[1:]), grads):
        P.assert_grad_close(g, ref["grad"][:, a:b], f"shard grad [{a},{b})")


@pytest.mark.parametrize("dt,V,a,eps", [("bf16", 64128, 0, 0.1), ("bf16", 64128, 64128, 0.0),
                                        ("bf16", 40003, 17, 0.1), ("f32", 20001, 3, 0.0)])
def test_backward_long_chunks(dt, V, a, eps):
    """Backward over rows long enough for the 1024-thread gradient shape
    (one column chunk per row once T >= 1024), for a shard of a wider
    vocabulary at an aligned or odd column offset; the gradient goes into a
    larger canary-filled buffer, which must keep its canary outside the
    [T, V] view."""
    T, Vt = 1030, a + V + 5
    base = S.PAGE if dt == "bf16" else S.TINY
    c, whole, target = _case(base, T, Vt, 610 + V % 89, eps=eps)
    logits = whole[:, a:a + V]
    _say(f"[long chunks] T={T} shard [{a},{a + V}) of {Vt} {dt} eps={eps}")
    # row constants of the whole vocabulary, then this shard's backward
    m = vce.forward(whole, target, label_smoothing=eps)
    out_dt = logits.dtype
    canary = 0x7FC5 if out_dt == torch.bfloat16 else 0x7FC00005
    ity = torch.int16 if out_dt == torch.bfloat16 else torch.int32
    # same residue mod 16 bytes as the logits view, so the vector path runs
    buf = torch.full((T + 1, Vt), canary, dtype=ity, device=DEV).view(out_dt)
    g = buf[:T, a:a + V]
    vce.backward(logits, target, m["fin"], m["n_valid"], vocab_start=a, V_total=Vt,
                 label_smoothing=eps, grad=g)
    torch.cuda.synchronize()
    raw = buf.view(ity)
    assert torch.all(raw[:T, :a] == canary), "write before the start of a row"
    assert torch.all(raw[:T, a + V:] == canary), "write past the end of a row"
    assert torch.all(raw[T] == canary), "write past the last row"
    # the oracle over the whole vocabulary; compare this shard's columns
    ref = P.oracle_for(whole, target, eps=eps)
    P.assert_grad_close(g, ref["grad"][:, a:a + V], f"long chunks [{a},{a + V})")


def test_fused_equals_unfused_equals_shards_loss():
    """Three paths to the same loss (fp32 rounding apart)."""
    c, logits, target = _case(S.PAGE, 600, 64128, 99)
    a = vce.fused_fwd_bwd(logits, target)
    f = vce.forward(logits, target)
    s1 = vce.forward(logits[:, :32064], target, vocab_start=0, V_total=64128)
    s2 = vce.forward(logits[:, 32064:], target, vocab_start=32064, V_total=64128)
    m = vce.merge_shard_stats([s1["stats"], s2["stats"]], target, 64128)
    torch.cuda.synchronize()
    la, lf, lm = a["loss"].item(), f["loss"].item(), m["loss"].item()
    assert abs(la - lf) <= 1e-5 * abs(lf) and abs(lm - lf) <= 1e-5 * abs(lf)


# --------------------------------------------------------------------------
# edge cases
# --------------------------------------------------------------------------

def test_empty_batch():
    logits = torch.empty((0, 100), dtype=torch.bfloat16, device=DEV)
    target = torch.empty((0,), dtype=torch.int64, device=DEV)
    out = vce.fused_fwd_bwd(logits, target)
    torch.cuda.synchronize()
    assert math.isnan(out["loss"].item()) and out["n_valid"].item() == 0
    out = vce.fused_fwd_bwd(logits, target, reduction="sum")
    torch.cuda.synchronize()
    assert out["loss"].item() == 0.0


def test_single_column_and_all_ignored():
    logits = torch.randn((5, 1), device=DEV)
    target = torch.zeros(5, dtype=torch.int64, device=DEV)
    out = vce.fused_fwd_bwd(logits, target, label_smoothing=0.1)
    torch.cuda.synchronize()
    assert torch.all(out["loss_rows"] == 0) and torch.all(out["grad"] == 0)
    logits = torch.randn((7, 300), device=DEV).to(torch.bfloat16)
    target = torch.full((7,), -100, dtype=torch.int64, device=DEV)
    out = vce.fused_fwd_bwd(logits, target)
    torch.cuda.synchronize()
    assert math.isnan(out["loss"].item()) and torch.all(out["grad"] == 0)


def test_bad_targets_counted():
    logits = torch.randn((8, 500), device=DEV)
    target = torch.tensor([0, 1, 500, -1, -100, 7, 10**12, 3], dtype=torch.int64, device=DEV)
    out = vce.fused_fwd_bwd(logits, target, reduction="sum")
    torch.cuda.synchronize()
    assert out["err_count"].item() == 3 and out["n_valid"].item() == 4
    lr = out["loss_rows"].cpu()
    assert torch.isnan(lr[[2, 3, 6]]).all() and lr[4].item() == 0.0
    assert torch.all(out["grad"][[2, 3, 4, 6]] == 0)
    assert math.isnan(out["loss"].item())


@pytest.mark.parametrize("T", [5, 1024, 1025])
def test_batch_count_in_kernel_and_by_launch(T):
    """Batches of up to 1024 rows on the register-resident kernel count their
    targets inside it (workgroup 0, which takes row 0, writes the count);
    longer ones in a launch of their own.  Row 0 holds a bad target, so the
    workgroup writing the count takes the zero-gradient exit; the mean
    reduction makes every gradient row depend on the count."""
    c, logits, target = _case(S.MID, T, 3000, 11)
    target[0] = 3000
    target[1::7] = c.ignore_index
    c = dataclasses.replace(c, reduction="mean")
    _fused_check(c, logits, target, what=f"count T={T}")


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_minus_inf_logits(dt):
    """Rows with -inf fallback logits (torchtitan PR Test Plan)."""
    g = torch.Generator().manual_seed(5)
    z = torch.randn((520, 700), generator=g) * 2
    target = torch.randint(0, 700, (520,), generator=g)
    z[0, :350] = -math.inf                  # half the row at -inf
    z[1, :] = -math.inf
    z[1, target[1]] = 1.0                   # only the target is finite
    z[2, target[2]] = -math.inf             # target at -inf: loss +inf
    target[3] = -100
    z[3, :] = -math.inf                     # ignored row of -inf
    z = z.to(dt)
    if z[0, target[0]] == -math.inf:
        target[0] = 400
    logits, tgt = z.to(DEV), target.to(DEV)
    out = vce.fused_fwd_bwd(logits, tgt, reduction="none")
    torch.cuda.synchronize()
    ref = P.oracle_for(logits, tgt, reduction="none")
    lr = out["loss_rows"].cpu()
    assert lr[1].item() == 0.0 and torch.all(out["grad"][1] == 0)
    assert lr[2].item() == math.inf and lr[3].item() == 0.0
    keep = [i for i in range(520) if i != 2]
    rows = ref["status"].copy()
    rows[2] = 0  # the +inf row is compared exactly above
    fake = dict(ref)
    fake["status"] = rows
    fake["loss_rows"] = ref["loss_rows"].copy()
    fake["loss_rows"][2] = 0.0
    lr2 = out["loss_rows"].clone()
    lr2[2] = 0.0
    P.assert_loss_rows(lr2, fake, "-inf")
    P.assert_grad_close(out["grad"][keep], ref["grad"][keep], "-inf grad")
    assert float(out["grad"][2, tgt[2]]) == -1.0


@pytest.mark.parametrize("dt,V,eps", [
    (torch.float32, 700, 0.1),     # fp32 register-resident, fp64 exponentials
    (torch.bfloat16, 700, 0.1),    # bf16 register-resident with smoothing
    (torch.float32, 70001, 0.1),   # fp32 rows streamed: online fp64 sums
    (torch.bfloat16, 700, 0.0),    # bf16 fast path
])
def test_plus_inf_logit_gives_nan_row(dt, V, eps):
    """A +inf non-target logit makes its row's loss NaN (inf - inf in the
    softmax), as in the oracle; the other rows are unaffected."""
    c, logits, target = _case(S.PAGE if dt == torch.bfloat16 else S.TINY, 520, V, 909, eps=eps,
                              dtype=dt)
    target[0] = 10
    logits[0, 5] = math.inf
    target[1] = -100
    logits[1, 3] = math.inf                   # an ignored row: still exactly zero
    out = vce.fused_fwd_bwd(logits, target, label_smoothing=eps, reduction="none")
    torch.cuda.synchronize()
    ref = P.oracle_for(logits, target, eps=eps, reduction="none")
    assert math.isnan(ref["loss_rows"][0])
    lr = out["loss_rows"].cpu()
    _say(f"[+inf] {dt} V={V} eps={eps}: row 0 loss {lr[0].item()}")
    assert math.isnan(lr[0].item()), f"+inf row: loss {lr[0].item()} instead of NaN"
    assert lr[1].item() == 0.0 and torch.all(out["grad"][1] == 0)
    rest = list(range(2, 520))
    sub = {k: (v[rest] if isinstance(v, np.ndarray) and v.shape[:1] == (520,) else v)
           for k, v in ref.items()}
    P.assert_loss_rows(out["loss_rows"][2:], sub, "+inf other rows")
    P.assert_grad_close(out["grad"][2:], ref["grad"][2:], "+inf other rows grad")


def test_side_stream_calls_match_current_stream():
    """stream= runs a call on another stream: its outputs and workspace are
    allocated there, so allocations on the current stream made while it runs
    cannot take them over.  The split-V grid keeps partial statistics in the
    workspace; results equal a current-stream call bit for bit and the
    oracle within the usual bounds."""
    c, logits, target = _case(S.PAGE, 40, 128256, 905, eps=0.1)
    ref = vce.fused_fwd_bwd(logits, target, label_smoothing=0.1)
    f_ref = vce.forward(logits, target, label_smoothing=0.1)
    g_ref = vce.backward(logits, target, f_ref["fin"], f_ref["n_valid"], label_smoothing=0.1)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    out = vce.fused_fwd_bwd(logits, target, label_smoothing=0.1, stream=s)
    f = vce.forward(logits, target, label_smoothing=0.1, stream=s)
    g = vce.backward(logits, target, f["fin"], f["n_valid"], label_smoothing=0.1, stream=s)
    junk = [torch.full((1 << 22,), 7.0, device=DEV) for _ in range(8)]
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    del junk
    for k in ("loss", "loss_rows", "n_valid"):
        assert torch.equal(out[k], ref[k]), k
    assert torch.equal(out["grad"].view(torch.int16), ref["grad"].view(torch.int16))
    assert torch.equal(f["loss"], f_ref["loss"])
    assert torch.equal(g.view(torch.int16), g_ref.view(torch.int16))
    oracle = P.oracle_for(logits, target, eps=0.1)
    P.assert_loss_rows(out["loss_rows"], oracle, "side stream")
    P.assert_grad_close(out["grad"], oracle["grad"], "side stream grad")


def test_deterministic_run_to_run():
    c, logits, target = _case(S.PAGE, 700, 50000, 123, eps=0.1)
    a = vce.fused_fwd_bwd(logits, target, label_smoothing=0.1)
    b = vce.fused_fwd_bwd(logits, target, label_smoothing=0.1)
    torch.cuda.synchronize()
    for k in ("loss", "loss_rows", "grad"):
        assert torch.equal(a[k].view(torch.uint8), b[k].view(torch.uint8)), k


def test_subnormal_gradients_round_correctly():
    """Probabilities far below 2^-126 come out as the right subnormals (or
    zero) in both output dtypes, not flushed early."""
    z = torch.zeros((520, 600))
    z[:, 1:300] = torch.linspace(-95.0, -80.0, 299)   # p ~ 1e-42 .. 1e-35
    z[:, 300:] = torch.linspace(-110.0, -100.0, 300)  # below the smallest subnormal
    target = torch.zeros(520, dtype=torch.int64)
    for dt in (torch.float32, torch.bfloat16):
        logits = z.to(dt).to(DEV)
        tgt = target.to(DEV)
        out = vce.fused_fwd_bwd(logits, tgt, reduction="sum")
        torch.cuda.synchronize()
        ref = P.oracle_for(logits, tgt, reduction="sum")
        P.assert_grad_close(out["grad"], ref["grad"], f"subnormal {dt}")
        if dt == torch.float32:
            g = out["grad"].cpu().double().numpy()
            err = np.abs(g - ref["grad"]) - 1e-5 * np.abs(ref["grad"])
            assert err.max() <= 2.0 ** -149, "fp32 subnormal gradients"
            assert (g[:, 1:300] > 0).all(), "subnormal gradients flushed to zero"


def test_api_errors_raise():
    logits = torch.randn((4, 10), device=DEV)
    target = torch.zeros(4, dtype=torch.int64, device=DEV)
    with pytest.raises(vce.CEError):
        vce.fused_fwd_bwd(logits, target, label_smoothing=1.0)
    # grad overlapping the logits other than exactly (in place is allowed)
    buf = torch.randn((4, 11), device=DEV)
    with pytest.raises(vce.CEError):
        vce.fused_fwd_bwd(buf[:, :10], target, grad=buf[:, 1:])


# --------------------------------------------------------------------------
# writes stay inside [T, V] of the gradient view
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T,V,in_dt,out_dt", [
    (520, 128256, torch.bfloat16, torch.bfloat16),   # register + LDS rows, 2 per CU
    (520, 128257, torch.bfloat16, torch.bfloat16),   # ... with a scalar tail
    (520, 100003, torch.bfloat16, torch.float32),
    (520, 40001, torch.float32, torch.bfloat16),
    (520, 3000, torch.bfloat16, torch.bfloat16),     # register-resident rows
    (520, 64128, torch.bfloat16, torch.bfloat16),
    (24, 128256, torch.bfloat16, torch.bfloat16),    # split-V grid
])
def test_writes_stay_inside_the_gradient_rows(T, V, in_dt, out_dt):
    """The gradient rows sit in a larger buffer (row stride V + 64, one
    extra row) filled with a NaN-payload canary; after the call every
    element outside the [T, V] view still holds it, and the view matches
    the oracle."""
    base = S.PAGE if in_dt == torch.bfloat16 else S.TINY
    c, logits, target = _case(base, T, V, 500 + V % 97)
    pad = 64
    canary = 0x7FC5 if out_dt == torch.bfloat16 else 0x7FC00005
    ity = torch.int16 if out_dt == torch.bfloat16 else torch.int32
    buf = torch.full((T + 1, V + pad), canary, dtype=ity, device=DEV).view(out_dt)
    g = buf[:T, :V]
    _say(f"[canary] T={T} V={V} {in_dt}->{out_dt}")
    out = vce.fused_fwd_bwd(logits, target, grad=g)
    torch.cuda.synchronize()
    raw = buf.view(ity)
    assert torch.all(raw[:T, V:] == canary), "write past the end of a row"
    assert torch.all(raw[T] == canary), "write past the last row"
    ref = P.oracle_for(logits, target)
    P.assert_grad_close(out["grad"], ref["grad"], f"canary view T={T} V={V}")
    P.assert_loss_rows(out["loss_rows"], ref, "canary")


def _table_edge_rows(logits, target):
    """Rows 0-7 rewritten with the values the table of e^z treats apart:
    zeros, |z| around 2^-16, |z| >= 512, -inf, a tiny-valued row, values
    just below 512 and +-1000."""
    z = logits.float().cpu()
    t = target.cpu()

    def put(r, cols, vals):
        for col, v in zip(cols, vals):
            if int(t[r]) != col:
                z[r, col] = v
    put(0, range(0, 400, 4), [0.0] * 100)
    put(1, [3, 9, 27, 81, 243], [1e-6, -1e-6, 2.0 ** -16, -(2.0 ** -16), 3e-5])
    put(2, [10], [600.0])
    put(3, [20], [-700.0])
    put(4, [5, 6], [-math.inf, -math.inf])
    z[5] *= 1e-6
    put(6, [30, 31, 32], [510.0, -510.0, 511.0])
    put(7, [1, 2], [-1000.0, 1000.0])
    return z.to(torch.bfloat16).to(DEV)


@pytest.mark.parametrize("V", [12000, 30001])
def test_smoothed_fused_table_edge_values(V):
    """Fused forward + backward of smoothed bf16 rows with 16384 < V <= 32768
    (the row-resident kernel that sums e^z from the LDS table; 30001: an odd
    width, so rows have a peeled head and a scalar tail), and 12000 (fp64
    exponentials), on the table's edge values."""
    c, logits, target = _case(S.PAGE, 64, V, 137, eps=0.1)
    logits = _table_edge_rows(logits, target)
    _fused_check(c, logits, target, what=f"table edges fused V={V}")


@pytest.mark.parametrize("shard", [False, True])
def test_smoothed_bf16_statistics_edge_values(shard):
    """The smoothed bf16 statistics read e^z from a table of bf16 patterns
    with 2^-16 <= |z| < 2^9: zeros and values below 2^-16 take a series,
    values of magnitude >= 512 send the chunk to the online form, -inf
    logits and the target read the table's zero entry."""
    c, logits, target = _case(S.PAGE, 64, 5000, 131, eps=0.1)
    logits = _table_edge_rows(logits, target)
    t = target.cpu()
    eps = 0.1
    ref = P.oracle_for(logits, target, eps=eps)
    if shard:
        edges = [0, 2504, 5000]
        stats = [vce.forward(logits[:, a:b], target, vocab_start=a, V_total=5000,
                             label_smoothing=eps)["stats"] for a, b in zip(edges[:-1], edges[1:])]
        m = vce.merge_shard_stats(stats, target, 5000, label_smoothing=eps)
        fin, nv, lr = m["fin"], m["n_valid"], m["loss_rows"]
    else:
        f = vce.forward(logits, target, label_smoothing=eps)
        fin, nv, lr = f["fin"], f["n_valid"], f["loss_rows"]
        zz = to_numpy_logits(logits)
        _stats_check(f["stats"], O.shard_stats(zz, t.numpy(), 0), t.numpy(), 5000,
                     "table stats", eps)
    g = vce.backward(logits, target, fin, nv, label_smoothing=eps)
    torch.cuda.synchronize()
    P.assert_loss_rows(lr, ref, "table edges")
    P.assert_grad_close(g, ref["grad"], "table edges grad")


def test_smoothed_bf16_statistics_max_by_sign():
    """The smoothed bf16 statistics take the running max of the patterns
    read as another 16-bit float format; the max must come out right
    whatever the signs: rows all negative, all positive, negative but for
    one small positive logit, and negative but for a large positive target
    (which the non-target max leaves out).  40000 columns: four whole
    groups of vectors per row, then the per-vector tail."""
    c, logits, target = _case(S.PAGE, 64, 40000, 149, eps=0.1)
    g = torch.Generator().manual_seed(149)
    z = logits.float().cpu()
    t = target.cpu()
    a = z.abs()
    z[0:16] = -a[0:16] - 1.0
    z[16:32] = a[16:32] + 1.0
    z[32:48] = -a[32:48] - 2.0
    cols = torch.randint(0, 40000, (16,), generator=g)
    for i in range(16):
        r = 32 + i
        col = int(cols[i]) if int(cols[i]) != int(t[r]) else (int(cols[i]) + 1) % 40000
        z[r, col] = 0.0078125 * (i + 1)
    z[48:64] = -a[48:64] - 3.0
    for r in range(48, 64):
        if 0 <= int(t[r]) < 40000:
            z[r, int(t[r])] = 50.0
    logits = z.to(torch.bfloat16).to(DEV)
    eps = 0.1
    f = vce.forward(logits, target, label_smoothing=eps)
    torch.cuda.synchronize()
    zz = to_numpy_logits(logits)
    _stats_check(f["stats"], O.shard_stats(zz, t.numpy(), 0), t.numpy(), 40000,
                 "max by sign", eps)
    ref = P.oracle_for(logits, target, eps=eps)
    P.assert_loss_rows(f["loss_rows"], ref, "max by sign")


@pytest.mark.parametrize("V", [6144, 24576])
@pytest.mark.parametrize("eps", [0.1, 0.6])
def test_smoothed_gradient_where_p_meets_eps_over_v(eps, V):
    """With smoothing, a non-target gradient is k (p_j - eps/V), which cancels
    where p_j is close to eps/V.  Each row holds 4096 zeros and a sweep of
    2048 logits through [-3, 1] (shifted a little per row), so that p_j
    passes eps/V in bf16 steps: some entries fall inside the window where the
    difference is rebuilt from log2(p/u) (|log2(p/u)| < 2^-6), many just
    outside it, where the plain form must already be within a bf16 ulp.
    V = 24576 takes the fused kernel that sums e^z from the LDS table."""
    T = 8
    z = torch.zeros(T, V)
    sweep = torch.linspace(-3.0, 1.0, 2048)
    for r in range(T):
        z[r, V - 2048:] = sweep + r * 2.0 ** -9
    logits = z.to(torch.bfloat16).to(DEV)
    target = torch.tensor([17 * (r + 1) for r in range(T)], dtype=torch.int64, device=DEV)
    zz = logits.double().cpu().numpy()
    lse = np.log(np.exp(zz).sum(axis=1, keepdims=True))
    w = (zz - lse - math.log(np.float32(eps) / V)) / math.log(2.0)
    inside = int((np.abs(w) < 2.0 ** -6).sum())
    near = int(((np.abs(w) >= 2.0 ** -6) & (np.abs(w) < 0.5)).sum())
    _say(f"[p ~ eps/V] eps={eps}: {inside} entries inside the window, {near} within 0.5")
    assert inside >= 8 and near >= 400
    ref = P.oracle_for(logits, target, eps=eps)
    out = vce.fused_fwd_bwd(logits, target, label_smoothing=eps)
    f = vce.forward(logits, target, label_smoothing=eps)
    g = vce.backward(logits, target, f["fin"], f["n_valid"], label_smoothing=eps)
    torch.cuda.synchronize()
    P.assert_loss_rows(out["loss_rows"], ref, "p ~ eps/V fused")
    P.assert_grad_close(out["grad"], ref["grad"], "p ~ eps/V fused grad")
    P.assert_grad_close(g, ref["grad"], "p ~ eps/V streaming grad")


@pytest.mark.parametrize("T,V,dt,eps", [
    (300, 128256, torch.bfloat16, 0.0),    # two rows per CU, row split register/LDS
    (96, 32000, torch.bfloat16, 0.1),      # register-resident with smoothing
    (64, 1000, torch.float32, 0.0),        # fp32, register-resident
    (40, 128256, torch.bfloat16, 0.1),     # split-V grid (streaming kernels)
])
def test_in_place_gradient_matches_out_of_place(T, V, dt, eps):
    """grad == logits: the gradient overwrites the logits (same pointer,
    stride and dtype).  Every element of the in-place result is checked
    against the fp64 oracle on the original logits (kept on the host before
    the call), and it also equals the out-of-place result bit for bit."""
    c, logits, target = _case(S.PAGE, T, V, 151 + T, eps=eps, dtype=dt)
    _say(f"[in place] T={T} V={V} {dt} eps={eps}")
    ref = vce.fused_fwd_bwd(logits, target, label_smoothing=eps)
    oracle = P.oracle_for(logits, target, eps=eps)
    buf = logits.clone()
    out = vce.fused_fwd_bwd(buf, target, label_smoothing=eps, grad=buf)
    torch.cuda.synchronize()
    assert out["grad"].data_ptr() == buf.data_ptr()
    # against the oracle: losses, counts and every gradient element
    assert int(out["n_valid"].item()) == oracle["n_valid"]
    P.assert_loss_rows(out["loss_rows"], oracle, f"in place T={T} V={V}")
    P.assert_scalar_loss(out["loss"].item(), oracle["loss"], f"in place T={T} V={V}")
    P.assert_grad_close(buf, oracle["grad"], f"in place T={T} V={V} grad")
    # and the same bits as the out-of-place call
    assert torch.equal(out["loss_rows"], ref["loss_rows"])
    assert torch.equal(out["loss"], ref["loss"])
    assert torch.equal(buf.view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                       ref["grad"].view(torch.int16 if dt == torch.bfloat16 else torch.int32))


def test_in_place_backward_on_shards():
    """Per-shard backward written over each shard's own logits."""
    c, logits, target = _case(S.PAGE, 200, 128256, 163, eps=0.1)
    V, cut = 128256, 64128
    stats = [vce.forward(logits[:, a:b], target, vocab_start=a, V_total=V,
                         label_smoothing=0.1)["stats"] for a, b in ((0, cut), (cut, V))]
    m = vce.merge_shard_stats(stats, target, V, label_smoothing=0.1)
    ref = [vce.backward(logits[:, a:b], target, m["fin"], m["n_valid"], vocab_start=a,
                        V_total=V, label_smoothing=0.1) for a, b in ((0, cut), (cut, V))]
    buf = logits.clone()
    for a, b in ((0, cut), (cut, V)):
        view = buf[:, a:b]
        vce.backward(view, target, m["fin"], m["n_valid"], vocab_start=a, V_total=V,
                     label_smoothing=0.1, grad=view)
    torch.cuda.synchronize()
    assert torch.equal(buf[:, :cut].view(torch.int16), ref[0].view(torch.int16))
    assert torch.equal(buf[:, cut:].view(torch.int16), ref[1].view(torch.int16))


# --------------------------------------------------------------------------
# HIP graph capture: a captured call replays like an eager one
# --------------------------------------------------------------------------

@pytest.mark.parametrize("V,eps", [(128256, 0.0), (24000, 0.1), (150001, 0.1)])
def test_graph_replay_matches_eager(V, eps):
    """The library allocates nothing, never synchronises and launches only
    on the caller's stream, so a call can be captured into a HIP graph.
    Each replay (with new logits copied into the captured input between
    replays, eagerly) must equal an eager call on the same bytes, bit for
    bit: the fused register + LDS kernel, the smoothed table kernel, and the
    streaming path (column-chunk statistics, merge, gradient)."""
    T = 300
    cases = [_case(S.PAGE, T, V, 700 + k, eps=eps) for k in range(3)]
    x = cases[0][1].clone()
    tg = cases[0][2].clone()
    # warm-up outside the capture (per-device launch caches, LDS limits)
    vce.fused_fwd_bwd(x, tg, label_smoothing=eps)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            out = vce.fused_fwd_bwd(x, tg, label_smoothing=eps)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for k, (c, logits, target) in enumerate(cases):
        x.copy_(logits)
        tg.copy_(target)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = vce.fused_fwd_bwd(logits, target, label_smoothing=eps)
        torch.cuda.synchronize()
        _say(f"[graph] V={V} eps={eps} replay {k}: loss {out['loss'].item():.6f}")
        assert torch.equal(out["loss"], ref["loss"]), f"replay {k}: loss"
        assert torch.equal(out["loss_rows"], ref["loss_rows"]), f"replay {k}: loss rows"
        assert torch.equal(out["n_valid"], ref["n_valid"]), f"replay {k}: n_valid"
        assert torch.equal(out["grad"].view(torch.int16), ref["grad"].view(torch.int16)), \
            f"replay {k}: gradient"


# --------------------------------------------------------------------------
# the autograd wrapper: forward and backward through the C ABI
# --------------------------------------------------------------------------

@pytest.mark.parametrize("reduction,eps", [("mean", 0.0), ("sum", 0.1), ("none", 0.0)])
def test_autograd_cross_entropy(reduction, eps):
    """vce.cross_entropy under torch autograd: the loss of ce_forward, and a
    gradient from ce_backward with the incoming gradient as grad_output
    (3 x the loss, or per-row weights for reduction none)."""
    c, logits, target = _case(S.PAGE, 400, 50257, 171, eps=eps)
    x = logits.clone().requires_grad_(True)
    loss = vce.cross_entropy(x, target, label_smoothing=eps, reduction=reduction)
    if reduction == "none":
        w = torch.linspace(-1.0, 2.0, c.T, device=DEV)
        (loss * w).sum().backward()
        go = w
    else:
        (3.0 * loss).backward()
        go = 3.0
    torch.cuda.synchronize()
    ref = P.oracle_for(logits, target, eps=eps, reduction=reduction, grad_output=go)
    if reduction == "none":
        P.assert_loss_rows(loss.detach(), ref, f"autograd {reduction}")
    else:
        P.assert_scalar_loss(loss.item(), ref["loss"], f"autograd {reduction}")
    assert x.grad.dtype == logits.dtype
    P.assert_grad_close(x.grad, ref["grad"], f"autograd {reduction} grad")


def test_timed_call_events_bracket_the_kernel():
    """ce_fused_fwd_bwd_timed (measurement only): the events it records
    around the fused call's main kernel time it (a positive duration below
    the whole call's), and its results are bit-identical to ce_fused_fwd_bwd."""
    c, logits, target = _case(S.PAGE, 600, 128256, 181)
    ref = vce.fused_fwd_bwd(logits, target)
    T, V = logits.shape
    prob = vce.make_problem(T, V, ignore_index=c.ignore_index, reduction="mean")
    nws = vce.ce_workspace_bytes(prob, vce.CE_OP_FUSED)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=DEV)
    loss = torch.empty(1, dtype=torch.float32, device=DEV)
    rows = torch.empty(T, dtype=torch.float32, device=DEV)
    nv = torch.empty(1, dtype=torch.int32, device=DEV)
    err = torch.empty(1, dtype=torch.int32, device=DEV)
    grad = torch.empty_like(logits)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    b.record()
    torch.cuda.synchronize()
    w0.record()
    vce.ce_fused_fwd_bwd_timed(prob, logits, vce.CE_BF16, target, None, rows, loss, nv, err,
                               grad, vce.CE_BF16, V, ws, nws, None, a.cuda_event, b.cuda_event)
    w1.record()
    torch.cuda.synchronize()
    k, whole = a.elapsed_time(b), w0.elapsed_time(w1)
    _say(f"[events] fused kernel {k * 1e3:.1f} us of a {whole * 1e3:.1f} us call")
    assert 0.0 < k < whole
    assert torch.equal(loss, ref["loss"])
    assert torch.equal(rows, ref["loss_rows"])
    assert torch.equal(grad.view(torch.int16), ref["grad"].view(torch.int16))


@pytest.mark.parametrize("V,eps,out_dt", [(70001, 0.1, torch.float32), (70001, 0.0, torch.bfloat16),
                                          (100000, 0.2, torch.float32)])
def test_fp32_rows_too_long_for_registers(V, eps, out_dt):
    """fp32 logits longer than the register-resident kernels hold (65536
    columns) stream: column-chunk statistics (fp64 online sums with
    smoothing), the on-device merge, the gradient pass; odd widths peel
    each row's head."""
    c, logits, target = _case(S.TINY, 300, V, 191 + V % 7, eps=eps)
    target[0] = V - 1
    _fused_check(c, logits, target, grad_dtype=out_dt, what=f"fp32 long rows V={V} eps={eps}")


def test_fp32_shards_with_smoothing():
    """fp32 logits as three vocabulary shards of unequal width with
    smoothing: per-shard statistics, merge, per-shard backward."""
    c, logits, target = _case(S.TINY, 500, 30000, 197, eps=0.1)
    V = c.V
    edges = [0, 7001, 20000, V]
    stats = [vce.forward(logits[:, a:b], target, vocab_start=a, V_total=V,
                         label_smoothing=0.1)["stats"] for a, b in zip(edges[:-1], edges[1:])]
    m = vce.merge_shard_stats(stats, target, V, label_smoothing=0.1)
    grads = [vce.backward(logits[:, a:b], target, m["fin"], m["n_valid"], vocab_start=a,
                          V_total=V, label_smoothing=0.1) for a, b in zip(edges[:-1], edges[1:])]
    torch.cuda.synchronize()
    ref = P.oracle_for(logits, target, eps=0.1)
    P.assert_loss_rows(m["loss_rows"], ref, "fp32 shards")
    P.assert_scalar_loss(m["loss"].item(), ref["loss"], "fp32 shards")
    for (a, b), g in zip(zip(edges[:-1], edges[1:]), grads):
        P.assert_grad_close(g, ref["grad"][:, a:b], f"fp32 shard [{a},{b})")


def test_ignore_index_inside_the_vocabulary_and_per_row_grad_output_on_shards():
    """ignore_index is a parameter and may be a class id (7 here): rows whose
    target is 7 are ignored on every path.  With reduction none, the shard
    backward scales row r by grad_output[r]."""
    c, logits, target = _case(S.PAGE, 640, 50000, 199, eps=0.1)
    target[target == -100] = 11  # -100 would be a bad target once 7 is the ignore index
    target[::9] = 7
    t = target.cpu().numpy()
    go = torch.linspace(-1.5, 2.5, c.T, device=DEV)
    # fused, mean
    out = vce.fused_fwd_bwd(logits, target, ignore_index=7, label_smoothing=0.1)
    torch.cuda.synchronize()
    ref = P.oracle_for(logits, target, ignore_index=7, eps=0.1)
    assert int(out["n_valid"].item()) == ref["n_valid"] == int((t != 7).sum())
    P.assert_loss_rows(out["loss_rows"], ref, "ignore 7 fused")
    P.assert_grad_close(out["grad"], ref["grad"], "ignore 7 fused grad")
    assert torch.all(out["grad"].cpu()[torch.from_numpy(t == 7)] == 0)
    # two shards, reduction none with a per-row grad_output
    V, h = c.V, 23456
    stats = [vce.forward(logits[:, a:b], target, vocab_start=a, V_total=V, ignore_index=7,
                         label_smoothing=0.1, reduction="none")["stats"]
             for a, b in ((0, h), (h, V))]
    m = vce.merge_shard_stats(stats, target, V, ignore_index=7, label_smoothing=0.1,
                              reduction="none")
    grads = [vce.backward(logits[:, a:b], target, m["fin"], m["n_valid"], grad_output=go,
                          vocab_start=a, V_total=V, ignore_index=7, label_smoothing=0.1,
                          reduction="none") for a, b in ((0, h), (h, V))]
    torch.cuda.synchronize()
    ref = P.oracle_for(logits, target, ignore_index=7, eps=0.1, reduction="none",
                       grad_output=go)
    P.assert_loss_rows(m["loss_rows"], ref, "ignore 7 shards")
    P.assert_grad_close(grads[0], ref["grad"][:, :h], "ignore 7 shard 0")
    P.assert_grad_close(grads[1], ref["grad"][:, h:], "ignore 7 shard 1")


@pytest.mark.parametrize("V,dt,eps", [(128256, "bf16", 0.0), (128256, "bf16", 0.1),
                                      (1000, "f32", 0.0), (2, "bf16", 0.1), (40001, "f32", 0.1)])
def test_single_row(V, dt, eps):
    """One row (T = 1): the split-V grid for long rows, the resident kernel
    for short ones, and the smallest vocabulary with a real softmax."""
    base = S.PAGE if dt == "bf16" else S.TINY
    c, logits, target = _case(base, 1, V, 211 + V % 5, eps=eps)
    if int(target[0]) == -100:
        target[0] = V - 1
    _fused_check(c, logits, target, what=f"T=1 V={V} {dt} eps={eps}")
    f = vce.forward(logits, target, label_smoothing=eps)
    g = vce.backward(logits, target, f["fin"], f["n_valid"], label_smoothing=eps)
    torch.cuda.synchronize()
    ref = P.oracle_for(logits, target, eps=eps)
    P.assert_loss_rows(f["loss_rows"], ref, "T=1 unfused")
    P.assert_grad_close(g, ref["grad"], "T=1 unfused grad")


# --------------------------------------------------------------------------
# small batches: row tails inside aligned rows, the most rows of a short
# width, per-row weights, a single row
# --------------------------------------------------------------------------

@pytest.mark.parametrize("in_dt,out_dt,T,V,ld,reduction", [
    (torch.float32, torch.float32, 64, 1000, 1000, "mean"),    # the tiny workload's shape
    (torch.bfloat16, torch.bfloat16, 300, 1003, 1008, "mean"),  # a 3-logit tail per row
    (torch.bfloat16, torch.float32, 1024, 120, 120, "sum"),
    (torch.float32, torch.bfloat16, 33, 2048, 2048, "none"),    # 8 vectors per lane
    (torch.bfloat16, torch.bfloat16, 1, 64, 64, "mean"),
    (torch.bfloat16, torch.bfloat16, 1025, 120, 120, "mean"),
])
def test_small_batch_single_launch(in_dt, out_dt, T, V, ld, reduction):
    """Small batches with the gradient rows at the logits' stride (so a
    short tail sits inside 16-byte aligned rows): every output against the
    oracle, including ignored rows, a confident row and per-row weights."""
    base = S.TINY if in_dt == torch.float32 else S.MID
    c = S.scaled(base, T, ld, 930 + T, dtype=in_dt, reduction=reduction)
    full, target = S.generate(c)
    logits = full.to(DEV)[:, :V]
    target = target.clamp(max=V - 1)
    target[target < 0] = -100
    target = target.to(DEV)
    if T > 2:
        target[1] = -100
        logits[2, int(target[2]) if int(target[2]) >= 0 else 0] = 30.0   # a confident row
    go = None
    if reduction == "none":
        go = torch.linspace(-1.0, 2.0, T, device=DEV)
    elif reduction == "sum":
        go = torch.tensor([0.5], device=DEV)
    what = f"small {in_dt}->{out_dt} {T}x{V}"
    _say(f"[small] {what} ld={ld} {reduction}")
    # the gradient rows share the logits' stride, so both stay 16-byte aligned
    grad = torch.empty((T, ld), dtype=out_dt, device=DEV)[:, :V]
    out = vce.fused_fwd_bwd(logits, target, reduction=reduction, grad_output=go, grad=grad)
    torch.cuda.synchronize()
    ref = P.oracle_for(logits, target, reduction=reduction,
                       grad_output=1.0 if go is None else go)
    assert int(out["n_valid"].item()) == ref["n_valid"]
    assert int(out["err_count"].item()) == ref["n_bad"]
    P.assert_loss_rows(out["loss_rows"], ref, what)
    if reduction != "none":
        P.assert_scalar_loss(out["loss"].item(), ref["loss"], what)
    P.assert_grad_close(out["grad"], ref["grad"], what)
    P.assert_collapse_rows(out["loss_rows"], out["grad"].cpu(), target.cpu(), ref,
                           P.collapse_rows(logits, target), what)


def test_small_batch_edge_rows():
    """Small batches: bad targets, an all-ignored batch (mean NaN), -inf
    logits and an in-place gradient."""
    logits = torch.randn((8, 512), device=DEV)
    target = torch.tensor([0, 1, 512, -1, -100, 7, 10**12, 3], dtype=torch.int64, device=DEV)
    out = vce.fused_fwd_bwd(logits, target, reduction="sum")
    torch.cuda.synchronize()
    assert out["err_count"].item() == 3 and out["n_valid"].item() == 4
    lr = out["loss_rows"].cpu()
    assert torch.isnan(lr[[2, 3, 6]]).all() and lr[4].item() == 0.0
    assert torch.all(out["grad"][[2, 3, 4, 6]] == 0) and math.isnan(out["loss"].item())
    allign = torch.full((8,), -100, dtype=torch.int64, device=DEV)
    out = vce.fused_fwd_bwd(logits.to(torch.bfloat16), allign)
    torch.cuda.synchronize()
    assert math.isnan(out["loss"].item()) and int(out["n_valid"].item()) == 0
    assert torch.all(out["grad"] == 0)
    z = torch.randn((40, 704), device=DEV) * 2
    t = torch.randint(0, 704, (40,), device=DEV)
    z[0, :300] = -math.inf
    z[0, int(t[0])] = 1.0
    z[1, :] = -math.inf
    z[1, int(t[1])] = 1.0
    out = vce.fused_fwd_bwd(z, t, reduction="none")
    torch.cuda.synchronize()
    ref = P.oracle_for(z, t, reduction="none")
    P.assert_loss_rows(out["loss_rows"], ref, "small -inf")
    P.assert_grad_close(out["grad"], ref["grad"], "small -inf grad")
    buf = z.clone()
    ip = vce.fused_fwd_bwd(buf, t, reduction="none", grad=buf)
    torch.cuda.synchronize()
    assert torch.equal(buf, out["grad"]) and torch.equal(ip["loss_rows"], out["loss_rows"])
