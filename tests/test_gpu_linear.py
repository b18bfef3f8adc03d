"""GPU parity of the linear-classifier cross-entropy (ce_linear_fwd_bwd)
against the fp64 oracle, through the C ABI.

Loss: every valid row within 1e-5 relative (ignored rows exactly +0, bad
targets NaN), the reduced loss within 1e-5.  dE and dC: the bound of
``parity_util.assert_linear_grad_close`` (G is a bf16 operand of the
backward products).  Shapes cover padding in every dimension (tokens not a
multiple of 256, hidden size not a multiple of 64, classes not a multiple
of 256), several vocabulary chunks with a ragged last one, both dE
accumulation modes, label smoothing, every reduction, the toy shape of
apple/ml-cross-entropy issue #14, every element of dE and dC at the
workload's 8192 tokens and hidden size 2048 (1000 classes), and the full
8192 x 2048 x 128256 workload (sampled rows of dE, a zero-sum property of
dC; full gradients at 16 rows of the full width).
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import vocab_softmax_cross_row_amd as vce
from vocab_softmax_cross_row_amd import _binding as B
from synth import ce_inputs as S
from tests.parity_util import (LOSS_RTOL, assert_linear_grad_close, assert_loss_rows,
                               assert_scalar_loss, linear_oracle_for)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _case(N, D, V, seed, n_ignored=None, **kw):
    base = S.LINEAR
    if n_ignored is None:
        n_ignored = max(1, round(N * base.n_ignored / base.N))
    return dataclasses.replace(base, name=f"lin_{N}x{D}x{V}", N=N, D=D, V=V, seed=seed,
                               n_ignored=n_ignored, **kw)


def _run(case, *, accum="fp32", grad_output=None, backward=True):
    print(f"[linear] {case.name} eps={case.eps} red={case.reduction} accum={accum}", flush=True)
    E, C, t = S.generate_linear(case, device=DEV)
    go = grad_output
    out = vce.linear_cross_entropy(E, C, t, ignore_index=case.ignore_index,
                                   label_smoothing=case.eps, reduction=case.reduction,
                                   grad_output=go, backward=backward, accum=accum)
    torch.cuda.synchronize()
    return E, C, t, out


def _check(case, E, C, t, out, grad_output=1.0, what=""):
    ref = linear_oracle_for(E, C, t, ignore_index=case.ignore_index, eps=case.eps,
                            reduction=case.reduction, grad_output=grad_output)
    assert_loss_rows(out["loss_rows"], {"loss_rows": ref["loss_rows"], "status": ref["status"]},
                     what)
    if case.reduction != "none":
        assert_scalar_loss(out["loss"].item(), ref["loss"], what)
    assert int(out["n_valid"].item()) == ref["n_valid"]
    assert int(out["err_count"].item()) == ref["n_bad"]
    if out["dE"] is not None:
        assert_linear_grad_close(out["dE"], ref["dE"], ref["rsE"], what + " dE")
        assert_linear_grad_close(out["dC"], ref["dC"], ref["rsC"], what + " dC")
    return ref


def test_ragged_in_every_dimension():
    case = _case(300, 72, 1000, 2101)
    E, C, t, out = _run(case)
    _check(case, E, C, t, out, what="300x72x1000")


@pytest.mark.parametrize("accum", ["fp32", "kahan"])
def test_several_chunks_with_smoothing(accum):
    # 2 vocabulary chunks, the second ragged; sum with a grad_output of 0.5
    case = _case(512, 256, B.CE_LINEAR_CHUNK + 300, 2102, eps=0.1, reduction="sum")
    go = torch.tensor([0.5], device=DEV)
    E, C, t, out = _run(case, accum=accum, grad_output=go)
    _check(case, E, C, t, out, grad_output=go, what=f"chunks {accum}")


@pytest.mark.parametrize("accum", ["fp32", "kahan"])
def test_mean_with_smoothing_over_two_chunks(accum):
    # mean over the non-ignored rows with smoothing; the vocabulary spans one
    # full backward chunk and a ragged second one
    case = _case(300, 128, B.CE_LINEAR_CHUNK + 3616, 2105, eps=0.1)
    E, C, t, out = _run(case, accum=accum)
    _check(case, E, C, t, out, what=f"mean smoothing {accum}")


def test_reduction_none_per_row_grad_output():
    case = _case(260, 64, 700, 2103, reduction="none")
    go = torch.linspace(0.25, 2.0, 260, device=DEV)
    E, C, t, out = _run(case, grad_output=go)
    _check(case, E, C, t, out, grad_output=go, what="none")


def test_cce_issue_toy_shape():
    # apple/ml-cross-entropy issue #14: 8191 shifted rows, hidden 128, 32 classes
    case = dataclasses.replace(S.CCE_TOY)
    E, C, t, out = _run(case)
    _check(case, E, C, t, out, what="cce toy")


def test_kahan_and_fp32_agree_closely():
    case = _case(256, 128, 3 * B.CE_LINEAR_CHUNK, 2104)
    E, C, t, a = _run(case, accum="fp32")
    b = vce.linear_cross_entropy(E, C, t, accum="kahan")
    torch.cuda.synchronize()
    assert torch.equal(a["dC"], b["dC"])          # dC rows are complete in one chunk
    assert torch.equal(a["loss_rows"], b["loss_rows"])
    d = (a["dE"] - b["dE"]).abs().max().item()
    assert d <= 1e-6 * b["dE"].abs().max().item()


def test_loss_only_matches_backward_call():
    case = _case(300, 72, 1000, 2105)
    E, C, t, out = _run(case, backward=False)
    assert out["dE"] is None and out["dC"] is None
    _, _, _, full = _run(case)
    assert torch.equal(out["loss_rows"], full["loss_rows"])
    assert torch.equal(out["loss"], full["loss"])


def test_bad_targets_and_all_ignored():
    case = _case(200, 64, 500, 2106)
    E, C, t = S.generate_linear(case, device=DEV)
    t = t.clone()
    t[3] = 500          # out of range
    t[7] = -5
    out = vce.linear_cross_entropy(E, C, t)
    torch.cuda.synchronize()
    ref = _check(case, E, C, t, out, what="bad targets")
    assert ref["n_bad"] == 2 and int(out["err_count"].item()) == 2
    assert math.isnan(out["loss"].item())
    t_all = torch.full_like(t, -100)
    out = vce.linear_cross_entropy(E, C, t_all)
    torch.cuda.synchronize()
    assert math.isnan(out["loss"].item()) and int(out["n_valid"].item()) == 0
    assert torch.all(out["dE"] == 0) and torch.all(out["dC"] == 0)


def test_deterministic():
    case = _case(300, 136, 2000, 2107)
    E, C, t, a = _run(case)
    b = vce.linear_cross_entropy(E, C, t)
    torch.cuda.synchronize()
    for k in ("loss_rows", "dE", "dC"):
        assert torch.equal(a[k], b[k]), k


def test_full_width_sixteen_rows():
    # the full hidden size and vocabulary, in the launch configuration of the
    # full workload, at 16 rows: full dE and dC parity
    case = dataclasses.replace(S.LINEAR, name="linear_16rows", N=16, n_ignored=1)
    E, C, t, out = _run(case)
    _check(case, E, C, t, out, what="16 x 2048 x 128256")


@pytest.fixture(scope="module")
def long_tokens():
    """The linear workload's token count and hidden size (8192 x 2048) with
    1000 classes (three full 256-class tiles and a ragged one, one
    vocabulary chunk), and its oracle: small enough for the fp64 oracle to
    give every element of dE and dC in seconds."""
    case = _case(8192, 2048, 1000, 2110)
    E, C, t = S.generate_linear(case, device=DEV)
    print(f"[linear] oracle for {case.name}", flush=True)
    ref = linear_oracle_for(E, C, t, ignore_index=case.ignore_index)
    return case, E, C, t, ref


@pytest.mark.parametrize("accum", ["fp32", "kahan"])
def test_long_token_accumulation_every_element(long_tokens, accum):
    """dC summed over 8192 tokens at hidden size 2048, the accumulation the
    apple/ml-cross-entropy issue #14 report finds broken in low precision:
    every element of dC and dE against the oracle, in both dE modes."""
    case, E, C, t, ref = long_tokens
    print(f"[linear] {case.name} accum={accum}", flush=True)
    out = vce.linear_cross_entropy(E, C, t, ignore_index=case.ignore_index, accum=accum)
    torch.cuda.synchronize()
    assert_loss_rows(out["loss_rows"], {"loss_rows": ref["loss_rows"], "status": ref["status"]},
                     f"long tokens {accum}")
    assert_scalar_loss(out["loss"].item(), ref["loss"], f"long tokens {accum}")
    assert int(out["n_valid"].item()) == ref["n_valid"]
    assert_linear_grad_close(out["dE"], ref["dE"], ref["rsE"], f"long tokens {accum} dE")
    assert_linear_grad_close(out["dC"], ref["dC"], ref["rsC"], f"long tokens {accum} dC")


def test_full_workload_sampled_rows():
    case = S.LINEAR
    E, C, t, out = _run(case)
    n_valid = int((t != case.ignore_index).sum().item())
    assert int(out["n_valid"].item()) == n_valid
    g = torch.Generator().manual_seed(7)
    rows = torch.randperm(case.N, generator=g)[:8].tolist()
    rows[0] = int(torch.nonzero(t.cpu() == case.ignore_index)[0, 0])  # one ignored row
    ref = linear_oracle_for(E[rows], C, t[rows], n_valid=n_valid, dC=False)
    sel = torch.tensor(rows)
    assert_loss_rows(out["loss_rows"].cpu()[sel], {"loss_rows": ref["loss_rows"],
                                                   "status": ref["status"]}, "sampled")
    assert_linear_grad_close(out["dE"].cpu()[sel], ref["dE"], ref["rsE"], "sampled dE")
    # the mean over all rows agrees with the per-row losses it is made of
    lr = out["loss_rows"].double()
    assert abs(out["loss"].item() - lr.sum().item() / n_valid) <= LOSS_RTOL * abs(out["loss"].item())
    assert torch.isfinite(out["dC"]).all()
    # every class row of dC is a sum over the valid tokens of G E: with logits
    # of spread about 0.9 every class has gradient mass, so no row is zero
    assert (out["dC"].abs().sum(dim=1) > 0).all()
    # A property of dC at any size: each row of G sums to zero (softmax minus
    # a distribution that sums to one), so sum_v dC[v, d] = sum_r E[r, d]
    # sum_v G[r, v] vanishes up to the bf16 rounding of G, which leaves at
    # most 2^-9 sum_v |G[r, v]| <= 2^-8 |k_r| per row: the column sums are
    # bounded by 2^-8 sum_r |k_r| |E[r, d]| (plus fp32 accumulation, far
    # below).  A dropped or doubled term in any row breaks this.
    k = 1.0 / n_valid
    valid = (t != case.ignore_index).to(torch.float64)
    bound = 2.0 ** -8 * k * (valid[:, None] * E.double().abs()).sum(dim=0)
    col = out["dC"].double().sum(dim=0)
    assert torch.all(col.abs() <= bound + 1e-12), \
        f"dC column sums {col.abs().max().item():.3e} beyond {bound.min().item():.3e}"


# --------------------------------------------------------------------------
# gradient filtering (filter_eps > 0)
# --------------------------------------------------------------------------
TAU = 2.0 ** -8


def _targets_in(t, ranges, seed):
    """Redraw the non-ignored targets uniformly from the union of `ranges`,
    leaving class tiles outside them without targets (their blocks then
    hold only softmax values far below TAU)."""
    g = torch.Generator().manual_seed(seed)
    pool = torch.cat([torch.arange(a, b) for a, b in ranges])
    t = t.clone().cpu()
    keep = t != -100
    t[keep] = pool[torch.randint(0, len(pool), (int(keep.sum()),), generator=g)]
    return t.to(DEV)


@pytest.mark.parametrize("accum", ["fp32", "kahan"])
def test_filtering_that_keeps_every_block_is_exact(accum):
    """A threshold below every entry keeps every block: the filtered K walk
    (lists of kept tiles) must then reproduce the unfiltered products bit
    for bit: 3 token tiles (the last ragged), 2 vocabulary chunks."""
    case = _case(600, 256, B.CE_LINEAR_CHUNK + 700, 2120)
    E, C, t = S.generate_linear(case, device=DEV)
    a = vce.linear_cross_entropy(E, C, t, accum=accum)
    b = vce.linear_cross_entropy(E, C, t, accum=accum, filter_eps=1e-30)
    torch.cuda.synchronize()
    for k in ("loss", "loss_rows", "dE", "dC"):
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("eps,reduction,accum,go", [(0.0, "mean", "fp32", None),
                                                    (0.1, "sum", "kahan", 0.5)])
def test_filtering_against_oracle(eps, reduction, accum, go):
    """Filtering at 2^-8 on 556 tokens x 18384 classes (two chunks, ragged
    in tokens and classes), targets drawn from classes 0..1499 and
    16400..17099 only: the blocks of the other class tiles hold softmax
    values near 1/V and are dropped, the others are kept.  The oracle applies
    the same rule; every decision is first checked to sit far from the
    threshold, then dE and dC are compared with the filtered oracle at the
    usual bound, and they must differ from the unfiltered result."""
    case = _case(556, 256, B.CE_LINEAR_CHUNK + 2000, 2121, eps=eps, reduction=reduction)
    E, C, t = S.generate_linear(case, device=DEV)
    t = _targets_in(t, [(0, 1500), (16400, 17100)], 2122)
    gout = None if go is None else torch.tensor([go], device=DEV)
    print(f"[linear filter] eps={eps} {reduction} {accum}", flush=True)
    out = vce.linear_cross_entropy(E, C, t, label_smoothing=eps, reduction=reduction,
                                   grad_output=gout, accum=accum, filter_eps=TAU)
    exact = vce.linear_cross_entropy(E, C, t, label_smoothing=eps, reduction=reduction,
                                     grad_output=gout, accum=accum)
    torch.cuda.synchronize()
    ref = linear_oracle_for(E, C, t, eps=eps, reduction=reduction,
                            grad_output=1.0 if go is None else go)
    Eb = E.cpu().view(torch.int16).numpy().view(np.uint16)
    Cb = C.cpu().view(torch.int16).numpy().view(np.uint16)
    from oracle import ce_oracle as O
    fref = O.linear_fwd_bwd(Eb, Cb, t.cpu().numpy(), eps=float(np.float32(eps)),
                            reduction=reduction, grad_output=1.0 if go is None else go,
                            filter_eps=TAU)
    bm = fref["block_max"]
    assert np.all((bm < TAU / 2) | (bm > 2 * TAU)), "a block decision too close to the threshold"
    assert fref["keep"].any() and not fref["keep"].all()
    assert_loss_rows(out["loss_rows"], {"loss_rows": ref["loss_rows"], "status": ref["status"]},
                     "filtered")
    assert torch.equal(out["loss_rows"], exact["loss_rows"])
    assert_linear_grad_close(out["dE"], fref["dE"], fref["rsE"], "filtered dE")
    assert_linear_grad_close(out["dC"], fref["dC"], fref["rsC"], "filtered dC")
    assert not torch.equal(out["dC"], exact["dC"])
    # rows of dC whose class tiles were dropped for every token tile are zero
    dropped_cols = np.nonzero(fref["keep"].max(axis=0) == 0)[0]
    assert len(dropped_cols) > 0
    for j in dropped_cols[:3]:
        assert torch.all(out["dC"][256 * j:256 * (j + 1)] == 0)


def test_filtering_full_workload_one_token_tile():
    """The full 8192 x 2048 x 128256 workload with filtering at 2^-8, in the
    launch configuration of the benchmark: every dE entry of one token tile
    (rows 2048 .. 2303; a block's decision depends only on its own 256
    rows) against the oracle applying the same rule to those rows, with the
    batch's N_valid for the mean."""
    case = S.LINEAR
    E, C, t = S.generate_linear(case, device=DEV)
    out = vce.linear_cross_entropy(E, C, t, filter_eps=TAU)
    torch.cuda.synchronize()
    n_valid = int((t != case.ignore_index).sum().item())
    rows = slice(2048, 2304)
    Eb = E[rows].cpu().view(torch.int16).numpy().view(np.uint16)
    Cb = C.cpu().view(torch.int16).numpy().view(np.uint16)
    from oracle import ce_oracle as O
    print("[linear filter] oracle for one token tile at full width", flush=True)
    fref = O.linear_fwd_bwd(Eb, Cb, t[rows].cpu().numpy(), n_valid=n_valid, dC=False,
                            filter_eps=TAU)
    bm = fref["block_max"]
    assert np.all((bm < TAU / 2) | (bm > 2 * TAU)), "a block decision too close to the threshold"
    print(f"[linear filter] {int(fref['keep'].sum())} of {fref['keep'].size} blocks kept",
          flush=True)
    assert_loss_rows(out["loss_rows"][rows], {"loss_rows": fref["loss_rows"],
                                              "status": fref["status"]}, "filtered full")
    assert_linear_grad_close(out["dE"][rows], fref["dE"], fref["rsE"], "filtered full dE")


def test_filtering_with_per_row_grad_output():
    """reduction none with per-row weights (some zero, some negative): a
    row's threshold scales with |k_r|, so the decisions are those of the
    unscaled gradient; dE and dC against the filtered oracle."""
    case = _case(300, 128, B.CE_LINEAR_CHUNK + 500, 2123, reduction="none")
    E, C, t = S.generate_linear(case, device=DEV)
    t = _targets_in(t, [(0, 700), (16500, 16884)], 2124)
    go = torch.linspace(-1.5, 2.0, 300, device=DEV)
    go[::7] = 0.0
    out = vce.linear_cross_entropy(E, C, t, reduction="none", grad_output=go, filter_eps=TAU)
    torch.cuda.synchronize()
    Eb = E.cpu().view(torch.int16).numpy().view(np.uint16)
    Cb = C.cpu().view(torch.int16).numpy().view(np.uint16)
    from oracle import ce_oracle as O
    fref = O.linear_fwd_bwd(Eb, Cb, t.cpu().numpy(), reduction="none",
                            grad_output=go.cpu().double().numpy(), filter_eps=TAU)
    bm = fref["block_max"]
    assert np.all((bm < TAU / 2) | (bm > 2 * TAU)), "a block decision too close to the threshold"
    assert fref["keep"].any() and not fref["keep"].all()
    assert_loss_rows(out["loss_rows"], {"loss_rows": fref["loss_rows"], "status": fref["status"]},
                     "filtered none")
    assert_linear_grad_close(out["dE"], fref["dE"], fref["rsE"], "filtered none dE")
    assert_linear_grad_close(out["dC"], fref["dC"], fref["rsC"], "filtered none dC")
