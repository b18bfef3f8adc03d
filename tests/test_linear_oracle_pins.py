"""Pins of the oracle's linear-classifier cross-entropy (logits z = E C^T,
apple/ml-cross-entropy issue #14, linear_cross_entropy) to facts outside
itself, no GPU needed: a closed form at C = 0, central finite differences in
fp64, torch's float64 autograd through matmul + cross_entropy on the CPU,
numpy's matmul for the two contractions, and the zero column sums of dC.
A transposed operand, a dropped scale, a wrong smoothing weight or a G row
that does not sum to zero fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch

from oracle import ce_oracle as O


def _case(n=6, D=5, V=9, seed=0, scale=0.7):
    rng = np.random.default_rng(seed)
    E = rng.standard_normal((n, D))
    C = rng.standard_normal((V, D)) * scale
    t = rng.integers(0, V, n)
    t[1] = -100
    return E, C, t


@pytest.mark.parametrize("eps", [0.0, 0.1])
def test_zero_classifier_closed_form(eps):
    """C = 0: every row is uniform, so loss_r = log V, dE = 0 and
    dC[v] = sum_r k (1 - eps) (1/V - [t_r = v]) E_r."""
    E, _, t = _case()
    V = 9
    C = np.zeros((V, E.shape[1]))
    o = O.linear_fwd_bwd(E, C, t, eps=eps, reduction="sum")
    valid = t != -100
    assert np.allclose(o["loss_rows"][valid], math.log(V), rtol=1e-14, atol=0)
    assert np.all(o["loss_rows"][~valid] == 0.0)
    assert np.all(o["dE"] == 0.0)
    want = np.zeros((V, E.shape[1]))
    for r in np.nonzero(valid)[0]:
        for v in range(V):
            want[v] += (1.0 - eps) * ((1.0 / V) - (1.0 if v == t[r] else 0.0)) * E[r]
    assert np.allclose(o["dC"], want, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("reduction", ["sum", "mean", "none"])
@pytest.mark.parametrize("eps", [0.0, 0.2])
def test_matches_torch_float64_autograd(reduction, eps):
    """Loss and both gradients against torch's float64 matmul + cross_entropy
    and its autograd (CPU), with a grad_output that is not 1."""
    E, C, t = _case(n=7, D=6, V=11, seed=3)
    go = 0.75 if reduction != "none" else np.linspace(0.5, 1.5, 7)
    o = O.linear_fwd_bwd(E, C, t, eps=eps, reduction=reduction, grad_output=go)
    Et = torch.tensor(E, requires_grad=True)
    Ct = torch.tensor(C, requires_grad=True)
    loss = torch.nn.functional.cross_entropy(Et @ Ct.T, torch.tensor(t), ignore_index=-100,
                                             label_smoothing=eps, reduction=reduction)
    loss.backward(torch.tensor(go, dtype=torch.float64))
    if reduction == "none":
        assert np.allclose(o["loss_rows"], loss.detach().numpy(), rtol=1e-13, atol=1e-15)
    else:
        assert abs(o["loss"] - loss.item()) <= 1e-13 * abs(loss.item())
    assert np.allclose(o["dE"], Et.grad.numpy(), rtol=1e-11, atol=1e-14)
    assert np.allclose(o["dC"], Ct.grad.numpy(), rtol=1e-11, atol=1e-14)


@pytest.mark.parametrize("eps", [0.0, 0.1])
def test_central_finite_differences(eps):
    """d(sum of losses)/dE and /dC against central differences in fp64."""
    E, C, t = _case(n=4, D=3, V=5, seed=5)
    o = O.linear_fwd_bwd(E, C, t, eps=eps, reduction="sum")
    h = 1e-6

    def total(E_, C_):
        return O.linear_fwd_bwd(E_, C_, t, eps=eps, reduction="sum", grads=False)["loss"]

    for (r, d) in [(0, 0), (2, 1), (3, 2)]:
        Ep, Em = E.copy(), E.copy()
        Ep[r, d] += h
        Em[r, d] -= h
        fd = (total(Ep, C) - total(Em, C)) / (2 * h)
        assert abs(fd - o["dE"][r, d]) <= 1e-7 * max(1.0, abs(fd))
    for (v, d) in [(0, 0), (int(t[0]), 2), (4, 1)]:
        Cp, Cm = C.copy(), C.copy()
        Cp[v, d] += h
        Cm[v, d] -= h
        fd = (total(E, Cp) - total(E, Cm)) / (2 * h)
        assert abs(fd - o["dC"][v, d]) <= 1e-7 * max(1.0, abs(fd))


def test_agrees_with_stored_logits_oracle():
    """The logits E C^T formed by numpy's matmul and rounded to fp32, fed to
    the stored-logits oracle, give the same per-row loss as the linear
    oracle up to the fp32 rounding of the logits."""
    E, C, t = _case(n=8, D=16, V=40, seed=7)
    o = O.linear_fwd_bwd(E, C, t, grads=False)
    z = (E @ C.T).astype(np.float32)
    f = O.forward(z, t)
    v = f["status"] == 1
    assert np.array_equal(f["status"], o["status"])
    assert np.allclose(o["loss_rows"][v], f["loss"][v], rtol=1e-5)


def test_contractions_and_scales_match_numpy():
    """dE = G C, dC = G^T E, rsE = sqrt(G^2 C^2), rsC = sqrt((G^2)^T E^2)
    with numpy's matmul on the oracle's own G; dC's columns sum to zero."""
    E, C, t = _case(n=9, D=7, V=13, seed=11)
    o = O.linear_fwd_bwd(E, C, t, eps=0.1)
    G = o["G"]
    assert np.allclose(o["dE"], G @ C, rtol=1e-12, atol=1e-15)
    assert np.allclose(o["dC"], G.T @ E, rtol=1e-12, atol=1e-15)
    assert np.allclose(o["rsE"], np.sqrt((G * G) @ (C * C)), rtol=1e-12, atol=1e-15)
    assert np.allclose(o["rsC"], np.sqrt((G * G).T @ (E * E)), rtol=1e-12, atol=1e-15)
    colsum = o["dC"].sum(axis=0)
    assert np.all(np.abs(colsum) <= 1e-14 * np.abs(o["dC"]).sum(axis=0) + 1e-16)
    assert np.allclose(G.sum(axis=1), 0.0, atol=1e-15)


def test_bf16_inputs_are_decoded_exactly():
    """bf16 bit patterns give the same results as their exact fp64 values."""
    E, C, t = _case(n=5, D=8, V=10, seed=13)
    Eb, Cb = O.to_bf16(E), O.to_bf16(C)
    a = O.linear_fwd_bwd(Eb, Cb, t, eps=0.1)
    b = O.linear_fwd_bwd(O.bf16_to_f64(Eb), O.bf16_to_f64(Cb), t, eps=0.1)
    for key in ("loss_rows", "dE", "dC", "rsE"):
        assert np.array_equal(a[key], b[key])


def test_ignored_and_bad_rows():
    """Ignored rows: loss +0, G row +0, no contribution to dC; a target
    outside [0, V) is status -1 and NaN loss."""
    E, C, t = _case(n=6, D=4, V=7, seed=17)
    t = t.copy()
    t[3] = 7
    o = O.linear_fwd_bwd(E, C, t, reduction="sum")
    assert o["status"][1] == 0 and o["loss_rows"][1] == 0.0
    assert o["status"][3] == -1 and math.isnan(o["loss_rows"][3])
    assert np.all(o["G"][1] == 0.0) and np.all(o["G"][3] == 0.0)
    assert np.all(o["dE"][1] == 0.0) and np.all(o["dE"][3] == 0.0)
    keep = [r for r in range(6) if r not in (1, 3)]
    o2 = O.linear_fwd_bwd(E[keep], C, t[keep], reduction="sum")
    assert np.allclose(o["dC"], o2["dC"], rtol=1e-13, atol=1e-16)


def _filter_case(seed):
    """300 rows x 600 classes (2 x 3 blocks of 256, both ragged), D = 8, in
    fp64.  Rows 0..255 draw targets from classes 0..255 and rows 256..299
    from 512..599, so blocks (0, 0) and (1, 2) hold targets (|u| near 1) and
    the other four hold only softmax values of at most about 3.5e-3, more
    than 2 times below 2^-7: every decision has a wide margin."""
    rng = np.random.default_rng(seed)
    n, V, D = 300, 600, 8
    E = rng.standard_normal((n, D))
    C = rng.standard_normal((V, D)) * 0.05
    t = np.concatenate([rng.integers(0, 256, 256), rng.integers(512, 600, n - 256)])
    t[7] = -100
    return E, C, t


@pytest.mark.parametrize("eps,reduction,go", [(0.0, "mean", 1.0), (0.1, "sum", 0.5)])
def test_gradient_filtering_against_independent_blocks(eps, reduction, go):
    """Gradient filtering (the reading: drop 256 x 256 blocks of the unscaled
    gradient whose entries are all below tau) against the same rule applied
    by hand to torch's float64 autograd gradient of cross_entropy(E C^T):
    block maxima, keep mask, and dE, dC from the masked gradient by numpy."""
    tau = 2.0 ** -7
    E, C, t = _filter_case(5)
    o = O.linear_fwd_bwd(E, C, t, eps=eps, reduction=reduction, grad_output=go, filter_eps=tau)
    z = torch.tensor(E @ C.T, requires_grad=True)
    loss = torch.nn.functional.cross_entropy(z, torch.tensor(t), ignore_index=-100,
                                             label_smoothing=eps, reduction=reduction)
    loss.backward(torch.tensor(go, dtype=torch.float64))
    G = z.grad.numpy()
    k = go if reduction == "sum" else go / int((t != -100).sum())
    U = np.abs(G / k)
    n, V = G.shape
    bm = np.zeros((2, 3))
    for i in range(2):
        for j in range(3):
            bm[i, j] = U[256 * i:256 * (i + 1), 256 * j:256 * (j + 1)].max()
    assert np.allclose(o["block_max"], bm, rtol=1e-12, atol=1e-15)
    keep = bm >= tau
    assert keep.any() and (~keep).any()
    assert np.all((bm < tau / 2) | (bm > 2 * tau)), "a decision too close to the threshold"
    assert np.array_equal(o["keep"], keep.astype(np.int32))
    Gf = G.copy()
    for i in range(2):
        for j in range(3):
            if not keep[i, j]:
                Gf[256 * i:256 * (i + 1), 256 * j:256 * (j + 1)] = 0.0
    assert np.allclose(o["G"], Gf, rtol=1e-11, atol=1e-17)
    assert np.allclose(o["dE"], Gf @ C, rtol=1e-10, atol=1e-15)
    assert np.allclose(o["dC"], Gf.T @ E, rtol=1e-10, atol=1e-15)
    # and the filtered result really differs from the exact one
    ex = O.linear_fwd_bwd(E, C, t, eps=eps, reduction=reduction, grad_output=go)
    assert np.abs(ex["dC"] - o["dC"]).max() > 1e-6 * np.abs(ex["dC"]).max()


def test_gradient_filtering_limits():
    """tau = 0 is the exact path bit for bit; a tau above every entry drops
    every block (zero gradients), the loss untouched either way."""
    E, C, t = _filter_case(6)
    ex = O.linear_fwd_bwd(E, C, t)
    z0 = O.linear_fwd_bwd(E, C, t, filter_eps=0.0)
    for key in ("G", "dE", "dC", "loss_rows"):
        assert np.array_equal(ex[key], z0[key]), key
    assert np.all(z0["keep"] == 1)
    big = O.linear_fwd_bwd(E, C, t, filter_eps=2.0)
    assert np.all(big["keep"] == 0)
    assert np.all(big["dE"] == 0.0) and np.all(big["dC"] == 0.0)
    assert np.array_equal(big["loss_rows"], ex["loss_rows"])


def test_gradient_filtering_with_per_row_weights():
    """reduction none with per-row weights, some zero and some negative: the
    unscaled gradient of a row is its autograd gradient divided by its
    weight, and a row of weight zero (an all-zero gradient) keeps no block.
    Every row of block row 0 except those of weight zero has targets in class
    block 0 only, so with the zero-weight rows voting, block (0, 1) would be
    kept by the target of a zero-weight row placed there."""
    tau = 2.0 ** -7
    E, C, t = _filter_case(7)
    n = len(t)
    go = np.linspace(-1.5, 2.0, n)
    go[::5] = 0.0
    t[10] = 300                       # a zero-weight row (10 % 5 == 0) targets class block 1
    o = O.linear_fwd_bwd(E, C, t, reduction="none", grad_output=go, filter_eps=tau)
    z = torch.tensor(E @ C.T, requires_grad=True)
    loss = torch.nn.functional.cross_entropy(z, torch.tensor(t), ignore_index=-100,
                                             reduction="none")
    loss.backward(torch.tensor(go))
    G = z.grad.numpy()
    vote = (go != 0.0) & (t != -100)
    U = np.zeros_like(G)
    U[vote] = np.abs(G[vote] / go[vote, None])
    bm = np.zeros((2, 3))
    for i in range(2):
        for j in range(3):
            bm[i, j] = U[256 * i:256 * (i + 1), 256 * j:256 * (j + 1)].max()
    keep = bm >= tau
    assert not keep[0, 1], "the zero-weight row must not keep block (0, 1)"
    assert np.all((bm < tau / 2) | (bm > 2 * tau))
    assert np.allclose(o["block_max"], bm, rtol=1e-12, atol=1e-15)
    assert np.array_equal(o["keep"], keep.astype(np.int32))
    Gf = G.copy()
    for i in range(2):
        for j in range(3):
            if not keep[i, j]:
                Gf[256 * i:256 * (i + 1), 256 * j:256 * (j + 1)] = 0.0
    assert np.allclose(o["dE"], Gf @ C, rtol=1e-10, atol=1e-15)
    assert np.allclose(o["dC"], Gf.T @ E, rtol=1e-10, atol=1e-15)
