"""GPU parity at the measured workload's full size, in the launch
configuration the benchmark times: T = 16384 rows, V = 128256 bf16 logits
(fused), and the same bytes as two 64128-column shards with label smoothing
0.1 (forward per shard, on-device merge, backward per shard).

The oracle recomputes a sample of rows one by one (every kind of row:
ordinary, confident-target, ignored) and the whole-batch loss; properties
that hold at any size cover the rest (counts, zero rows, unchanged input).
"""
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


@pytest.fixture(scope="module")
def page():
    print("[full] generating T=16384 V=128256 bf16 on the GPU", flush=True)
    logits, target = S.generate(S.PAGE, device=DEV, block_rows=2048)
    torch.cuda.synchronize()
    return logits, target


def _sample_rows(target, logits):
    t = target.cpu().numpy()
    rng = np.random.default_rng(2024)
    ign = np.nonzero(t == -100)[0]
    valid = np.nonzero(t != -100)[0]
    # confident rows: the target logit far above the row's typical maximum
    zt = logits[torch.arange(logits.shape[0], device=DEV),
                torch.clamp(target, min=0)].float().cpu().numpy()
    conf = valid[zt[valid] > 22.0]
    rows = np.concatenate([valid[:8], rng.choice(conf, 16, replace=False),
                           rng.choice(ign, 6, replace=False),
                           rng.choice(valid, 12, replace=False), [t.shape[0] - 1]])
    return np.unique(rows)


def _checksum(x):
    return int(x.view(torch.int16).to(torch.int64).sum().item())


def test_fused_full_size(page):
    logits, target = page
    T, V = logits.shape
    ck = _checksum(logits)
    print("[full] fused fwd+bwd", flush=True)
    out = vce.fused_fwd_bwd(logits, target)
    torch.cuda.synchronize()
    assert _checksum(logits) == ck, "logits modified"
    t = target.cpu().numpy()
    n_valid = int((t != -100).sum())
    assert out["n_valid"].item() == n_valid and out["err_count"].item() == 0
    lr = out["loss_rows"].double().cpu().numpy()
    assert np.all(lr[t == -100] == 0.0)
    # property: the loss is the mean of the per-row losses over valid rows
    assert abs(out["loss"].item() - lr.sum() / n_valid) <= 1e-6 * abs(out["loss"].item())
    rows = _sample_rows(target, logits)
    idx = torch.from_numpy(rows).to(DEV)
    sub_logits, sub_t = logits[idx], target[idx]
    ref = P.oracle_for(sub_logits, sub_t, n_valid=n_valid)
    P.assert_loss_rows(out["loss_rows"][idx], ref, "full-size sample")
    P.assert_grad_close(out["grad"][idx], ref["grad"], "full-size sample grad")
    conf = P.collapse_rows(sub_logits, sub_t)     # indices into the sample
    assert len(conf) >= 8
    P.assert_collapse_rows(out["loss_rows"][idx], out["grad"][idx].cpu(), sub_t.cpu(), ref,
                           conf, "full-size collapse rows")
    # the whole-batch loss from the oracle over every row
    print("[full] oracle over all rows", flush=True)
    z = to_numpy_logits(logits)
    f = O.forward(z, t)
    loss, nv, _ = O.reduce(f["loss"], f["status"], "mean")
    assert nv == n_valid
    P.assert_scalar_loss(out["loss"].item(), loss, "full-size loss")


def test_fused_full_size_every_element(page):
    """Every per-row loss and every one of the 2.1e9 gradient elements of
    the page-scale fused call against the oracle, in blocks of 1024 rows
    (the oracle's gradient of a block is 1 GB of fp64)."""
    logits, target = page
    T, V = logits.shape
    out = vce.fused_fwd_bwd(logits, target)
    torch.cuda.synchronize()
    t = target.cpu().numpy()
    n_valid = int((t != -100).sum())
    worst, ones = 0, 0
    for r0 in range(0, T, 1024):
        r1 = min(T, r0 + 1024)
        ref = P.oracle_for(logits[r0:r1], target[r0:r1], n_valid=n_valid)
        P.assert_loss_rows(out["loss_rows"][r0:r1], ref, f"rows [{r0},{r1})")
        g = P.ordered_bf16(P.bf16_bits(out["grad"][r0:r1]))
        d = np.abs(g - P.ordered_bf16(O.to_bf16(ref["grad"])))
        worst = max(worst, int(d.max()))
        ones += int((d == 1).sum())
        assert worst <= P.BF16_ULPS, f"rows [{r0},{r1}): bf16 gradient off by {worst} ulp"
        if r0 % 4096 == 0:
            print(f"[full] every element: rows [0,{r1}) checked, max {worst} ulp", flush=True)
    print(f"[full] every element: {T * V} gradients, max {worst} ulp, {ones} at 1 ulp",
          flush=True)


def test_split_vocabulary_full_size(page):
    logits, target = page
    T, V = logits.shape
    half = V // 2
    eps = 0.1
    print("[full] split-V shards, eps=0.1", flush=True)
    s1 = vce.forward(logits[:, :half], target, vocab_start=0, V_total=V, label_smoothing=eps)
    s2 = vce.forward(logits[:, half:], target, vocab_start=half, V_total=V,
                     label_smoothing=eps)
    m = vce.merge_shard_stats([s1["stats"], s2["stats"]], target, V, label_smoothing=eps)
    g1 = vce.backward(logits[:, :half], target, m["fin"], m["n_valid"], vocab_start=0,
                      V_total=V, label_smoothing=eps)
    g2 = vce.backward(logits[:, half:], target, m["fin"], m["n_valid"], vocab_start=half,
                      V_total=V, label_smoothing=eps)
    torch.cuda.synchronize()
    t = target.cpu().numpy()
    n_valid = int((t != -100).sum())
    assert m["n_valid"].item() == n_valid
    rows = _sample_rows(target, logits)
    idx = torch.from_numpy(rows).to(DEV)
    ref = P.oracle_for(logits[idx], target[idx], eps=eps, n_valid=n_valid)
    P.assert_loss_rows(m["loss_rows"][idx], ref, "split full-size sample")
    P.assert_grad_close(g1[idx], ref["grad"][:, :half], "split shard 0")
    P.assert_grad_close(g2[idx], ref["grad"][:, half:], "split shard 1")
    lr = m["loss_rows"].double().cpu().numpy()
    assert abs(m["loss"].item() - lr.sum() / n_valid) <= 1e-6 * abs(m["loss"].item())


def test_mid_workload_full_size():
    """T = 4096, V = 32000 bf16 logits ~ N(0, 2^2), 82 ignored rows, mean,
    bf16 gradient: every loss and every gradient element against the
    oracle over the whole batch (it finishes in seconds at this size)."""
    c = S.MID
    print(f"[full] mid workload T={c.T} V={c.V}", flush=True)
    logits, target = S.generate(c, device=DEV, block_rows=1024)
    lg, tg = logits, target
    out = vce.fused_fwd_bwd(lg, tg)
    torch.cuda.synchronize()
    ref = P.oracle_for(lg, tg)
    assert int(out["n_valid"].item()) == ref["n_valid"] == c.T - c.n_ignored
    assert int(out["err_count"].item()) == 0
    P.assert_loss_rows(out["loss_rows"], ref, "mid full size")
    P.assert_scalar_loss(out["loss"].item(), ref["loss"], "mid full size")
    P.assert_grad_close(out["grad"], ref["grad"], "mid full size grad")


def test_beyond_2_31_elements():
    """T = 17000 rows of V = 128256 bf16 logits: 2.18e9 elements, so the
    last rows start beyond 2^31 elements (and 2^32 bytes) of the logits and
    of the gradient.  The fused call and the separate forward / backward
    calls are checked on rows at both ends against the oracle; the batch
    loss is the mean of the per-row losses."""
    c = S.scaled(S.PAGE, 17000, 128256, 1011)
    print(f"[full] T={c.T} V={c.V}: {c.T * c.V / 2 ** 31:.3f} x 2^31 elements", flush=True)
    logits, target = S.generate(c, device=DEV, block_rows=2048)
    T, V = logits.shape
    first_far = (2 ** 31 + V - 1) // V          # first row starting beyond 2^31 elements
    rows = np.array([0, 1, 2, T // 2, first_far - 1, first_far, first_far + 1, T - 3, T - 2,
                     T - 1])
    idx = torch.from_numpy(rows).to(DEV)
    t = target.cpu().numpy()
    n_valid = int((t != -100).sum())
    out = vce.fused_fwd_bwd(logits, target)
    torch.cuda.synchronize()
    ref = P.oracle_for(logits[idx], target[idx], n_valid=n_valid)
    P.assert_loss_rows(out["loss_rows"][idx], ref, "beyond 2^31: fused")
    P.assert_grad_close(out["grad"][idx], ref["grad"], "beyond 2^31: fused grad")
    lr = out["loss_rows"].double().cpu().numpy()
    assert out["n_valid"].item() == n_valid
    assert abs(out["loss"].item() - lr.sum() / n_valid) <= 1e-6 * abs(out["loss"].item())
    grad = out["grad"]
    del out
    print("[full] forward, then backward", flush=True)
    f = vce.forward(logits, target)
    vce.backward(logits, target, f["fin"], f["n_valid"], grad=grad)
    torch.cuda.synchronize()
    P.assert_loss_rows(f["loss_rows"][idx], ref, "beyond 2^31: forward")
    P.assert_grad_close(grad[idx], ref["grad"], "beyond 2^31: backward grad")


def test_split_vocabulary_full_size_every_element(page):
    """The split-vocabulary step with smoothing 0.1 (two 64128-column shards,
    merge, per-shard backward): every per-row loss and every gradient
    element against the oracle over the whole vocabulary, in row blocks."""
    logits, target = page
    T, V = logits.shape
    half, eps = V // 2, 0.1
    s1 = vce.forward(logits[:, :half], target, vocab_start=0, V_total=V, label_smoothing=eps)
    s2 = vce.forward(logits[:, half:], target, vocab_start=half, V_total=V,
                     label_smoothing=eps)
    m = vce.merge_shard_stats([s1["stats"], s2["stats"]], target, V, label_smoothing=eps)
    grad = torch.empty_like(logits)
    vce.backward(logits[:, :half], target, m["fin"], m["n_valid"], vocab_start=0, V_total=V,
                 label_smoothing=eps, grad=grad[:, :half])
    vce.backward(logits[:, half:], target, m["fin"], m["n_valid"], vocab_start=half,
                 V_total=V, label_smoothing=eps, grad=grad[:, half:])
    torch.cuda.synchronize()
    t = target.cpu().numpy()
    n_valid = int((t != -100).sum())
    worst, ones = 0, 0
    for r0 in range(0, T, 1024):
        r1 = min(T, r0 + 1024)
        ref = P.oracle_for(logits[r0:r1], target[r0:r1], eps=eps, n_valid=n_valid)
        P.assert_loss_rows(m["loss_rows"][r0:r1], ref, f"shards rows [{r0},{r1})")
        g = P.ordered_bf16(P.bf16_bits(grad[r0:r1]))
        d = np.abs(g - P.ordered_bf16(O.to_bf16(ref["grad"])))
        worst = max(worst, int(d.max()))
        ones += int((d == 1).sum())
        assert worst <= P.BF16_ULPS, f"shards rows [{r0},{r1}): off by {worst} ulp"
        if r0 % 4096 == 0:
            print(f"[full] shards, every element: rows [0,{r1}) checked", flush=True)
    print(f"[full] shards, every element: {T * V} gradients, max {worst} ulp, {ones} at 1 ulp",
          flush=True)
