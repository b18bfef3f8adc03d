"""ce_fused_fwd_bwd_noalloc (the entry point for callers that cannot
allocate) against ce_fused_fwd_bwd, through the C ABI: two calls in a row on
the same GPU, the second with a smaller input, each compared bit for bit
with the workspace entry point on the same bytes (same kernels, same
arithmetic), and with the fp64 oracle within the usual bounds."""
import numpy as np
import pytest
import torch

from synth import ce_inputs as S
from tests import parity_util as P
from vocab_softmax_cross_row_amd import _binding as B

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _buffers(T, dt):
    return {"loss": torch.empty(1, dtype=torch.float32, device=DEV),
            "loss_rows": torch.empty(T, dtype=torch.float32, device=DEV),
            "n_valid": torch.empty(1, dtype=torch.int32, device=DEV),
            "err": torch.empty(1, dtype=torch.int32, device=DEV)}


def _run(case, noalloc):
    logits, target = S.generate(case)
    logits, target = logits.to(DEV), target.to(DEV)
    T, V = logits.shape
    prob = B.make_problem(T, V, ignore_index=case.ignore_index, label_smoothing=case.eps,
                          reduction=case.reduction)
    dt = B.dtype_code(logits.dtype)
    o = _buffers(T, dt)
    grad = torch.empty_like(logits)
    stream = torch.cuda.current_stream()
    if noalloc:
        B.ce_fused_fwd_bwd_noalloc(prob, logits, dt, target, None, o["loss_rows"], o["loss"],
                                   o["n_valid"], o["err"], grad, dt, V, stream)
    else:
        nws = B.ce_workspace_bytes(prob, B.CE_OP_FUSED)
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=DEV)
        B.ce_fused_fwd_bwd(prob, logits, dt, target, None, o["loss_rows"], o["loss"],
                           o["n_valid"], o["err"], grad, dt, V, ws, nws, stream)
    torch.cuda.synchronize()
    o["grad"] = grad
    return logits, target, o


def _same(a, b, what):
    for k in ("loss", "loss_rows", "n_valid", "err"):
        assert torch.equal(a[k].view(torch.uint8), b[k].view(torch.uint8)), f"{what}: {k}"
    assert torch.equal(a["grad"].view(torch.uint8), b["grad"].view(torch.uint8)), f"{what}: grad"


def test_noalloc_matches_workspace_entry_point_twice():
    # first call: 300 rows of 128256 bf16 columns take the split-V grid
    # (column-chunk statistics, merge, gradient), which keeps partial
    # statistics, row constants and per-row losses in the scratch array;
    # second call: fewer rows, smoothing (the e^z table in scratch too)
    cases = [S.scaled(S.PAGE, 300, 128256, 4401),
             S.scaled(S.PAGE, 40, 50000, 4402, eps=0.1)]
    for k, c in enumerate(cases):
        print(f"[no-alloc] call {k}: T={c.T} V={c.V} eps={c.eps}", flush=True)
        logits, target, got = _run(c, noalloc=True)
        _, _, ref = _run(c, noalloc=False)
        _same(got, ref, f"call {k}")
        oracle = P.oracle_for(logits, target, ignore_index=c.ignore_index, eps=c.eps)
        assert int(got["n_valid"].item()) == oracle["n_valid"]
        P.assert_loss_rows(got["loss_rows"], oracle, f"no-alloc call {k}")
        P.assert_scalar_loss(got["loss"].item(), oracle["loss"], f"no-alloc call {k}")
        P.assert_grad_close(got["grad"], oracle["grad"], f"no-alloc call {k}")


def test_noalloc_register_resident_rows():
    # the resident kernels use only loss rows and the count from the scratch
    c = S.scaled(S.MID, 700, 32000, 4403)
    print(f"[no-alloc] resident T={c.T} V={c.V}", flush=True)
    _, _, got = _run(c, noalloc=True)
    _, _, ref = _run(c, noalloc=False)
    _same(got, ref, "resident")


def test_noalloc_call_replays_from_a_graph():
    """The entry point's use case: a call captured into a HIP graph (it
    allocates nothing and clears nothing with a memset) and replayed on new
    inputs copied into the captured buffers, with eager work between the
    replays; every replay equals the workspace entry point on the same
    bytes, bit for bit.  Split-V grid shape (scratch holds partial
    statistics) and smoothing (scratch holds the e^z table)."""
    cases = [S.scaled(S.PAGE, 300, 128256, 4410 + k, eps=0.1) for k in range(3)]
    data = [tuple(x.to(DEV) for x in S.generate(c)) for c in cases]
    T, V = data[0][0].shape
    prob = B.make_problem(T, V, label_smoothing=0.1)
    x = data[0][0].clone()
    tg = data[0][1].clone()
    o = _buffers(T, B.CE_BF16)
    grad = torch.empty_like(x)
    stream = torch.cuda.Stream()

    def call(s):
        B.ce_fused_fwd_bwd_noalloc(prob, x, B.CE_BF16, tg, None, o["loss_rows"], o["loss"],
                                   o["n_valid"], o["err"], grad, B.CE_BF16, V, s)

    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        call(stream)                       # warm-up outside the capture
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            call(stream)
    torch.cuda.synchronize()
    for k, (c, (logits, target)) in enumerate(zip(cases, data)):
        x.copy_(logits)
        tg.copy_(target)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"[no-alloc graph] replay {k}: loss {o['loss'].item():.6f}", flush=True)
        _, _, ref = _run(c, noalloc=False)
        got = dict(o, grad=grad)
        _same(got, ref, f"graph replay {k}")
