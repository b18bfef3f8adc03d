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
