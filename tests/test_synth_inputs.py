"""The seeded input generator: deterministic, and the target mix it promises."""
import numpy as np
import torch

from synth import ce_inputs as S


def test_generator_is_deterministic_and_mix_is_as_stated():
    case = S.scaled(S.PAGE, 200, 3000, seed=77)
    a, ta = S.generate(case)
    b, tb = S.generate(case)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)) and torch.equal(ta, tb)
    assert a.dtype == torch.bfloat16 and ta.dtype == torch.int64
    assert int((ta == -100).sum()) == case.n_ignored
    z = a.to(torch.float64)
    valid = ta != -100
    margins = []
    for r in torch.nonzero(valid).flatten().tolist():
        row = z[r].clone()
        zt = row[ta[r]].item()
        row[ta[r]] = -float("inf")
        margins.append(zt - row.max().item())
    margins = np.array(margins)
    # confident rows: margin in [10, 40] up to the bf16 rounding of z_t
    conf = margins > 5
    assert conf.sum() == case.n_margin
    assert margins[conf].min() >= 10 - 0.25 and margins[conf].max() <= 40 + 0.25


def test_tiny_case_rowmax_plus_25():
    logits, target = S.generate(S.TINY)
    assert logits.shape == (64, 1000) and logits.dtype == torch.float32
    assert int((target == -100).sum()) == 4
    rows = 0
    for r in range(64):
        t = int(target[r])
        if t < 0:
            continue
        row = logits[r].clone()
        zt = row[t].item()
        row[t] = -float("inf")
        if zt - row.max().item() > 20:
            rows += 1
            assert abs(zt - row.max().item() - 25.0) < 1e-5
    assert rows == 8
