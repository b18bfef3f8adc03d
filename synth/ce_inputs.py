"""Seeded synthetic cross-entropy workloads.

This module only draws inputs.  It holds none of the loss or gradient
arithmetic and is the one module both the HIP path's tests and the oracle's
tests take inputs from.

Shapes follow the measured workload of torchtitan PR "[loss] fix softmax
collapse with improved ce perf" (H100 table: T = 16384 tokens, V = 128256,
bf16 logits, vocabulary split in two shards of 64128), which measured on an
unnamed benchmark input and trained on C4 with Qwen3-0.6B; neither dataset
nor weights are used here.  Gaussian logits stand in for a language model's
bulk, and a fraction of rows gets a confident target (a large target margin)
to reach the collapse regime the PR's opening summary describes.

Recipe of every case (all draws from one ``torch.Generator`` seeded with
``seed``, in this order):
  1. logits  ~ N(0, sigma^2), drawn in fp32 row blocks, then rounded to the
     storage dtype (round-to-nearest-even for bf16);
  2. targets ~ uniform integers in [0, V);
  3. a random permutation of the rows: the first ``n_ignored`` rows get
     ``ignore_index``; the next ``n_margin`` rows get a confident target;
  4. margins ~ U[margin_lo, margin_hi) (one per confident row);
  5. a confident row's target logit becomes
        ``margin_ref`` = "nontarget": max over the other columns + margin
        ``margin_ref`` = "rowmax":    max over the whole row + margin
     rounded to the storage dtype.
"""
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch


@dataclass
class CECase:
    name: str
    T: int
    V: int
    dtype: torch.dtype           # logits storage dtype
    sigma: float
    n_ignored: int
    n_margin: int
    margin_lo: float
    margin_hi: float
    margin_ref: str              # "nontarget" or "rowmax"
    seed: int
    ignore_index: int = -100
    eps: float = 0.0             # label smoothing
    reduction: str = "mean"
    grad_dtype: Optional[torch.dtype] = None
    n_shards: int = 1
    extra: dict = field(default_factory=dict)

    @property
    def out_dtype(self):
        return self.grad_dtype if self.grad_dtype is not None else self.dtype


# The five workloads (shapes, value distributions and target mix) the
# measured configuration and its smaller parity cases are defined by.
TINY = CECase("tiny", 64, 1000, torch.float32, 1.0, 4, 8, 25.0, 25.0, "rowmax", 1001)
MID = CECase("mid", 4096, 32000, torch.bfloat16, 2.0, 82, 0, 0.0, 0.0, "nontarget", 1002)
PAGE = CECase("page", 16384, 128256, torch.bfloat16, 3.0, 164, 1638, 10.0, 40.0,
              "nontarget", 1003)
SPLIT = CECase("split_v", 16384, 128256, torch.bfloat16, 3.0, 164, 1638, 10.0, 40.0,
               "nontarget", 1003, eps=0.1, n_shards=2)
CONFIGS = {c.name: c for c in (TINY, MID, PAGE, SPLIT)}


def scaled(base: CECase, T: int, V: int, seed: int, **kw) -> CECase:
    """A smaller case with ``base``'s distributions and target mix, the
    ignored and confident fractions kept (at least one row each when the
    base has any)."""
    def frac(k):
        if k == 0:
            return 0
        return max(1, round(k * T / base.T))
    d = dict(base.__dict__)
    d.update(name=f"{base.name}_{T}x{V}", T=T, V=V, seed=seed,
             n_ignored=frac(base.n_ignored), n_margin=frac(base.n_margin), extra={})
    d.update(kw)
    return CECase(**d)


def generate(case: CECase, device="cpu", block_rows: int = 1024):
    """Draw (logits [T, V] in case.dtype, target [T] int64) on ``device``."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(case.seed)
    T, V = case.T, case.V
    logits = torch.empty((T, V), dtype=case.dtype, device=dev)
    for r0 in range(0, T, block_rows):
        r1 = min(T, r0 + block_rows)
        blk = torch.randn((r1 - r0, V), generator=g, device=dev, dtype=torch.float32)
        blk.mul_(case.sigma)
        logits[r0:r1].copy_(blk)
        del blk
    target = torch.randint(0, V, (T,), generator=g, device=dev, dtype=torch.int64)
    perm = torch.randperm(T, generator=g, device=dev)
    ign = perm[:case.n_ignored]
    conf = perm[case.n_ignored:case.n_ignored + case.n_margin]
    margins = torch.rand((conf.numel(),), generator=g, device=dev, dtype=torch.float64)
    margins = case.margin_lo + (case.margin_hi - case.margin_lo) * margins
    if conf.numel():
        rows = logits[conf].to(torch.float64)
        tc = target[conf]
        ar = torch.arange(conf.numel(), device=dev)
        if case.margin_ref == "nontarget":
            rows[ar, tc] = -float("inf")
        ref = rows.max(dim=1).values
        logits[conf, tc] = (ref + margins).to(case.dtype)
    target[ign] = case.ignore_index
    return logits, target


def to_numpy_logits(x: torch.Tensor) -> np.ndarray:
    """Host numpy view of logits in the oracle's convention: float32 stays
    float32, bf16 becomes its uint16 bit patterns."""
    x = x.detach().to("cpu").contiguous()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view(np.uint16)
    if x.dtype == torch.float32:
        return x.numpy()
    raise TypeError(f"unsupported logits dtype {x.dtype}")


# ---------------------------------------------------------------------------
# Linear-classifier workloads (embeddings E [N, D], classifier C [V, D]).
# ---------------------------------------------------------------------------

@dataclass
class LinearCase:
    """Recipe (draws from one ``torch.Generator`` seeded with ``seed``, in
    this order): E ~ N(0, sigma_e^2) and C ~ N(0, sigma_c^2), both drawn in
    fp32 row blocks and rounded to bf16 (RNE); targets ~ uniform integers in
    [0, V); a random permutation of the rows whose first ``n_ignored`` get
    ``ignore_index``.  With sigma_e = 1 and sigma_c = 0.02 the logits have
    standard deviation about 0.02 sqrt(D) (0.905 at D = 2048)."""
    name: str
    N: int
    D: int
    V: int
    sigma_e: float
    sigma_c: float
    n_ignored: int
    seed: int
    ignore_index: int = -100
    eps: float = 0.0
    reduction: str = "mean"


# The fused linear-classifier workload (embeddings [8192, 2048], classifier
# [128256, 2048], 1% of rows ignored), and the toy shape of
# apple/ml-cross-entropy issue #14 (8191 shifted rows of a 128-wide
# embedding, 32 classes).
LINEAR = LinearCase("linear", 8192, 2048, 128256, 1.0, 0.02, 82, 1005)
CCE_TOY = LinearCase("cce_toy", 8191, 128, 32, 1.0, 0.1, 0, 1006)


def generate_linear(case: LinearCase, device="cpu", block_rows: int = 4096):
    """Draw (E [N, D] bf16, C [V, D] bf16, target [N] int64) on ``device``."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(case.seed)

    def draw(rows, sigma):
        out = torch.empty((rows, case.D), dtype=torch.bfloat16, device=dev)
        for r0 in range(0, rows, block_rows):
            r1 = min(rows, r0 + block_rows)
            blk = torch.randn((r1 - r0, case.D), generator=g, device=dev, dtype=torch.float32)
            out[r0:r1].copy_(blk.mul_(sigma))
        return out

    E = draw(case.N, case.sigma_e)
    C = draw(case.V, case.sigma_c)
    target = torch.randint(0, case.V, (case.N,), generator=g, device=dev, dtype=torch.int64)
    perm = torch.randperm(case.N, generator=g, device=dev)
    target[perm[:case.n_ignored]] = case.ignore_index
    return E, C, target
