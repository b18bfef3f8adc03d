"""Numerically stable large-vocabulary softmax cross-entropy for AMD
Instinct MI355X (gfx950): a HIP library behind a C ABI (include/vocab_ce.h)
and a ctypes binding with the same entry-point names.
"""
from ._binding import (CE_BF16, CE_F32, CE_OP_BACKWARD, CE_OP_FORWARD, CE_OP_FUSED,  # noqa: F401
                       CE_OP_MERGE, CE_RED_MEAN, CE_RED_NONE, CE_RED_SUM, CEError,
                       CELinearProblem, CEProblem, ce_backward, ce_forward, ce_fused_fwd_bwd,
                       ce_linear_fwd_bwd, ce_linear_workspace_bytes, ce_merge_shard_stats,
                       ce_fused_fwd_bwd_timed, ce_status_str, ce_version, ce_workspace_bytes,
                       make_linear_problem,
                       make_problem, read_final, read_stats)
from .api import (CrossEntropy, backward, cross_entropy, forward, fused_fwd_bwd,  # noqa: F401
                  linear_cross_entropy, merge_shard_stats)
