"""High-precision brute force for tiny rows (test infrastructure only).

Evaluates the textbook definition directly, with no stabilising rearrangement:

    p_j   = exp(z_j) / sum_i exp(z_i)
    loss  = sum_j q_j * (-log p_j),   q = (1 - eps) onehot(t) + eps / V
    grad  = p - q

in Python ``decimal`` arithmetic at 60 significant digits.  ``exp`` and
``ln`` of ``decimal`` are correctly rounded, and every binary64 input
converts to a Decimal exactly, so the only error is the 60-digit rounding:
far below what fp64 can resolve even at target margins of 40, where
1 - p_t is about 4e-18.  Used to pin the fp64 oracle (which uses the
cancellation-free form of torchtitan PR "[loss] fix softmax collapse with
improved ce perf", Numerics) against an independent evaluation.
"""
from decimal import Decimal, localcontext


def ce_row(z, t, eps=0.0, prec=60):
    """Return (loss, grad) of one row as Decimals; z is a sequence of finite
    floats, t the target column, eps the label-smoothing weight."""
    V = len(z)
    with localcontext() as ctx:
        ctx.prec = prec
        zd = [Decimal(float(v)) for v in z]
        e = [v.exp() for v in zd]
        total = sum(e, Decimal(0))
        log_total = total.ln()
        neg_logp = [log_total - v for v in zd]       # -log p_j
        p = [v / total for v in e]
        eps_d = Decimal(float(eps))
        u = eps_d / V
        loss = (1 - eps_d) * neg_logp[t] + u * sum(neg_logp, Decimal(0))
        q = [u] * V
        q[t] += 1 - eps_d
        grad = [p[j] - q[j] for j in range(V)]
        return +loss, [+g for g in grad]
