/*
 * ce_oracle.c -- plain, slow, fp64 CPU reference for numerically stable
 * softmax cross-entropy over a logits matrix [n, V].
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * constant with the HIP library; the two meet only through the seeded input
 * generators, which hold none of the arithmetic below.
 *
 * Every quantity is the textbook definition written out row by row in
 * double precision, in the form that does not cancel:
 *
 *   torchtitan PR "[loss] fix softmax collapse with improved ce perf",
 *   Numerics section: the per-row loss is softplus of (log-sum-exp over the
 *   non-target logits minus the target logit); the target term is left out
 *   of the sum, so nothing small is added to exp(0) = 1.  That is exactly
 *   -log softmax(z)_t rearranged, not an approximation.
 *
 *   Megatron-core core.tensor_parallel.cross_entropy, VocabParallelCrossEntropy
 *   (calculate_logits_max, gather_predicted_logits,
 *   calculate_cross_entropy_loss): per-shard max, per-shard target logit
 *   (zero on shards that do not own the target), sums merged across shards.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - the stabilising shift is the NON-target max m (mathematically
 *     irrelevant; it keeps the dominant non-target term at exp(0));
 *   - label smoothing eps spreads eps/V uniformly over all V classes, the
 *     target included: loss = sum_j q_j * (-log p_j),
 *     q = (1 - eps) * onehot(t) + eps / V;
 *   - a target equal to ignore_index gives loss +0 and gradient +0;
 *   - a target outside [0, V) is an error: status -1, loss NaN, gradient 0;
 *   - the mean divides by the number of rows whose status is 1.
 *
 * No -ffast-math: inf/NaN semantics and log1p matter here.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_F64 2 /* logits computed here (the linear classifier below) */

#define ORACLE_RED_NONE 0
#define ORACLE_RED_SUM 1
#define ORACLE_RED_MEAN 2

/* One logits element as an exact double.  bf16 is the top half of an
 * IEEE binary32, so widening it is exact; so is float -> double. */
static double load_elem(const void *base, int dtype, int64_t i)
{
    if (dtype == ORACLE_F64)
        return ((const double *)base)[i];
    if (dtype == ORACLE_F32)
        return (double)((const float *)base)[i];
    uint32_t w = (uint32_t)((const uint16_t *)base)[i] << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* Neumaier's compensated summation (Neumaier 1974). */
typedef struct { double sum, comp; } nsum;

static void nsum_add(nsum *a, double v)
{
    double t = a->sum + v;
    if (fabs(a->sum) >= fabs(v))
        a->comp += (a->sum - t) + v;
    else
        a->comp += (v - t) + a->sum;
    a->sum = t;
}

static double nsum_value(const nsum *a)
{
    /* an infinite sum must not turn into NaN through the correction term */
    if (!isfinite(a->sum))
        return a->sum;
    return a->sum + a->comp;
}

/* softplus(x) = log(1 + e^x), evaluated without overflow or cancellation. */
static double softplus(double x)
{
    if (x == -INFINITY)
        return 0.0;
    if (x == INFINITY)
        return INFINITY;
    return fmax(x, 0.0) + log1p(exp(-fabs(x)));
}

/* logistic sigma(x) = 1 / (1 + e^-x) */
static double sigmoid(double x)
{
    if (x >= 0.0)
        return 1.0 / (1.0 + exp(-x));
    double e = exp(x);
    return e / (1.0 + e);
}

/* ------------------------------------------------------------------------ */
/* Per-row statistics over a column range (one shard, or the whole row).     */
/* ------------------------------------------------------------------------ */

/* Statistics of one row restricted to columns [0, V_local) of a shard:
 *   m   = max over non-target columns (-inf if there is none),
 *   s   = sum over non-target columns of exp(z_j - m) (0 if m = -inf),
 *   zt  = z at the target if this shard owns it, else 0,
 *   own = 1 if this shard owns the target, else 0,
 *   sz  = sum of z over all columns of the shard (target included).
 * t_local is the target's column inside the shard, or -1 if not owned. */
static void shard_row_stats(const void *row, int dtype, int64_t V_local, int64_t t_local,
                            double *m, double *s, double *zt, int32_t *own, double *sz)
{
    double mx = -INFINITY;
    for (int64_t j = 0; j < V_local; ++j) {
        if (j == t_local)
            continue;
        double z = load_elem(row, dtype, j);
        if (z > mx)
            mx = z;
    }
    nsum es = {0.0, 0.0}, zs = {0.0, 0.0};
    for (int64_t j = 0; j < V_local; ++j) {
        double z = load_elem(row, dtype, j);
        nsum_add(&zs, z);
        if (j == t_local || mx == -INFINITY)
            continue;
        nsum_add(&es, exp(z - mx));
    }
    *m = mx;
    *s = nsum_value(&es);
    *zt = (t_local >= 0) ? load_elem(row, dtype, t_local) : 0.0;
    *own = (t_local >= 0) ? 1 : 0;
    *sz = nsum_value(&zs);
}

/* ------------------------------------------------------------------------ */
/* Finalize: from (m, s, z_t, sum z) of the whole row to the loss.           */
/* ------------------------------------------------------------------------ */

typedef struct {
    double x;    /* lse over non-targets minus z_t */
    double nll;  /* -log p_t = softplus(x) */
    double lse;  /* log-sum-exp of the whole row */
    double loss; /* smoothed per-row loss */
} row_final;

static void finalize_row(double m, double s, double zt, double sz, int64_t V_total,
                         double eps, row_final *f)
{
    double x;
    if (s == 0.0)                 /* no non-target mass at all */
        x = (zt == -INFINITY) ? NAN : -INFINITY;
    else if (zt == -INFINITY)     /* the target has probability 0 */
        x = INFINITY;
    else
        x = (m - zt) + log(s);
    double nll = softplus(x);
    double lse;
    if (zt == -INFINITY)
        lse = (s == 0.0) ? NAN : m + log(s);
    else
        lse = zt + nll;
    /* sum_j q_j (-log p_j) with q = (1-eps) onehot + eps/V and
     * -log p_j = lse - z_j  =>  (1-eps) nll + eps (lse - mean_j z_j) */
    double loss = (eps == 0.0) ? nll
                               : (1.0 - eps) * nll + eps * (lse - sz / (double)V_total);
    f->x = x;
    f->nll = nll;
    f->lse = lse;
    f->loss = loss;
}

/* ------------------------------------------------------------------------ */
/* Exported: whole-row forward.                                              */
/* ------------------------------------------------------------------------ */

/* Forward over n rows of V columns (row stride ld elements).
 * Outputs (each [n], any may be NULL except loss and status):
 *   loss   per-row smoothed loss (+0 ignored, NaN bad target)
 *   status 1 valid, 0 ignored, -1 target outside [0, V)
 *   m, s, zt, sz, x, lse  per-row diagnostics (0 on non-valid rows). */
void oracle_forward(const void *logits, int dtype, int64_t n, int64_t V, int64_t ld,
                    const int64_t *target, int64_t ignore_index, double eps,
                    double *loss, int32_t *status, double *m_out, double *s_out,
                    double *zt_out, double *sz_out, double *x_out, double *lse_out)
{
    const size_t esz = (dtype == ORACLE_F32) ? 4 : 2;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t r = 0; r < n; ++r) {
        const char *row = (const char *)logits + (size_t)r * (size_t)ld * esz;
        int64_t t = target[r];
        double m = 0, s = 0, zt = 0, sz = 0;
        row_final f = {0, 0, 0, 0};
        int32_t st;
        if (t == ignore_index) {
            st = 0;
        } else if (t < 0 || t >= V) {
            st = -1;
            f.loss = NAN;
        } else {
            int32_t own;
            shard_row_stats(row, dtype, V, t, &m, &s, &zt, &own, &sz);
            finalize_row(m, s, zt, sz, V, eps, &f);
            st = 1;
        }
        loss[r] = f.loss;
        status[r] = st;
        if (m_out) m_out[r] = m;
        if (s_out) s_out[r] = s;
        if (zt_out) zt_out[r] = zt;
        if (sz_out) sz_out[r] = sz;
        if (x_out) x_out[r] = f.x;
        if (lse_out) lse_out[r] = f.lse;
    }
}

/* ------------------------------------------------------------------------ */
/* Exported: gradient rows.                                                  */
/* ------------------------------------------------------------------------ */

/* d loss_r / d z_rj scaled by k[r], written as doubles into grad [n, V]:
 *   j != t : k * (p_j - eps/V),           p_j = exp(z_j - lse)
 *   j == t : k * (p_t - 1 + eps (V-1)/V), p_t - 1 = -sigma(x) exactly.
 * Rows whose status is not 1 are written as +0.  x and lse are the values
 * oracle_forward returned for the same rows. */
void oracle_grad(const void *logits, int dtype, int64_t n, int64_t V, int64_t ld,
                 const int64_t *target, const int32_t *status, const double *x,
                 const double *lse, double eps, const double *k, double *grad)
{
    const size_t esz = (dtype == ORACLE_F32) ? 4 : 2;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t r = 0; r < n; ++r) {
        const char *row = (const char *)logits + (size_t)r * (size_t)ld * esz;
        double *g = grad + (size_t)r * (size_t)V;
        if (status[r] != 1) {
            for (int64_t j = 0; j < V; ++j)
                g[j] = 0.0;
            continue;
        }
        const double kr = k[r];
        const double u = eps / (double)V;
        for (int64_t j = 0; j < V; ++j) {
            double p = exp(load_elem(row, dtype, j) - lse[r]);
            g[j] = kr * (p - u);
        }
        const int64_t t = target[r];
        g[t] = kr * (-sigmoid(x[r]) + eps * (double)(V - 1) / (double)V);
    }
}

/* ------------------------------------------------------------------------ */
/* Exported: shard emulation and merge.                                      */
/* ------------------------------------------------------------------------ */

/* Statistics of columns [vocab_start, vocab_start + V_local) of a
 * V_total-column matrix, given as an [n, V_local] view with stride ld.
 * A target is owned when it is not ignore_index and falls in the range. */
void oracle_shard_stats(const void *logits, int dtype, int64_t n, int64_t V_local,
                        int64_t ld, int64_t vocab_start, const int64_t *target,
                        int64_t ignore_index, double *m, double *s, double *zt,
                        int32_t *own, double *sz)
{
    const size_t esz = (dtype == ORACLE_F32) ? 4 : 2;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t r = 0; r < n; ++r) {
        const char *row = (const char *)logits + (size_t)r * (size_t)ld * esz;
        int64_t t = target[r];
        int64_t tl = -1;
        if (t != ignore_index && t >= vocab_start && t < vocab_start + V_local)
            tl = t - vocab_start;
        shard_row_stats(row, dtype, V_local, tl, &m[r], &s[r], &zt[r], &own[r], &sz[r]);
    }
}

/* Merge S shards' statistics ([S][n] each, shard-major) and finalize:
 *   M = max_s m_s;  s = sum_s s_s exp(m_s - M) (shards with m_s = -inf add 0);
 *   zt = sum_s zt_s;  own = sum_s own_s;  sz = sum_s sz_s.
 * A row is ignored if its target is ignore_index, an error if not exactly
 * one shard owns its target, else valid.  Outputs as oracle_forward. */
void oracle_merge(int64_t S, int64_t n, const double *m, const double *s, const double *zt,
                  const int32_t *own, const double *sz, const int64_t *target,
                  int64_t ignore_index, int64_t V_total, double eps, double *loss,
                  int32_t *status, double *m_out, double *s_out, double *zt_out,
                  double *sz_out, double *x_out, double *lse_out)
{
    for (int64_t r = 0; r < n; ++r) {
        double M = -INFINITY;
        for (int64_t k = 0; k < S; ++k)
            if (m[k * n + r] > M)
                M = m[k * n + r];
        nsum ss = {0, 0}, zs = {0, 0};
        double ztm = 0.0;
        int32_t ow = 0;
        for (int64_t k = 0; k < S; ++k) {
            double mk = m[k * n + r];
            if (mk != -INFINITY)
                nsum_add(&ss, s[k * n + r] * exp(mk - M));
            ztm += zt[k * n + r];
            ow += own[k * n + r];
            nsum_add(&zs, sz[k * n + r]);
        }
        row_final f = {0, 0, 0, 0};
        int32_t st;
        double sv = nsum_value(&ss), szv = nsum_value(&zs);
        if (target[r] == ignore_index) {
            st = 0;
        } else if (ow != 1) {
            st = -1;
            f.loss = NAN;
        } else {
            finalize_row(M, sv, ztm, szv, V_total, eps, &f);
            st = 1;
        }
        loss[r] = f.loss;
        status[r] = st;
        if (m_out) m_out[r] = (st == 1) ? M : 0.0;
        if (s_out) s_out[r] = (st == 1) ? sv : 0.0;
        if (zt_out) zt_out[r] = (st == 1) ? ztm : 0.0;
        if (sz_out) sz_out[r] = (st == 1) ? szv : 0.0;
        if (x_out) x_out[r] = f.x;
        if (lse_out) lse_out[r] = f.lse;
    }
}

/* ------------------------------------------------------------------------ */
/* Exported: reductions.                                                     */
/* ------------------------------------------------------------------------ */

/* Scalar loss over the rows that are not ignored (status != 0; a bad
 * target's NaN therefore reaches the sum).  reduction: 1 sum, 2 mean over
 * the rows whose status is 1 (NaN when there are none).  Returns the loss;
 * *n_valid and *n_bad receive the counts of status 1 and status -1. */
double oracle_reduce(const double *loss, const int32_t *status, int64_t n, int reduction,
                     int64_t *n_valid, int64_t *n_bad)
{
    nsum acc = {0, 0};
    int64_t nv = 0, nb = 0;
    int any_nan = 0;
    for (int64_t r = 0; r < n; ++r) {
        if (status[r] == 0)
            continue;
        if (status[r] == 1)
            ++nv;
        else
            ++nb;
        if (isnan(loss[r]))
            any_nan = 1;
        else
            nsum_add(&acc, loss[r]);
    }
    *n_valid = nv;
    *n_bad = nb;
    double total = any_nan ? NAN : nsum_value(&acc);
    if (reduction == ORACLE_RED_MEAN)
        return total / (double)nv; /* 0/0 = NaN when nothing is valid */
    return total;
}

/* ------------------------------------------------------------------------ */
/* Exported: cross-entropy of a linear classifier, logits z = E C^T.         */
/* ------------------------------------------------------------------------ */

/* apple/ml-cross-entropy issue #14 (linear_cross_entropy(embeddings,
 * classifier weight, labels), and the reference it is checked against there:
 * logits = embeddings times the transposed classifier, then cross-entropy):
 * row r's logits are z_rv = sum_d E[r,d] C[v,d] for the V classifier rows;
 * the loss is the per-row loss above on those logits; by the chain rule the
 * gradients are dE = G C and dC = G^T E with G = d loss / d z (the rows
 * oracle_grad writes).  Everything is written out directly in fp64: each
 * logit is a plain dot product (products of bf16 or fp32 inputs are exact in
 * fp64), the row statistics and finalize are the ones above, then the two
 * contractions as plain sums.  E and C share one dtype (bf16, fp32 or fp64;
 * fp64 inputs serve the finite-difference checks). */

/* A matrix [rows, cols] as exact doubles, row-major (the caller frees). */
static double *decode_matrix(const void *X, int dtype, int64_t rows, int64_t cols)
{
    const int64_t n = rows * cols;
    double *out = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = load_elem(X, dtype, i);
    return out;
}

/* z[v] = E_r . C_v for v in [0, V), the sum over d in increasing order */
static void linear_row_logits(const double *E, const double *C, int64_t r, int64_t D, int64_t V,
                              double *z)
{
    const double *e = E + (size_t)r * (size_t)D;
    for (int64_t v = 0; v < V; ++v) {
        const double *c = C + (size_t)v * (size_t)D;
        double acc = 0.0;
        for (int64_t d = 0; d < D; ++d)
            acc += e[d] * c[d];
        z[v] = acc;
    }
}

/* Forward over the n rows of E [n, D] against C [V, D].  Outputs as
 * oracle_forward (loss, status required; x, lse may be NULL). */
void oracle_linear_forward(const void *E, const void *C, int dtype, int64_t n, int64_t D,
                           int64_t V, const int64_t *target, int64_t ignore_index, double eps,
                           double *loss, int32_t *status, double *x_out, double *lse_out)
{
    double *Ed = decode_matrix(E, dtype, n, D), *Cd = decode_matrix(C, dtype, V, D);
#pragma omp parallel
    {
        double *z = (double *)malloc((size_t)V * sizeof(double));
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n; ++r) {
            const int64_t t = target[r];
            row_final f = {0, 0, 0, 0};
            int32_t st;
            if (t == ignore_index) {
                st = 0;
            } else if (t < 0 || t >= V) {
                st = -1;
                f.loss = NAN;
            } else {
                double m, s, zt, sz;
                int32_t own;
                linear_row_logits(Ed, Cd, r, D, V, z);
                shard_row_stats(z, ORACLE_F64, V, t, &m, &s, &zt, &own, &sz);
                finalize_row(m, s, zt, sz, V, eps, &f);
                st = 1;
            }
            loss[r] = f.loss;
            status[r] = st;
            if (x_out) x_out[r] = f.x;
            if (lse_out) lse_out[r] = f.lse;
        }
        free(z);
    }
    free(Ed);
    free(Cd);
}

/* Gradients, from the status, x and lse oracle_linear_forward returned and
 * the per-row scale k:
 *   G [n, V]  d loss_r / d z_rv times k_r (written; +0 on rows whose status
 *             is not 1), the same formula as oracle_grad;
 *   dE [n, D] = G C            (may be NULL)
 *   dC [V, D] = G^T E          (may be NULL)
 *   rsE [n, D] = sqrt(sum_v (G[r,v] C[v,d])^2),
 *   rsC [V, D] = sqrt(sum_r (G[r,v] E[r,d])^2)   (may be NULL): the scales of
 *             the rounding error a bf16 copy of G brings into each sum.
 *
 * Gradient filtering (apple/ml-cross-entropy issue #14: the default
 * implementation filters gradients; impl="cce_exact" turns it off).  The
 * page does not define the rule; the reading taken: the unscaled gradient
 * u_rv = d loss_r / d z_rv (softmax minus the smoothed one-hot, the target
 * entry -sigma(x) + eps (V-1)/V) is cut into blocks of 256 rows x 256
 * classes, block (i, j) holding rows 256 i .. 256 i + 255 and classes
 * 256 j .. 256 j + 255 (the last ones ragged); with tau > 0 a block is
 * dropped when |u_rv| < tau for every row r of the block whose gradient is
 * not identically zero (status 1 and k_r != 0): its G entries are taken as
 * zero in both contractions.  tau <= 0 keeps every block (the exact
 * gradients).
 *   keep      [ceil(n/256), ceil(V/256)] int32, 1 kept / 0 dropped (may be NULL)
 *   block_max same shape, fp64: max |u_rv| over those rows of the block (0
 *             when there are none) (may be NULL) */
void oracle_linear_backward(const void *E, const void *C, int dtype, int64_t n, int64_t D,
                            int64_t V, const int64_t *target, const int32_t *status,
                            const double *x, const double *lse, double eps, const double *k,
                            double tau, double *G, double *dE, double *dC, double *rsE,
                            double *rsC, int32_t *keep, double *block_max)
{
    const double u = eps / (double)V;
    const int64_t B = 256, nbr = (n + B - 1) / B, nbv = (V + B - 1) / B;
    double *Ed = decode_matrix(E, dtype, n, D), *Cd = decode_matrix(C, dtype, V, D);
    /* the unscaled gradient rows */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n; ++r) {
        double *g = G + (size_t)r * (size_t)V;
        if (status[r] != 1) {
            for (int64_t v = 0; v < V; ++v)
                g[v] = 0.0;
        } else {
            linear_row_logits(Ed, Cd, r, D, V, g);
            for (int64_t v = 0; v < V; ++v)
                g[v] = exp(g[v] - lse[r]) - u;
            g[target[r]] = -sigmoid(x[r]) + eps * (double)(V - 1) / (double)V;
        }
    }
    /* the block decisions */
    int32_t *kp = (int32_t *)malloc((size_t)(nbr * nbv) * sizeof(int32_t));
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bi = 0; bi < nbr; ++bi) {
        for (int64_t bj = 0; bj < nbv; ++bj) {
            double m = 0.0;
            for (int64_t r = bi * B; r < n && r < (bi + 1) * B; ++r) {
                if (status[r] != 1 || k[r] == 0.0)
                    continue; /* an all-zero gradient row keeps no block */
                for (int64_t v = bj * B; v < V && v < (bj + 1) * B; ++v)
                    m = fmax(m, fabs(G[(size_t)r * (size_t)V + v]));
            }
            kp[bi * nbv + bj] = (tau <= 0.0) || (m >= tau);
            if (keep) keep[bi * nbv + bj] = kp[bi * nbv + bj];
            if (block_max) block_max[bi * nbv + bj] = m;
        }
    }
    /* scaled by k_r; dropped blocks are zero */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n; ++r) {
        double *g = G + (size_t)r * (size_t)V;
        if (status[r] != 1)
            continue;
        for (int64_t v = 0; v < V; ++v)
            g[v] = kp[(r / B) * nbv + v / B] ? k[r] * g[v] : 0.0;
    }
    free(kp);
    /* dE[r, d] = sum over v = 0, 1, ..., V-1 of G[r, v] C[v, d]: the D sums
     * of a row advance together, v in the outer loop, so C is read row by
     * row; each sum still takes its terms in increasing v. */
    if (dE || rsE) {
#pragma omp parallel
        {
            double *acc = (double *)malloc((size_t)D * sizeof(double));
            double *sq = (double *)malloc((size_t)D * sizeof(double));
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < n; ++r) {
                const double *g = G + (size_t)r * (size_t)V;
                for (int64_t d = 0; d < D; ++d)
                    acc[d] = sq[d] = 0.0;
                for (int64_t v = 0; v < V; ++v) {
                    const double *c = Cd + (size_t)v * (size_t)D;
                    for (int64_t d = 0; d < D; ++d) {
                        const double p = g[v] * c[d];
                        acc[d] += p;
                        sq[d] += p * p;
                    }
                }
                for (int64_t d = 0; d < D; ++d) {
                    if (dE) dE[r * D + d] = acc[d];
                    if (rsE) rsE[r * D + d] = sqrt(sq[d]);
                }
            }
            free(acc);
            free(sq);
        }
    }
    free(Cd);
    if (!dC && !rsC) {
        free(Ed);
        return;
    }
    /* dC[v, d] = sum over r = 0, 1, ..., n-1 of G[r, v] E[r, d].  Column v of G
     * and column d of E are first copied out contiguously, so the sum walks
     * memory in order; the terms and their order are those of the definition. */
    double *GT = (double *)malloc((size_t)V * (size_t)n * sizeof(double));
    double *ET = (double *)malloc((size_t)D * (size_t)n * sizeof(double));
#pragma omp parallel for schedule(static)
    for (int64_t v = 0; v < V; ++v)
        for (int64_t r = 0; r < n; ++r)
            GT[(size_t)v * (size_t)n + r] = G[(size_t)r * (size_t)V + v];
#pragma omp parallel for schedule(static)
    for (int64_t d = 0; d < D; ++d)
        for (int64_t r = 0; r < n; ++r)
            ET[(size_t)d * (size_t)n + r] = Ed[(size_t)r * (size_t)D + d];
    free(Ed);
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t v = 0; v < V; ++v) {
        const double *gv = GT + (size_t)v * (size_t)n;
        for (int64_t d = 0; d < D; ++d) {
            const double *ed = ET + (size_t)d * (size_t)n;
            double acc = 0.0, sq = 0.0;
            for (int64_t r = 0; r < n; ++r) {
                const double p = gv[r] * ed[r];
                acc += p;
                sq += p * p;
            }
            if (dC) dC[v * D + d] = acc;
            if (rsC) rsC[v * D + d] = sqrt(sq);
        }
    }
    free(GT);
    free(ET);
}

/* ------------------------------------------------------------------------ */
/* Exported: fp64 -> bf16 round-to-nearest-even, in one rounding.            */
/* ------------------------------------------------------------------------ */

/* bf16 keeps binary32's exponent range with an 8-bit significand.  The
 * quantum of a normal value in [2^e, 2^(e+1)) is 2^(e-7); below 2^-126
 * every value is a multiple of 2^-133.  nearbyint() rounds half to even in
 * the default rounding mode, and every scaling here is by a power of two,
 * so the only rounding is the one wanted. */
void oracle_to_bf16(const double *v, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) {
        double x = v[i];
        float f;
        if (isnan(x)) {
            f = NAN;
        } else if (x == 0.0 || isinf(x)) {
            f = (float)x;
        } else {
            int e;
            frexp(fabs(x), &e);      /* |x| = mant * 2^e, mant in [0.5, 1) */
            int q = e - 1 - 7;       /* quantum exponent for [2^(e-1), 2^e) */
            if (q < -133)
                q = -133;
            double r = nearbyint(ldexp(x, -q));
            double y = ldexp(r, q);
            /* overflow: anything that rounds to 2^128 or above is inf */
            if (fabs(y) >= 0x1p128)
                y = copysign(INFINITY, x);
            f = (float)y;            /* exact: y has at most 8 significant bits */
        }
        uint32_t w;
        memcpy(&w, &f, sizeof w);
        if (isnan(x))
            w = 0x7fc00000u | (w & 0x80000000u);
        out[i] = (uint16_t)(w >> 16);
    }
}

/* Number of OpenMP threads the row loops above run on. */
int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the number of OpenMP threads later calls use (n >= 1); used to time
 * the oracle on one host core.  No effect on any result. */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
