/*
 * vocab_ce.h -- C ABI of libvocab_ce.so: numerically stable softmax
 * cross-entropy forward and backward over a logits matrix [T, V] on one
 * AMD Instinct MI355X (gfx950) GPU.
 *
 * What is computed, per row r with target t (ignore_index rows excepted):
 *
 *   m   = max over non-target columns of z          (the stabilising shift)
 *   s   = sum over non-target columns of exp(z_j - m)
 *   x   = (m - z_t) + log s                          (= lse_{j != t} - z_t)
 *   nll = softplus(x)                                (= -log p_t)
 *   lse = z_t + nll
 *   loss_r = (1 - eps) nll + eps (lse - mean_j z_j)  (eps: label smoothing)
 *   grad_rj = k_r (p_j - eps/V)              j != t, p_j = exp(z_j - lse)
 *   grad_rt = k_r (g_t + eps (V-1)/V),  g_t = p_t - 1 if p_t < 1/4, else -p_nt
 *
 * with k_r = grad_output (sum), grad_output / N_valid (mean) or
 * grad_output[r] (none).
 *
 *   torchtitan PR "[loss] fix softmax collapse with improved ce perf":
 *     opening summary -- the forward computes the non-target mass and
 *       prepares the backward instead of saving log-probabilities;
 *     Numerics -- NLL = softplus(lse over non-targets - z_t) with the target
 *       dropped before the sum; target gradient p_t - 1 below p_t = 1/4,
 *       else minus the non-target probability; ignored labels are targets
 *       on no shard and get zero loss and gradient;
 *     Memory/perf -- input logits are never modified; bf16 logits are
 *       upcast inside, never copied to fp32; the forward reads the logits
 *       once and the backward rebuilds the gradient in one pass.
 *   Megatron-core core.tensor_parallel.cross_entropy:
 *     VocabParallelCrossEntropy -- per-shard max, per-shard target logit
 *       (zero where the shard does not own the target), sums combined over
 *       the vocabulary shards; scale_gradients_inplace scales by grad_output;
 *     vocab_parallel_cross_entropy -- label_smoothing in [0, 1); logits are
 *       [sequence, batch, vocab / ranks], flattened here to T rows.
 *
 * Conventions shared by every entry point:
 *   - Every pointer argument not marked "host" is a DEVICE pointer.  The
 *     caller owns and allocates every buffer; the library never allocates,
 *     frees or synchronises, and launches all work on `stream` (a
 *     hipStream_t; NULL is the default stream).  Calls are asynchronous.
 *   - Inputs are const and never written, with one opt-in exception: the
 *     gradient may be written in place over the logits (grad == logits,
 *     ldg == ld, grad_dtype == logits_dtype), as the torchtitan PR's eager
 *     path and Megatron-core's in-place methods do, halving the memory of a
 *     fused step.  Any other overlap of outputs with inputs or with each
 *     other is an error.
 *   - Logits: row r, column j of this call lives at logits[r * ld + j]
 *     (elements, not bytes), j in [0, V_local).  Any alignment is accepted;
 *     16-byte aligned rows take the vectorised path.
 *   - Targets are int64 [T]; a target equal to ignore_index marks an
 *     ignored row; any other target outside [0, V_total) is a bad target.
 *   - Return value: CE_OK (0) or a negative ce_status.  Arguments are
 *     checked on the host before anything is launched; a failed check
 *     launches nothing.  CE_ERR_HIP reports a failed launch.
 *   - Bad targets are data errors found on the device: such a row gets
 *     status -1, loss_r = NaN (so a sum or mean over it is NaN) and a
 *     gradient row of zeros, and is counted in *err_count.
 *   - T == 0 is a successful no-op except that scalar outputs are written
 *     (loss 0 for sum, NaN for mean, n_valid 0, err_count 0).
 *   - Results are deterministic: fixed reduction trees, no float atomics.
 */
#ifndef VOCAB_CE_H
#define VOCAB_CE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CE_F32 = 0,  /* IEEE binary32 */
    CE_BF16 = 1  /* bfloat16: the top 16 bits of a binary32; outputs are
                    rounded to nearest, ties to even */
} ce_dtype;

typedef enum {
    CE_RED_NONE = 0, /* per-row losses only; k_r = grad_output[r] */
    CE_RED_SUM = 1,  /* loss = sum over non-ignored rows; k_r = grad_output[0] */
    CE_RED_MEAN = 2  /* loss = that sum / N_valid; k_r = grad_output[0] / N_valid */
} ce_reduction;

typedef enum {
    CE_OK = 0,
    CE_ERR_NULL = -1,      /* a required pointer is NULL */
    CE_ERR_SHAPE = -2,     /* T < 0, V_local < 1, ld < V_local, ldg < V_local,
                              vocab_start < 0, vocab_start + V_local > V_total,
                              or a size too large for the kernels' indexing */
    CE_ERR_SMOOTHING = -3, /* label_smoothing not in [0, 1) or not finite */
    CE_ERR_DTYPE = -4,     /* unknown ce_dtype */
    CE_ERR_REDUCTION = -5, /* unknown ce_reduction */
    CE_ERR_WORKSPACE = -6, /* workspace NULL or smaller than ce_workspace_bytes */
    CE_ERR_SHARDS = -7,    /* n_shards < 1 or > CE_MAX_SHARDS */
    CE_ERR_ALIAS = -8,     /* grad overlaps logits other than exactly in place */
    CE_ERR_HIP = -9,       /* a HIP launch failed */
    CE_ERR_ARG = -10       /* an output given where the call cannot produce it
                              (e.g. finalize outputs of a split-vocabulary
                              ce_forward, or the whole-vocabulary fused call
                              given a shard) */
} ce_status;

#define CE_MAX_SHARDS 64

/* The problem one call works on.  A host struct, passed by pointer. */
typedef struct {
    int64_t T;            /* rows */
    int64_t V_local;      /* columns handled by this call */
    int64_t ld;           /* row stride of the logits, in elements (>= V_local) */
    int64_t vocab_start;  /* global column of this call's column 0 */
    int64_t V_total;      /* vocabulary size across all shards */
    int64_t ignore_index; /* target value that marks an ignored row, e.g. -100 */
    float label_smoothing;/* eps in [0, 1) */
    int32_t reduction;    /* ce_reduction */
} ce_problem;

/* Partial statistics of one row over this call's columns (one vocabulary
 * shard): the forward's output when the vocabulary is split, merged by
 * ce_merge_shard_stats.  32 bytes, device memory, [T] per shard.  A row
 * whose target is ignore_index or outside [0, V_total) is not read: its
 * statistics are m = -inf, s = 0, zt = 0, own = 0, sz = 0. */
typedef struct {
    float m;          /* max over this shard's non-target columns; -inf if none */
    float zt;         /* z at the target if this shard owns it, else 0 */
    int32_t own;      /* 1 if this shard owns the target, else 0 */
    int32_t reserved; /* 0 */
    double s;         /* sum over the same columns of exp(z_j - m); 0 if m = -inf */
    double sz;        /* sum of z over all of this shard's columns; computed
                         only when label_smoothing > 0 (else 0) */
} ce_row_stats;

/* What the forward prepares for the backward, per row.  24 bytes, device
 * memory, [T]. */
typedef struct {
    double lse;     /* log-sum-exp of the whole row (all shards) */
    double gt;      /* target gradient before the row scale k_r: p_t - 1 or
                       -p_nt by the 1/4 select, plus eps (V-1)/V */
    float m;        /* the merged non-target max */
    int32_t status; /* 1 valid, 0 ignored, -1 bad target */
} ce_row_final;

/* Workspace, in bytes, that `op` needs for `prob` (0 if none).  `op` is one
 * of the CE_OP_* values.  Host function; never fails (an invalid problem
 * yields 0 and the entry point then reports the problem's error). */
enum { CE_OP_FORWARD = 0, CE_OP_BACKWARD = 1, CE_OP_FUSED = 2, CE_OP_MERGE = 3 };
size_t ce_workspace_bytes(const ce_problem *prob, int op);

/* Forward: one read of the logits.
 *   stats   [T] out, required: this call's partial row statistics.
 *   When the call covers the whole vocabulary (vocab_start == 0 and
 *   V_local == V_total) it also finalizes, writing whichever of these are
 *   non-NULL:
 *     fin       [T] ce_row_final for ce_backward;
 *     loss_rows [T] float per-row loss (+0 ignored, NaN bad target);
 *     loss      [1] float reduced loss (sum or mean; not written for none);
 *     n_valid   [1] int32 number of rows with status 1;
 *     err_count [1] int32 number of bad targets.
 *   When the vocabulary is split, those outputs must be NULL and
 *   ce_merge_shard_stats produces them from all shards' stats.
 *   ws/ws_bytes: workspace of at least ce_workspace_bytes(prob, CE_OP_FORWARD).
 * Megatron-core VocabParallelCrossEntropy.calculate_logits_max and
 * gather_predicted_logits (per-shard max and owned target logit);
 * torchtitan PR Numerics (non-target mass, target dropped before the sum). */
int ce_forward(const ce_problem *prob, const void *logits, int logits_dtype,
               const int64_t *target, ce_row_stats *stats, ce_row_final *fin,
               float *loss_rows, float *loss, int32_t *n_valid, int32_t *err_count,
               void *ws, size_t ws_bytes, void *stream);

/* Merge the partial statistics of n_shards vocabulary shards, in shard
 * order 0..n_shards-1, and finalize:
 *   M = max_s m_s;  s = sum_s s_s exp(m_s - M);  zt = sum_s zt_s;
 *   own = sum_s own_s (a non-ignored row is valid only if own == 1);
 *   sz = sum_s sz_s;  then x, nll, lse, loss_r, the target select.
 *   shard_stats [n_shards][T], shard-major (shard k's row r at k * T + r).
 *   prob->V_total is the full vocabulary; V_local, ld, vocab_start unused.
 *   fin [T] required; loss_rows, loss, n_valid, err_count optional.
 *   ws/ws_bytes: at least ce_workspace_bytes(prob, CE_OP_MERGE).
 * On one GPU this replaces the vocabulary-parallel all-reduce of
 * Megatron-core vocab_parallel_cross_entropy (tp_group). */
int ce_merge_shard_stats(const ce_problem *prob, int n_shards,
                         const ce_row_stats *shard_stats, const int64_t *target,
                         ce_row_final *fin, float *loss_rows, float *loss,
                         int32_t *n_valid, int32_t *err_count, void *ws, size_t ws_bytes,
                         void *stream);

/* Backward: one read of the logits and one write of the gradient.
 *   fin         [T] from ce_forward (unsharded) or ce_merge_shard_stats.
 *   n_valid     [1] device int32, required for CE_RED_MEAN (else may be NULL).
 *   grad_output device float: [1] for sum and mean, [T] for none; NULL
 *               means 1.0 everywhere.
 *   grad        [T, V_local] out, row stride ldg elements, grad_dtype;
 *               may be the logits themselves (same pointer, ldg == ld,
 *               same dtype: the gradient overwrites them); any other
 *               overlap is CE_ERR_ALIAS.
 * Ignored and bad-target rows get +0 everywhere.
 * Megatron-core VocabParallelCrossEntropy.prepare_gradient_calculation_operands,
 * calculate_gradients, scale_gradients_inplace; torchtitan PR Numerics
 * (target select) and Memory/perf (one fused gradient pass). */
int ce_backward(const ce_problem *prob, const void *logits, int logits_dtype,
                const int64_t *target, const ce_row_final *fin, const int32_t *n_valid,
                const float *grad_output, void *grad, int grad_dtype, int64_t ldg,
                void *stream);

/* Fused forward + backward over the whole vocabulary (vocab_start == 0,
 * V_local == V_total): reads each logits row once and writes its gradient
 * once.  loss_rows, loss, n_valid, err_count optional (loss is not written
 * for CE_RED_NONE); grad_output as in ce_backward; grad as in ce_backward.
 * ws/ws_bytes: at least ce_workspace_bytes(prob, CE_OP_FUSED).
 * torchtitan PR opening summary (the forward prepares the backward) and
 * Memory/perf (one read of the logits, one fused gradient pass). */
int ce_fused_fwd_bwd(const ce_problem *prob, const void *logits, int logits_dtype,
                     const int64_t *target, const float *grad_output, float *loss_rows,
                     float *loss, int32_t *n_valid, int32_t *err_count, void *grad,
                     int grad_dtype, int64_t ldg, void *ws, size_t ws_bytes,
                     void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation and results as ce_fused_fwd_bwd, with no workspace argument.
 * Its scratch memory is a static device array of CE_NOALLOC_SCRATCH_BYTES
 * in the library, one per GPU, held until the process ends; the call
 * allocates nothing.  The caller still passes inputs and outputs.
 *   - Problems whose ce_workspace_bytes(prob, CE_OP_FUSED) exceeds
 *     CE_NOALLOC_SCRATCH_BYTES (about 139,000 rows at any row length)
 *     return CE_ERR_WORKSPACE before any launch.
 *   - The stream must belong to the current device (CE_ERR_ARG otherwise).
 *   - Every call on one GPU shares that GPU's array: calls that overlap in
 *     time on one GPU (two streams, two threads) race and give wrong
 *     results.  Calls in order on one stream are safe; nothing in the
 *     array needs to start at zero, every byte read is first written by
 *     the same call.
 *   - The first call on a device looks the array's address up once
 *     (hipGetSymbolAddress) and keeps it. */
#define CE_NOALLOC_SCRATCH_BYTES (8u << 20)
int ce_fused_fwd_bwd_noalloc(const ce_problem *prob, const void *logits, int logits_dtype,
                             const int64_t *target, const float *grad_output, float *loss_rows,
                             float *loss, int32_t *n_valid, int32_t *err_count, void *grad,
                             int grad_dtype, int64_t ldg, void *stream);

/* ------------------------------------------------------------------------ */
/* Cross-entropy of a linear classifier, logits = E C^T never stored.        */
/* ------------------------------------------------------------------------ */

/* apple/ml-cross-entropy issue #14: linear_cross_entropy(embeddings,
 * classifier weight, labels) fuses the classifier product with the loss so
 * that the [N, V] logits are never materialised; the thread's fix keeps the
 * dC and dE accumulations out of low precision (fp32 accumulators, optional
 * Kahan compensation: use_kahan; impl="cce_exact" also turns off gradient
 * filtering, which is opt-in here through filter_eps).
 *
 *   z_rv = sum_d E[r,d] C[v,d]     (bf16 inputs, fp32 accumulation, MFMA)
 *   loss_r, the 1/4 target select, ignore_index, label smoothing and the
 *   row scale k_r exactly as for ce_fused_fwd_bwd on those logits;
 *   G = k (softmax(z) - q), rounded to bf16 (round-to-nearest-even) as the
 *   operand of the two backward products;
 *   dE = G C   [N, D] fp32,  dC = G^T E  [V, D] fp32.
 *
 * The backward processes the vocabulary in chunks of at most
 * CE_LINEAR_CHUNK classes, fewer when the chunk's bf16 G and G^T would pass
 * 256 MiB (8192 classes at 8192 tokens): dC rows of a chunk are complete
 * after it, dE is summed over the chunks in fp32 or, with CE_ACC_KAHAN,
 * with a Kahan compensation term (one more [N, D] fp32 workspace buffer).
 * Everything is deterministic (no atomics). */
#define CE_LINEAR_CHUNK 16384

typedef enum {
    CE_ACC_FP32 = 0, /* dE summed over vocabulary chunks in fp32 */
    CE_ACC_KAHAN = 1 /* ... with Kahan compensation */
} ce_accum;

typedef struct {
    int64_t N;            /* rows of E (tokens) */
    int64_t D;            /* hidden size: columns of E and C; a multiple of 8 */
    int64_t V;            /* classes: rows of C */
    int64_t ignore_index; /* target value that marks an ignored row */
    float label_smoothing;/* eps in [0, 1) */
    int32_t reduction;    /* ce_reduction */
    int32_t accum;        /* ce_accum */
    float filter_eps;     /* gradient filtering threshold; 0 = off (exact) */
} ce_linear_problem;

/* Gradient filtering (filter_eps > 0; apple/ml-cross-entropy issue #14:
 * the fused loss filters gradients by default, and impl="cce_exact" turns
 * that off -- the page does not state the rule; this is the reading taken):
 * the unscaled gradient u = softmax(z) - q (G = k u, target entries from
 * the 1/4 select) is cut into blocks of 256 tokens x 256 classes aligned at
 * token 0 and class 0; a block in which every entry of every valid row with
 * k_r != 0 has |u| < filter_eps is dropped -- taken as zero in both backward
 * products, whose work for it is skipped.  (A row with k_r = 0, e.g. a zero
 * per-row grad_output, has an all-zero gradient and keeps no block.)  The loss is exact either way.  2^-8 (the
 * bf16 unit roundoff) drops blocks whose entries all vanish next to a unit
 * entry at bf16 resolution.  The error this brings into an entry of dE or
 * dC is at most the sum over the dropped blocks' entries of |G| times the
 * matching |C| or |E| entries.  filter_eps = 0 gives results bit-identical
 * to a call without filtering.  Must be finite and >= 0 (else CE_ERR_ARG). */

/* Workspace bytes ce_linear_fwd_bwd needs; `backward` = 0 when dE and dC
 * are both NULL (loss only).  Host function; 0 for an invalid problem. */
size_t ce_linear_workspace_bytes(const ce_linear_problem *prob, int backward);

/* Loss and, if dE or dC is non-NULL, both gradients.
 *   E [N, D] bf16, row-major, row stride D; C [V, D] bf16, row stride D;
 *   both 16-byte aligned.
 *   target [N] int64.
 *   grad_output: as in ce_backward (device; NULL means 1).
 *   loss_rows [N], loss [1], n_valid [1], err_count [1]: optional outputs
 *   as in ce_fused_fwd_bwd.
 *   dE [N, D] fp32 and dC [V, D] fp32, row-major: either both or neither.
 *   ws/ws_bytes: at least ce_linear_workspace_bytes(prob, dE != NULL).
 * Errors: CE_ERR_NULL (E, C or target NULL, or only one of dE and dC),
 * CE_ERR_SHAPE (N < 0, D < 8 or not a multiple of 8, V < 1, sizes beyond
 * the kernels' 32-bit block offsets), CE_ERR_SMOOTHING, CE_ERR_REDUCTION,
 * CE_ERR_ARG (unknown accum, filter_eps negative or not finite),
 * CE_ERR_WORKSPACE, CE_ERR_HIP. */
int ce_linear_fwd_bwd(const ce_linear_problem *prob, const void *E, const void *C,
                      const int64_t *target, const float *grad_output, float *loss_rows,
                      float *loss, int32_t *n_valid, int32_t *err_count, float *dE, float *dC,
                      void *ws, size_t ws_bytes, void *stream);

/* Human-readable name of a ce_status.  Host function, static storage. */
const char *ce_status_str(int status);

/* Library version as MAJOR * 10000 + MINOR * 100 + PATCH.  Host function. */
int ce_version(void);

/* ======================================================================== */
/* MEASUREMENT ONLY -- not part of the computation.                          */
/* ======================================================================== */

/* ce_fused_fwd_bwd, plus two HIP events (hipEvent_t handles created and
 * owned by the caller, passed as void *) recorded on `stream`: ev_start just
 * before the call's main kernels (after the count of valid targets when
 * that is a launch of its own; batches of at most 1024 rows on the
 * register-resident kernels count inside them) and ev_stop just after them
 * (before the loss reduction), so that a benchmark
 * can time the fused kernel alone with hipEventElapsedTime.  Both NULL: the
 * same as ce_fused_fwd_bwd.  CE_ERR_ARG if exactly one is NULL.  Results
 * are bit-identical to ce_fused_fwd_bwd; the library keeps no state. */
int ce_fused_fwd_bwd_timed(const ce_problem *prob, const void *logits, int logits_dtype,
                           const int64_t *target, const float *grad_output, float *loss_rows,
                           float *loss, int32_t *n_valid, int32_t *err_count, void *grad,
                           int grad_dtype, int64_t ldg, void *ws, size_t ws_bytes, void *stream,
                           void *ev_start, void *ev_stop);

#ifdef __cplusplus
}
#endif

#endif /* VOCAB_CE_H */
