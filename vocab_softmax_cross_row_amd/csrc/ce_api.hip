// C ABI of libvocab_ce.so (declared in include/vocab_ce.h): argument checks,
// workspace layout and the order of launches for each entry point.  No
// allocation, no host synchronisation; everything goes on the caller's
// stream.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "ce_launch.h"
#include "vocab_ce.h"

namespace {

using namespace vce;

// Split-V grid: rows shorter than this many workgroups' worth of work are
// split into column chunks so the streaming kernels still fill the GPU.
constexpr int64_t kTargetBlocks = 1024;
constexpr int64_t kMinChunkCols = 4096;
constexpr int64_t kMaxChunks = 64;
// The fused entry point prefers the split-V grid over the row-resident
// kernel when there are fewer rows than this and rows are long.
constexpr int64_t kResidentMinRows = 512;
constexpr int64_t kResidentSplitCols = 16384;
// bf16 rows with label smoothing longer than this go to the streaming path:
// its statistics read e^z from an LDS table, while the resident kernel
// takes an fp64 exponential per logit, and from about 64K columns the extra
// pass costs less than those exponentials (page scale 2.4 against 3.7 ms).
constexpr int64_t kSmoothedResidentMaxCols = 32768;

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Plan {
    int nchunks;
    int64_t chunk_cols;
};

Plan plan_chunks(int64_t T, int64_t V_local) {
    Plan p{1, V_local};
    if (T <= 0 || T >= kTargetBlocks) return p;
    int64_t n = (kTargetBlocks + T - 1) / T;
    n = std::min(n, V_local / kMinChunkCols);
    n = std::min(n, kMaxChunks);
    if (n <= 1) return p;
    int64_t cc = (V_local + n - 1) / n;
    cc = (cc + 7) / 8 * 8; // chunk starts stay 16-byte aligned for either dtype
    p.chunk_cols = cc;
    p.nchunks = (int)((V_local + cc - 1) / cc);
    return p;
}

size_t elem_size(int dt) { return dt == CE_BF16 ? 2 : 4; }
bool dtype_ok(int dt) { return dt == CE_F32 || dt == CE_BF16; }

int check_problem(const ce_problem *p) {
    if (!p) return CE_ERR_NULL;
    if (p->reduction != CE_RED_NONE && p->reduction != CE_RED_SUM &&
        p->reduction != CE_RED_MEAN)
        return CE_ERR_REDUCTION;
    if (!std::isfinite(p->label_smoothing) || p->label_smoothing < 0.0f ||
        p->label_smoothing >= 1.0f)
        return CE_ERR_SMOOTHING;
    if (p->T < 0 || p->V_local < 1 || p->ld < p->V_local || p->vocab_start < 0 ||
        p->V_total < 1 || p->vocab_start > p->V_total - p->V_local)
        return CE_ERR_SHAPE;
    // grid and count limits: blocks are rows x chunks, counts are int32
    if (p->T > (int64_t)INT32_MAX / kMaxChunks || p->V_total > ((int64_t)1 << 40) ||
        p->ld > ((int64_t)1 << 40))
        return CE_ERR_SHAPE;
    return CE_OK;
}

bool aligned(const void *p, int64_t ld_bytes, size_t a) {
    return (reinterpret_cast<uintptr_t>(p) % a) == 0 && (ld_bytes % (int64_t)a) == 0;
}

// logits rows 16-byte aligned and gradient rows aligned to one vector store
bool vec_ok(const void *logits, int64_t ld, int in_dt, const void *grad, int64_t ldg,
            int out_dt) {
    if (!aligned(logits, ld * (int64_t)elem_size(in_dt), 16)) return false;
    if (!grad) return true;
    const size_t epv = in_dt == CE_BF16 ? 8 : 4;
    const size_t a = std::min<size_t>(16, epv * elem_size(out_dt));
    return aligned(grad, ldg * (int64_t)elem_size(out_dt), a);
}

// The streaming kernels' vector path: it starts each row (chunk) at the
// logits' first 16-byte boundary, so logits rows need only be element
// aligned; gradient rows must then be aligned for their vector stores at the
// same columns: already so, or the same element size with the same address
// residue mod 16 in every row (a contiguous gradient of a contiguous, odd
// width logits tensor, or the logits themselves).
bool stream_vec_ok(const void *logits, int64_t ld, int in_dt, const void *grad, int64_t ldg,
                   int out_dt) {
    if (vec_ok(logits, ld, in_dt, grad, ldg, out_dt)) return true;
    const size_t in_size = elem_size(in_dt), out_size = elem_size(out_dt);
    if (reinterpret_cast<uintptr_t>(logits) % in_size != 0) return false;
    if (!grad) return true;
    if (in_size != out_size) return false;
    const intptr_t d = reinterpret_cast<intptr_t>(grad) - reinterpret_cast<intptr_t>(logits);
    return d % 16 == 0 && ((ldg - ld) * (int64_t)in_size) % 16 == 0;
}

// The gradient overwrites the logits in place: same address, stride and
// dtype.  Every kernel reads an element before it writes that element's
// gradient (a row is read whole before its gradient is written), and no
// element is read by one thread and written by another.
bool in_place(const void *logits, int64_t ld, int in_dt, const void *grad, int64_t ldg,
              int out_dt) {
    return logits == grad && ld == ldg && in_dt == out_dt;
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

size_t matrix_bytes(int64_t T, int64_t cols, int64_t ld, size_t esz) {
    return T <= 0 ? 0 : ((size_t)(T - 1) * (size_t)ld + (size_t)cols) * esz;
}

// Workspace layout of an entry point.
struct Layout {
    size_t partial;   // [nchunks][T] ce_row_stats
    size_t fin;       // [T] ce_row_final
    size_t loss_rows; // [T] float
    size_t n_valid;   // [1] int32
    size_t total;
};

Layout layout(const ce_problem *p, int op) {
    Layout l{0, 0, 0, 0, 0};
    const int64_t T = std::max<int64_t>(p->T, 0);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align_up(bytes);
        return o;
    };
    const Plan pl = plan_chunks(T, p->V_local);
    if (op == CE_OP_FORWARD) {
        l.partial = take(pl.nchunks > 1 ? (size_t)pl.nchunks * T * sizeof(ce_row_stats) : 0);
        l.loss_rows = take((size_t)T * sizeof(float));
        l.n_valid = take(sizeof(int32_t));
    } else if (op == CE_OP_FUSED) {
        l.partial = take((size_t)std::max(pl.nchunks, 1) * T * sizeof(ce_row_stats));
        l.fin = take((size_t)T * sizeof(ce_row_final));
        l.loss_rows = take((size_t)T * sizeof(float));
        l.n_valid = take(sizeof(int32_t));
    } else if (op == CE_OP_MERGE) {
        l.loss_rows = take((size_t)T * sizeof(float));
        l.n_valid = take(sizeof(int32_t));
    }
    l.total = off;
    return l;
}

int check_ws(const ce_problem *p, int op, void *ws, size_t ws_bytes, Layout *l) {
    *l = layout(p, op);
    if (l->total == 0) return CE_OK;
    if (!ws || ws_bytes < l->total || reinterpret_cast<uintptr_t>(ws) % 16 != 0)
        return CE_ERR_WORKSPACE;
    return CE_OK;
}

template <class T>
T *at(void *ws, size_t off) {
    return reinterpret_cast<T *>(static_cast<char *>(ws) + off);
}


// ---- linear classifier ------------------------------------------------------
int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

int check_linear(const ce_linear_problem *p) {
    if (!p) return CE_ERR_NULL;
    if (p->reduction != CE_RED_NONE && p->reduction != CE_RED_SUM &&
        p->reduction != CE_RED_MEAN)
        return CE_ERR_REDUCTION;
    if (!std::isfinite(p->label_smoothing) || p->label_smoothing < 0.0f ||
        p->label_smoothing >= 1.0f)
        return CE_ERR_SMOOTHING;
    if (p->accum != CE_ACC_FP32 && p->accum != CE_ACC_KAHAN) return CE_ERR_ARG;
    if (!std::isfinite(p->filter_eps) || p->filter_eps < 0.0f) return CE_ERR_ARG;
    if (p->N < 0 || p->D < 8 || p->D % 8 != 0 || p->V < 1) return CE_ERR_SHAPE;
    // fragment-major operands: 16 row blocks of 16 rows x (padded K) bf16 must
    // stay below 2^31 bytes (32-bit buffer offsets); counts are int32
    const int64_t kmax = ((int64_t)1 << 31) / 512 - 256;
    if (round_up(p->N, 256) > kmax || round_up(p->V, 256) > kmax ||
        round_up(p->D, 256) > kmax || p->N > INT32_MAX)
        return CE_ERR_SHAPE;
    return CE_OK;
}

// Padded sizes and workspace layout of ce_linear_fwd_bwd.
struct LinLayout {
    int64_t Np;  // tokens padded to 256: rows of Ef and G, K of ETf and GT
    int64_t Dp;  // hidden size padded to 64: K of Ef and Cf
    int64_t Dr;  // hidden size padded to 256: rows of ETf and CTf
    int64_t Vp;  // classes padded to 256: rows of Cf, K of CTf
    int64_t Vc;  // classes per backward chunk
    int64_t tiles_v;
    size_t Ef, Cf, stats, fin, loss_rows, counts, ETf, CTf, rows, G, GT, comp;
    size_t flags, list_e, cnt_e, list_c, cnt_c; // gradient filtering, per chunk
    size_t total;
};

LinLayout linear_layout(const ce_linear_problem *p, bool backward) {
    LinLayout l{};
    const int64_t N = std::max<int64_t>(p->N, 0);
    l.Np = round_up(std::max<int64_t>(N, 1), 256);
    l.Dp = round_up(p->D, 64);
    l.Dr = round_up(p->D, 256);
    l.Vp = round_up(p->V, 256);
    // classes per backward chunk: CE_LINEAR_CHUNK, fewer when one chunk's G
    // and G^T (4 Np Vc bytes) would pass kLinGBudget
    const int64_t fit = kLinGBudget / (4 * l.Np) / 256 * 256;
    l.Vc = std::min<int64_t>(std::min<int64_t>(CE_LINEAR_CHUNK, l.Vp),
                             std::max<int64_t>(256, fit));
    l.tiles_v = l.Vp / 256;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align_up(bytes);
        return o;
    };
    l.Ef = take((size_t)l.Np * l.Dp * 2);
    l.Cf = take((size_t)l.Vp * l.Dp * 2);
    l.stats = take((size_t)l.tiles_v * N * sizeof(LinTileStats));
    l.fin = take((size_t)N * sizeof(ce_row_final));
    l.loss_rows = take((size_t)N * sizeof(float));
    l.counts = take(2 * sizeof(int32_t));
    if (backward) {
        l.ETf = take((size_t)l.Dr * l.Np * 2);
        l.CTf = take((size_t)l.Dr * l.Vc * 2); // C^T of one chunk
        l.rows = take((size_t)N * kLinRowBytes);
        l.G = take((size_t)l.Np * l.Vc * 2);
        l.GT = take((size_t)l.Vc * l.Np * 2);
        l.comp = take(p->accum == CE_ACC_KAHAN ? (size_t)N * p->D * sizeof(float) : 0);
        if (p->filter_eps > 0.0f) {
            const size_t tm = (size_t)(l.Np / 256), tn = (size_t)(l.Vc / 256);
            l.flags = take(tm * tn * 4 * sizeof(int32_t));
            l.list_e = take(tm * tn * sizeof(uint16_t));
            l.cnt_e = take(tm * sizeof(int32_t));
            l.list_c = take(tn * tm * sizeof(uint16_t));
            l.cnt_c = take(tn * sizeof(int32_t));
        }
    }
    l.total = off;
    return l;
}

// Device memory of ce_fused_fwd_bwd_noalloc: one array per device, loaded
// with the code object and held until the process ends.  Host code never
// uses this name as an address: the device address comes from
// hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) unsigned char scratch[CE_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The scratch array's device address on the current device, which must be
// the stream's device (NULL stream: the current device's default stream).
int scratch_address(hipStream_t s, void **out) {
    int dev = 0;
    if (current_device(&dev) != hipSuccess) return CE_ERR_HIP;
    if (s) {
        hipDevice_t sdev = 0;
        if (hipStreamGetDevice(s, &sdev) != hipSuccess) return CE_ERR_HIP;
        if ((int)sdev != dev) return CE_ERR_ARG;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CE_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return CE_OK;
}

#define VCE_TRY(expr)                                                                            \
    do {                                                                                         \
        const hipError_t e_ = (expr);                                                            \
        if (e_ != hipSuccess) return CE_ERR_HIP;                                                 \
    } while (0)

} // namespace

extern "C" {

size_t ce_workspace_bytes(const ce_problem *prob, int op) {
    if (check_problem(prob) != CE_OK) return 0;
    if (op != CE_OP_FORWARD && op != CE_OP_BACKWARD && op != CE_OP_FUSED && op != CE_OP_MERGE)
        return 0;
    return layout(prob, op).total;
}

int ce_forward(const ce_problem *prob, const void *logits, int logits_dtype,
               const int64_t *target, ce_row_stats *stats, ce_row_final *fin, float *loss_rows,
               float *loss, int32_t *n_valid, int32_t *err_count, void *ws, size_t ws_bytes,
               void *stream) {
    int rc = check_problem(prob);
    if (rc != CE_OK) return rc;
    if (!dtype_ok(logits_dtype)) return CE_ERR_DTYPE;
    const ce_problem &p = *prob;
    const bool whole = p.vocab_start == 0 && p.V_local == p.V_total;
    if (!whole && (fin || loss_rows || loss || n_valid || err_count)) return CE_ERR_ARG;
    if (p.T > 0 && (!logits || !target || !stats)) return CE_ERR_NULL;
    Layout l;
    if ((rc = check_ws(prob, CE_OP_FORWARD, ws, ws_bytes, &l)) != CE_OK) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);

    int32_t *nv = n_valid ? n_valid : at<int32_t>(ws, l.n_valid);
    if (p.T == 0) {
        if (whole) {
            VCE_TRY(launch_count(target, p.T, p.ignore_index, p.V_total, nv, err_count, s));
            if (loss && p.reduction != CE_RED_NONE)
                VCE_TRY(launch_reduce(nullptr, 0, p.reduction, nv, loss, s));
        }
        return CE_OK;
    }

    const Plan pl = plan_chunks(p.T, p.V_local);
    StatsArgs sa;
    sa.logits = logits;
    sa.ld = p.ld;
    sa.V_local = p.V_local;
    sa.vocab_start = p.vocab_start;
    sa.V_total = p.V_total;
    sa.target = target;
    sa.ignore_index = p.ignore_index;
    sa.T = p.T;
    sa.nchunks = pl.nchunks;
    sa.chunk_cols = pl.chunk_cols;
    sa.out = pl.nchunks > 1 ? at<ce_row_stats>(ws, l.partial) : stats;
    sa.smoothing = p.label_smoothing > 0.0f;
    sa.exp_tab = nullptr;
    const bool vec = stream_vec_ok(logits, p.ld, logits_dtype, nullptr, 0, CE_F32);
    if (sa.smoothing && vec && logits_dtype == CE_BF16)
        VCE_TRY(exp_table_address(s, &sa.exp_tab));
    VCE_TRY(launch_stats(sa, logits_dtype, vec, s));

    MergeArgs ma;
    ma.T = p.T;
    ma.target = target;
    ma.ignore_index = p.ignore_index;
    ma.V_total = p.V_total;
    ma.eps = p.label_smoothing;
    if (pl.nchunks > 1) {
        // column chunks -> this call's statistics (and the finalize if whole)
        ma.in = sa.out;
        ma.S = pl.nchunks;
        ma.stats_out = stats;
    } else {
        ma.in = stats;
        ma.S = 1;
        ma.stats_out = nullptr;
    }
    ma.fin = whole ? fin : nullptr;
    float *lr = loss_rows ? loss_rows : at<float>(ws, l.loss_rows);
    ma.loss_rows = whole ? lr : nullptr;
    // a whole-vocabulary call also counts its targets, in the merge launch
    ma.count = whole ? 1 : 0;
    ma.n_valid = nv;
    ma.err_count = err_count;
    if (ma.stats_out || ma.fin || ma.loss_rows) VCE_TRY(launch_merge(ma, s));

    if (whole && loss && p.reduction != CE_RED_NONE)
        VCE_TRY(launch_reduce(lr, p.T, p.reduction, nv, loss, s));
    return CE_OK;
}

int ce_merge_shard_stats(const ce_problem *prob, int n_shards, const ce_row_stats *shard_stats,
                         const int64_t *target, ce_row_final *fin, float *loss_rows, float *loss,
                         int32_t *n_valid, int32_t *err_count, void *ws, size_t ws_bytes,
                         void *stream) {
    int rc = check_problem(prob);
    if (rc != CE_OK) return rc;
    if (n_shards < 1 || n_shards > CE_MAX_SHARDS) return CE_ERR_SHARDS;
    const ce_problem &p = *prob;
    if (p.T > 0 && (!shard_stats || !target || !fin)) return CE_ERR_NULL;
    Layout l;
    if ((rc = check_ws(prob, CE_OP_MERGE, ws, ws_bytes, &l)) != CE_OK) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);

    int32_t *nv = n_valid ? n_valid : at<int32_t>(ws, l.n_valid);
    float *lr = loss_rows ? loss_rows : at<float>(ws, l.loss_rows);
    if (p.T == 0) VCE_TRY(launch_count(target, p.T, p.ignore_index, p.V_total, nv, err_count, s));
    if (p.T > 0) {
        MergeArgs ma;
        ma.in = shard_stats;
        ma.S = n_shards;
        ma.T = p.T;
        ma.target = target;
        ma.ignore_index = p.ignore_index;
        ma.V_total = p.V_total;
        ma.eps = p.label_smoothing;
        ma.stats_out = nullptr;
        ma.fin = fin;
        ma.loss_rows = lr;
        // the target count runs as one more workgroup of the merge
        ma.count = 1;
        ma.n_valid = nv;
        ma.err_count = err_count;
        VCE_TRY(launch_merge(ma, s));
    }
    if (loss && p.reduction != CE_RED_NONE)
        VCE_TRY(launch_reduce(lr, p.T, p.reduction, nv, loss, s));
    return CE_OK;
}

int ce_backward(const ce_problem *prob, const void *logits, int logits_dtype,
                const int64_t *target, const ce_row_final *fin, const int32_t *n_valid,
                const float *grad_output, void *grad, int grad_dtype, int64_t ldg,
                void *stream) {
    int rc = check_problem(prob);
    if (rc != CE_OK) return rc;
    if (!dtype_ok(logits_dtype) || !dtype_ok(grad_dtype)) return CE_ERR_DTYPE;
    const ce_problem &p = *prob;
    if (ldg < p.V_local) return CE_ERR_SHAPE;
    if (p.T == 0) return CE_OK;
    if (!logits || !target || !fin || !grad) return CE_ERR_NULL;
    if (p.reduction == CE_RED_MEAN && !n_valid) return CE_ERR_NULL;
    if (!in_place(logits, p.ld, logits_dtype, grad, ldg, grad_dtype) &&
        overlaps(logits, matrix_bytes(p.T, p.V_local, p.ld, elem_size(logits_dtype)), grad,
                 matrix_bytes(p.T, p.V_local, ldg, elem_size(grad_dtype))))
        return CE_ERR_ALIAS;
    hipStream_t s = static_cast<hipStream_t>(stream);

    const Plan pl = plan_chunks(p.T, p.V_local);
    GradArgs ga;
    ga.logits = logits;
    ga.ld = p.ld;
    ga.V_local = p.V_local;
    ga.vocab_start = p.vocab_start;
    ga.V_total = p.V_total;
    ga.target = target;
    ga.fin = fin;
    ga.n_valid = n_valid;
    ga.grad_output = grad_output;
    ga.reduction = p.reduction;
    ga.eps = p.label_smoothing;
    ga.grad = grad;
    ga.ldg = ldg;
    ga.nchunks = pl.nchunks;
    ga.chunk_cols = pl.chunk_cols;
    const bool vec = stream_vec_ok(logits, p.ld, logits_dtype, grad, ldg, grad_dtype);
    VCE_TRY(launch_grad(ga, logits_dtype, grad_dtype, vec, p.T, s));
    return CE_OK;
}

} // extern "C"

namespace {

// ce_fused_fwd_bwd, with optional events recorded on the stream just before
// and just after the main kernels (everything between the count of valid
// targets and the loss reduction); NULL events are not recorded.
int fused_fwd_bwd(const ce_problem *prob, const void *logits, int logits_dtype,
                  const int64_t *target, const float *grad_output, float *loss_rows, float *loss,
                  int32_t *n_valid, int32_t *err_count, void *grad, int grad_dtype, int64_t ldg,
                  void *ws, size_t ws_bytes, hipStream_t s, hipEvent_t ev_start,
                  hipEvent_t ev_stop) {
    int rc = check_problem(prob);
    if (rc != CE_OK) return rc;
    if (!dtype_ok(logits_dtype) || !dtype_ok(grad_dtype)) return CE_ERR_DTYPE;
    const ce_problem &p = *prob;
    if (p.vocab_start != 0 || p.V_local != p.V_total) return CE_ERR_ARG;
    if (ldg < p.V_local) return CE_ERR_SHAPE;
    if (p.T > 0 && (!logits || !target || !grad)) return CE_ERR_NULL;
    Layout l;
    if ((rc = check_ws(prob, CE_OP_FUSED, ws, ws_bytes, &l)) != CE_OK) return rc;
    if (p.T > 0 && !in_place(logits, p.ld, logits_dtype, grad, ldg, grad_dtype) &&
        overlaps(logits, matrix_bytes(p.T, p.V_local, p.ld, elem_size(logits_dtype)), grad,
                 matrix_bytes(p.T, p.V_local, ldg, elem_size(grad_dtype))))
        return CE_ERR_ALIAS;

    int32_t *nv = n_valid ? n_valid : at<int32_t>(ws, l.n_valid);
    float *lr = loss_rows ? loss_rows : at<float>(ws, l.loss_rows);
    const bool vec = p.T > 0 && vec_ok(logits, p.ld, logits_dtype, grad, ldg, grad_dtype);
    const bool svec = p.T > 0 && stream_vec_ok(logits, p.ld, logits_dtype, grad, ldg, grad_dtype);
    const bool split = p.T < kResidentMinRows && p.V_local >= kResidentSplitCols;
    const bool smoothed_long = p.label_smoothing > 0.0f && logits_dtype == CE_BF16 &&
                               p.V_local > kSmoothedResidentMaxCols;
    const bool resident = p.T > 0 && svec && !split && !smoothed_long &&
                          fused_fits(logits_dtype, p.V_local, vec, p.label_smoothing > 0.0f);
    // The count of valid targets comes first, from its own launch, except
    // where a later kernel of this call takes it over: a small batch's
    // register-resident kernel, or the merge of the streaming form.
    const bool count_inline = resident && p.T <= kInlineCountMaxRows;
    if (p.T == 0 || (resident && !count_inline))
        VCE_TRY(launch_count(target, p.T, p.ignore_index, p.V_total, nv, err_count, s));

    if (p.T > 0 && ev_start) VCE_TRY(hipEventRecord(ev_start, s));
    if (p.T > 0) {
        if (resident) {
            FusedArgs fa;
            fa.logits = logits;
            fa.ld = p.ld;
            fa.V = p.V_local;
            fa.target = target;
            fa.ignore_index = p.ignore_index;
            fa.grad = grad;
            fa.ldg = ldg;
            fa.grad_output = grad_output;
            fa.n_valid = nv;
            fa.loss_rows = lr;
            fa.reduction = p.reduction;
            fa.eps = p.label_smoothing;
            fa.exp_tab = nullptr;
            fa.count_inline = count_inline ? 1 : 0;
            fa.T = p.T;
            fa.count_out = nv;
            fa.err_out = err_count;
            if (p.label_smoothing > 0.0f && fused_table(logits_dtype, p.V_local)) {
                // the smoothed sums read e^z from the code object's table
                VCE_TRY(exp_table_address(s, &fa.exp_tab));
            }
            VCE_TRY(launch_fused_resident(fa, logits_dtype, grad_dtype, p.T, vec, s));
        } else {
            // streaming: stats (column chunks) -> merge + finalize -> gradient
            const Plan pl = plan_chunks(p.T, p.V_local);
            StatsArgs sa;
            sa.logits = logits;
            sa.ld = p.ld;
            sa.V_local = p.V_local;
            sa.vocab_start = 0;
            sa.V_total = p.V_total;
            sa.target = target;
            sa.ignore_index = p.ignore_index;
            sa.T = p.T;
            sa.nchunks = pl.nchunks;
            sa.chunk_cols = pl.chunk_cols;
            sa.out = at<ce_row_stats>(ws, l.partial);
            sa.smoothing = p.label_smoothing > 0.0f;
            sa.exp_tab = nullptr;
            if (sa.smoothing && svec && logits_dtype == CE_BF16)
                VCE_TRY(exp_table_address(s, &sa.exp_tab));
            VCE_TRY(launch_stats(sa, logits_dtype, svec, s));

            ce_row_final *fin = at<ce_row_final>(ws, l.fin);
            MergeArgs ma;
            ma.in = sa.out;
            ma.S = pl.nchunks;
            ma.T = p.T;
            ma.target = target;
            ma.ignore_index = p.ignore_index;
            ma.V_total = p.V_total;
            ma.eps = p.label_smoothing;
            ma.stats_out = nullptr;
            ma.fin = fin;
            ma.loss_rows = lr;
            // the target count runs as one more workgroup of the merge
            ma.count = 1;
            ma.n_valid = nv;
            ma.err_count = err_count;
            VCE_TRY(launch_merge(ma, s));

            GradArgs ga;
            ga.logits = logits;
            ga.ld = p.ld;
            ga.V_local = p.V_local;
            ga.vocab_start = 0;
            ga.V_total = p.V_total;
            ga.target = target;
            ga.fin = fin;
            ga.n_valid = nv;
            ga.grad_output = grad_output;
            ga.reduction = p.reduction;
            ga.eps = p.label_smoothing;
            ga.grad = grad;
            ga.ldg = ldg;
            ga.nchunks = pl.nchunks;
            ga.chunk_cols = pl.chunk_cols;
            VCE_TRY(launch_grad(ga, logits_dtype, grad_dtype, svec, p.T, s));
        }
    }
    if (p.T > 0 && ev_stop) VCE_TRY(hipEventRecord(ev_stop, s));
    if (loss && p.reduction != CE_RED_NONE)
        VCE_TRY(launch_reduce(lr, p.T, p.reduction, nv, loss, s));
    return CE_OK;
}

} // namespace

extern "C" {

int ce_fused_fwd_bwd(const ce_problem *prob, const void *logits, int logits_dtype,
                     const int64_t *target, const float *grad_output, float *loss_rows,
                     float *loss, int32_t *n_valid, int32_t *err_count, void *grad,
                     int grad_dtype, int64_t ldg, void *ws, size_t ws_bytes, void *stream) {
    return fused_fwd_bwd(prob, logits, logits_dtype, target, grad_output, loss_rows, loss, n_valid,
                         err_count, grad, grad_dtype, ldg, ws, ws_bytes,
                         static_cast<hipStream_t>(stream), nullptr, nullptr);
}

int ce_fused_fwd_bwd_noalloc(const ce_problem *prob, const void *logits, int logits_dtype,
                             const int64_t *target, const float *grad_output, float *loss_rows,
                             float *loss, int32_t *n_valid, int32_t *err_count, void *grad,
                             int grad_dtype, int64_t ldg, void *stream) {
    int rc = check_problem(prob);
    if (rc != CE_OK) return rc;
    if (layout(prob, CE_OP_FUSED).total > (size_t)CE_NOALLOC_SCRATCH_BYTES) return CE_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void *ws = nullptr;
    if ((rc = scratch_address(s, &ws)) != CE_OK) return rc;
    return fused_fwd_bwd(prob, logits, logits_dtype, target, grad_output, loss_rows, loss, n_valid,
                         err_count, grad, grad_dtype, ldg, ws, CE_NOALLOC_SCRATCH_BYTES, s,
                         nullptr, nullptr);
}

int ce_fused_fwd_bwd_timed(const ce_problem *prob, const void *logits, int logits_dtype,
                           const int64_t *target, const float *grad_output, float *loss_rows,
                           float *loss, int32_t *n_valid, int32_t *err_count, void *grad,
                           int grad_dtype, int64_t ldg, void *ws, size_t ws_bytes, void *stream,
                           void *ev_start, void *ev_stop) {
    if ((ev_start == nullptr) != (ev_stop == nullptr)) return CE_ERR_ARG;
    return fused_fwd_bwd(prob, logits, logits_dtype, target, grad_output, loss_rows, loss, n_valid,
                         err_count, grad, grad_dtype, ldg, ws, ws_bytes,
                         static_cast<hipStream_t>(stream), static_cast<hipEvent_t>(ev_start),
                         static_cast<hipEvent_t>(ev_stop));
}

size_t ce_linear_workspace_bytes(const ce_linear_problem *prob, int backward) {
    if (check_linear(prob) != CE_OK) return 0;
    return linear_layout(prob, backward != 0).total;
}

int ce_linear_fwd_bwd(const ce_linear_problem *prob, const void *E, const void *C,
                      const int64_t *target, const float *grad_output, float *loss_rows,
                      float *loss, int32_t *n_valid, int32_t *err_count, float *dE, float *dC,
                      void *ws, size_t ws_bytes, void *stream) {
    int rc = check_linear(prob);
    if (rc != CE_OK) return rc;
    const ce_linear_problem &p = *prob;
    if ((dE == nullptr) != (dC == nullptr)) return CE_ERR_NULL;
    const bool bwd = dE != nullptr;
    if (!E || !C || (p.N > 0 && !target)) return CE_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(E) % 16 || reinterpret_cast<uintptr_t>(C) % 16 ||
        reinterpret_cast<uintptr_t>(dE) % 16 || reinterpret_cast<uintptr_t>(dC) % 16)
        return CE_ERR_SHAPE;
    const LinLayout l = linear_layout(prob, bwd);
    if (!ws || ws_bytes < l.total || reinterpret_cast<uintptr_t>(ws) % 256 != 0)
        return CE_ERR_WORKSPACE;
    if (bwd && (overlaps(dE, (size_t)p.N * p.D * 4, E, (size_t)p.N * p.D * 2) ||
                overlaps(dE, (size_t)p.N * p.D * 4, C, (size_t)p.V * p.D * 2) ||
                overlaps(dC, (size_t)p.V * p.D * 4, E, (size_t)p.N * p.D * 2) ||
                overlaps(dC, (size_t)p.V * p.D * 4, C, (size_t)p.V * p.D * 2) ||
                overlaps(dE, (size_t)p.N * p.D * 4, dC, (size_t)p.V * p.D * 4)))
        return CE_ERR_ALIAS;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t N = p.N, D = p.D, V = p.V;

    int32_t *nv = n_valid ? n_valid : at<int32_t>(ws, l.counts);
    VCE_TRY(launch_count(target, N, p.ignore_index, V, nv, err_count, s));
    float *lr = loss_rows ? loss_rows : at<float>(ws, l.loss_rows);
    if (N == 0) {
        if (loss && p.reduction != CE_RED_NONE)
            VCE_TRY(launch_reduce(nullptr, 0, p.reduction, nv, loss, s));
        if (bwd)
            VCE_TRY(launch_zero_f32(dC, V * D, s));
        return CE_OK;
    }
    uint16_t *Ef = at<uint16_t>(ws, l.Ef), *Cf = at<uint16_t>(ws, l.Cf);
    const uint16_t *Eh = static_cast<const uint16_t *>(E), *Ch = static_cast<const uint16_t *>(C);
    uint16_t *ETf = bwd ? at<uint16_t>(ws, l.ETf) : nullptr;
    uint16_t *CTf = bwd ? at<uint16_t>(ws, l.CTf) : nullptr;
    if (bwd) {
        // both operand forms of E from one read; C^T is formed per chunk below
        VCE_TRY(launch_relayout(RelayoutArgs{Eh, N, D, D, ETf, l.Dr, l.Np}, true, s, Ef, l.Dp));
    } else {
        VCE_TRY(launch_relayout(RelayoutArgs{Eh, N, D, D, Ef, l.Np, l.Dp}, false, s));
    }
    VCE_TRY(launch_relayout(RelayoutArgs{Ch, V, D, D, Cf, l.Vp, l.Dp}, false, s));

    // forward: per (256-class tile, row) statistics of the logits, merged
    const bool ls = p.label_smoothing > 0.0f;
    LinTileStats *stats = at<LinTileStats>(ws, l.stats);
    GemmArgs fg{};
    fg.A = Ef;
    fg.B = Cf;
    fg.a_ks = fg.b_ks = l.Dp;
    fg.K = l.Dp;
    fg.M = N;
    fg.N = V;
    fg.tiles_m = (int)(l.Np / 256);
    fg.tiles_n = (int)l.tiles_v;
    fg.target = target;
    fg.col_base = 0;
    fg.stats = stats;
    VCE_TRY(launch_gemm(fg, GEMM_STATS, ls, false, s));

    ce_row_final *fin = at<ce_row_final>(ws, l.fin);
    LinMergeArgs ma{stats, (int)l.tiles_v, N, V, target, p.ignore_index, p.label_smoothing,
                    fin, lr};
    VCE_TRY(launch_linear_merge(ma, s));
    if (loss && p.reduction != CE_RED_NONE)
        VCE_TRY(launch_reduce(lr, N, p.reduction, nv, loss, s));
    if (!bwd) return CE_OK;

    // backward: per class chunk, G and G^T (bf16), then dC rows and dE
    void *rows = at<char>(ws, l.rows);
    LinRowArgs ra{fin, target, nv, grad_output, p.reduction, p.label_smoothing, N, V, rows};
    VCE_TRY(launch_linear_rowconst(ra, s));
    void *G = at<char>(ws, l.G), *GT = at<char>(ws, l.GT);
    float *comp = p.accum == CE_ACC_KAHAN ? at<float>(ws, l.comp) : nullptr;
    const bool filt = p.filter_eps > 0.0f;
    const int64_t tiles_tok = l.Np / 256, tiles_chunk = l.Vc / 256;
    int32_t *flags = filt ? at<int32_t>(ws, l.flags) : nullptr;
    uint16_t *list_e = filt ? at<uint16_t>(ws, l.list_e) : nullptr;
    uint16_t *list_c = filt ? at<uint16_t>(ws, l.list_c) : nullptr;
    int32_t *cnt_e = filt ? at<int32_t>(ws, l.cnt_e) : nullptr;
    int32_t *cnt_c = filt ? at<int32_t>(ws, l.cnt_c) : nullptr;
    for (int64_t c0 = 0; c0 < V; c0 += l.Vc) {
        const int64_t w = std::min(l.Vc, V - c0), wp = round_up(w, 256);
        GemmArgs gg{};
        gg.A = Ef;
        gg.B = reinterpret_cast<const char *>(Cf) + (c0 / 16) * (l.Dp / 32) * 1024;
        gg.a_ks = gg.b_ks = l.Dp;
        gg.K = l.Dp;
        gg.M = N;
        gg.N = w;
        gg.tiles_m = (int)(l.Np / 256);
        gg.tiles_n = (int)(wp / 256);
        gg.col_base = c0;
        gg.rows = rows;
        gg.G = G;
        gg.ldg = wp;
        gg.GT = GT;
        gg.ldgt = l.Np;
        gg.keep_flags = flags;
        gg.filter_eps = p.filter_eps;
        VCE_TRY(launch_gemm(gg, GEMM_GRAD, ls, filt, s));
        if (filt) {
            FilterListArgs fl{flags, tiles_tok, wp / 256, list_e, cnt_e, tiles_chunk,
                              list_c, cnt_c, tiles_tok};
            VCE_TRY(launch_filter_lists(fl, s));
        }

        GemmArgs cg{}; // dC[c0 .. c0 + w) = G^T E
        cg.A = GT;
        cg.B = ETf;
        cg.a_ks = cg.b_ks = l.Np;
        cg.K = l.Np;
        cg.M = w;
        cg.N = D;
        cg.tiles_m = (int)(wp / 256);
        cg.tiles_n = (int)(l.Dr / 256);
        cg.out = dC + c0 * D;
        cg.ldo = D;
        cg.klist = list_c;
        cg.kcnt = cnt_c;
        cg.klist_pitch = tiles_tok;
        VCE_TRY(launch_gemm(cg, GEMM_STORE, false, filt, s));

        // C^T of this chunk's classes, fragment-major (rows D, K the classes)
        VCE_TRY(launch_relayout(RelayoutArgs{Ch + c0 * D, w, D, D, CTf, l.Dr, wp}, true, s));
        GemmArgs eg{}; // dE += G C[c0 .. c0 + w)
        eg.A = G;
        eg.B = CTf;
        eg.a_ks = wp;
        eg.b_ks = wp;
        eg.b_kb0 = 0;
        eg.K = wp;
        eg.M = N;
        eg.N = D;
        eg.tiles_m = (int)(l.Np / 256);
        eg.tiles_n = (int)(l.Dr / 256);
        eg.out = dE;
        eg.ldo = D;
        eg.comp = comp;
        eg.first = c0 == 0;
        eg.klist = list_e;
        eg.kcnt = cnt_e;
        eg.klist_pitch = tiles_chunk;
        VCE_TRY(launch_gemm(eg, comp ? GEMM_KAHAN : GEMM_ADD, false, filt, s));
    }
    return CE_OK;
}

const char *ce_status_str(int status) {
    switch (status) {
    case CE_OK: return "CE_OK";
    case CE_ERR_NULL: return "CE_ERR_NULL: a required pointer is NULL";
    case CE_ERR_SHAPE: return "CE_ERR_SHAPE: invalid or too large shape, stride or vocabulary range";
    case CE_ERR_SMOOTHING: return "CE_ERR_SMOOTHING: label_smoothing must be finite and in [0, 1)";
    case CE_ERR_DTYPE: return "CE_ERR_DTYPE: unknown dtype";
    case CE_ERR_REDUCTION: return "CE_ERR_REDUCTION: unknown reduction";
    case CE_ERR_WORKSPACE: return "CE_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case CE_ERR_SHARDS: return "CE_ERR_SHARDS: n_shards out of range";
    case CE_ERR_ALIAS: return "CE_ERR_ALIAS: grad overlaps logits other than exactly in place";
    case CE_ERR_HIP: return "CE_ERR_HIP: a HIP launch failed";
    case CE_ERR_ARG: return "CE_ERR_ARG: output requested that this call cannot produce";
    default: return "unknown ce_status";
    }
}

int ce_version(void) { return 100; }

} // extern "C"
