// Launch interface between the C ABI (ce_api.hip) and the kernels
// (ce_kernels.hip).  Internal to libvocab_ce.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

#include "vocab_ce.h"

namespace vce {

// ---------------------------------------------------------------------------
// Per-device launch facts, computed once per device (host side).
// ---------------------------------------------------------------------------
constexpr int kMaxDevices = 64;

inline hipError_t current_device(int *dev) {
    hipError_t e = hipGetDevice(dev);
    if (e == hipSuccess && (*dev < 0 || *dev >= kMaxDevices)) e = hipErrorInvalidDevice;
    return e;
}

// Workgroups of `kern` (threads per workgroup, dynamic LDS bytes) the current
// device holds at once: its CUs times the kernel's occupancy per CU; `cache`
// has one entry per device.
inline hipError_t device_slots(const void *kern, int threads, size_t lds, std::atomic<int> *cache,
                               int64_t *slots) {
    int dev = 0;
    hipError_t e = current_device(&dev);
    if (e != hipSuccess) return e;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v <= 0) {
        int cus = 0, per_cu = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, lds);
        if (e != hipSuccess) return e;
        v = std::max(cus, 1) * std::max(per_cu, 1);
        cache[dev].store(v, std::memory_order_relaxed);
    }
    *slots = v;
    return hipSuccess;
}

// Raises `kern`'s dynamic LDS ceiling to `bytes`, once per device.
inline hipError_t raise_lds_once(const void *kern, int bytes, std::atomic<bool> *done) {
    int dev = 0;
    hipError_t e = current_device(&dev);
    if (e != hipSuccess) return e;
    if (done[dev].load(std::memory_order_relaxed)) return hipSuccess;
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess) done[dev].store(true, std::memory_order_relaxed);
    return e;
}


struct FusedArgs {
    const void *logits;
    int64_t ld;
    int64_t V;
    const int64_t *target;
    int64_t ignore_index;
    void *grad;
    int64_t ldg;
    const float *grad_output;
    const int32_t *n_valid;
    float *loss_rows;
    int reduction;
    float eps;
    // smoothing, bf16 rows: e^z per bf16 pattern (kExpTabN entries, the
    // code object's table, exp_table_address), or NULL for fp64 exponentials
    const double *exp_tab = nullptr;
    // count_inline (batches of at most kInlineCountMaxRows rows): each
    // workgroup counts the batch's T targets itself instead of reading
    // n_valid, and workgroup 0 writes the count to count_out and the bad
    // targets to err_out (if not NULL), so no count launch precedes the
    // kernel.  The register-resident kernels only: launch_fused_resident
    // launches the count itself before the LDS-split kernel.
    int count_inline = 0;
    int64_t T = 0;
    int32_t *count_out = nullptr;
    int32_t *err_out = nullptr;
};
// Up to this many rows a workgroup reads every target of the batch (8 KB)
// rather than wait for a count launch.
constexpr int64_t kInlineCountMaxRows = 1024;

struct StatsArgs {
    const void *logits;
    int64_t ld;
    int64_t V_local;     // columns of this call
    int64_t vocab_start; // global column of column 0
    int64_t V_total;
    const int64_t *target;
    int64_t ignore_index;
    int64_t T;
    int nchunks;          // column chunks per row
    int64_t chunk_cols;   // columns per chunk (multiple of the vector width)
    ce_row_stats *out;    // [nchunks][T]
    int smoothing;        // label smoothing on: fp64 sums, and the row sum of z
    const double *exp_tab; // smoothing, bf16 rows: e^z per bf16 pattern (kExpTabN), or NULL
};

// Table of e^z for the bf16 patterns with 2^-16 <= |z| < 2^9, used by the
// smoothed statistics of bf16 rows.  Entry 2 off + sign holds the pattern
// (kExpTabLo + off) | sign << 15, off < kExpTabHalf; the two entries after
// them (off = kExpTabHalf) are NaN: a read clamped to them marks its sum.
// gen_exp_table.py writes the values (its LO and HALF are these constants).
constexpr uint32_t kExpTabLo = 0x3780; // bf16 bits of 2^-16
constexpr int kExpTabHalf = 3200;      // magnitudes up to 2^9
constexpr int kExpTabNaN = 2 * kExpTabHalf;
constexpr int kExpTabN = 2 * kExpTabHalf + 2;

struct MergeArgs {
    const ce_row_stats *in; // [S][T]
    int S;
    int64_t T;
    const int64_t *target;
    int64_t ignore_index;
    int64_t V_total;
    float eps;
    ce_row_stats *stats_out; // merged statistics (or NULL)
    ce_row_final *fin;       // finalize outputs (or NULL)
    float *loss_rows;
    // count: one more workgroup writes the valid-row count and bad-target
    // count of the batch (as launch_count does); 0 leaves them alone
    int count = 0;
    int32_t *n_valid = nullptr;
    int32_t *err_count = nullptr;
};

struct GradArgs {
    const void *logits;
    int64_t ld;
    int64_t V_local;
    int64_t vocab_start;
    int64_t V_total;
    const int64_t *target;
    const ce_row_final *fin;
    const int32_t *n_valid;
    const float *grad_output;
    int reduction;
    float eps;
    void *grad;
    int64_t ldg;
    int nchunks;
    int64_t chunk_cols;
};

// ---- linear classifier (ce_linear.hip) ------------------------------------
constexpr int kLinRowBytes = 48;         // per-row gradient constants
// bytes one backward chunk's G and G^T may take (the chunk is narrowed for
// many tokens: at 8192 tokens, 8192 classes)
constexpr int64_t kLinGBudget = (int64_t)256 << 20;
constexpr int kGemmLdsBytes = 147456;    // 144 KB of the CU's 160 KB
enum { GEMM_STATS = 0, GEMM_GRAD = 1, GEMM_STORE = 2, GEMM_ADD = 3, GEMM_KAHAN = 4 };

// X [R, K] row-major bf16 (stride ld) -> fragment-major Y padded to [Rp, Kp]
// (of X, or of X^T when transposed: then Y's rows are X's columns)
struct RelayoutArgs {
    const uint16_t *X;
    int64_t R, K, ld;
    uint16_t *Y;
    int64_t Rp, Kp;
};

struct LinRowArgs {
    const ce_row_final *fin;
    const int64_t *target;
    const int32_t *n_valid;
    const float *grad_output;
    int reduction;
    float eps;
    int64_t N, V;
    void *rows; // [N] x kLinRowBytes
};

// Statistics of one row over one 256-class tile of the linear classifier's
// logits (fp32, as computed): non-target max m, sum of exp(z - m) over the
// non-target columns, the target logit if the tile holds the target column
// (else 0), and the sum of all its logits (label smoothing; else 0).
struct LinTileStats {
    float m, s, zt, sz;
};

// out[M, N] = A[M, K] B[N, K]^T, A and B fragment-major bf16
struct GemmArgs {
    const void *A, *B;
    int64_t a_ks, b_ks; // stored (padded) K of A and B: the row pitch of the blocks
    int a_kb0, b_kb0;   // first 32-column K block this product reads
    int64_t K;          // K of the product (multiple of 64)
    int64_t M, N;       // valid output rows and columns
    int tiles_m, tiles_n;
    // GEMM_STATS
    const int64_t *target;
    int64_t col_base;   // class of output column 0
    LinTileStats *stats; // [M][tiles_n]
    // GEMM_GRAD
    const void *rows;   // per-row constants [M]
    void *G;            // fragment-major, rows = tokens, K = classes (ldg)
    int64_t ldg;
    void *GT;           // fragment-major, rows = classes, K = tokens (ldgt)
    int64_t ldgt;
    // GEMM_STORE / ADD / KAHAN
    float *out;
    int64_t ldo;
    float *comp;
    int first;
    // gradient filtering: GEMM_GRAD writes one keep flag per wave and tile
    // ([tiles_m][tiles_n][4]) for |G| >= filter_eps |k|; the backward
    // products walk kcnt[tm] K tiles of 256 listed at klist + tm * klist_pitch
    int32_t *keep_flags;
    float filter_eps;
    const uint16_t *klist;
    const int32_t *kcnt;
    int64_t klist_pitch;
};

// lists of kept 256-wide K tiles from the keep flags of one class chunk
struct FilterListArgs {
    const int32_t *flags;  // [tiles_m][tiles_n][4]
    int64_t tiles_m;       // token tiles
    int64_t tiles_n;       // class tiles of the chunk
    uint16_t *list_e;      // [tiles_m][pitch_e] kept class tiles of token tile i
    int32_t *cnt_e;        // [tiles_m]
    int64_t pitch_e;
    uint16_t *list_c;      // [tiles_n][pitch_c] kept token tiles of class tile j
    int32_t *cnt_c;        // [tiles_n]
    int64_t pitch_c;
};

struct LinMergeArgs {
    const LinTileStats *stats; // [N][S]
    int S;
    int64_t N, V;
    const int64_t *target;
    int64_t ignore_index;
    float eps;
    ce_row_final *fin;
    float *loss_rows;
};

hipError_t launch_linear_merge(const LinMergeArgs &a, hipStream_t stream);
// transpose with Yn: also the plain fragment-major form of X into Yn (rows
// padded to a.Kp, K padded to Kn, Kn <= a.Rp), from the same reads of X
hipError_t launch_relayout(const RelayoutArgs &a, bool transpose, hipStream_t stream,
                           uint16_t *Yn = nullptr, int64_t Kn = 0);
hipError_t launch_linear_rowconst(const LinRowArgs &a, hipStream_t stream);
hipError_t launch_gemm(const GemmArgs &g, int epi, bool ls, bool filt, hipStream_t stream);
hipError_t launch_filter_lists(const FilterListArgs &a, hipStream_t stream);
hipError_t launch_zero_f32(float *p, int64_t n, hipStream_t stream);

hipError_t launch_count(const int64_t *target, int64_t T, int64_t ignore_index, int64_t V_total,
                        int32_t *n_valid, int32_t *err_count, hipStream_t stream);
hipError_t launch_reduce(const float *loss_rows, int64_t T, int reduction, const int32_t *n_valid,
                         float *loss, hipStream_t stream);
// Threads x vectors per thread of the row-resident kernel for V columns of
// dtype in_dt, or 0 if the row does not fit in registers.
int resident_threads(int in_dt, int64_t V);
// whether a fused kernel takes rows of V columns (aligned: 16-byte aligned
// rows; smoothing: label smoothing on)
bool fused_fits(int in_dt, int64_t V, bool aligned, bool smoothing);
// whether the row-resident kernel with smoothing sums e^z from the table
// (FusedArgs::exp_tab) for rows of V columns of dtype in_dt
bool fused_table(int in_dt, int64_t V);
hipError_t launch_fused_resident(const FusedArgs &a, int in_dt, int out_dt, int64_t T,
                                 bool aligned, hipStream_t stream);
// vec: 16-byte vectors (rows aligned) rather than single elements
hipError_t launch_stats(const StatsArgs &a, int in_dt, bool vec, hipStream_t stream);
hipError_t launch_merge(const MergeArgs &a, hipStream_t stream);
// device address of the e^z table (kExpTabN entries) on the stream's device
hipError_t exp_table_address(hipStream_t stream, const double **out);
hipError_t launch_grad(const GradArgs &a, int in_dt, int out_dt, bool vec, int64_t T,
                       hipStream_t stream);

} // namespace vce
