// Launch interface between the C ABI (ce_api.hip) and the kernels
// (ce_kernels.hip).  Internal to libvocab_ce.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vocab_ce.h"

namespace vce {

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
};

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
};

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

hipError_t launch_count(const int64_t *target, int64_t T, int64_t ignore_index, int64_t V_total,
                        int32_t *n_valid, int32_t *err_count, hipStream_t stream);
hipError_t launch_reduce(const float *loss_rows, int64_t T, int reduction, const int32_t *n_valid,
                         float *loss, hipStream_t stream);
// Threads x vectors per thread of the row-resident kernel for V columns of
// dtype in_dt, or 0 if the row does not fit in registers.
int resident_threads(int in_dt, int64_t V);
hipError_t launch_fused_resident(const FusedArgs &a, int in_dt, int out_dt, int64_t T,
                                 hipStream_t stream);
// vec: 16-byte vectors (rows aligned) rather than single elements
hipError_t launch_stats(const StatsArgs &a, int in_dt, bool vec, hipStream_t stream);
hipError_t launch_merge(const MergeArgs &a, hipStream_t stream);
hipError_t launch_grad(const GradArgs &a, int in_dt, int out_dt, bool vec, int64_t T,
                       hipStream_t stream);

} // namespace vce
