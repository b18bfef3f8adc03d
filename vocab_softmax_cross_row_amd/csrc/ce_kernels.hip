// Cross-entropy kernels for gfx950 and the C ABI declared in vocab_ce.h.
//
// Paths
//   fused, row resident: one workgroup per row holds the whole row in
//     registers (16-byte vectors, up to 16 per thread), so the logits are
//     read from HBM once and the gradient written once: a max sweep, a
//     sum-of-exponentials sweep, an fp64 finalize by one thread, then the
//     gradient sweep, all from registers (torchtitan PR "[loss] fix softmax
//     collapse with improved ce perf", Memory/perf: one read of the logits,
//     the backward rebuilt in one fused pass).
//   streaming: the stats kernel (one read, online max / sum per thread),
//     the finalize kernel (merge of column-chunk or shard statistics, fp64
//     finalize) and the gradient kernel (one read, one write).  They serve
//     ce_forward / ce_merge_shard_stats / ce_backward, and the fused entry
//     point when the row does not fit in registers, when rows are not
//     16-byte aligned, or when there are too few rows to fill the GPU (then
//     each row is split into column chunks: the split-V grid).
//   count and reduce: N_valid / bad-target counts before the gradient needs
//     them, and the deterministic loss sum.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>

#include "ce_device.h"
#include "ce_launch.h"
#include "vocab_ce.h"

namespace vce {

// ===========================================================================
// count: N_valid and bad targets (one workgroup, any T)
// ===========================================================================
// Each thread issues kPerThread independent target loads per round, so the
// whole batch is in flight at once instead of one round trip per target.
constexpr int kCountThreads = 1024;
constexpr int kPerThread = 16;

__global__ __launch_bounds__(kCountThreads) void k_count(const int64_t *__restrict__ target,
                                                         int64_t T, int64_t ignore_index,
                                                         int64_t V_total, int32_t *n_valid,
                                                         int32_t *err_count) {
    int nv = 0, nb = 0;
    for (int64_t base = 0; base < T; base += (int64_t)kCountThreads * kPerThread) {
        int64_t t[kPerThread];
#pragma unroll
        for (int u = 0; u < kPerThread; ++u) {
            const int64_t r = base + (int64_t)u * kCountThreads + threadIdx.x;
            t[u] = (r < T) ? target[r] : ignore_index;
        }
#pragma unroll
        for (int u = 0; u < kPerThread; ++u) {
            if (t[u] == ignore_index) continue;
            if (t[u] >= 0 && t[u] < V_total)
                ++nv;
            else
                ++nb;
        }
    }
    nv = wave_sum(nv);
    nb = wave_sum(nb);
    __shared__ int part[2][kCountThreads / kWave];
    const int wv = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) {
        part[0][wv] = nv;
        part[1][wv] = nb;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int x = 0, y = 0;
        for (int i = 0; i < kCountThreads / kWave; ++i) {
            x += part[0][i];
            y += part[1][i];
        }
        if (n_valid) *n_valid = x;
        if (err_count) *err_count = y;
    }
}

// ===========================================================================
// reduce: loss = sum of loss_rows (fp64, fixed order), / N_valid for mean
// ===========================================================================
constexpr int kReduceThreads = 1024;

__global__ __launch_bounds__(kReduceThreads) void k_reduce(const float *__restrict__ loss_rows,
                                                           int64_t T, int reduction,
                                                           const int32_t *n_valid, float *loss) {
    __shared__ BlockRed<kReduceThreads> red;
    double acc = 0.0;
    for (int64_t base = 0; base < T; base += (int64_t)kReduceThreads * kPerThread) {
        float x[kPerThread];
#pragma unroll
        for (int u = 0; u < kPerThread; ++u) {
            const int64_t r = base + (int64_t)u * kReduceThreads + threadIdx.x;
            x[u] = (r < T) ? loss_rows[r] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kPerThread; ++u) acc += (double)x[u];
    }
    acc = block_sum_d(acc, red, 0);
    if (threadIdx.x == 0) {
        if (reduction == CE_RED_MEAN) acc /= (double)(*n_valid);
        *loss = (float)acc;
    }
}

// ===========================================================================
// fused, row resident
// ===========================================================================

// One workgroup per row; the row lives in registers from its load to its
// gradient store.  FAST = bf16 gradient without smoothing: fp32 finalize
// and the biased exponent form (see GradConst); otherwise fp64 finalize.
template <int IN, int OUT, int THREADS, int NV, bool LS>
__global__ __launch_bounds__(THREADS) void k_fused_resident(FusedArgs a) {
    using In = Elem<IN>;
    constexpr int EPV = In::kVec;
    using Ch = Chunk<IN, EPV>;
    using St = Store<OUT, EPV, true>;
    constexpr int kOutSize = (OUT == CE_BF16) ? 2 : 4;
    constexpr bool FAST = (OUT == CE_BF16) && !LS;

    __shared__ BlockRed<THREADS> red;
    __shared__ GradConst gc_sh;

    const int tid = threadIdx.x;
    const int64_t row = xcd_major(blockIdx.x, gridDim.x);
    const int V = (int)a.V;
    const int nvec = V / EPV;
    const int tail0 = nvec * EPV;
    const int ntail = V - tail0;
    const char *zrow = static_cast<const char *>(a.logits) + row * a.ld * In::kSize;
    char *grow = static_cast<char *>(a.grad) + row * a.ldg * kOutSize;

    const int64_t t64 = a.target[row];
    if (t64 == a.ignore_index || t64 < 0 || t64 >= V) {
        // ignored row or bad target: zero gradient, no reads of the row
        float zero[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) zero[e] = 0.0f;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int vi = i * THREADS + tid;
            if (vi < nvec) St::put(grow + vi * EPV * kOutSize, zero);
        }
        if (tid < ntail) Store<OUT, 1>::put(grow + (tail0 + tid) * kOutSize, zero);
        if (tid == 0) a.loss_rows[row] = (t64 == a.ignore_index) ? 0.0f : __builtin_nanf("");
        return;
    }
    const int t = (int)t64;

    // ---- load the row into registers (streamed: read once) ----------------
    Ch v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int vi = i * THREADS + tid;
        if (vi < nvec)
            v[i].template load<true>(zrow + vi * EPV * In::kSize);
        else
            v[i].fill_ninf();
    }
    float ztail = ninf();
    if (tid < ntail) ztail = In::load1(zrow + (tail0 + tid) * In::kSize);

    // where the target sits: vector tv = slot t_slot of thread t_thread
    // (wave t_wave), element te; or the scalar tail.  t is the same for the
    // whole workgroup, and readfirstlane makes the slot and wave tests
    // scalar branches, so only the owner wave does any work for it.
    const int tv = t / EPV;
    const int te = __builtin_amdgcn_readfirstlane(t - tv * EPV);
    const bool t_in_vec = t < tail0;
    const int t_slot = __builtin_amdgcn_readfirstlane(t_in_vec ? tv / THREADS : -1);
    const int t_thread = tv - (tv / THREADS) * THREADS;
    const int t_wave = __builtin_amdgcn_readfirstlane(t_thread / kWave);
    const int my_wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const bool t_wave_mine = t_in_vec && my_wave == t_wave;
    const bool t_lane_mine = (tid & (kWave - 1)) == (t_thread & (kWave - 1));

    // ---- sum of the whole row (smoothing only), before the target is masked
    double sz = 0.0;
    if constexpr (LS) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int vi = i * THREADS + tid;
            float p[EPV];
#pragma unroll
            for (int e = 0; e < EPV; ++e) p[e] = v[i].get(e);
#pragma unroll
            for (int h = EPV / 2; h > 0; h >>= 1)
#pragma unroll
                for (int e = 0; e < h; ++e) p[e] += p[e + h];
            sz += (vi < nvec) ? (double)p[0] : 0.0;
        }
        if (tid < ntail) sz += (double)ztail;
    }

    // ---- drop the target before any reduction ------------------------------
    if (t_wave_mine) {
#pragma unroll
        for (int i = 0; i < NV; ++i)
            if (i == t_slot && t_lane_mine) v[i].kill(te);
    }
    if (!t_in_vec && tid == t - tail0) ztail = ninf();

#pragma unroll
    for (int i = 0; i < NV; ++i) v[i].fence();

    // ---- non-target max ---------------------------------------------------
    float mx = ztail;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int e = 0; e < EPV; ++e) mx = fmaxf(mx, v[i].get(e));
    mx = block_max<THREADS>(mx, red, 0);
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i].fence();

    // ---- non-target sum of exponentials ----------------------------------
    double sd = 0.0;
    float s = 0.0f;
    if constexpr (LS) {
        // With smoothing the gradient k (p_j - eps/V) cancels where p_j is
        // close to eps/V and magnifies any error of lse there, so the sum is
        // taken with fp64 exponentials and fp64 accumulation.
        if (mx != ninf()) {
            const double md = (double)mx;
#pragma unroll
            for (int i = 0; i < NV; ++i)
#pragma unroll
                for (int e = 0; e < EPV; ++e) sd += exp_nonpos((double)v[i].get(e) - md);
            sd += exp_nonpos((double)ztail - md);
        }
        sd = block_sum_d<THREADS>(sd, red, 0);
        sz = block_sum_d<THREADS>(sz, red, 1);
    } else {
        if (mx != ninf()) {
            const float K = mx * kL2E;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                float p[EPV];
#pragma unroll
                for (int e = 0; e < EPV; ++e) p[e] = fast_exp2(fmaf(v[i].get(e), kL2E, -K));
#pragma unroll
                for (int h = EPV / 2; h > 0; h >>= 1)
#pragma unroll
                    for (int e = 0; e < h; ++e) p[e] += p[e + h];
                s += p[0];
            }
            s += fast_exp2(fmaf(ztail, kL2E, -K));
        }
        s = block_sum<THREADS>(s, red, 1);
        if (mx != ninf()) {
            // the terms were 2^(z kL2E - K) with K = fl(mx kL2E): undo the
            // rounding of K (the residual is exact)
            const float K = mx * kL2E;
            s *= fast_exp2(-fmaf(mx, kL2E, -K));
        }
        sd = (double)s;
    }

    // ---- finalize (one thread) -----------------------------------------------
    if (tid == 0) {
        const float zt = In::load1(zrow + (int64_t)t * In::kSize);
        const double k = row_scale(a.reduction, a.grad_output, a.n_valid, row);
        if constexpr (FAST) {
            const FastFinal f = finalize_fast(mx, s, zt, k);
            a.loss_rows[row] = f.loss;
            GradConst c;
            c.cb = f.cb;
            c.scale = f.scale;
            c.gk = f.gk;
            c.ch = c.cl = c.k = c.ku = c.lu = c.d2hi = c.d2lo = 0.0f;
            gc_sh = c;
        } else {
            const RowFinal f =
                finalize_row((double)mx, sd, (double)zt, sz, (double)V, (double)a.eps);
            a.loss_rows[row] = (float)f.loss;
            gc_sh = grad_constants(f.lse, f.gt, k, (double)a.eps, (double)V);
        }
    }
    __syncthreads();
    const GradConst c = gc_sh;
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i].fence();

    // ---- gradient sweep from registers ------------------------------------
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int vi = i * THREADS + tid;
        float g[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) g[e] = grad_elem<OUT, LS>(v[i].get(e), c);
        if (t_wave_mine && i == t_slot) {
            if (t_lane_mine) {
#pragma unroll
                for (int e = 0; e < EPV; ++e)
                    if (e == te) g[e] = c.gk;
            }
        }
        if (vi < nvec) St::put(grow + vi * EPV * kOutSize, g);
    }
    if (tid < ntail) {
        const float g = (!t_in_vec && tid == t - tail0) ? c.gk : grad_elem<OUT, LS>(ztail, c);
        Store<OUT, 1>::put(grow + (tail0 + tid) * kOutSize, &g);
    }
}

// ===========================================================================
// fused, row split between registers and LDS, two workgroups per CU
// ===========================================================================
// For rows of more than 8192 16-byte vectors (V > 65536 bf16) a register-
// resident row needs 1024 threads and fills the register file, so each CU
// holds one row and its barriers, finalize and exponentials cannot overlap
// another row's memory traffic.  Here a 512-thread workgroup keeps NR
// vectors per lane in registers and the rest of the row in LDS (filled by
// direct buffer->LDS loads), and two workgroups share a CU.  Buffer
// addressing keeps every slot at one VGPR offset; the SGPR slot offset is
// not covered by the buffer range check, so every possibly partial slot is
// guarded explicitly.
constexpr int kLdsThreads = 512;
constexpr int kLdsRegSlots = 22;
constexpr int kBufNT = 2; // buffer cache policy: non-temporal
typedef __attribute__((address_space(3))) void lds_void_t;

template <int IN, int OUT, int NR>
__global__ __launch_bounds__(kLdsThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
void k_fused_lds(FusedArgs a) {
    using In = Elem<IN>;
    constexpr int TH = kLdsThreads;
    constexpr int EPV = In::kVec;
    using Ch = Chunk<IN, EPV>;
    constexpr int kOutSize = (OUT == CE_BF16) ? 2 : 4;
    constexpr int kOutVec = EPV * kOutSize; // bytes of one gradient vector
    constexpr bool FAST = (OUT == CE_BF16);
    extern __shared__ u32x4 lbuf[];
    __shared__ BlockRed<TH> red;
    __shared__ GradConst gc_sh;

    const int tid = threadIdx.x;
    const int64_t row = xcd_major(blockIdx.x, gridDim.x);
    const int V = (int)a.V;
    const int nvec = V / EPV;
    const int tail0 = nvec * EPV;
    const int ntail = V - tail0;
    const int nl = (nvec - NR * TH + TH - 1) / TH; // LDS slots (last one partial)
    const char *zrow = static_cast<const char *>(a.logits) + row * a.ld * In::kSize;
    char *grow = static_cast<char *>(a.grad) + row * a.ldg * kOutSize;
    const __amdgpu_buffer_rsrc_t rin =
        __builtin_amdgcn_make_buffer_rsrc((void *)zrow, 0, tail0 * In::kSize, 0x00020000);
    const __amdgpu_buffer_rsrc_t rout =
        __builtin_amdgcn_make_buffer_rsrc((void *)grow, 0, tail0 * kOutSize, 0x00020000);
    const int voff = tid * 16;
    const int goff = tid * kOutVec;

    auto put = [&](int slot, const float *g) {
        if (slot * TH + tid >= nvec) return;
        if constexpr (OUT == CE_BF16 && EPV == 8) {
            u32x4 o;
#pragma unroll
            for (int k = 0; k < 4; ++k) o[k] = pack_bf16x2(g[2 * k], g[2 * k + 1]);
            __builtin_amdgcn_raw_buffer_store_b128(o, rout, goff, slot * TH * kOutVec, kBufNT);
        } else if constexpr (OUT == CE_F32 && EPV == 4) {
            u32x4 o;
#pragma unroll
            for (int k = 0; k < 4; ++k) o[k] = __float_as_uint(g[k]);
            __builtin_amdgcn_raw_buffer_store_b128(o, rout, goff, slot * TH * kOutVec, kBufNT);
        } else {
            Store<OUT, EPV, true>::put(grow + (int64_t)(slot * TH + tid) * kOutVec, g);
        }
    };

    const int64_t t64 = a.target[row];
    if (t64 == a.ignore_index || t64 < 0 || t64 >= V) {
        float zero[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) zero[e] = 0.0f;
#pragma unroll
        for (int i = 0; i < NR; ++i) put(i, zero);
        for (int q = 0; q < nl; ++q) put(NR + q, zero);
        if (tid < ntail) Store<OUT, 1>::put(grow + (tail0 + tid) * kOutSize, zero);
        if (tid == 0) a.loss_rows[row] = (t64 == a.ignore_index) ? 0.0f : __builtin_nanf("");
        return;
    }
    const int t = (int)t64;

    // ---- loads: register slots first (needed first), then the LDS part.
    // While a wave issues memory instructions it runs at raised priority, so
    // the other workgroup's arithmetic on this CU does not delay the requests.
    __builtin_amdgcn_s_setprio(1);
    Ch v[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        if (i * TH + tid < nvec)
            v[i].v = __builtin_amdgcn_raw_buffer_load_b128(rin, voff, i * TH * 16, kBufNT);
        else
            v[i].fill_ninf();
    }
    const int wave_base = __builtin_amdgcn_readfirstlane((tid / kWave) * kWave);
    for (int q = 0; q < nl; ++q)
        if ((NR + q) * TH + tid < nvec)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rin, (lds_void_t *)(lbuf + q * TH + wave_base),
                                                     16, voff, (NR + q) * TH * 16, 0, kBufNT);
    float ztail = ninf();
    if (tid < ntail) ztail = In::load1(zrow + (tail0 + tid) * In::kSize);
    __builtin_amdgcn_s_setprio(0);

    // ---- target location (wave-uniform tests; see k_fused_resident) ----------
    const int tv = t / EPV;
    const int te = __builtin_amdgcn_readfirstlane(t - tv * EPV);
    const bool t_in_vec = t < tail0;
    const int t_slot = __builtin_amdgcn_readfirstlane(t_in_vec ? tv / TH : -1);
    const int t_thread = tv - (tv / TH) * TH;
    const int t_wave = __builtin_amdgcn_readfirstlane(t_thread / kWave);
    const int my_wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const bool t_wave_mine = t_in_vec && my_wave == t_wave;
    const bool t_lane_mine = (tid & (kWave - 1)) == (t_thread & (kWave - 1));

    if (t_wave_mine) {
#pragma unroll
        for (int i = 0; i < NR; ++i)
            if (i == t_slot && t_lane_mine) v[i].kill(te);
    }
    if (!t_in_vec && tid == t - tail0) ztail = ninf();
#pragma unroll
    for (int i = 0; i < NR; ++i) v[i].fence();

    // ---- non-target max: registers, then (once this wave's LDS part has
    // landed) the LDS slots; each lane reads back only what it loaded ----
    float mx = ztail;
#pragma unroll
    for (int i = 0; i < NR; ++i)
#pragma unroll
        for (int e = 0; e < EPV; ++e) mx = fmaxf(mx, v[i].get(e));
    __builtin_amdgcn_s_waitcnt(0);
    if (t_wave_mine && t_slot >= NR && t_lane_mine) {
        Ch w;
        w.v = lbuf[(t_slot - NR) * TH + tid];
        w.kill(te);
        lbuf[(t_slot - NR) * TH + tid] = w.v;
    }
    auto lds_vec = [&](int q) {
        Ch w;
        if ((NR + q) * TH + tid < nvec)
            w.v = lbuf[q * TH + tid];
        else
            w.fill_ninf();
        return w;
    };
#pragma unroll 1
    for (int q = 0; q < nl; ++q) {
        const Ch w = lds_vec(q);
#pragma unroll
        for (int e = 0; e < EPV; ++e) mx = fmaxf(mx, w.get(e));
    }
    mx = block_max<TH>(mx, red, 0);
#pragma unroll
    for (int i = 0; i < NR; ++i) v[i].fence();

    // ---- non-target sum of exponentials ----------------------------------
    float s = 0.0f;
    if (mx != ninf()) {
        const float K = mx * kL2E;
        auto sumvec = [&](const Ch &w) {
            float p[EPV];
#pragma unroll
            for (int e = 0; e < EPV; ++e) p[e] = fast_exp2(fmaf(w.get(e), kL2E, -K));
#pragma unroll
            for (int h = EPV / 2; h > 0; h >>= 1)
#pragma unroll
                for (int e = 0; e < h; ++e) p[e] += p[e + h];
            s += p[0];
        };
#pragma unroll
        for (int i = 0; i < NR; ++i) sumvec(v[i]);
#pragma unroll 1
        for (int q = 0; q < nl; ++q) sumvec(lds_vec(q));
        s += fast_exp2(fmaf(ztail, kL2E, -K));
    }
    s = block_sum<TH>(s, red, 1);
    if (mx != ninf()) {
        const float K = mx * kL2E;
        s *= fast_exp2(-fmaf(mx, kL2E, -K));
    }

    // ---- finalize (one thread) ---------------------------------------------
    if (tid == 0) {
        const float zt = In::load1(zrow + (int64_t)t * In::kSize);
        const double k = row_scale(a.reduction, a.grad_output, a.n_valid, row);
        if constexpr (FAST) {
            const FastFinal f = finalize_fast(mx, s, zt, k);
            a.loss_rows[row] = f.loss;
            GradConst c;
            c.cb = f.cb;
            c.scale = f.scale;
            c.gk = f.gk;
            c.ch = c.cl = c.k = c.ku = c.lu = c.d2hi = c.d2lo = 0.0f;
            gc_sh = c;
        } else {
            const RowFinal f = finalize_row((double)mx, (double)s, (double)zt, 0.0, (double)V, 0.0);
            a.loss_rows[row] = (float)f.loss;
            gc_sh = grad_constants(f.lse, f.gt, k, 0.0, (double)V);
        }
    }
    __syncthreads();
    const GradConst c = gc_sh;
#pragma unroll
    for (int i = 0; i < NR; ++i) v[i].fence();

    // ---- gradient sweep -----------------------------------------------------
    auto gradvec = [&](const Ch &w, int slot) {
        float g[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) g[e] = grad_elem<OUT, false>(w.get(e), c);
        if (t_wave_mine && slot == t_slot) {
            if (t_lane_mine) {
#pragma unroll
                for (int e = 0; e < EPV; ++e)
                    if (e == te) g[e] = c.gk;
            }
        }
        put(slot, g);
    };
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < NR; ++i) gradvec(v[i], i);
#pragma unroll 1
    for (int q = 0; q < nl; ++q) gradvec(lds_vec(q), NR + q);
    if (tid < ntail) {
        const float g = (!t_in_vec && tid == t - tail0) ? c.gk : grad_elem<OUT, false>(ztail, c);
        Store<OUT, 1>::put(grow + (tail0 + tid) * kOutSize, &g);
    }
}

// ===========================================================================
// streaming stats: one workgroup per (row, column chunk)
// ===========================================================================

// Per-thread online (max, sum of exponentials).  The fast form keeps the sum
// in fp32 relative to K = fl(m kL2E); the precise form (label smoothing,
// where the gradient needs lse to ~1e-12) uses fp64 exponentials and sums.
template <bool PRECISE>
struct Online;

template <>
struct Online<false> {
    float m = -__builtin_inff(), K = -__builtin_inff(), s = 0.0f;
    __device__ __forceinline__ void rescale(float vm) {
        if (vm > m) {
            const float K2 = vm * kL2E;
            s = (m == ninf()) ? 0.0f : s * fast_exp2(K - K2);
            m = vm;
            K = K2;
        }
    }
    __device__ __forceinline__ float term(float z) const { return fast_exp2(fmaf(z, kL2E, -K)); }
    __device__ __forceinline__ void add(float t) { s += t; }
    __device__ __forceinline__ MaxSum result() const {
        if (m == ninf()) return {m, 0.0};
        // undo the rounding of K (the residual is exact)
        return {m, (double)s * exp2(-(double)fmaf(m, kL2E, -K))};
    }
};

template <>
struct Online<true> {
    float m = -__builtin_inff();
    double md = -__builtin_inf(), s = 0.0;
    __device__ __forceinline__ void rescale(float vm) {
        if (vm > m) {
            s = (m == ninf()) ? 0.0 : s * exp_nonpos(md - (double)vm);
            m = vm;
            md = (double)vm;
        }
    }
    __device__ __forceinline__ double term(float z) const { return exp_nonpos((double)z - md); }
    __device__ __forceinline__ void add(double t) { s += t; }
    __device__ __forceinline__ MaxSum result() const { return {m, s}; }
};

// Online (max, sum of exponentials) of the columns [c0, c1) of one row with
// column tc (if in range) left out, and the sum of all of them (smoothing);
// every thread of the workgroup calls it and gets the workgroup's result.
template <int IN, int EPV, int THREADS, int UNROLL, bool LS>
__device__ __forceinline__ void stats_online(const char *zrow, int64_t c0, int64_t c1,
                                             int64_t tc, BlockRed<THREADS> &red, MaxSum &ms_out,
                                             double &sz_out) {
    using In = Elem<IN>;
    using Ch = Chunk<IN, EPV>;
    const int tid = threadIdx.x;
    const int64_t nv = (c1 - c0) / EPV; // full vectors of this chunk
    const int64_t tail0 = c0 + nv * EPV;
    Online<LS> acc;
    double sz = 0.0;
    for (int64_t base = 0; base < nv; base += (int64_t)UNROLL * THREADS) {
        Ch v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int64_t vi = base + (int64_t)u * THREADS + tid;
            if (vi < nv)
                v[u].load(zrow + (c0 + vi * EPV) * In::kSize);
            else
                v[u].fill_ninf();
        }
        // one rescale per UNROLL vectors: the max of the whole group first;
        // the target test is uniform over the group's column span first
        const bool t_here = tc >= c0 + base * EPV && tc < c0 + (base + (int64_t)UNROLL * THREADS) * EPV;
        float vm = ninf();
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int64_t vi = base + (int64_t)u * THREADS + tid;
            const int64_t col = c0 + vi * EPV;
            if (LS && vi < nv) {
                float p[EPV];
#pragma unroll
                for (int e = 0; e < EPV; ++e) p[e] = v[u].get(e);
#pragma unroll
                for (int h = EPV / 2; h > 0; h >>= 1)
#pragma unroll
                    for (int e = 0; e < h; ++e) p[e] += p[e + h];
                sz += (double)p[0];
            }
            if (t_here && tc >= col && tc < col + EPV) v[u].kill((int)(tc - col));
#pragma unroll
            for (int e = 0; e < EPV; ++e) vm = fmaxf(vm, v[u].get(e));
        }
        acc.rescale(vm);
        if (acc.m != ninf()) {
#pragma unroll
            for (int u = 0; u < UNROLL; ++u)
#pragma unroll
                for (int e = 0; e < EPV; ++e) acc.add(acc.term(v[u].get(e)));
        }
    }
    // scalar tail of the chunk
    for (int64_t col = tail0 + tid; col < c1; col += THREADS) {
        float z = In::load1(zrow + col * In::kSize);
        if (LS) sz += (double)z;
        if (col == tc) z = ninf();
        acc.rescale(z);
        if (acc.m != ninf()) acc.add(acc.term(z));
    }
    const MaxSum ms = block_combine<THREADS>(acc.result(), red);
    if (LS) sz = block_sum_d<THREADS>(sz, red, 1);
    ms_out = ms;
    sz_out = sz;
}

template <int IN, int EPV, int THREADS, int UNROLL, bool LS>
__global__ __launch_bounds__(THREADS) void k_stats(StatsArgs a) {
    using In = Elem<IN>;
    using Ch = Chunk<IN, EPV>;
    __shared__ BlockRed<THREADS> red;

    const int tid = threadIdx.x;
    const int64_t unit = xcd_major(blockIdx.x, gridDim.x);
    const int64_t row = unit / a.nchunks;
    const int ch = (int)(unit % a.nchunks);
    const int64_t c0 = (int64_t)ch * a.chunk_cols;
    const int64_t c1 = std::min(a.V_local, c0 + a.chunk_cols);
    const int64_t t = a.target[row];
    ce_row_stats *o = a.out + (int64_t)ch * a.T + row;

    if (t == a.ignore_index || t < 0 || t >= a.V_total) {
        // no row statistics are needed: the row is ignored or an error
        if (tid == 0) {
            ce_row_stats z;
            z.m = ninf();
            z.zt = 0.0f;
            z.own = 0;
            z.reserved = 0;
            z.s = 0.0;
            z.sz = 0.0;
            *o = z;
        }
        return;
    }
    const int64_t tl = t - a.vocab_start; // target column in this call
    const int64_t tc = (tl >= c0 && tl < c1) ? tl : -1;

    const char *zrow = static_cast<const char *>(a.logits) + row * a.ld * In::kSize;
    MaxSum ms;
    double sz;
    stats_online<IN, EPV, THREADS, UNROLL, LS>(zrow, c0, c1, tc, red, ms, sz);
    if (tid == 0) {
        ce_row_stats r;
        r.m = ms.m;
        r.zt = (tc >= 0) ? In::load1(zrow + tc * In::kSize) : 0.0f;
        r.own = (tc >= 0) ? 1 : 0;
        r.reserved = 0;
        r.s = ms.s;
        r.sz = sz;
        *o = r;
    }
}

// ===========================================================================
// smoothed statistics of bf16 rows from a table of e^z
// ===========================================================================
// With smoothing the row sum must be fp64-exact (the gradient k (p - eps/V)
// cancels near p = eps/V).  A bf16 logit is one of 65536 values; those with
// 2^-16 <= |z| < 2^9 are 2 x 3200 bit patterns, whose e^z (fp64, from the
// math library) make a 50 KB table in LDS.  The row sum is taken unshifted,
// sum_j e^{z_j} (fp64 spans e^{-512} .. e^{512}), and scaled by e^{-m} at
// the end: one LDS read and one fp64 add per element instead of an fp64
// exponential.  The target and -inf logits read the table's zero entry.
// |z| < 2^-16 takes e^z = 1 + z + z^2/2 (error below 1e-15); a chunk with
// |z| >= 512, +inf or NaN is recomputed with the online form.

__global__ __launch_bounds__(256) void k_exp_table(double *tab) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= kExpTabN) return;
    if (i == kExpTabZero) {
        tab[i] = 0.0;
        return;
    }
    const uint32_t b = (kExpTabLo + (uint32_t)(i % kExpTabHalf)) | (i >= kExpTabHalf ? 0x8000u : 0u);
    tab[i] = exp((double)__uint_as_float(b << 16));
}

template <int THREADS, int UNROLL>
__global__ __launch_bounds__(THREADS) void k_stats_tab(StatsArgs a, const double *tab_g) {
    using Ch = Chunk<CE_BF16, 8>;
    __shared__ BlockRed<THREADS> red;
    __shared__ double tab[kExpTabN];

    const int tid = threadIdx.x;
    const int64_t unit = xcd_major(blockIdx.x, gridDim.x);
    const int64_t row = unit / a.nchunks;
    const int ch = (int)(unit % a.nchunks);
    const int64_t c0 = (int64_t)ch * a.chunk_cols;
    const int64_t c1 = std::min(a.V_local, c0 + a.chunk_cols);
    const int64_t t = a.target[row];
    ce_row_stats *o = a.out + (int64_t)ch * a.T + row;

    if (t == a.ignore_index || t < 0 || t >= a.V_total) {
        if (tid == 0) {
            ce_row_stats z;
            z.m = ninf();
            z.zt = 0.0f;
            z.own = 0;
            z.reserved = 0;
            z.s = 0.0;
            z.sz = 0.0;
            *o = z;
        }
        return;
    }
    for (int i = tid; i < kExpTabN; i += THREADS) tab[i] = tab_g[i];
    const int64_t tl = t - a.vocab_start;
    const int64_t tc = (tl >= c0 && tl < c1) ? tl : -1;
    const char *zrow = static_cast<const char *>(a.logits) + row * a.ld * 2;
    const int64_t nv = (c1 - c0) / 8;
    const int64_t tail0 = c0 + nv * 8;
    __syncthreads();

    // table index of one bf16 pattern; sets *rare when it is outside the table
    // (the zero entry is read then, and the rare path below corrects it)
    auto index = [&](uint32_t b, bool &rare) {
        const uint32_t off = (b & 0x7fffu) - kExpTabLo;
        const bool in = off < (uint32_t)kExpTabHalf;
        rare |= !in;
        return in ? (int)(off + (b >> 15) * kExpTabHalf) : kExpTabZero;
    };
    // the exact term of a pattern outside the table, and whether the online
    // form is needed instead
    auto rare_term = [&](uint32_t b, bool &redo) {
        const uint32_t mag = b & 0x7fffu;
        if (b == 0xff80u) return 0.0;                    // -inf (or the target)
        if (mag < kExpTabLo) {                           // |z| < 2^-16, or 0
            const double z = (double)__uint_as_float(b << 16);
            return 1.0 + z * (1.0 + 0.5 * z);
        }
        if (mag < (uint32_t)(kExpTabLo + kExpTabHalf)) return 0.0; // in the table
        redo = true;                                     // |z| >= 512, +inf, NaN
        return 0.0;
    };

    double s = 0.0, sz = 0.0;
    float mx = ninf();
    bool redo = false;
    // One vector of 8 logits.  The common path adds the table entries of all
    // 8 and takes their max; a vector with a pattern outside the table, or
    // holding the target, is redone element by element (the target left out).
    auto vec = [&](const Ch &v, int64_t col) {
        float zf[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) zf[e] = v.get(e);
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = zf[e];
#pragma unroll
        for (int hh = 4; hh > 0; hh >>= 1)
#pragma unroll
            for (int e = 0; e < hh; ++e) p[e] += p[e + hh];
        sz += (double)p[0];
        bool rare = tc >= col && tc < col + 8;
        double sv = 0.0;
        float vm = zf[0];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (e) vm = fmaxf(vm, zf[e]);
            const uint32_t w = v.v[e >> 1];
            sv += tab[index((e & 1) ? (w >> 16) : (w & 0xffffu), rare)];
        }
        if (__builtin_expect(rare, 0)) {
            sv = 0.0;
            vm = ninf();
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if (col + e == tc) continue;
                const uint32_t w = v.v[e >> 1];
                const uint32_t b = (e & 1) ? (w >> 16) : (w & 0xffffu);
                bool r2 = false;
                const double tv = tab[index(b, r2)];
                sv += r2 ? rare_term(b, redo) : tv;
                vm = fmaxf(vm, zf[e]);
            }
        }
        s += sv;
        mx = fmaxf(mx, vm);
    };
    const int64_t step = (int64_t)UNROLL * THREADS;
    const int64_t nfull = nv / step * step; // vectors covered by whole iterations
    // the next group's loads are issued before the current group's work
    Ch va[UNROLL], vb[UNROLL];
    auto load_group = [&](Ch *v, int64_t base) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
            v[u].load(zrow + (c0 + (base + (int64_t)u * THREADS + tid) * 8) * 2);
    };
    auto work_group = [&](Ch *v, int64_t base) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) vec(v[u], c0 + (base + (int64_t)u * THREADS + tid) * 8);
    };
    if (nfull > 0) load_group(va, 0);
    for (int64_t base = 0; base < nfull; base += 2 * step) {
        if (base + step < nfull) load_group(vb, base + step);
        work_group(va, base);
        if (base + step < nfull) {
            if (base + 2 * step < nfull) load_group(va, base + 2 * step);
            work_group(vb, base + step);
        }
    }
    for (int64_t vi = nfull + tid; vi < nv; vi += THREADS) {
        Ch v;
        v.load(zrow + (c0 + vi * 8) * 2);
        vec(v, c0 + vi * 8);
    }
    // scalar tail of the chunk
    for (int64_t col = tail0 + tid; col < c1; col += THREADS) {
        const uint32_t b = *reinterpret_cast<const uint16_t *>(zrow + col * 2);
        const float z = __uint_as_float(b << 16);
        sz += (double)z;
        if (col == tc) continue;
        mx = fmaxf(mx, z);
        bool rare = false;
        const double tv = tab[index(b, rare)];
        s += rare ? rare_term(b, redo) : tv;
    }
    // a thread that saw |z| >= 512, +inf or NaN sends the chunk to the online form
    const float redo_all = block_max<THREADS>(redo ? 1.0f : 0.0f, red, 0);
    MaxSum ms;
    if (redo_all > 0.0f) {
        __syncthreads();
        stats_online<CE_BF16, 8, THREADS, UNROLL, true>(zrow, c0, c1, tc, red, ms, sz);
    } else {
        const float M = block_max<THREADS>(mx, red, 1);
        __syncthreads();
        const double S = block_sum_d<THREADS>(s, red, 0);
        sz = block_sum_d<THREADS>(sz, red, 1);
        // e^{-M}: -M is a bf16 value (M is a max of bf16 values)
        double scale = 0.0;
        if (M != ninf()) {
            const uint32_t mb = (__float_as_uint(M) >> 16) ^ 0x8000u;
            bool rare = false;
            bool unused = false;
            const double tv = tab[index(mb, rare)];
            scale = rare ? rare_term(mb, unused) : tv;
        }
        ms.m = M;
        ms.s = (M == ninf()) ? 0.0 : S * scale;
    }
    if (tid == 0) {
        ce_row_stats r;
        r.m = ms.m;
        r.zt = (tc >= 0) ? __uint_as_float((uint32_t)(*reinterpret_cast<const uint16_t *>(zrow + tc * 2)) << 16) : 0.0f;
        r.own = (tc >= 0) ? 1 : 0;
        r.reserved = 0;
        r.s = ms.s;
        r.sz = sz;
        *o = r;
    }
}

// ===========================================================================
// merge of partial statistics ([S][T], in order) + optional finalize
// ===========================================================================

constexpr int kMergeThreads = 256;

__global__ __launch_bounds__(kMergeThreads) void k_merge(MergeArgs a) {
    const int64_t r = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
    if (r >= a.T) return;
    double M = -__builtin_inf();
    for (int k = 0; k < a.S; ++k) M = fmax(M, (double)a.in[(int64_t)k * a.T + r].m);
    double s = 0.0, zt = 0.0, sz = 0.0;
    int own = 0;
    for (int k = 0; k < a.S; ++k) {
        const ce_row_stats p = a.in[(int64_t)k * a.T + r];
        if (p.m != ninf()) s += p.s * exp((double)p.m - M);
        zt += (double)p.zt;
        own += p.own;
        sz += p.sz;
    }
    if (a.stats_out) {
        ce_row_stats o;
        o.m = (float)M;
        o.zt = (float)zt;
        o.own = own;
        o.reserved = 0;
        o.s = s;
        o.sz = sz;
        a.stats_out[r] = o;
    }
    if (a.fin || a.loss_rows) {
        const int64_t t = a.target[r];
        ce_row_final fo;
        fo.lse = 0.0;
        fo.gt = 0.0;
        fo.m = 0.0f;
        float loss;
        if (t == a.ignore_index) {
            fo.status = 0;
            loss = 0.0f;
        } else if (t < 0 || t >= a.V_total || own != 1) {
            fo.status = -1;
            loss = __builtin_nanf("");
        } else {
            const RowFinal f = finalize_row(M, s, zt, sz, (double)a.V_total, (double)a.eps);
            fo.lse = f.lse;
            fo.gt = f.gt;
            fo.m = (float)M;
            fo.status = 1;
            loss = (float)f.loss;
        }
        if (a.fin) a.fin[r] = fo;
        if (a.loss_rows) a.loss_rows[r] = loss;
    }
}

// ===========================================================================
// streaming gradient: one workgroup per (row, column chunk)
// ===========================================================================

template <int IN, int OUT, int EPV, int THREADS, int UNROLL, bool LS>
__global__ __launch_bounds__(THREADS) void k_grad(GradArgs a) {
    using In = Elem<IN>;
    using Ch = Chunk<IN, EPV>;
    using St = Store<OUT, EPV>;
    constexpr int kOutSize = (OUT == CE_BF16) ? 2 : 4;
    __shared__ GradConst gc_sh;

    const int tid = threadIdx.x;
    const int64_t unit = xcd_major(blockIdx.x, gridDim.x);
    const int64_t row = unit / a.nchunks;
    const int ch = (int)(unit % a.nchunks);
    const int64_t c0 = (int64_t)ch * a.chunk_cols;
    const int64_t c1 = std::min(a.V_local, c0 + a.chunk_cols);
    const int64_t nv = (c1 - c0) / EPV;
    const int64_t tail0 = c0 + nv * EPV;
    const char *zrow = static_cast<const char *>(a.logits) + row * a.ld * In::kSize;
    char *grow = static_cast<char *>(a.grad) + row * a.ldg * kOutSize;

    const ce_row_final f = a.fin[row];
    if (f.status != 1) {
        float zero[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) zero[e] = 0.0f;
        for (int64_t vi = tid; vi < nv; vi += THREADS) St::put(grow + (c0 + vi * EPV) * kOutSize, zero);
        for (int64_t col = tail0 + tid; col < c1; col += THREADS)
            Store<OUT, 1>::put(grow + col * kOutSize, zero);
        return;
    }
    if (tid == 0) {
        const double k = row_scale(a.reduction, a.grad_output, a.n_valid, row);
        gc_sh = grad_constants(f.lse, f.gt, k, (double)a.eps, (double)a.V_total);
    }
    __syncthreads();
    const GradConst c = gc_sh;
    const int64_t tl = a.target[row] - a.vocab_start;
    const int64_t tc = (tl >= c0 && tl < c1) ? tl : -1;

    for (int64_t base = 0; base < nv; base += (int64_t)UNROLL * THREADS) {
        Ch v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int64_t vi = base + (int64_t)u * THREADS + tid;
            if (vi < nv) v[u].load(zrow + (c0 + vi * EPV) * In::kSize);
        }
        const bool t_here = tc >= c0 + base * EPV && tc < c0 + (base + (int64_t)UNROLL * THREADS) * EPV;
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int64_t vi = base + (int64_t)u * THREADS + tid;
            if (vi >= nv) continue;
            const int64_t col = c0 + vi * EPV;
            float g[EPV];
#pragma unroll
            for (int e = 0; e < EPV; ++e) g[e] = grad_elem<OUT, LS>(v[u].get(e), c);
            if (t_here && tc >= col && tc < col + EPV) {
#pragma unroll
                for (int e = 0; e < EPV; ++e)
                    if (col + e == tc) g[e] = c.gk;
            }
            St::put(grow + col * kOutSize, g);
        }
    }
    for (int64_t col = tail0 + tid; col < c1; col += THREADS) {
        const float z = In::load1(zrow + col * In::kSize);
        float g;
        g = (col == tc) ? c.gk : grad_elem<OUT, LS>(z, c);
        Store<OUT, 1>::put(grow + col * kOutSize, &g);
    }
}

} // namespace vce

// ===========================================================================
// launchers
// ===========================================================================
namespace vce {

hipError_t launch_count(const int64_t *target, int64_t T, int64_t ignore_index, int64_t V_total,
                        int32_t *n_valid, int32_t *err_count, hipStream_t stream) {
    hipLaunchKernelGGL(k_count, dim3(1), dim3(kCountThreads), 0, stream, target, T, ignore_index,
                       V_total, n_valid, err_count);
    return hipGetLastError();
}

hipError_t launch_reduce(const float *loss_rows, int64_t T, int reduction, const int32_t *n_valid,
                         float *loss, hipStream_t stream) {
    hipLaunchKernelGGL(k_reduce, dim3(1), dim3(kReduceThreads), 0, stream, loss_rows, T,
                       reduction, n_valid, loss);
    return hipGetLastError();
}

// (threads, vectors per thread) of the row-resident kernel, smallest first
struct ResidentShape {
    int threads, nv;
};
constexpr ResidentShape kResident[] = {{256, 1}, {256, 2},  {256, 4},  {256, 8},
                                       {256, 16}, {512, 16}, {1024, 16}};

static int resident_index(int in_dt, int64_t V) {
    const int64_t epv = (in_dt == CE_BF16) ? 8 : 4;
    const int64_t nvec = V / epv;
    for (int i = 0; i < (int)(sizeof(kResident) / sizeof(kResident[0])); ++i)
        if ((int64_t)kResident[i].threads * kResident[i].nv >= nvec &&
            kResident[i].threads >= V - nvec * epv)
            return i;
    return -1;
}

int resident_threads(int in_dt, int64_t V) {
    const int i = resident_index(in_dt, V);
    return i < 0 ? 0 : kResident[i].threads;
}

template <int IN, int OUT, bool LS>
static hipError_t fused_dispatch(const FusedArgs &a, int64_t T, hipStream_t stream) {
    const int i = resident_index(IN, a.V);
    const dim3 grid((unsigned)T);
#define VCE_RES(TH, NV)                                                                         \
    hipLaunchKernelGGL((k_fused_resident<IN, OUT, TH, NV, LS>), grid, dim3(TH), 0, stream, a); \
    break;
    switch (i) {
    case 0: VCE_RES(256, 1)
    case 1: VCE_RES(256, 2)
    case 2: VCE_RES(256, 4)
    case 3: VCE_RES(256, 8)
    case 4: VCE_RES(256, 16)
    case 5: VCE_RES(512, 16)
    case 6: VCE_RES(1024, 16)
    default: return hipErrorInvalidValue;
    }
#undef VCE_RES
    return hipGetLastError();
}

// LDS bytes per workgroup the split kernel needs for V columns (0 if the
// row is not in its range).
static int lds_split_bytes(int in_dt, int64_t V) {
    const int64_t epv = (in_dt == CE_BF16) ? 8 : 4;
    const int64_t nvec = V / epv;
    const int64_t reg = (int64_t)kLdsRegSlots * kLdsThreads;
    if (nvec <= 8192 || nvec <= reg) return 0;
    const int64_t bytes = (nvec - reg) * 16;
    // two workgroups per CU: half of the 160 KB LDS each, less the static part
    if (bytes > 163840 / 2 - 512) return 0;
    return (int)bytes;
}

template <int IN, int OUT>
static hipError_t launch_lds(const FusedArgs &a, int64_t T, int lds, hipStream_t stream) {
    static bool configured = false;
    if (!configured) {
        const hipError_t e = hipFuncSetAttribute(
            (const void *)k_fused_lds<IN, OUT, kLdsRegSlots>,
            hipFuncAttributeMaxDynamicSharedMemorySize, 163840 / 2 - 512);
        if (e != hipSuccess) return e;
        configured = true;
    }
    hipLaunchKernelGGL((k_fused_lds<IN, OUT, kLdsRegSlots>), dim3((unsigned)T), dim3(kLdsThreads),
                       lds, stream, a);
    return hipGetLastError();
}

hipError_t launch_fused_resident(const FusedArgs &a, int in_dt, int out_dt, int64_t T,
                                 hipStream_t stream) {
    const bool ls = a.eps > 0.0f;
    const int lds = ls ? 0 : lds_split_bytes(in_dt, a.V);
    if (lds > 0) {
        if (in_dt == CE_BF16)
            return out_dt == CE_BF16 ? launch_lds<CE_BF16, CE_BF16>(a, T, lds, stream)
                                     : launch_lds<CE_BF16, CE_F32>(a, T, lds, stream);
        return out_dt == CE_BF16 ? launch_lds<CE_F32, CE_BF16>(a, T, lds, stream)
                                 : launch_lds<CE_F32, CE_F32>(a, T, lds, stream);
    }
    if (in_dt == CE_BF16) {
        if (out_dt == CE_BF16)
            return ls ? fused_dispatch<CE_BF16, CE_BF16, true>(a, T, stream)
                      : fused_dispatch<CE_BF16, CE_BF16, false>(a, T, stream);
        return ls ? fused_dispatch<CE_BF16, CE_F32, true>(a, T, stream)
                  : fused_dispatch<CE_BF16, CE_F32, false>(a, T, stream);
    }
    if (out_dt == CE_BF16)
        return ls ? fused_dispatch<CE_F32, CE_BF16, true>(a, T, stream)
                  : fused_dispatch<CE_F32, CE_BF16, false>(a, T, stream);
    return ls ? fused_dispatch<CE_F32, CE_F32, true>(a, T, stream)
              : fused_dispatch<CE_F32, CE_F32, false>(a, T, stream);
}

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 4;

template <int IN, bool LS>
static void stats_dispatch(const StatsArgs &a, bool vec, dim3 grid, hipStream_t stream) {
    constexpr int EPV = Elem<IN>::kVec;
    if (vec)
        hipLaunchKernelGGL((k_stats<IN, EPV, kStreamThreads, kStreamUnroll, LS>), grid,
                           dim3(kStreamThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((k_stats<IN, 1, kStreamThreads, 16, LS>), grid, dim3(kStreamThreads),
                           0, stream, a);
}

hipError_t launch_exp_table(double *tab, hipStream_t stream) {
    hipLaunchKernelGGL(k_exp_table, dim3((kExpTabN + 255) / 256), dim3(256), 0, stream, tab);
    return hipGetLastError();
}

hipError_t launch_stats(const StatsArgs &a, int in_dt, bool vec, hipStream_t stream) {
    const dim3 grid((unsigned)(a.T * a.nchunks));
    const bool ls = a.smoothing != 0;
    if (ls && vec && in_dt == CE_BF16 && a.exp_tab) {
        hipLaunchKernelGGL((k_stats_tab<kStreamThreads, kStreamUnroll>), grid,
                           dim3(kStreamThreads), 0, stream, a, a.exp_tab);
        return hipGetLastError();
    }
    if (in_dt == CE_BF16)
        ls ? stats_dispatch<CE_BF16, true>(a, vec, grid, stream)
           : stats_dispatch<CE_BF16, false>(a, vec, grid, stream);
    else
        ls ? stats_dispatch<CE_F32, true>(a, vec, grid, stream)
           : stats_dispatch<CE_F32, false>(a, vec, grid, stream);
    return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs &a, hipStream_t stream) {
    const dim3 grid((unsigned)((a.T + kMergeThreads - 1) / kMergeThreads));
    hipLaunchKernelGGL(k_merge, grid, dim3(kMergeThreads), 0, stream, a);
    return hipGetLastError();
}

template <int IN, int OUT, bool LS>
static void grad_dispatch(const GradArgs &a, bool vec, dim3 grid, hipStream_t stream) {
    constexpr int EPV = Elem<IN>::kVec;
    if (vec)
        hipLaunchKernelGGL((k_grad<IN, OUT, EPV, kStreamThreads, kStreamUnroll, LS>), grid,
                           dim3(kStreamThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((k_grad<IN, OUT, 1, kStreamThreads, 16, LS>), grid,
                           dim3(kStreamThreads), 0, stream, a);
}

hipError_t launch_grad(const GradArgs &a, int in_dt, int out_dt, bool vec, int64_t T,
                       hipStream_t stream) {
    const dim3 grid((unsigned)(T * a.nchunks));
    const bool ls = a.eps > 0.0f;
    if (in_dt == CE_BF16) {
        if (out_dt == CE_BF16)
            ls ? grad_dispatch<CE_BF16, CE_BF16, true>(a, vec, grid, stream)
               : grad_dispatch<CE_BF16, CE_BF16, false>(a, vec, grid, stream);
        else
            ls ? grad_dispatch<CE_BF16, CE_F32, true>(a, vec, grid, stream)
               : grad_dispatch<CE_BF16, CE_F32, false>(a, vec, grid, stream);
    } else {
        if (out_dt == CE_BF16)
            ls ? grad_dispatch<CE_F32, CE_BF16, true>(a, vec, grid, stream)
               : grad_dispatch<CE_F32, CE_BF16, false>(a, vec, grid, stream);
        else
            ls ? grad_dispatch<CE_F32, CE_F32, true>(a, vec, grid, stream)
               : grad_dispatch<CE_F32, CE_F32, false>(a, vec, grid, stream);
    }
    return hipGetLastError();
}

} // namespace vce
