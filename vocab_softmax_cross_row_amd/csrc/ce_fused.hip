// Fused cross-entropy forward + backward for gfx950: one workgroup per row
// keeps the row on chip from its one read to its one gradient write
// (torchtitan PR "[loss] fix softmax collapse with improved ce perf",
// Memory/perf: one read of the logits, the backward rebuilt in one fused
// pass):
//   k_fused_lds: 65536 < V <= 130944 bf16 without smoothing; two 512-thread
//     workgroups per CU, the row split between registers and LDS;
//   k_fused_resident: other row lengths, smoothing and fp32 gradients; the
//     whole row in registers (up to 16 vectors of 16 bytes per thread).
// Sweeps: non-target max, sum of exponentials, an fp32 or fp64 finalize by
// one thread, then the gradient.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>

#include "ce_device.h"
#include "ce_launch.h"
#include "vocab_ce.h"

namespace vce {

// ===========================================================================
// fused, row resident
// ===========================================================================

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// e^z of one bf16 pattern b from the LDS table of e^z (see kExpTabLo): the
// table's entry, 0 for -inf, 1 + z + z^2/2 for |z| < 2^-16 (error below
// 1e-15); |z| >= 512, +inf and NaN set `bad` (the caller recomputes).
__device__ __forceinline__ double tab_exp1(uint32_t b, const double *tab, bool &bad) {
    const uint32_t mag = b & 0x7fffu;
    const uint32_t off = mag - kExpTabLo;
    if (off < (uint32_t)kExpTabHalf) return tab[2 * off + (b >> 15)];
    if (b == 0xff80u) return 0.0;
    if (mag < kExpTabLo) {
        const double z = (double)__uint_as_float(b << 16);
        return 1.0 + z * (1.0 + 0.5 * z);
    }
    bad = true;
    return 0.0;
}

// Sum of e^z over the 8 bf16 logits of one 16-byte vector, from the table.
// Two logits per 32-bit word: byte offset 16 (|pattern| - kExpTabLo),
// clamped to the NaN entries, plus 8 for a negative logit; all 8 table
// reads are issued together.  Returns false (and a sum to be ignored) when
// a pattern lies outside the table: the killed target, padding, |z| < 2^-16
// or |z| >= 512; tab_exp8_slow then takes the vector logit by logit.
__device__ __forceinline__ bool tab_exp8(const u32x4 &w, const double *tab, double &sum) {
    const char *tabc = reinterpret_cast<const char *>(tab);
    u16x2 omax = {0, 0};
    double t[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const u16x2 off =
            __builtin_bit_cast(u16x2, w[q] & 0x7fff7fffu) - (u16x2)(uint16_t)kExpTabLo;
        omax = __builtin_elementwise_max(omax, off);
        const u16x2 c = __builtin_elementwise_min(off, (u16x2)(uint16_t)kExpTabHalf);
        const uint32_t a2 =
            __builtin_bit_cast(uint32_t, c << (uint16_t)4) | ((w[q] >> 12) & 0x00080008u);
        t[2 * q] = *reinterpret_cast<const double *>(tabc + (a2 & 0xffffu));
        t[2 * q + 1] = *reinterpret_cast<const double *>(tabc + (a2 >> 16));
    }
    sum = ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
    return omax.x < (uint16_t)kExpTabHalf && omax.y < (uint16_t)kExpTabHalf;
}

__device__ __forceinline__ double tab_exp8_slow(const u32x4 &w, const double *tab, bool &bad) {
    double s = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t x = w[e >> 1];
        s += tab_exp1((e & 1) ? (x >> 16) : (x & 0xffffu), tab, bad);
    }
    return s;
}

// One row, resident in registers from its load to its gradient store; the
// workgroup's threads all call it.  FAST = bf16 gradient without smoothing:
// fp32 finalize and the biased exponent form (see GradConst); otherwise
// fp64 finalize.  TAB (bf16 with smoothing): the fp64 sum of exponentials
// reads e^z from the LDS table `tab` instead of an fp64 exponential per
// logit.
// The batch's count of valid and of bad targets, by one workgroup (every
// thread gets both): small batches count in the fused kernel itself.
template <int THREADS>
__device__ __forceinline__ void inline_count(const FusedArgs &a, int &n_valid, int &n_bad) {
    int nv = 0, nb = 0;
    for (int64_t r = threadIdx.x; r < a.T; r += THREADS) {
        const int64_t t = a.target[r];
        if (t == a.ignore_index) continue;
        if (t >= 0 && t < a.V)
            ++nv;
        else
            ++nb;
    }
    nv = wave_sum(nv);
    nb = wave_sum(nb);
    __shared__ int part[2][THREADS / kWave];
    const int wv = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) {
        part[0][wv] = nv;
        part[1][wv] = nb;
    }
    __syncthreads();
    n_valid = n_bad = 0;
#pragma unroll
    for (int i = 0; i < THREADS / kWave; ++i) {
        n_valid += part[0][i];
        n_bad += part[1][i];
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        *a.count_out = n_valid;
        if (a.err_out) *a.err_out = n_bad;
    }
}

// Scale k_r of a row's gradient from a count already at hand.
__device__ __forceinline__ double row_scale_n(int reduction, const float *grad_output, int n_valid,
                                              int64_t row) {
    double g = 1.0;
    if (reduction == CE_RED_NONE) {
        if (grad_output) g = (double)grad_output[row];
        return g;
    }
    if (grad_output) g = (double)grad_output[0];
    if (reduction == CE_RED_MEAN) g /= (double)n_valid;
    return g;
}

template <int IN, int OUT, int THREADS, int NV, bool LS, bool TAB>
__device__ __forceinline__ void fused_row(const FusedArgs &a, int64_t row,
                                          BlockRed<THREADS> &red, GradConst &gc_sh,
                                          double *tab) {
    using In = Elem<IN>;
    constexpr int EPV = In::kVec;
    using Ch = Chunk<IN, EPV>;
    using St = Store<OUT, EPV, true>;
    constexpr int kOutSize = (OUT == CE_BF16) ? 2 : 4;
    constexpr bool FAST = (OUT == CE_BF16) && !LS;
    static_assert(!TAB || (LS && IN == CE_BF16), "the table holds e^z of bf16 logits");

    const int tid = threadIdx.x;
    const int V = (int)a.V;
    const char *zrow = static_cast<const char *>(a.logits) + row * a.ld * In::kSize;
    char *grow = static_cast<char *>(a.grad) + row * a.ldg * kOutSize;
    // Vectors start at the row's first 16-byte boundary (rows of odd width
    // are not aligned; the host takes this kernel for them only when the
    // gradient row is then aligned too).  The head before it and the tail
    // after the last vector are scalar slots, one per thread: slot k is
    // column k of the head, or column tail0 + (k - head) of the tail.
    const int head = (int)head_elems<In::kSize, EPV>(zrow, V);
    const int nvec = (V - head) / EPV;
    const int tail0 = head + nvec * EPV;
    const int nscal = head + (V - tail0);
    const int scol = tid < head ? tid : tail0 + (tid - head); // this thread's scalar slot
    const char *zvec = zrow + head * In::kSize;
    char *gvec = grow + head * kOutSize;

    const int64_t t64 = a.target[row];
    if (t64 == a.ignore_index || t64 < 0 || t64 >= V) {
        // ignored row or bad target: zero gradient, no reads of the row;
        // workgroup 0 still writes the batch's count
        if (a.count_inline && blockIdx.x == 0) {
            int nv, nb;
            inline_count<THREADS>(a, nv, nb);
        }
        float zero[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) zero[e] = 0.0f;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int vi = i * THREADS + tid;
            if (vi < nvec) St::put(gvec + vi * EPV * kOutSize, zero);
        }
        if (tid < nscal) Store<OUT, 1>::put(grow + scol * kOutSize, zero);
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
            v[i].template load<true>(zvec + vi * EPV * In::kSize);
        else
            v[i].fill_ninf();
    }
    float ztail = ninf(); // this thread's scalar slot
    if (tid < nscal) ztail = In::load1(zrow + scol * In::kSize);
    if constexpr (TAB) {
        // the table of e^z: global -> LDS directly (no registers), behind
        // the row's loads; waited for just before the sum of exponentials
        constexpr int kTabVecs = (kExpTabN * 8 + 15) / 16;
        const __amdgpu_buffer_rsrc_t rt =
            __builtin_amdgcn_make_buffer_rsrc((void *)a.exp_tab, 0, kExpTabN * 8, 0x00020000);
        const int wave_base = __builtin_amdgcn_readfirstlane((tid / kWave) * kWave);
        u32x4 *tv = reinterpret_cast<u32x4 *>(tab);
#pragma unroll 1
        for (int q = 0; q * THREADS < kTabVecs; ++q)
            if (q * THREADS + tid < kTabVecs)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rt, (__attribute__((address_space(3))) void *)(tv + q * THREADS + wave_base), 16,
                    (q * THREADS + tid) * 16, 0, 0, 0);
    }

    // the batch's count, counted here while the row's loads are in flight
    int n_valid = 0, n_bad = 0;
    if (a.count_inline && (blockIdx.x == 0 || a.reduction == CE_RED_MEAN))
        inline_count<THREADS>(a, n_valid, n_bad);

    // where the target sits: vector tv = slot t_slot of thread t_thread
    // (wave t_wave), element te; or the scalar tail.  t is the same for the
    // whole workgroup, and readfirstlane makes the slot and wave tests
    // scalar branches, so only the owner wave does any work for it.
    const int tv = (t - head) / EPV;
    const int te = __builtin_amdgcn_readfirstlane((t - head) - tv * EPV);
    const bool t_in_vec = t >= head && t < tail0;
    const int t_scal = t < head ? t : head + (t - tail0); // its scalar slot otherwise
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
        if (tid < nscal) sz += (double)ztail;
    }

    // ---- drop the target before any reduction ------------------------------
    if (t_wave_mine) {
#pragma unroll
        for (int i = 0; i < NV; ++i)
            if (i == t_slot && t_lane_mine) v[i].kill(te);
    }
    if (!t_in_vec && tid == t_scal) ztail = ninf();

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
        // taken with fp64 exponentials (or table entries) and fp64
        // accumulation.
        bool online = !TAB;
        if constexpr (TAB) {
            // unshifted: sum of e^z (fp64 spans e^-512 .. e^512), then times
            // e^-mx (-mx is a bf16 value: mx is a max of bf16 logits)
            __builtin_amdgcn_s_waitcnt(0); // this wave's part of the table has landed
            __syncthreads();               // and every other wave's
            if (mx != ninf()) {
                bool bad = false;
                // branch-free table sums first; vectors with a pattern outside
                // the table are marked and summed logit by logit afterwards
                uint32_t slow = 0;
#pragma unroll
                for (int i = 0; i < NV; ++i) {
                    double si;
                    const bool ok = tab_exp8(v[i].v, tab, si);
                    sd += ok ? si : 0.0;
                    slow |= (ok ? 0u : 1u) << i;
                }
                if (slow) {
#pragma unroll
                    for (int i = 0; i < NV; ++i)
                        if ((slow >> i) & 1u) sd += tab_exp8_slow(v[i].v, tab, bad);
                }
                sd += tab_exp1(__float_as_uint(ztail) >> 16, tab, bad);
                sd *= tab_exp1((__float_as_uint(mx) >> 16) ^ 0x8000u, tab, bad);
                online = block_max<THREADS>(bad ? 1.0f : 0.0f, red, 1) > 0.0f;
            }
        }
        if (online) {
            // |z| >= 512, +inf or NaN somewhere in the row (TAB): the whole
            // row again with fp64 exponentials
            sd = 0.0;
            if (mx != ninf()) {
                const double md = (double)mx;
#pragma unroll
                for (int i = 0; i < NV; ++i)
#pragma unroll
                    for (int e = 0; e < EPV; ++e) sd += exp_nonpos((double)v[i].get(e) - md);
                sd += exp_nonpos((double)ztail - md);
            }
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
        const double k = a.count_inline ? row_scale_n(a.reduction, a.grad_output, n_valid, row)
                                        : row_scale(a.reduction, a.grad_output, a.n_valid, row);
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
        if (vi < nvec) St::put(gvec + vi * EPV * kOutSize, g);
    }
    if (tid < nscal) {
        const float g = (!t_in_vec && tid == t_scal) ? c.gk : grad_elem<OUT, LS>(ztail, c);
        Store<OUT, 1>::put(grow + scol * kOutSize, &g);
    }
}

template <int IN, int OUT, int THREADS, int NV, bool LS>
__global__ __launch_bounds__(THREADS) void k_fused_resident(FusedArgs a) {
    __shared__ BlockRed<THREADS> red;
    __shared__ GradConst gc_sh;
    fused_row<IN, OUT, THREADS, NV, LS, false>(a, xcd_major(blockIdx.x, gridDim.x), red, gc_sh,
                                               nullptr);
}

// bf16 rows with smoothing, 16384 < V <= 32768: one row per workgroup, as
// k_fused_resident, with the table of e^z (51 KB, read from L2 by each
// workgroup) in LDS.  The table allows 3 workgroups per CU, so registers are
// capped for 3 waves per SIMD.  A persistent form (the table loaded once per
// workgroup, rows in a loop) kept row-loop invariants in registers: 129 VGPRs
// before any of the row.
constexpr int kTabThreads = 256;

template <int OUT, int NV>
__global__ __launch_bounds__(kTabThreads) __attribute__((amdgpu_waves_per_eu(3, 3)))
void k_fused_resident_tab(FusedArgs a) {
    __shared__ BlockRed<kTabThreads> red;
    __shared__ GradConst gc_sh;
    __shared__ u32x4 tab[(kExpTabN * 8 + 15) / 16];
    fused_row<CE_BF16, OUT, kTabThreads, NV, true, true>(a, xcd_major(blockIdx.x, gridDim.x), red,
                                                         gc_sh, reinterpret_cast<double *>(tab));
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


} // namespace vce

// ===========================================================================
// launchers
// ===========================================================================
namespace vce {

// (threads, vectors per thread) of the row-resident kernel, smallest first.
// Short rows take small workgroups: a 256-thread workgroup per 1000-column
// row left half of its threads idle (65536 x 1000 bf16: 157 us at 256 x 1,
// 85 us at 64 x 2).  With smoothing the fp64 work per logit makes 64-thread
// workgroups pay up to 4096 columns (65536 x 4096: 381 -> 333 us); without
// it 256 x 2 stays best there (204 against 215 us).  Rows of 8K to 32K
// columns without smoothing take 512 threads (65536 x 12000 bf16: 567 ->
// 546 us at 512 x 4; 65536 x 32000: 1453 -> 1432 us at 512 x 8); 512 x 2
// was slower at 6000 columns, and with smoothing 512 x 4 was slower.
struct ResidentShape {
    int threads, nv;
};
constexpr ResidentShape kResident[] = {{64, 1},   {64, 2},   {128, 2},   {256, 2}, {256, 4},
                                       {512, 4},  {512, 8},  {512, 16},  {1024, 16}};
constexpr ResidentShape kResidentLS[] = {{64, 1},  {64, 2},   {64, 4},    {64, 8},  {256, 4},
                                         {256, 8}, {256, 16}, {512, 16},  {1024, 16}};
constexpr int kNumResident = sizeof(kResident) / sizeof(kResident[0]);
static_assert(kNumResident == sizeof(kResidentLS) / sizeof(kResidentLS[0]), "table sizes");

static const ResidentShape *resident_table(bool ls) { return ls ? kResidentLS : kResident; }

static int resident_index(int in_dt, int64_t V, bool ls) {
    const ResidentShape *tab = resident_table(ls);
    const int64_t epv = (in_dt == CE_BF16) ? 8 : 4;
    const int64_t nvec = V / epv;
    for (int i = 0; i < kNumResident; ++i)
        if ((int64_t)tab[i].threads * tab[i].nv >= nvec && tab[i].threads >= V - nvec * epv)
            return i;
    return -1;
}

int resident_threads(int in_dt, int64_t V) {
    const int i = resident_index(in_dt, V, false);
    return i < 0 ? 0 : kResident[i].threads;
}

template <int IN, int OUT, bool LS>
static hipError_t fused_dispatch(const FusedArgs &a, int64_t T, hipStream_t stream) {
    const int i = resident_index(IN, a.V, LS);
    const dim3 grid((unsigned)T);
#define VCE_RES(TH, NV)                                                                         \
    hipLaunchKernelGGL((k_fused_resident<IN, OUT, TH, NV, LS>), grid, dim3(TH), 0, stream, a); \
    break;
    if constexpr (LS) {
        switch (i) {
        case 0: VCE_RES(64, 1)
        case 1: VCE_RES(64, 2)
        case 2: VCE_RES(64, 4)
        case 3: VCE_RES(64, 8)
        case 4: VCE_RES(256, 4)
        case 5: VCE_RES(256, 8)
        case 6: VCE_RES(256, 16)
        case 7: VCE_RES(512, 16)
        case 8: VCE_RES(1024, 16)
        default: return hipErrorInvalidValue;
        }
    } else {
        switch (i) {
        case 0: VCE_RES(64, 1)
        case 1: VCE_RES(64, 2)
        case 2: VCE_RES(128, 2)
        case 3: VCE_RES(256, 2)
        case 4: VCE_RES(256, 4)
        case 5: VCE_RES(512, 4)
        case 6: VCE_RES(512, 8)
        case 7: VCE_RES(512, 16)
        case 8: VCE_RES(1024, 16)
        default: return hipErrorInvalidValue;
        }
    }
#undef VCE_RES
    return hipGetLastError();
}

// LDS bytes per workgroup the split kernel needs for V columns (0 if the
// row is not in its range).
// Up to half of the 160 KB LDS (less the static part) two workgroups share a
// CU; longer rows (to about 171K bf16 columns) run one workgroup per CU,
// which still reads each row once, rather than stream it three times.
constexpr int kLdsMaxBytes = 163840 - 512;

static int lds_split_bytes(int in_dt, int64_t V) {
    const int64_t epv = (in_dt == CE_BF16) ? 8 : 4;
    const int64_t nvec = V / epv;
    const int64_t reg = (int64_t)kLdsRegSlots * kLdsThreads;
    if (nvec <= 8192 || nvec <= reg) return 0;
    const int64_t bytes = (nvec - reg) * 16;
    if (bytes > kLdsMaxBytes) return 0;
    return (int)bytes;
}

bool fused_table(int in_dt, int64_t V) {
    const int i = resident_index(in_dt, V, true);
    return in_dt == CE_BF16 && i >= 0 && kResidentLS[i].threads == kTabThreads &&
           kResidentLS[i].nv == 16;
}

bool fused_fits(int in_dt, int64_t V, bool aligned, bool smoothing) {
    if (aligned && !smoothing && lds_split_bytes(in_dt, V) > 0) return true;
    return resident_threads(in_dt, V) > 0;
}

template <int IN, int OUT>
static hipError_t launch_lds(const FusedArgs &a, int64_t T, int lds, hipStream_t stream) {
    static std::atomic<bool> configured[kMaxDevices];
    const hipError_t e =
        raise_lds_once((const void *)k_fused_lds<IN, OUT, kLdsRegSlots>, kLdsMaxBytes, configured);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_fused_lds<IN, OUT, kLdsRegSlots>), dim3((unsigned)T), dim3(kLdsThreads),
                       lds, stream, a);
    return hipGetLastError();
}

template <int OUT>
static hipError_t tab_dispatch(const FusedArgs &a, int64_t T, hipStream_t stream) {
    hipLaunchKernelGGL((k_fused_resident_tab<OUT, 16>), dim3((unsigned)T), dim3(kTabThreads), 0,
                       stream, a);
    return hipGetLastError();
}

hipError_t launch_fused_resident(const FusedArgs &a, int in_dt, int out_dt, int64_t T,
                                 bool aligned, hipStream_t stream) {
    const bool ls = a.eps > 0.0f;
    if (ls && in_dt == CE_BF16 && a.exp_tab) {
        // smoothed bf16 rows of the 256 x 16 shape (16384 < V <= 32768):
        // sums from the table.  Shorter rows keep fp64 exponentials: with
        // 256 x 8 (V <= 16384) the table, read per row, cost more than it
        // saved (32768 x 12000: 532 -> 601 us; 65536 x 32000: 2216 -> 1896)
        if (fused_table(in_dt, a.V))
            return out_dt == CE_BF16 ? tab_dispatch<CE_BF16>(a, T, stream)
                                     : tab_dispatch<CE_F32>(a, T, stream);
    }
    // the LDS-split kernel needs 16-byte aligned rows; rows that are not take
    // the register-resident kernel, which peels their heads
    const int lds = (ls || !aligned) ? 0 : lds_split_bytes(in_dt, a.V);
    if (lds > 0) {
        // this kernel reads the count from n_valid
        FusedArgs b = a;
        if (b.count_inline) {
            const hipError_t e = launch_count(a.target, a.T, a.ignore_index, a.V, a.count_out,
                                              a.err_out, stream);
            if (e != hipSuccess) return e;
            b.count_inline = 0;
        }
        if (in_dt == CE_BF16)
            return out_dt == CE_BF16 ? launch_lds<CE_BF16, CE_BF16>(b, T, lds, stream)
                                     : launch_lds<CE_BF16, CE_F32>(b, T, lds, stream);
        return out_dt == CE_BF16 ? launch_lds<CE_F32, CE_BF16>(b, T, lds, stream)
                                 : launch_lds<CE_F32, CE_F32>(b, T, lds, stream);
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

} // namespace vce
