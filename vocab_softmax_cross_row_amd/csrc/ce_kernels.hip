// Cross-entropy kernels for gfx950: the streaming paths and the counts.
//
//   streaming: the stats kernel (one read, online max / sum per thread, or
//     the e^z table for smoothed bf16 rows), the merge kernel (column-chunk
//     or shard statistics, fp64 finalize) and the gradient kernel (one
//     read, one write).  They serve ce_forward / ce_merge_shard_stats /
//     ce_backward, and the fused entry point when the row does not fit on
//     chip, when rows are not 16-byte aligned, or when there are too few
//     rows to fill the GPU (then each row is split into column chunks: the
//     split-V grid).
//   count and reduce: N_valid / bad-target counts before the gradient needs
//     them, and the deterministic loss sum.
//
// The fused, row-resident kernels are in ce_fused.hip.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <mutex>

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

// The count by one workgroup of THREADS threads (k_count, and the extra
// workgroup of k_merge).
template <int THREADS>
__device__ __forceinline__ void count_targets(const int64_t *__restrict__ target, int64_t T,
                                              int64_t ignore_index, int64_t V_total,
                                              int32_t *n_valid, int32_t *err_count) {
    int nv = 0, nb = 0;
    for (int64_t base = 0; base < T; base += (int64_t)THREADS * kPerThread) {
        int64_t t[kPerThread];
#pragma unroll
        for (int u = 0; u < kPerThread; ++u) {
            const int64_t r = base + (int64_t)u * THREADS + threadIdx.x;
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
    __shared__ int part[2][THREADS / kWave];
    const int wv = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) {
        part[0][wv] = nv;
        part[1][wv] = nb;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int x = 0, y = 0;
        for (int i = 0; i < THREADS / kWave; ++i) {
            x += part[0][i];
            y += part[1][i];
        }
        if (n_valid) *n_valid = x;
        if (err_count) *err_count = y;
    }
}

__global__ __launch_bounds__(kCountThreads) void k_count(const int64_t *__restrict__ target,
                                                         int64_t T, int64_t ignore_index,
                                                         int64_t V_total, int32_t *n_valid,
                                                         int32_t *err_count) {
    count_targets<kCountThreads>(target, T, ignore_index, V_total, n_valid, err_count);
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
    // vectors start at the first 16-byte boundary at or after c0; the head
    // before it (rows that are not 16-byte aligned) joins the scalar tail
    const int64_t v0 = c0 + head_elems<In::kSize, EPV>(zrow + c0 * In::kSize, c1 - c0);
    const int64_t nv = (c1 - v0) / EPV; // full vectors of this chunk
    const int64_t tail0 = v0 + nv * EPV;
    Online<LS> acc;
    double sz = 0.0;
    for (int64_t base = 0; base < nv; base += (int64_t)UNROLL * THREADS) {
        Ch v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int64_t vi = base + (int64_t)u * THREADS + tid;
            if (vi < nv)
                v[u].template load<true>(zrow + (v0 + vi * EPV) * In::kSize);
            else
                v[u].fill_ninf();
        }
        // one rescale per UNROLL vectors: the max of the whole group first;
        // the target test is uniform over the group's column span first
        const bool t_here = tc >= v0 + base * EPV && tc < v0 + (base + (int64_t)UNROLL * THREADS) * EPV;
        float vm = ninf();
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int64_t vi = base + (int64_t)u * THREADS + tid;
            const int64_t col = v0 + vi * EPV;
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
    // scalar head and tail of the chunk
    for (int64_t k = tid; k < (v0 - c0) + (c1 - tail0); k += THREADS) {
        const int64_t col = k < v0 - c0 ? c0 + k : tail0 + (k - (v0 - c0));
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
// exponential.  The target and -inf logits count zero, |z| < 2^-16 takes
// e^z = 1 + z + z^2/2 (error below 1e-15), and a chunk with |z| >= 512, +inf
// or NaN is recomputed with the online form.  The table's lower end keeps
// the element-by-element path rare: below 2^-16 it is a few logits in a
// million, and a wave pays for that path whenever one of its lanes needs it.

// Entry 2 off + sign holds e^z of the pattern (kExpTabLo + off) | sign << 15,
// off < kExpTabHalf, the double nearest to the exact value; the last two
// entries (off = kExpTabHalf) are NaN, so that a sum which took one of them
// shows it.  The values are written by gen_exp_table.py when the library is
// built, and live in the code object: no call builds the table.  Not const:
// a const array would have internal linkage, and since kernels read it only
// through a pointer argument the device compiler would drop it, leaving the
// runtime nothing to find when the host asks for its address.
__device__ double kExpTable[kExpTabN] = {
#include "ce_exp_table.inc"
};
static_assert(CE_EXP_TABLE_LO == kExpTabLo && CE_EXP_TABLE_HALF == kExpTabHalf &&
                  CE_EXP_TABLE_ENTRIES == kExpTabN,
              "ce_exp_table.inc was written for another table layout");

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// One (row, column chunk) unit of the smoothed bf16 statistics, with the
// table already in LDS.
template <int THREADS, int UNROLL>
__device__ __forceinline__ void stats_tab_unit(const StatsArgs &a, int64_t unit, const double *tab,
                                               BlockRed<THREADS> &red) {
    using Ch = Chunk<CE_BF16, 8>;
    const int tid = threadIdx.x;
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
    const int64_t tl = t - a.vocab_start;
    const int64_t tc = (tl >= c0 && tl < c1) ? tl : -1;
    const char *zrow = static_cast<const char *>(a.logits) + row * a.ld * 2;
    // vectors start at the first 16-byte boundary at or after c0; the head
    // before it joins the scalar tail
    const int64_t v0 = c0 + head_elems<2, 8>(zrow + c0 * 2, c1 - c0);
    const int64_t nv = (c1 - v0) / 8;
    const int64_t tail0 = v0 + nv * 8;

    // table index of one bf16 pattern; sets *rare when it is outside the table
    // (a NaN entry is read then, and the rare path below replaces it)
    auto index = [&](uint32_t b, bool &rare) {
        const uint32_t off = (b & 0x7fffu) - kExpTabLo;
        const bool in = off < (uint32_t)kExpTabHalf;
        rare |= !in;
        return in ? (int)(2 * off + (b >> 15)) : kExpTabNaN;
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
    // the vector (of this chunk's full vectors) that holds the target, or -1
    const int64_t tvec = tc >= v0 && tc < tail0 ? (tc - v0) / 8 : -1;
    const char *tabc = reinterpret_cast<const char *>(tab);
    // One vector of 8 logits, branch-free, so that a group's vectors keep all
    // their table reads in flight together.  Two logits are handled at a
    // time in the 16-bit lanes of a word:
    // - table byte offset: the pattern rotated left by one bit is
    //   2 |pattern| + sign (one packed multiply-add of the pattern by 2 and
    //   its sign bit); minus 2 kExpTabLo (wrapping below) that is the entry
    //   index 2 off + sign, clamped to 2 kExpTabHalf (a NaN entry), times 8;
    //   a pattern outside the table thus makes the vector's sum NaN, which
    //   the caller tests once per vector;
    // - max: a running max of the patterns read as fp16 numbers.  Like
    //   bf16, fp16 orders sign-magnitude patterns as their values, so the
    //   largest fp16 reading is the largest logit, for every pattern in the
    //   table (bf16 2^-16 .. 2^9 reads as a normal fp16: exponent field 13
    //   to 16); the NaN-propagating maximum takes two words per operation
    //   and needs no canonicalizing, and a pattern outside the table sends
    //   the group to the element-by-element form anyway;
    // - the sum of the logits: a bf16 dot product with (1, 1) into fp32.
    // It returns whether the target lies inside the vector.
    auto vec_common = [&](const Ch &v, int64_t vi, double &sv, f16x2 &hmax, float &zsum) {
        double t[8];
        const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
        float zs = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t w = v.v[q];
            // the compiler builds x * 2 + (x >> 15) from a shift, a shift
            // and an or; v_pk_mad_u16 does it in one operation
            const uint32_t sg = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, w) >> (uint16_t)15);
            uint32_t rot;
            asm("v_pk_mad_u16 %0, %1, %2, %3" : "=v"(rot) : "v"(w), "v"(0x00020002u), "v"(sg));
            const u16x2 ix = __builtin_bit_cast(u16x2, rot) - (u16x2)(uint16_t)(2 * kExpTabLo);
            const u16x2 c = __builtin_elementwise_min(ix, (u16x2)(uint16_t)(2 * kExpTabHalf));
            uint32_t a2 = __builtin_bit_cast(uint32_t, c << (uint16_t)3);
            // keeps the two offsets to one and and one shift
            asm("" : "+v"(a2));
            t[2 * q] = *reinterpret_cast<const double *>(tabc + (a2 & 0xffffu));
            t[2 * q + 1] = *reinterpret_cast<const double *>(tabc + (a2 >> 16));
            hmax = __builtin_elementwise_maximum(hmax, __builtin_bit_cast(f16x2, w));
            zs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), ones, zs, false);
        }
        zsum = zs;
        sv = ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
        return vi == tvec;
    };
    // the largest logit of vectors whose patterns all lie in the table
    auto max_value = [](f16x2 hmax) {
        const _Float16 m = hmax.x > hmax.y ? hmax.x : hmax.y;
        return __uint_as_float((uint32_t)__builtin_bit_cast(uint16_t, m) << 16);
    };
    const f16x2 hmax0 = {__builtin_bit_cast(_Float16, (uint16_t)0xfc00u),
                         __builtin_bit_cast(_Float16, (uint16_t)0xfc00u)}; // fp16 -inf
    // the element-by-element form of a vector (the target left out)
    auto vec_redo = [&](const Ch &v, int64_t vi, double &sv, float &vm) {
        const int64_t col = v0 + vi * 8;
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
            vm = fmaxf(vm, v.get(e));
        }
    };
    const int64_t step = (int64_t)UNROLL * THREADS;
    const int64_t nfull = nv / step * step; // vectors covered by whole iterations
    // the next group's loads are issued before the current group's work
    Ch va[UNROLL], vb[UNROLL];
    auto load_group = [&](Ch *v, int64_t base) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
            v[u].template load<true>(zrow + (v0 + (base + (int64_t)u * THREADS + tid) * 8) * 2);
    };
    auto work_group = [&](Ch *v, int64_t base) {
        double sv[UNROLL];
        float zs[UNROLL];
        f16x2 hmax = hmax0;
        bool rare[UNROLL], any = false;
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            rare[u] = vec_common(v[u], base + (int64_t)u * THREADS + tid, sv[u], hmax, zs[u]);
            rare[u] |= sv[u] != sv[u];
            any |= rare[u];
        }
        float vm = max_value(hmax);
        if (__builtin_expect(any, 0)) {
            // the group's max again, from the vectors' own element maxima
            vm = ninf();
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                float m;
                if (rare[u]) {
                    vec_redo(v[u], base + (int64_t)u * THREADS + tid, sv[u], m);
                } else {
                    m = v[u].get(0);
#pragma unroll
                    for (int e = 1; e < 8; ++e) m = fmaxf(m, v[u].get(e));
                }
                vm = fmaxf(vm, m);
            }
        }
        static_assert(UNROLL == 4, "the group sums below are written for 4 vectors");
        s += (sv[0] + sv[1]) + (sv[2] + sv[3]);
        sz += (double)((zs[0] + zs[1]) + (zs[2] + zs[3]));
        mx = fmaxf(mx, vm);
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
        v.load(zrow + (v0 + vi * 8) * 2);
        double sv;
        float zs;
        f16x2 hmax = hmax0;
        float vm;
        if (vec_common(v, vi, sv, hmax, zs) || sv != sv)
            vec_redo(v, vi, sv, vm);
        else
            vm = max_value(hmax);
        s += sv;
        sz += (double)zs;
        mx = fmaxf(mx, vm);
    }
    // scalar head and tail of the chunk
    for (int64_t k = tid; k < (v0 - c0) + (c1 - tail0); k += THREADS) {
        const int64_t col = k < v0 - c0 ? c0 + k : tail0 + (k - (v0 - c0));
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

// Persistent: each workgroup copies the table into LDS once and then walks
// units blockIdx.x, + gridDim.x, ...; the grid is sized to the workgroups
// the device holds at once.
template <int THREADS, int UNROLL>
__global__ __launch_bounds__(THREADS) void k_stats_tab(StatsArgs a, const double *tab_g) {
    __shared__ BlockRed<THREADS> red;
    __shared__ double tab[kExpTabN];
    for (int i = threadIdx.x; i < kExpTabN; i += THREADS) tab[i] = tab_g[i];
    __syncthreads();
    const int64_t units = a.T * a.nchunks;
    for (int64_t unit = blockIdx.x; unit < units; unit += gridDim.x) {
        stats_tab_unit<THREADS, UNROLL>(a, unit, tab, red);
        __syncthreads(); // the unit's reductions are read before `red` is reused
    }
}

// ===========================================================================
// merge of partial statistics ([S][T], in order) + optional finalize
// ===========================================================================

constexpr int kMergeThreads = 256;

__global__ __launch_bounds__(kMergeThreads) void k_merge(MergeArgs a) {
    if (a.count && blockIdx.x == gridDim.x - 1) {
        // the extra workgroup: the batch's target count, which needs no
        // statistics, beside the merge instead of in a launch of its own
        count_targets<kMergeThreads>(a.target, a.T, a.ignore_index, a.V_total, a.n_valid,
                                     a.err_count);
        return;
    }
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
    using St = Store<OUT, EPV, true>; // nontemporal: the gradient is not read back here
    constexpr int kOutSize = (OUT == CE_BF16) ? 2 : 4;
    __shared__ GradConst gc_sh;

    const int tid = threadIdx.x;
    const int64_t unit = xcd_major(blockIdx.x, gridDim.x);
    const int64_t row = unit / a.nchunks;
    const int ch = (int)(unit % a.nchunks);
    const int64_t c0 = (int64_t)ch * a.chunk_cols;
    const int64_t c1 = std::min(a.V_local, c0 + a.chunk_cols);
    const char *zrow = static_cast<const char *>(a.logits) + row * a.ld * In::kSize;
    char *grow = static_cast<char *>(a.grad) + row * a.ldg * kOutSize;
    // vectors start at the first 16-byte boundary of the logits at or after
    // c0 (the host only takes this kernel when the gradient row is then
    // aligned for its vector stores too); the head joins the scalar tail
    const int64_t v0 = c0 + head_elems<In::kSize, EPV>(zrow + c0 * In::kSize, c1 - c0);
    const int64_t nv = (c1 - v0) / EPV;
    const int64_t tail0 = v0 + nv * EPV;
    const int64_t nscalar = (v0 - c0) + (c1 - tail0);
    auto scalar_col = [&](int64_t k) { return k < v0 - c0 ? c0 + k : tail0 + (k - (v0 - c0)); };

    const ce_row_final f = a.fin[row];
    if (f.status != 1) {
        float zero[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) zero[e] = 0.0f;
        for (int64_t vi = tid; vi < nv; vi += THREADS) St::put(grow + (v0 + vi * EPV) * kOutSize, zero);
        for (int64_t k = tid; k < nscalar; k += THREADS)
            Store<OUT, 1>::put(grow + scalar_col(k) * kOutSize, zero);
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
            if (vi < nv) v[u].template load<true>(zrow + (v0 + vi * EPV) * In::kSize);
        }
        const bool t_here = tc >= v0 + base * EPV && tc < v0 + (base + (int64_t)UNROLL * THREADS) * EPV;
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int64_t vi = base + (int64_t)u * THREADS + tid;
            if (vi >= nv) continue;
            const int64_t col = v0 + vi * EPV;
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
    for (int64_t k = tid; k < nscalar; k += THREADS) {
        const int64_t col = scalar_col(k);
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

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 4;

// Long chunks without smoothing: 128 threads x 16 vectors per thread, more
// rows in flight per CU and a cheaper workgroup reduction (16384 x 128256
// bf16 forward: 723 -> 631 us against 256 x 4 with default loads; 256 x 8:
// 669, 64 x 16: 644).  The smoothed online form (fp64 exponentials) would
// need 200+ VGPRs in this shape and keeps 256 x 4.
constexpr int kLongStatsThreads = 128;
constexpr int kLongStatsUnroll = 16;
constexpr int64_t kLongStatsMinVecs = 4096;

template <int IN, bool LS>
static void stats_dispatch(const StatsArgs &a, bool vec, dim3 grid, hipStream_t stream) {
    constexpr int EPV = Elem<IN>::kVec;
    if (!LS && vec && a.chunk_cols / EPV >= kLongStatsMinVecs)
        hipLaunchKernelGGL((k_stats<IN, EPV, kLongStatsThreads, kLongStatsUnroll, LS>), grid,
                           dim3(kLongStatsThreads), 0, stream, a);
    else if (vec)
        hipLaunchKernelGGL((k_stats<IN, EPV, kStreamThreads, kStreamUnroll, LS>), grid,
                           dim3(kStreamThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((k_stats<IN, 1, kStreamThreads, 16, LS>), grid, dim3(kStreamThreads),
                           0, stream, a);
}

// The table's device address on the stream's device (each GPU holds its own
// copy of the code object's array), looked up once per device.
hipError_t exp_table_address(hipStream_t stream, const double **out) {
    static std::mutex mu;
    static const double *addr[kMaxDevices] = {};
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    int dev = cur;
    if (stream) {
        hipDevice_t sdev = 0;
        if ((e = hipStreamGetDevice(stream, &sdev)) != hipSuccess) return e;
        dev = (int)sdev;
    }
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(kExpTable));
        if (dev != cur) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = static_cast<const double *>(p);
    }
    *out = addr[dev];
    return hipSuccess;
}

hipError_t launch_stats(const StatsArgs &a, int in_dt, bool vec, hipStream_t stream) {
    const dim3 grid((unsigned)(a.T * a.nchunks));
    const bool ls = a.smoothing != 0;
    if (ls && vec && in_dt == CE_BF16 && a.exp_tab) {
        // as many workgroups as the device holds at once, with the units
        // spread evenly over them
        auto kern = k_stats_tab<kStreamThreads, kStreamUnroll>;
        static std::atomic<int> slot_cache[kMaxDevices];
        int64_t slots = 0;
        const hipError_t e = device_slots((const void *)kern, kStreamThreads, 0, slot_cache, &slots);
        if (e != hipSuccess) return e;
        const int64_t units = a.T * a.nchunks;
        const int64_t per_wg = (units + slots - 1) / slots;
        const int64_t wgs = (units + per_wg - 1) / per_wg;
        hipLaunchKernelGGL(kern, dim3((unsigned)wgs), dim3(kStreamThreads), 0, stream, a, a.exp_tab);
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
    const dim3 grid((unsigned)((a.T + kMergeThreads - 1) / kMergeThreads + (a.count ? 1 : 0)));
    hipLaunchKernelGGL(k_merge, grid, dim3(kMergeThreads), 0, stream, a);
    return hipGetLastError();
}

// Long chunks take 1024 threads x 8 vectors, so a 64128-column bf16 row is in
// flight whole before its first store (a 16384 x 64128 shard: 796 -> 722 us
// against 256 x 4); shorter chunks keep 256 x 4, which leaves more workgroups.
constexpr int kLongGradThreads = 1024;
constexpr int kLongGradUnroll = 8;
constexpr int64_t kLongGradMinVecs = 4096;

template <int IN, int OUT, bool LS>
static void grad_dispatch(const GradArgs &a, bool vec, dim3 grid, hipStream_t stream) {
    constexpr int EPV = Elem<IN>::kVec;
    if (vec && a.chunk_cols / EPV >= kLongGradMinVecs)
        hipLaunchKernelGGL((k_grad<IN, OUT, EPV, kLongGradThreads, kLongGradUnroll, LS>), grid,
                           dim3(kLongGradThreads), 0, stream, a);
    else if (vec)
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
