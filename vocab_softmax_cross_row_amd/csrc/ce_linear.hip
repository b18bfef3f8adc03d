// Cross-entropy of a linear classifier: the logits Z = E C^T are formed tile
// by tile on the matrix cores and never stored (apple/ml-cross-entropy issue
// #14, linear_cross_entropy(embeddings, classifier, labels)).
//
// Every product here is out[M, N] = A[M, K] B[N, K]^T with bf16 operands and
// fp32 accumulation on v_mfma_f32_16x16x32_bf16.  Operands are kept in a
// "fragment-major" layout: the matrix is cut into blocks of 16 rows x 32
// K-columns (1 KB), block (rb, kb) at byte (rb * Ks/32 + kb) * 1024 where Ks
// is the stored (padded) K, and inside a block lane L's 16 bytes at L * 16
// hold row rb*16 + L%16, K-columns kb*32 + 8*(L/16) .. +7 -- exactly the
// A or B register fragment of that MFMA.  One 16-byte load per lane moves a
// block as 1 KB of contiguous memory, straight into operand registers (A) or
// into LDS unchanged (B), where one conflict-free ds_read_b128 reads it back
// as a fragment.  Padding (rows to a multiple of 256, K to a multiple of 64)
// is zero, so loads need no bounds checks.
//
// Accumulator layout of v_mfma_f32_16x16x32_bf16 (16 x 16 fp32, 4 values
// per lane): register r of lane l holds row 4*(l/16) + r, column l%16.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "ce_device.h"
#include "ce_launch.h"

namespace vce {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGT = 256;                 // 4 waves, each 64 rows x 256 columns of the tile
constexpr int kTile = 256;               // output tile 256 x 256
constexpr int kBK = 64;                  // K per LDS stage
constexpr int kStage = 8 * 4 * 1024;     // one B stage in LDS: 8 row blocks x 4 K blocks
constexpr int kSuperM = 8, kSuperN = 4;  // 32 tiles one XCD works on together

struct LinRow {
    GradConst c;
    int32_t t;     // target class
    int32_t valid; // 1 if the row has a gradient
};
static_assert(sizeof(LinRow) == kLinRowBytes, "row constant size");
constexpr int kStages = 4;             // B stage buffers in LDS
static_assert(kGemmLdsBytes >= kStages * kStage + kTile * (int)sizeof(LinRow), "LDS budget");

__device__ __forceinline__ int64_t frag_off(int64_t rb, int64_t kb, int64_t Ks) {
    return (rb * (Ks / 32) + kb) * 1024;
}

// ---------------------------------------------------------------------------
// Re-layout of a row-major bf16 matrix X [R, K] (leading dimension ld, K a
// multiple of 8) into fragment-major form, padded to [Rp, Kp] with zeros.
// One thread writes one 16-byte fragment slot.
// ---------------------------------------------------------------------------
constexpr int kRelayoutThreads = 256;

__global__ __launch_bounds__(kRelayoutThreads) void k_relayout(RelayoutArgs a) {
    const int64_t s = (int64_t)blockIdx.x * kRelayoutThreads + threadIdx.x;
    if (s >= a.Rp * a.Kp / 8) return;
    const int64_t blk = s / 64;
    const int L = (int)(s % 64);
    const int64_t rb = blk / (a.Kp / 32), kb = blk % (a.Kp / 32);
    const int64_t r = rb * 16 + (L & 15);
    const int64_t k = kb * 32 + 8 * (L >> 4);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < a.R && k < a.K) v = *reinterpret_cast<const u32x4 *>(a.X + r * a.ld + k);
    *reinterpret_cast<u32x4 *>(a.Y + s * 8) = v;
}

// Transposed re-layout: Y = fragment-major form of X^T, padded to [Rp, Kp]
// (Y's rows are X's columns, Y's K is X's rows).  A workgroup moves a
// 64 x 64 tile through LDS: 16-byte row loads of X, 16-byte slot stores of Y.
// With Yn, the same loads also give the plain fragment-major form of X
// (rows padded to Kp, K padded to Kn): each 16-byte row load is one of its
// fragment slots, so X is read once for both forms.
__global__ __launch_bounds__(kRelayoutThreads) void k_relayout_t(RelayoutArgs a, uint16_t *Yn,
                                                                 int64_t Kn) {
    __shared__ uint16_t t[64][64 + 2];
    const int tid = threadIdx.x;
    const int64_t tiles_y = a.Rp / 64;                        // tiles along Y rows
    const int64_t x0 = (int64_t)(blockIdx.x / tiles_y) * 64; // X rows = Y K-columns
    const int64_t y0 = (int64_t)(blockIdx.x % tiles_y) * 64; // X cols = Y rows
    if (x0 >= a.Kp) return;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int slot = tid + q * kRelayoutThreads;
        const int lr = slot / 8, lc = (slot % 8) * 8;
        const int64_t r = x0 + lr, c = y0 + lc;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (r < a.R && c < a.K) v = *reinterpret_cast<const u32x4 *>(a.X + r * a.ld + c);
        if (Yn && c < Kn) {
            // lane (r % 16) + 16 ((c / 8) % 4) of block (r / 16, c / 32)
            const int L = (int)(r & 15) + 16 * (int)((c >> 3) & 3);
            *reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(Yn) + frag_off(r >> 4, c >> 5, Kn) +
                                       L * 16) = v;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            t[lr][lc + 2 * e] = (uint16_t)(v[e] & 0xffffu);
            t[lr][lc + 2 * e + 1] = (uint16_t)(v[e] >> 16);
        }
    }
    __syncthreads();
    // 4 row blocks x 2 K blocks of Y = 512 slots, 2 per thread
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int slot = tid + q * kRelayoutThreads;
        const int b = slot / 64, L = slot % 64;
        const int brow = b / 2, bk = b % 2;
        const int yr = brow * 16 + (L & 15);   // Y row in the tile  (X column)
        const int yk = bk * 32 + 8 * (L >> 4); // Y K in the tile    (X row)
        u32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            v[e] = (uint32_t)t[yk + 2 * e][yr] | ((uint32_t)t[yk + 2 * e + 1][yr] << 16);
        const int64_t off = frag_off((y0 >> 4) + brow, (x0 >> 5) + bk, a.Kp);
        *reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(a.Y) + off + L * 16) = v;
    }
}

// ---------------------------------------------------------------------------
// Per-row gradient constants after the merge.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_linear_rowconst(LinRowArgs a) {
    const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (r >= a.N) return;
    const ce_row_final f = a.fin[r];
    LinRow o;
    o.t = (int32_t)a.target[r];
    o.valid = (f.status == 1) ? 1 : 0;
    o.c = GradConst{};
    if (o.valid) {
        const double k = row_scale(a.reduction, a.grad_output, a.n_valid, r);
        o.c = grad_constants(f.lse, f.gt, k, (double)a.eps, (double)a.V);
    }
    reinterpret_cast<LinRow *>(a.rows)[r] = o;
}

// ---------------------------------------------------------------------------
// The GEMM, with its epilogues.
// ---------------------------------------------------------------------------

// Reductions over each group of 16 lanes (a DPP row), the result in all 16:
// swap neighbours, swap pairs, mirror within 8, mirror within 16.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, dpp_f<0xB1>(x));  // quad_perm [1, 0, 3, 2]
    x = fmaxf(x, dpp_f<0x4E>(x));  // quad_perm [2, 3, 0, 1]
    x = fmaxf(x, dpp_f<0x141>(x)); // row_half_mirror
    return fmaxf(x, dpp_f<0x140>(x)); // row_mirror
}
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_f<0xB1>(x);
    x += dpp_f<0x4E>(x);
    x += dpp_f<0x141>(x);
    return x + dpp_f<0x140>(x);
}

// Tile of workgroup b.  Workgroups go round-robin over the 8 XCDs; the 32
// consecutive workgroups of one XCD get one 8 x 4 super-tile (8 row tiles,
// 4 column tiles), so they share its A and B blocks in that XCD's L2.  Each
// B block then serves 8 tiles: B is the large operand of the forward and G
// products (the classifier, beyond the last-level cache), so this halves its
// HBM reads against 4 x 8.  False for the padding workgroups.
__device__ __forceinline__ bool tile_of(int64_t b, int tiles_m, int tiles_n, int &tm, int &tn) {
    const int64_t x = b % kXcds, j = b / kXcds;
    const int64_t s = (j / (kSuperM * kSuperN)) * kXcds + x;
    const int pos = (int)(j % (kSuperM * kSuperN));
    const int64_t sn_count = (tiles_n + kSuperN - 1) / kSuperN;
    const int64_t sm = s / sn_count, sn = s % sn_count;
    tm = (int)(sm * kSuperM + pos / kSuperN);
    tn = (int)(sn * kSuperN + pos % kSuperN);
    return tm < tiles_m && tn < tiles_n;
}

// Number of tile ids tile_of walks: whole groups of 8 super-tiles (one per
// XCD), padding included.
__host__ __device__ __forceinline__ int64_t tile_ids(int tiles_m, int tiles_n) {
    const int64_t supers = (int64_t)((tiles_m + kSuperM - 1) / kSuperM) * ((tiles_n + kSuperN - 1) / kSuperN);
    return (supers + kXcds - 1) / kXcds * kXcds * kSuperM * kSuperN;
}

// One 256 x 256 output tile: main loop and epilogue.  FILT (gradient
// filtering): for the G product, record whether the tile keeps any entry;
// for the backward products, walk only the K tiles listed for this output
// row tile (the kept 256-wide blocks of G), 4 stages each.
template <int EPI, bool LS, bool FILT>
__device__ __forceinline__ void gemm_tile(const GemmArgs &g, int tm, int tn, char *lbase) {
    // opaque per tile: values derived from the thread index are not hoisted
    // out of the tile loop, where they would stay live through every tile
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t row0 = (int64_t)tm * kTile, col0 = (int64_t)tn * kTile;

    // the 256 rows (16 row blocks) of A and of B this tile reads, as buffer resources
    const int64_t a_span = (int64_t)kTile * g.a_ks * 2, b_span = (int64_t)kTile * g.b_ks * 2;
    const char *abase = reinterpret_cast<const char *>(g.A) + (int64_t)tm * a_span;
    const char *bbase = reinterpret_cast<const char *>(g.B) + (int64_t)tn * b_span;
    const __amdgpu_buffer_rsrc_t ra =
        __builtin_amdgcn_make_buffer_rsrc((void *)abase, 0, (int)a_span, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb =
        __builtin_amdgcn_make_buffer_rsrc((void *)bbase, 0, (int)b_span, 0x00020000);
    int nk = (int)(g.K / kBK);
    const int a_kbs = (int)(g.a_ks / 32), b_kbs = (int)(g.b_ks / 32);
    // the filtered K walk belongs to the backward products only; the G
    // product with FILT records keep flags and walks all of K
    constexpr bool kWalk = FILT && (EPI == GEMM_STORE || EPI == GEMM_ADD || EPI == GEMM_KAHAN);

    // Filtered K walk: the kept 256-wide K tiles of this output row tile are
    // copied into LDS after the stage buffers (free during the main loop),
    // and stage kt reads stored stage kstage(kt) = 4 list[kt/4] + kt%4.
    // km1 / km2 hold kstage(kt + 1) and kstage(kt + 2) while stage kt runs;
    // each list entry is read from LDS one stage before it is needed.
    uint16_t *klds = reinterpret_cast<uint16_t *>(lbase + kStages * kStage);
    if constexpr (kWalk) {
        nk = 4 * g.kcnt[tm];
        const uint16_t *src = g.klist + (int64_t)tm * g.klist_pitch;
        for (int i = tid; i < nk / 4; i += kGT) klds[i] = src[i];
        __syncthreads();
        if (nk == 0) {
            // every K tile dropped: the product is zero; an addition of zero
            // is skipped, a store (or the first addition) writes zeros
            if constexpr (EPI == GEMM_ADD || EPI == GEMM_KAHAN) {
                if (!g.first) return;
            }
        }
    }
    auto kstage = [&](int kt) -> int {
        if constexpr (kWalk) {
            return 4 * __builtin_amdgcn_readfirstlane((int)klds[kt >> 2]) + (kt & 3);
        } else {
            return kt;
        }
    };

    // Wave w owns rows 64w .. 64w+63 of the tile (16-row blocks 4w .. 4w+3)
    // and all 256 columns: 4 x 16 accumulators of 16 x 16.  A stage is
    // 64 K deep, two K steps of 32; it is walked as 32 positions (K step
    // p / 16, column block p % 16), each 4 MFMAs, one per row block.
    // - A fragments are the wave's own: global memory straight into operand
    //   registers, each K step's four reloaded with the next stage right
    //   after the step's last MFMAs, so a load has half a stage to land.
    // - B is shared by the four waves: global -> LDS directly (buffer loads
    //   with the LDS as destination, no registers), four stage buffers
    //   (stage kt in buffer kt % 4).  Each lane owns 8 slots of 16 bytes per
    //   stage (row blocks 4w .. 4w+3, both K blocks); positions 0..7 of
    //   stage kt load the slots of stage kt+2, so a load has a stage and a
    //   half to land.
    // - B fragments are read from LDS kAhead positions before their MFMAs,
    //   one read per position, across the stage boundary too: a rolling
    //   window of kAhead + 1 fragments instead of two full sets.
    // - One barrier per stage, at position 32 - kAhead, just before the
    //   first read of stage kt+1's buffer: it first waits for this wave's
    //   slot loads of stage kt+1 (issued in stage kt-1; vector memory loads
    //   complete in order, so the loads issued after them may stay in
    //   flight), so the read sees every wave's slots.  A buffer is loaded
    //   again (stage kt+4, in stage kt+2) only after every wave has used its
    //   fragments in MFMAs and passed stage kt+1's barrier, so no load can
    //   overtake a read.
    // - Each MFMA is followed by at most one memory instruction
    //   (sched_group_barrier), so the matrix pipe never waits behind a
    //   burst of them.
    // Only B passes through LDS: half the LDS traffic of a 2 x 2 wave
    // layout.  Moving B is the dearest part of the loop: without its loads
    // and LDS writes the product would take 20% less time (measured), and
    // the direct-to-LDS form is cheaper than staging through registers.  A bf16 GEMM on this chip runs at a power-limited clock, and
    // the 16 x 16 x 32 instruction costs less energy per flop than the
    // 32 x 32 x 16 one (with random operands, MFMAs alone sustain 1.99
    // against 1.75 PFLOP/s, at 1.92 against 1.67 GHz).
    constexpr int kAhead = 8;
    bf16x8 fa[4][2]; // [row block][K step]
    // ks: stored stage index (kstage of the loop's stage)
    auto load_a = [&](int ks, int i, int st) {
        fa[i][st] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                        ra, lane * 16, ((4 * wave + i) * a_kbs + g.a_kb0 + ks * 2 + st) * 1024, 0));
    };
    // slot q of stage ks into buffer buf: each lane's 16 bytes land at its
    // own place in the 1 KB block (the wave-uniform block address goes to M0)
    typedef __attribute__((address_space(3))) void lds_void_t;
    auto load_b = [&](int ks, int buf, int q) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rb, (lds_void_t *)(lbase + buf * kStage + ((4 * wave + (q >> 1)) * 2 + (q & 1)) * 1024), 16,
            lane * 16, ((4 * wave + (q >> 1)) * b_kbs + g.b_kb0 + ks * 2 + (q & 1)) * 1024, 0, 0);
    };
    // the B fragment of position p of a stage buffer
    auto read_b = [&](int buf, int p) {
        return *reinterpret_cast<const bf16x8 *>(lbase + buf * kStage + ((p & 15) * 2 + (p >> 4)) * 1024 +
                                                 lane * 16);
    };
    f32x4 acc[4][16];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0f;
    bf16x8 carry[kAhead]; // B fragments of the next stage's first positions
    int km1 = 1, km2 = 2;
    if (nk > 0) {
    const int k0 = kstage(0);
    if constexpr (kWalk) {
        km1 = kstage(1);
        km2 = kstage(2);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) load_b(k0, 0, q);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int st = 0; st < 2; ++st) load_a(k0, i, st);
    if (nk > 1) {
#pragma unroll
        for (int q = 0; q < 8; ++q) load_b(km1, 1, q);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
#pragma unroll
    for (int x = 0; x < kAhead; ++x) carry[x] = read_b(0, x);

    // MORE1: stage kt+1 exists (load its A, read its first B fragments);
    // MORE2: stage kt+2 exists (load its B).  The flags are
    // compile-time so the loop body has no branches and every wait before a
    // use stays a constant count of later loads.
    auto run_stage = [&](int kt, auto MORE1, auto MORE2) {
        constexpr bool more1 = decltype(MORE1)::value, more2 = decltype(MORE2)::value;
        const int cb = kt % kStages, nb = (kt + 1) % kStages;
        // stored stage indices of stages kt + 1 and kt + 2
        const int s1 = kWalk ? km1 : kt + 1, s2 = kWalk ? km2 : kt + 2;
        bf16x8 f[32 + kAhead];
#pragma unroll
        for (int x = 0; x < kAhead; ++x) f[x] = carry[x];
#pragma unroll
        for (int p = 0; p < 32; ++p) {
            __builtin_amdgcn_sched_barrier(0);
            if (p == 32 - kAhead && more1) {
                // issued after this wave's slot loads of stage kt+1 (stage
                // kt-1, positions 0..7): stage kt-1's 8 A loads, this
                // stage's 8 slot loads when stage kt+2 exists, and this
                // stage's 4 A loads of position 15
                static_assert(32 - kAhead > 15, "the barrier follows position 15's A loads");
                if constexpr (more2) asm volatile("s_waitcnt vmcnt(20)\n\ts_barrier" ::: "memory");
                else asm volatile("s_waitcnt vmcnt(12)\n\ts_barrier" ::: "memory");
            }
            const int pr = p + kAhead;
            const bool rd = pr < 32 || more1;
            if (pr < 32) f[pr] = read_b(cb, pr);
            else if (more1) f[pr] = read_b(nb, pr - 32);
            const bool ld = p < 8 && more2;
            if (ld) load_b(s2, (kt + 2) % kStages, p);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[i][p & 15] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i][p >> 4], f[p],
                                                                         acc[i][p & 15], 0, 0, 0);
            const bool lda = (p & 15) == 15 && more1;
            if (lda) {
#pragma unroll
                for (int i = 0; i < 4; ++i) load_a(s1, i, p >> 4);
            }
            // issue order: MFMA, LDS read; MFMA; MFMA, B load; MFMA, the
            // four A loads
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (rd) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (ld) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (lda) __builtin_amdgcn_sched_group_barrier(0x020, 4, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (more1) {
#pragma unroll
            for (int x = 0; x < kAhead; ++x) carry[x] = f[32 + x];
        }
        if constexpr (kWalk) {
            // the next stage's pair (stage kt + 3 read from the list now)
            km1 = km2;
            if (kt + 3 < nk) km2 = kstage(kt + 3);
        }
    };
    using Yes = std::true_type;
    using No = std::false_type;
    // The first stage is peeled off so that the loop is entered with its
    // loads outstanding in the loop's own order, and the waits in the loop
    // stay the counts the steady state needs.
    if (nk >= 3) {
        run_stage(0, Yes{}, Yes{});
        for (int kt = 1; kt + 2 < nk; ++kt) run_stage(kt, Yes{}, Yes{});
    }
    if (nk >= 2) run_stage(nk - 2, Yes{}, No{});
    run_stage(nk - 1, No{}, No{});
    } // nk > 0
    // Every accumulator is pinned here.  MFMAs touch no memory, so a barrier
    // alone does not keep them above the epilogue: the compiler has sunk the
    // last ones into the epilogue, among its LDS writes of accumulators, and
    // a write issued that soon after the MFMA producing its source read a
    // stale value (the hazard padding inserted for it was too short).
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) asm volatile("" : "+a"(acc[i][j]));
    // and 32 wait states on top of the compiler's own padding, whatever the
    // order of the last position's MFMAs (once per tile)
#pragma unroll
    for (int q = 0; q < 4; ++q) asm volatile("s_nop 7");
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads(); // every wave is done with the operand stages

    // Epilogues work on one block e of 32 rows x 128 columns per wave at a
    // time: rows 64w + 32 (e/2) .., columns 128 (e%2) .. of the tile, staged
    // through the wave's own LDS slab so that the row-wise work and the
    // global accesses are contiguous: lanes 16q..16q+15 then own row
    // 4*it + q of the block and 8 consecutive columns each.
    constexpr int kPitch = 132; // floats per slab row (keeps 16-byte reads spread over banks)
    float *slab = reinterpret_cast<float *>(lbase) + wave * 32 * kPitch;
    const int sub = lane >> 4, c8 = (lane & 15) * 8; // row-pass lane role
    // accumulator (i, j) register r of lane l: tile row 16 i + 4 (l / 16) + r
    // of the wave's rows, column 16 j + l % 16
    auto stage = [&](int e) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii)
#pragma unroll
            for (int jj = 0; jj < 8; ++jj)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    slab[(16 * ii + 4 * sub + r) * kPitch + jj * 16 + (lane & 15)] =
                        acc[2 * (e >> 1) + ii][8 * (e & 1) + jj][r];
    };
    auto blk_row = [&](int e) { return wave * 64 + (e >> 1) * 32; }; // first tile row of block e
    auto blk_col = [&](int e) { return (e & 1) * 128; };            // first tile column

    if constexpr (EPI == GEMM_STATS) {
        // Per row of the tile: max and sum of exp over this tile's columns
        // with the target left out, the target logit, the sum of all
        // logits.  Straight from the accumulators: lane l holds, for row
        // block i and register r, tile row 64 w + 16 i + 4 (l / 16) + r at
        // the 16 columns 16 j + l % 16, so the 16 lanes of a DPP row hold a
        // tile row's 256 columns between them: a pass over 16 registers and
        // a 16-lane reduction, four rows at a time.
        const int q4 = lane >> 4, cl = lane & 15;
        int32_t *t_l = reinterpret_cast<int32_t *>(lbase); // [256] target column or -1
        {
            const int64_t r = row0 + tid;
            int32_t tl = -1;
            if (r < g.M) {
                const int64_t t = g.target[r] - g.col_base - col0;
                if (t >= 0 && t < kTile && col0 + t < g.N) tl = (int32_t)t;
            }
            t_l[tid] = tl;
        }
        __syncthreads();
        const bool full = col0 + kTile <= g.N;
        const int ncol = full ? kTile : (int)(g.N - col0); // columns inside N
        // pairwise sums and maxima of 16 registers
        auto tree_sum = [](const float *x) {
            float a[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) a[k] = x[k] + x[k + 8];
#pragma unroll
            for (int k = 0; k < 4; ++k) a[k] += a[k + 4];
            return (a[0] + a[2]) + (a[1] + a[3]);
        };
        auto tree_max = [](const float *x) {
            float a[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) a[k] = fmaxf(x[k], x[k + 8]);
#pragma unroll
            for (int k = 0; k < 4; ++k) a[k] = fmaxf(a[k], a[k + 4]);
            return fmaxf(fmaxf(a[0], a[2]), fmaxf(a[1], a[3]));
        };
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float v[4][16];
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int j = 0; j < 16; ++j) v[r][j] = acc[i][j][r];
            float m[4], sm[4], sz[4], zt[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (!full) {
#pragma unroll
                    for (int j = 0; j < 16; ++j)
                        if (16 * j + cl >= ncol) v[r][j] = LS ? 0.0f : ninf();
                }
                sz[r] = LS ? tree_sum(v[r]) : 0.0f; // every column inside N, the target too
                if (LS && !full) {
#pragma unroll
                    for (int j = 0; j < 16; ++j)
                        if (16 * j + cl >= ncol) v[r][j] = ninf();
                }
                zt[r] = 0.0f;
                const int tcol = t_l[wave * 64 + 16 * i + 4 * q4 + r];
                // the target's column is held by the lane with l % 16 = tcol % 16
                if (__builtin_expect(tcol >= 0 && (tcol & 15) == cl, 0)) {
                    const int jt = tcol >> 4;
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        if (j == jt) {
                            zt[r] = v[r][j];
                            v[r][j] = ninf();
                        }
                    }
                }
                m[r] = tree_max(v[r]);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) m[r] = row16_max(m[r]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float e[16];
                const float K = m[r] * kL2E;
#pragma unroll
                for (int j = 0; j < 16; ++j) e[j] = fast_exp2(fmaf(v[r][j], kL2E, -K));
                sm[r] = m[r] != ninf() ? tree_sum(e) : 0.0f;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sm[r] = row16_sum(sm[r]);
                zt[r] = row16_sum(zt[r]);
                if (LS) sz[r] = row16_sum(sz[r]);
            }
            if (cl == 0) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t row = row0 + wave * 64 + 16 * i + 4 * q4 + r;
                    if (row < g.M) {
                        LinTileStats o;
                        o.m = m[r];
                        o.s = sm[r];
                        o.zt = zt[r];
                        o.sz = sz[r];
                        g.stats[row * g.tiles_n + tn] = o;
                    }
                }
            }
        }
    } else if constexpr (EPI == GEMM_GRAD) {
        // G = k (softmax - q) of the tile, rounded to bf16 (RNE), written in
        // fragment-major form twice, straight from the accumulators (lane l
        // holds, for row block i and register r, token 64 w + 16 i + 4 (l/16)
        // + r of the tile at class 16 j + l % 16):
        // - GT (rows = classes, K = tokens): a fragment lane needs 8
        //   consecutive tokens of one class.  Lane groups q hold tokens
        //   4q .. 4q+3 of row blocks 2b and 2b+1; one v_permlane32_swap and
        //   one v_permlane16_swap per dword regroup them so that group q'
        //   holds tokens 8q' .. 8q'+7 of the 32-token block, with no LDS;
        // - G (rows = tokens, K = classes): neighbouring lanes swap one dword
        //   (DPP) to form bf16 pairs of adjacent classes of one token, which
        //   go to the wave's own token-major LDS region and are read back 16
        //   bytes (8 classes) per lane.
        constexpr int kGPitch = 528;                  // bytes per token row: 256 classes + 16 (banks)
        constexpr int kGRegion = 64 * kGPitch;        // one wave's 64 tokens
        static_assert(4 * kGRegion + kTile * (int)sizeof(LinRow) <= kGemmLdsBytes, "G epilogue LDS");
        LinRow *rc = reinterpret_cast<LinRow *>(lbase + 4 * kGRegion);
        {
            // rows past M get all-zero constants: valid = 0
            const int64_t r = row0 + tid;
            u32x4 v[3] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
            if (r < g.M) {
                const u32x4 *src = reinterpret_cast<const u32x4 *>(g.rows) + r * 3;
#pragma unroll
                for (int q = 0; q < 3; ++q) v[q] = src[q];
            }
            u32x4 *dst = reinterpret_cast<u32x4 *>(rc + tid);
#pragma unroll
            for (int q = 0; q < 3; ++q) dst[q] = v[q];
        }
        __syncthreads();
        char *GT = reinterpret_cast<char *>(g.GT);
        char *G = reinterpret_cast<char *>(g.G);
        char *greg = lbase + wave * kGRegion;
        const int q4 = lane >> 4, cl = lane & 15;
        const bool odd = (cl & 1) != 0;
        const bool full = col0 + kTile <= g.N;
        const int ncol = full ? kTile : (int)(g.N - col0); // classes inside N
        // gradient filtering: whether this lane saw an entry of a valid row
        // with k != 0 and |G| >= filter_eps |k| (|p - q| >= filter_eps
        // unscaled); a row with k = 0 has an all-zero gradient and keeps
        // nothing
        bool kept = false;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            // D[ii][j]: tokens (4q, 4q+1) and (4q+2, 4q+3) of row block
            // 2 tb + ii at class 16 j + l % 16, as bf16 pairs
            uint32_t D[2][16][2];
#pragma unroll
            for (int ii = 0; ii < 2; ++ii) {
                const int i = 2 * tb + ii;
                float gv[4][16];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const LinRow R = rc[wave * 64 + 16 * i + 4 * q4 + r];
#pragma unroll
                    for (int j = 0; j < 16; ++j) gv[r][j] = grad_elem<CE_BF16, LS>(acc[i][j][r], R.c);
                    if (!full) {
#pragma unroll
                        for (int j = 0; j < 16; ++j)
                            if (16 * j + cl >= ncol) gv[r][j] = 0.0f;
                    }
                    // the target's class is held by the lane with l % 16 = t % 16
                    const int64_t tcl = (int64_t)R.t - g.col_base - col0;
                    if (__builtin_expect(tcl >= 0 && tcl < ncol && (int)(tcl & 15) == cl, 0)) {
                        const int jt = (int)(tcl >> 4);
#pragma unroll
                        for (int j = 0; j < 16; ++j)
                            if (j == jt) gv[r][j] = R.c.gk;
                    }
                    if (!R.valid) {
#pragma unroll
                        for (int j = 0; j < 16; ++j) gv[r][j] = 0.0f;
                    }
                    if constexpr (FILT) {
                        const float thr = g.filter_eps * fabsf(R.c.k);
                        float mx = 0.0f;
#pragma unroll
                        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, fabsf(gv[r][j]));
                        kept = kept || (R.valid && R.c.k != 0.0f && mx >= thr);
                    }
                }
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    D[ii][j][0] = pack_bf16x2(gv[0][j], gv[1][j]);
                    D[ii][j][1] = pack_bf16x2(gv[2][j], gv[3][j]);
                }
            }
            // GT fragments of the 32-token block tb: class block j, lane l
            // at byte 16 l of the fragment (class l % 16, tokens 8 (l/16) ..)
            const int64_t n0 = row0 + wave * 64 + 32 * tb;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const auto s0 = __builtin_amdgcn_permlane32_swap(D[0][j][0], D[1][j][0], false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap(D[0][j][1], D[1][j][1], false, false);
                const auto x0 = __builtin_amdgcn_permlane16_swap(s0[0], s0[1], false, false);
                const auto x1 = __builtin_amdgcn_permlane16_swap(s1[0], s1[1], false, false);
                const u32x4 w = {(uint32_t)x0[0], (uint32_t)x1[0], (uint32_t)x0[1], (uint32_t)x1[1]};
                const int64_t c = col0 + 16 * j;
                *reinterpret_cast<u32x4 *>(GT + frag_off(c >> 4, n0 >> 5, g.ldgt) + lane * 16) = w;
            }
            // G: pairs of adjacent classes of one token into the LDS region;
            // an even lane writes tokens 4q, 4q+1 at classes (c, c+1), an
            // odd lane tokens 4q+2, 4q+3 at classes (c-1, c)
#pragma unroll
            for (int ii = 0; ii < 2; ++ii) {
                const int tok = 16 * (2 * tb + ii) + 4 * q4 + (odd ? 2 : 0);
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const uint32_t p0 = D[ii][j][0], p1 = D[ii][j][1];
                    const uint32_t give = odd ? p0 : p1, own = odd ? p1 : p0;
                    const uint32_t got = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)give, 0xB1, 0xf, 0xf, false);
                    const uint32_t lo = odd ? got : own, hi = odd ? own : got; // lower class first
                    const uint32_t w0 = (lo & 0xffffu) | (hi << 16);
                    const uint32_t w1 = (lo >> 16) | (hi & 0xffff0000u);
                    char *d = greg + tok * kGPitch + (16 * j + (cl & ~1)) * 2;
                    *reinterpret_cast<uint32_t *>(d) = w0;
                    *reinterpret_cast<uint32_t *>(d + kGPitch) = w1;
                }
            }
        }
        // the region is this wave's alone: its LDS writes and reads stay in
        // order, and the compiler may not move the reads above the writes
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // G fragments: token block tk (16 tokens), class block s (32
        // classes), lane l at byte 16 l (token l % 16, classes 8 (l/16) ..)
#pragma unroll
        for (int tk = 0; tk < 4; ++tk) {
            const int64_t n = row0 + wave * 64 + 16 * tk;
#pragma unroll
            for (int sb = 0; sb < 8; ++sb) {
                const u32x4 w = *reinterpret_cast<const u32x4 *>(
                    greg + (16 * tk + cl) * kGPitch + (32 * sb + 8 * q4) * 2);
                const int64_t v0 = col0 + 32 * sb;
                *reinterpret_cast<u32x4 *>(G + frag_off(n >> 4, v0 >> 5, g.ldg) + lane * 16) = w;
            }
        }
        if constexpr (FILT) {
            // one flag per wave (its 64 rows of the tile); the list kernel ORs them
            const bool any = __builtin_amdgcn_ballot_w64(kept) != 0;
            if (lane == 0)
                g.keep_flags[((int64_t)tm * g.tiles_n + tn) * 4 + wave] = any ? 1 : 0;
        }
    } else {
        // plain fp32 result: store, add, or add with Kahan compensation;
        // lanes write 16 bytes, a row's 128 columns are 512 contiguous bytes
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            __syncthreads();
            stage(e);
            __syncthreads();
#pragma unroll 2
            for (int it = 0; it < 8; ++it) {
                const int rl = 4 * it + sub;
                const int64_t row = row0 + blk_row(e) + rl;
                const int64_t col = col0 + blk_col(e) + c8;
                if (row >= g.M || col >= g.N) continue;
                const float *src = slab + rl * kPitch + c8;
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    u32x4 a = *reinterpret_cast<const u32x4 *>(src + 4 * hh);
                    u32x4 *o = reinterpret_cast<u32x4 *>(g.out + row * g.ldo + col + 4 * hh);
                    if constexpr (EPI == GEMM_STORE) {
                        *o = a;
                    } else if constexpr (EPI == GEMM_ADD) {
                        if (!g.first) {
                            const u32x4 b = *o;
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                a[e] = __float_as_uint(__uint_as_float(a[e]) + __uint_as_float(b[e]));
                        }
                        *o = a;
                    } else {
                        u32x4 *cp = reinterpret_cast<u32x4 *>(g.comp + row * g.ldo + col + 4 * hh);
                        if (g.first) {
                            *o = a;
                            *cp = u32x4{0u, 0u, 0u, 0u};
                        } else {
                            // Kahan: c carries what earlier additions lost
                            const u32x4 sv = *o, cv = *cp;
                            u32x4 so, co;
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const float sum = __uint_as_float(sv[e]);
                                const float y = __uint_as_float(a[e]) - __uint_as_float(cv[e]);
                                const float t = sum + y;
                                co[e] = __float_as_uint((t - sum) - y);
                                so[e] = __float_as_uint(t);
                            }
                            *o = so;
                            *cp = co;
                        }
                    }
                }
            }
        }
    }
}

// Persistent: one workgroup per CU walks tile ids blockIdx.x, + gridDim.x,
// ...; the grid is a multiple of 8, so a workgroup stays on one XCD and the
// ids of a round still form one super-tile per XCD.  The G epilogue keeps
// one tile per workgroup: inside a tile loop it would not fit the registers.
template <int EPI>
constexpr bool kGemmPersistent = EPI != GEMM_GRAD;

template <int EPI, bool LS, bool FILT>
__global__ __launch_bounds__(kGT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_gemm(GemmArgs g) {
    extern __shared__ __attribute__((aligned(16))) u32x4 lds[];
    char *lbase = reinterpret_cast<char *>(lds);
    int tm, tn;
    if constexpr (!kGemmPersistent<EPI>) {
        if (tile_of(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn))
            gemm_tile<EPI, LS, FILT>(g, tm, tn, lbase);
        return;
    }
    const int64_t ids = tile_ids(g.tiles_m, g.tiles_n);
    for (int64_t b = blockIdx.x; b < ids; b += gridDim.x) {
        if (!tile_of(b, g.tiles_m, g.tiles_n, tm, tn)) continue;
        gemm_tile<EPI, LS, FILT>(g, tm, tn, lbase);
        __syncthreads(); // the epilogue's LDS is the next tile's stage buffers
    }
}

// ---------------------------------------------------------------------------
// Gradient filtering: from the G product's per-wave keep flags of one class
// chunk ([tiles_m][tiles_n][4]), the kept K tiles of each backward output
// row tile, in increasing order: for dE (row tile = token tile i) the kept
// class tiles j, for dC (row tile = class tile j) the kept token tiles i.
// One wave per list: 64 candidates at a time, a ballot, and each kept one
// written at its rank among the kept lanes below it.
// ---------------------------------------------------------------------------
constexpr int kListWaves = 4;

__global__ __launch_bounds__(kListWaves * kWave) void k_filter_lists(FilterListArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t w = (int64_t)blockIdx.x * kListWaves + (threadIdx.x >> 6);
    auto keep = [&](int64_t i, int64_t j) {
        const u32x4 f = *reinterpret_cast<const u32x4 *>(a.flags + (i * a.tiles_n + j) * 4);
        return (f[0] | f[1] | f[2] | f[3]) != 0u;
    };
    const bool for_e = w < a.tiles_m;
    if (!for_e && w >= a.tiles_m + a.tiles_n) return;
    const int64_t n = for_e ? a.tiles_n : a.tiles_m;        // candidates of this list
    uint16_t *out = for_e ? a.list_e + w * a.pitch_e : a.list_c + (w - a.tiles_m) * a.pitch_c;
    int c = 0;
    for (int64_t base = 0; base < n; base += kWave) {
        const int64_t x = base + lane;
        const bool k = x < n && (for_e ? keep(w, x) : keep(x, w - a.tiles_m));
        const uint64_t b = __builtin_amdgcn_ballot_w64(k);
        const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32),
                                                        __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
        if (k) out[c + rank] = (uint16_t)x;
        c += __builtin_popcountll(b);
    }
    if (lane == 0) {
        if (for_e)
            a.cnt_e[w] = c;
        else
            a.cnt_c[w - a.tiles_m] = c;
    }
}

// ---------------------------------------------------------------------------
// Merge of the per-tile statistics of each row ([M][S], row-major) and the
// finalize: one wave per row, shards spread over the lanes, combined by a
// fixed butterfly (deterministic).  Same merge and finalize as the shard
// merge: M = max m_k, s = sum s_k exp(m_k - M), zt, own and sz summed.
// ---------------------------------------------------------------------------
constexpr int kMergeWaves = 4;

__global__ __launch_bounds__(kMergeWaves * kWave) void k_linear_merge(LinMergeArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t r = (int64_t)blockIdx.x * kMergeWaves + (threadIdx.x >> 6);
    if (r >= a.N) return;
    const LinTileStats *in = a.stats + r * a.S;
    float m = ninf();
    for (int k = lane; k < a.S; k += kWave) m = fmaxf(m, in[k].m);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
    const double M = (double)m;
    double s = 0.0, zt = 0.0, sz = 0.0;
    for (int k = lane; k < a.S; k += kWave) {
        const LinTileStats p = in[k];
        if (p.m != ninf()) s += (double)p.s * exp((double)p.m - M);
        zt += (double)p.zt; // 0 except in the tile that holds the target
        sz += (double)p.sz;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        s += __shfl_xor(s, o, kWave);
        zt += __shfl_xor(zt, o, kWave);
        sz += __shfl_xor(sz, o, kWave);
    }
    if (lane != 0) return;
    const int64_t t = a.target[r];
    // a target in [0, V) lies in exactly one tile, which recorded its logit
    const int own = (t >= 0 && t < a.V) ? 1 : 0;
    ce_row_final fo;
    fo.lse = 0.0;
    fo.gt = 0.0;
    fo.m = 0.0f;
    float loss;
    if (t == a.ignore_index) {
        fo.status = 0;
        loss = 0.0f;
    } else if (t < 0 || t >= a.V || own != 1) {
        fo.status = -1;
        loss = __builtin_nanf("");
    } else {
        const RowFinal f = finalize_row(M, s, zt, sz, (double)a.V, (double)a.eps);
        fo.lse = f.lse;
        fo.gt = f.gt;
        fo.m = (float)M;
        fo.status = 1;
        loss = (float)f.loss;
    }
    a.fin[r] = fo;
    a.loss_rows[r] = loss;
}

// zero-fill (a kernel rather than a memset node, so callers may capture it)
__global__ __launch_bounds__(256) void k_zero_f32(float *p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_linear_merge(const LinMergeArgs &a, hipStream_t stream) {
    const dim3 grid((unsigned)((a.N + kMergeWaves - 1) / kMergeWaves));
    hipLaunchKernelGGL(k_linear_merge, grid, dim3(kMergeWaves * kWave), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_zero_f32(float *p, int64_t n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_zero_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

hipError_t launch_relayout(const RelayoutArgs &a, bool transpose, hipStream_t stream,
                           uint16_t *Yn, int64_t Kn) {
    if (!transpose) {
        const int64_t slots = a.Rp * a.Kp / 8;
        const dim3 grid((unsigned)((slots + kRelayoutThreads - 1) / kRelayoutThreads));
        hipLaunchKernelGGL(k_relayout, grid, dim3(kRelayoutThreads), 0, stream, a);
    } else {
        const dim3 grid((unsigned)((a.Rp / 64) * (a.Kp / 64)));
        hipLaunchKernelGGL(k_relayout_t, grid, dim3(kRelayoutThreads), 0, stream, a, Yn, Kn);
    }
    return hipGetLastError();
}

hipError_t launch_linear_rowconst(const LinRowArgs &a, hipStream_t stream) {
    const dim3 grid((unsigned)((a.N + 255) / 256));
    hipLaunchKernelGGL(k_linear_rowconst, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <int EPI, bool LS, bool FILT = false>
static hipError_t gemm_launch(const GemmArgs &g, hipStream_t stream) {
    static std::atomic<bool> attr[kMaxDevices];
    static std::atomic<int> slot_cache[kMaxDevices];
    const void *kern = (const void *)k_gemm<EPI, LS, FILT>;
    hipError_t e = raise_lds_once(kern, kGemmLdsBytes, attr);
    if (e != hipSuccess) return e;
    // as many workgroups as the device holds at once, a multiple of 8
    int64_t held = 0;
    e = device_slots(kern, kGT, kGemmLdsBytes, slot_cache, &held);
    if (e != hipSuccess) return e;
    const int64_t ids = tile_ids(g.tiles_m, g.tiles_n);
    const int64_t slots = std::max<int64_t>(kXcds, held / kXcds * kXcds);
    const dim3 grid((unsigned)(kGemmPersistent<EPI> ? std::min(ids, slots) : ids));
    hipLaunchKernelGGL((k_gemm<EPI, LS, FILT>), grid, dim3(kGT), kGemmLdsBytes, stream, g);
    return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs &g, int epi, bool ls, bool filt, hipStream_t stream) {
    if (filt) {
        // the filtered kernels dereference their filtering buffers
        if (epi == GEMM_GRAD ? !g.keep_flags : (!g.klist || !g.kcnt)) return hipErrorInvalidValue;
        switch (epi) {
        case GEMM_GRAD: return ls ? gemm_launch<GEMM_GRAD, true, true>(g, stream)
                                  : gemm_launch<GEMM_GRAD, false, true>(g, stream);
        case GEMM_STORE: return gemm_launch<GEMM_STORE, false, true>(g, stream);
        case GEMM_ADD: return gemm_launch<GEMM_ADD, false, true>(g, stream);
        case GEMM_KAHAN: return gemm_launch<GEMM_KAHAN, false, true>(g, stream);
        }
        return hipErrorInvalidValue;
    }
    switch (epi) {
    case GEMM_STATS: return ls ? gemm_launch<GEMM_STATS, true>(g, stream)
                               : gemm_launch<GEMM_STATS, false>(g, stream);
    case GEMM_GRAD: return ls ? gemm_launch<GEMM_GRAD, true>(g, stream)
                              : gemm_launch<GEMM_GRAD, false>(g, stream);
    case GEMM_STORE: return gemm_launch<GEMM_STORE, false>(g, stream);
    case GEMM_ADD: return gemm_launch<GEMM_ADD, false>(g, stream);
    case GEMM_KAHAN: return gemm_launch<GEMM_KAHAN, false>(g, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_filter_lists(const FilterListArgs &a, hipStream_t stream) {
    const int64_t n = a.tiles_m + a.tiles_n; // one wave per list
    hipLaunchKernelGGL(k_filter_lists, dim3((unsigned)((n + kListWaves - 1) / kListWaves)),
                       dim3(kListWaves * kWave), 0, stream, a);
    return hipGetLastError();
}

} // namespace vce
