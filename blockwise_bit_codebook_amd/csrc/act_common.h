// Pieces shared by the activation-assignment kernels: the threshold tables
// for the 16 Lloyd-Max centroids, the row-buffer layout in LDS, the 16-point
// butterfly pass, the per-element assignment and the bit-plane packing.
//
// Assignment ([ORBIT] methodology audit: divide by max(norm, 1e-10) when
// choosing indices): z = RN(u / max(norm, 1e-10f)), idx = first-index
// argmin |RN(z - c_i)|, decided with the exact switching-point test of
// threshold.h (q = base + slope * z clamped into [2, 4)).  The slope is
// 0.99 / R for the smallest power of two R with every threshold inside
// 0.97 * (-R, R), so that the 128 buckets of q spread over the codebook's
// own range: the codebooks for rows of many Hadamard blocks are narrow
// (entries of z have about h/d of the variance of a one-block row).
// |z| <= sqrt(h) <= 128 for Hadamard
// blocks of h <= 16384 (|u| <= sqrt(h) * norm), so the distances round at
// <= 2^-17, far below the smallest centroid gap the fast path accepts.
// Rows whose norm is not finite, and codebooks that do not qualify, take
// the exact path (IEEE division and the full scan).
#pragma once

#include "device.h"
#include "threshold.h"

namespace kbit {
namespace act {

constexpr float kActEps = 1e-10f;
constexpr float kActBase = 3.0f + 0x1p-10f;   // q = kActBase + slope * z
constexpr float kActMinGap = 0x1p-12f;
constexpr float kQMax = 0x1.fffffep+1f;       // largest float below 4

using ActTables = ThresholdTables<16>;

// LDS position of element 256a + 16b + c of a row: 16 floats of padding per
// 256 keep the strided passes conflict-free, and the swizzle of the four
// 16-byte chunks of each 16 does the same for 16-byte-per-lane accesses.
__device__ __forceinline__ int swz(int a, int b, int c) { return 272 * a + 16 * b + (c ^ (((b >> 1) & 3) << 2)); }
__device__ __forceinline__ int swz_i(int i) { return swz(i >> 8, (i >> 4) & 15, i & 15); }

// Stages s = 1, 2, ..., N/2 of the butterfly over the first N entries of v
// (every output rounded to fp32; the stages keep their order).
template <int N>
__device__ __forceinline__ void fwht_pts(float (&v)[16]) {
#pragma unroll
    for (int h = 1; h < N; h <<= 1) {
#pragma unroll
        for (int j = 0; j < N; ++j) {
            if ((j & h) == 0) {
                const float a = v[j], b = v[j + h];
                v[j] = a + b;
                v[j + h] = a - b;
            }
        }
    }
}

__device__ __forceinline__ uint32_t nearest16_lds(const float* c, float z) {
    uint32_t best = 0;
    float bd = fabsf(z - c[0]);
#pragma unroll 1
    for (int i = 1; i < 16; ++i) {
        const float d = fabsf(z - c[i]);
        if (d < bd) {
            bd = d;
            best = i;
        }
    }
    return best;
}

// Whether the fast path applies, and its slope.
struct ActPlan {
    bool fast;
    float slope;
};

// The table build in three stages, for kernels that interleave it with
// other work between their own barriers.  Every thread of the workgroup
// (nthreads = blockDim.x, a multiple of 64 and at least 128) runs each
// stage, and a workgroup barrier separates stage 1 from 2, 2 from 3, and 3
// from the first use of the tables.
struct ActBuild {
    float c[16];
    bool fast;
    float slope;
};

// Stage 1: codebook checks, bucket slope, and the switching points (T.mid).
__device__ __forceinline__ void act_tables_search(ActTables& T, const float* __restrict__ cb, int nthreads,
                                                  ActBuild& B) {
    const int lane = __lane_id();
    // A local copy for the indexed store into T.code below (indexing the
    // struct's array would put it in scratch memory).
    float c[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) c[i] = cb[i];
#pragma unroll
    for (int i = 0; i < 16; ++i) B.c[i] = c[i];
    bool fast = true;
#pragma unroll
    for (int i = 1; i < 16; ++i) fast = fast && (c[i] == c[i - 1] || c[i] - c[i - 1] >= kActMinGap);
    // range R: a power of two (2^-20 .. 2^20) above the largest |threshold|
    float mmax = 0.0f;
#pragma unroll
    for (int i = 1; i < 16; ++i) {
        if (c[i] != c[i - 1]) mmax = fmaxf(mmax, fabsf((c[i - 1] + c[i]) * 0.5f));
    }
    int ex = 0;
    (void)frexpf(mmax / 0.97f, &ex);
    ex = min(max(ex, -20), 20);
    const float zr = ldexpf(1.0f, ex);
    const float slope = 0.99f / zr;
#pragma unroll
    for (int i = 1; i < 16; ++i) {
        const float m = (c[i - 1] + c[i]) * 0.5f;
        fast = fast && (c[i] == c[i - 1] || (m > -0.97f * zr && m < 0.97f * zr));
    }
    if (threadIdx.x == 0) T.fail = 0;
    if (threadIdx.x < 16) T.code[threadIdx.x] = c[threadIdx.x];
    // One half-wave per threshold, all searched at once; a failed search
    // leaves the sentinel, which fails the table.
    {
        const int groups = 2 * nthreads / kWave;
        const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / kWave));
        for (int i0 = 1; i0 < 16; i0 += groups) {  // uniform trip count
            // the wave's thresholds ib and ib + 1 from three uniform (scalar)
            // loads: per-lane loads would wait behind the first row's loads
            const int ib = i0 + 2 * wave;
            const float a = cb[min(ib - 1, 15)], b = cb[min(ib, 15)], d = cb[min(ib + 1, 15)];
            const bool upper = lane >= 32;
            const int i = ib + (upper ? 1 : 0);
            const bool real = i < 16;
            const float lo = real ? (upper ? b : a) : 0.0f, hi = real ? (upper ? d : b) : 0.0f;
            uint64_t m = 0;
            const bool ok = threshold_mid_group<32>(lo, hi, m);  // every lane calls it
            if (real && (lane & 31) == 0) T.mid[i] = (fast && lo != hi) ? (ok ? m : kNoMid) : 0u;
        }
    }
    if (threadIdx.x == 0) T.mid[0] = 0;
    B.fast = fast;
    B.slope = slope;
}

// Stage 2: failed searches, and the bucket entries (T.master).
__device__ __forceinline__ void act_tables_entries(ActTables& T, const ActBuild& B) {
    if (threadIdx.x < 16 && T.mid[threadIdx.x] == kNoMid) T.fail = 1;
    if (B.fast && threadIdx.x < kBuckets) {
        u32x4 e;
        if (!build_entry<16, false>(B.c, T.mid, threadIdx.x, B.slope, kActBase, e)) T.fail = 1;
        T.master[threadIdx.x] = e;
    }
}

// Stage 3: whether the fast path applies, and the bank-spread copies.
__device__ __forceinline__ ActPlan act_tables_copies(ActTables& T, const ActBuild& B, int nthreads) {
    const bool fast = B.fast && (T.fail == 0);
    if (fast) {
        for (int i = threadIdx.x; i < kBuckets * kCopies; i += nthreads) T.row[i] = T.master[i / kCopies];
    }
    return ActPlan{fast, B.slope};
}

// Builds T for the codebook cb: the three stages with their barriers.
__device__ __forceinline__ ActPlan build_act_tables(ActTables& T, const float* __restrict__ cb, int nthreads) {
    ActBuild B;
    act_tables_search(T, cb, nthreads, B);
    __syncthreads();
    act_tables_entries(T, B);
    __syncthreads();
    const ActPlan plan = act_tables_copies(T, B, nthreads);
    __syncthreads();
    return plan;
}

// The tables in a form built once per codebook (act_tables_kernel) and
// loaded by every workgroup instead of its own build: the 128 bucket
// entries, then {fast, slope bits, 0, 0}, then the codebook as 4 vectors.
constexpr int kActPrepEntries = kBuckets + 1 + 4;  // u32x4 each: 2,128 bytes

// Writes the prepared form of T (built with plan) to out; threads of one
// workgroup, after the build's last barrier.
__device__ __forceinline__ void store_act_tables(const ActTables& T, const ActPlan& plan, u32x4* __restrict__ out,
                                                 int nthreads) {
    for (int i = threadIdx.x; i < kBuckets; i += nthreads) out[i] = T.master[i];
    if (threadIdx.x == 0) out[kBuckets] = u32x4{plan.fast ? 1u : 0u, __float_as_uint(plan.slope), 0u, 0u};
    if (threadIdx.x < 4) {
        const int i = 4 * threadIdx.x;
        out[kBuckets + 1 + threadIdx.x] = u32x4{__float_as_uint(T.code[i]), __float_as_uint(T.code[i + 1]),
                                                __float_as_uint(T.code[i + 2]), __float_as_uint(T.code[i + 3])};
    }
}

// Fills T's bank-spread rows and codebook from the prepared form and
// returns the plan.  Every thread of the workgroup calls it; a workgroup
// barrier must separate it from the first use of T.
// Every load goes out before the first LDS write, so that the copy costs one
// load latency: item i (of kBuckets * 4) is bucket i / 4's entry, which its
// thread writes to copies 4(i % 4) .. 4(i % 4) + 3.  A thread takes items
// threadIdx.x and threadIdx.x + nthreads (nthreads >= 256 covers all of
// them; the loop after it takes any left for smaller groups).
__device__ __forceinline__ ActPlan load_act_tables(ActTables& T, const u32x4* __restrict__ prep, int nthreads) {
    static_assert(kCopies == 16, "four copies per item");
    constexpr int kItems = kBuckets * 4;
    const int i0 = threadIdx.x, i1 = threadIdx.x + nthreads;
    u32x4 e0 = {0u, 0u, 0u, 0u}, e1 = {0u, 0u, 0u, 0u};
    if (i0 < kItems) e0 = prep[i0 >> 2];
    if (i1 < kItems) e1 = prep[i1 >> 2];
    const bool has_code = threadIdx.x < 16;
    const uint32_t cw = has_code ? prep[kBuckets + 1 + threadIdx.x / 4][threadIdx.x % 4] : 0u;
    const u32x4 pl = prep[kBuckets];
    auto put = [&](int i, const u32x4& e) {
        u32x4* dst = T.row + (i >> 2) * kCopies + (i & 3) * 4;
#pragma unroll
        for (int c = 0; c < 4; ++c) dst[c] = e;
    };
    if (i0 < kItems) put(i0, e0);
    if (i1 < kItems) put(i1, e1);
    for (int i = threadIdx.x + 2 * nthreads; i < kItems; i += nthreads) put(i, prep[i >> 2]);
    if (has_code) T.code[threadIdx.x] = __uint_as_float(cw);
    return ActPlan{pl[0] != 0u, __uint_as_float(pl[1])};
}

// Indices of the 16 transformed values v of a row with norm `norm`, as two
// plane accumulators: bit k of byte j of acc[h] is plane j of element
// 8h + k.  Every lane of the wave must work on the same row (the finite-norm
// test is a wave vote).
__device__ __forceinline__ void assign16(const float (&v)[16], float norm, const ActPlan& plan,
                                         const ActTables& T, uint32_t (&acc)[2]) {
    const uint32_t lane_off = static_cast<uint32_t>(__lane_id() & (kCopies - 1)) * 16u;
    const char* tab = reinterpret_cast<const char*>(T.row);
    // max(norm, eps) with a NaN norm kept NaN (fmaxf would drop it)
    const float den = norm < kActEps ? kActEps : norm;
    acc[0] = 0u;
    acc[1] = 0u;
    if (plan.fast && __builtin_amdgcn_ballot_w64(!(norm < __builtin_inff())) == 0) {
        const float r = __builtin_amdgcn_rcpf(den) * plan.slope;
        const double d64 = static_cast<double>(den);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int k = 7; k >= 0; --k) {
                const float z = v[8 * h + k];
                const float q = __builtin_amdgcn_fmed3f(__builtin_fmaf(z, r, kActBase), 2.0f, kQMax);
                const Decision d = decide(z, q, d64, tab, lane_off);
                const uint32_t sel = d.up ? d.e[3] : d.e[2];
                acc[h] = k == 7 ? sel : shl1_or(acc[h], sel);
            }
        }
    } else {
        // one element per iteration (rare path): rotate a copy so that the
        // element in use is always y[0]
        float y[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) y[i] = v[i];
#pragma unroll 1
        for (int k = 0; k < 16; ++k) {
            acc[k >> 3] |= spread4(nearest16_lds(T.code, y[0] / den)) << (k & 7);
#pragma unroll
            for (int i = 0; i < 15; ++i) y[i] = y[i + 1];
        }
    }
}

// The 4 plane words of a group of 32 elements from the two lanes 2g (first
// 16) and 2g + 1 (last 16); `odd` is the lane's parity.  Both lanes of the
// pair must be active.  The lane gets words 2*odd and 2*odd + 1.
__device__ __forceinline__ uint2 pack_pair(const uint32_t (&acc)[2], bool odd) {
    // per lane: plane j's 16 bits = [acc0 byte j, acc1 byte j]
    const uint32_t h01 = __builtin_amdgcn_perm(acc[1], acc[0], 0x05010400u);
    const uint32_t h23 = __builtin_amdgcn_perm(acc[1], acc[0], 0x07030602u);
    const uint32_t mine = odd ? h23 : h01;
    const uint32_t recv = dpp_u32<kDppXor1>(odd ? h01 : h23);
    const uint32_t lo = odd ? recv : mine, hi = odd ? mine : recv;  // even lane's half first
    return make_uint2(__builtin_amdgcn_perm(hi, lo, 0x05040100u), __builtin_amdgcn_perm(hi, lo, 0x07060302u));
}

// Sum of the lanes' values over each aligned group of 16 lanes, as a tree
// of contiguous halves (pairs, then quads, eights, sixteens).
__device__ __forceinline__ float sum16_tree(float S) {
    S = S + dpp_f32<kDppXor1>(S);
    S = S + dpp_f32<kDppXor2>(S);
    S = S + dpp_f32<kDppHalfMirror>(S);
    S = S + dpp_f32<kDppMirror>(S);
    return S;
}

}  // namespace act
}  // namespace kbit
