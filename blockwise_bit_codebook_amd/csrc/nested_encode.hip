// Nested (double-quantized) state encoder for gfx950: from the fp32
// per-block absmax to the 8-bit codes, the group absmax2 and the mean offset
// that the fused nested dequantize consumes ([PR2051] Summary: per-block
// scales are 8-bit codes over groups of 256 blocks plus a mean offset; the
// encoder itself is not on the pages).  What is computed:
//   offset      = RN32( (exact sum of absmax) / nb )
//                 (NaN if any value is NaN or both infinities occur; an
//                 infinity if only that one occurs)
//   r_b         = RN(absmax_b - offset)
//   absmax2_g   = max |r_b| over group g (blocks 256g .. 256g+255; the last
//                 group may be short; NaN propagates)
//   code_b      = smallest i minimising |RN(RN(r_b / max(absmax2_g, 1e-8f))
//                 - qmap2_i)|
//
// How: two launches on one stream.
//   1. Each workgroup (1024 threads) sums its values exactly into
//      32-bit-limb accumulators of the positive and the negative values
//      (exact_mean.h): per round of 4 values per lane, each wave adds the
//      integer significands of the values within 24 binades of its largest
//      one into 64-bit register sums (shifted to the window's bottom), sums
//      those across the wave and adds them to the limbs; values further down
//      go to LDS bins by (sign, exponent), folded into the limbs at the end.
//      The limbs, carried into 32-bit digits, and the NaN/infinity flags go
//      to the workspace: 25 32-bit words per workgroup.
//   2. Every workgroup (1024 threads, at most 512 workgroups) first adds
//      the records (a half wave per word) and rounds the mean itself (the
//      records are complete: they come from the previous launch; the
//      division by nb is a multiply-high by a constant the host computes);
//      workgroup 0 stores it.  Then one wave per group of 256 blocks: four
//      blocks per lane, the group max from the group's value range (taken
//      while the mean is pending), IEEE division, and the nearest code: a
//      count over 15 map entries held in registers, a binary search in LDS
//      inside the block of 16 it picks, and a walk to the lowest index with
//      the same rounded distance (a full scan if the map is not sorted).
// The workspace holds only the records (scratch, no initialisation).  A
// variant keeps it in a static device array instead (one per GPU, for
// callers that cannot allocate).
#include "device.h"
#include "exact_mean.h"
#include "kbit_internal.h"

#include <atomic>

namespace kbit {
namespace {

constexpr int kBinThreads = 1024;
constexpr int kBinWaves = kBinThreads / kWave;
constexpr int kMaxBinGroups = 256;  // workgroups of launch 1 (the workspace holds one record each)
constexpr int kLimbWords = kWideLimbs + 2;
constexpr int kRecordWords = 2 * kLimbWords + 1;  // uint32: digits[sign][i], then the flags
constexpr int kEncThreads = 1024;                       // launch 2: one group of 256 blocks per wave
constexpr int kEncWaves = kEncThreads / kWave;
constexpr int kEncMaxGrid = 512;                        // each workgroup of launch 2 re-reads the records
constexpr int kOffsetParts = 32;                        // lanes per record word in the mean (a half wave)
constexpr int kOffsetLoads = kMaxBinGroups / kOffsetParts;  // records per such lane
static_assert(kRecordWords * kOffsetParts <= kEncThreads, "a half wave per record word");
constexpr int kGroup2 = 256;
constexpr float kEps2 = 1e-8f;
constexpr uint32_t kFlagNan = 1, kFlagPosInf = 2, kFlagNegInf = 4;

constexpr int kBinVecs = 1;      // 16-byte loads per lane per round (4 values)
constexpr int kWindowBits = 24;  // binades below the wave's top one that the register sums take
constexpr int64_t kRoundValues = static_cast<int64_t>(kBinThreads) * kBinVecs * 4;  // per workgroup

int bin_groups(int64_t nb) {
    const int64_t g = (nb + kRoundValues - 1) / kRoundValues;
    return static_cast<int>(g < 1 ? 1 : (g > kMaxBinGroups ? kMaxBinGroups : g));
}

// Lane i of each row of 16 gets lane i - 1's value, lane 0 of a row gets 0
// (DPP row_shr:1; with bound_ctrl set, a source lane outside the row reads
// as zero).
__device__ __forceinline__ uint32_t row_shr1_or_zero(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x111, 0xF, 0xF, true));
}

template <int CTRL>
__device__ __forceinline__ int32_t dpp_i32(int32_t v) {
    return static_cast<int32_t>(dpp_u32<CTRL>(static_cast<uint32_t>(v)));
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    return (static_cast<uint64_t>(dpp_u32<CTRL>(static_cast<uint32_t>(v >> 32))) << 32) |
           dpp_u32<CTRL>(static_cast<uint32_t>(v));
}

__device__ __forceinline__ uint32_t readlane_u32(uint32_t v, int lane) {
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), lane));
}

// Sum over the wave (every lane active), returned uniform: DPP within each
// row of 16 lanes, then the four row totals read out.
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
    v += dpp_u64<kDppXor1>(v);
    v += dpp_u64<kDppXor2>(v);
    v += dpp_u64<kDppHalfMirror>(v);
    v += dpp_u64<kDppMirror>(v);
    uint64_t t = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        t += (static_cast<uint64_t>(readlane_u32(static_cast<uint32_t>(v >> 32), 16 * r)) << 32) |
             readlane_u32(static_cast<uint32_t>(v), 16 * r);
    }
    return t;
}

// Maximum over the wave (every lane active), returned uniform.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp_u32<kDppXor1>(v));
    v = max(v, dpp_u32<kDppXor2>(v));
    v = max(v, dpp_u32<kDppHalfMirror>(v));
    v = max(v, dpp_u32<kDppMirror>(v));
    return max(max(readlane_u32(v, 0), readlane_u32(v, 16)), max(readlane_u32(v, 32), readlane_u32(v, 48)));
}

// Launch 1.  Per round a wave holds 4 values per lane.  A finite nonzero
// value with biased exponent e and integer significand m is m * 2^(e' - 1)
// in units of 2^-149, e' = max(e, 1).  With E the wave's largest e' and
// e0 = max(E - 24, 1), every value with e' >= e0 adds m << (e' - e0) (below
// 2^48) to the register sum of its sign, in units of 2^(e0 - 1); the wave's
// two sums (below 2^56) go into the wave's own limb accumulators in LDS
// once per round, as three pieces below 2^33 (lane 0 alone writes them, so
// no atomics).  Values further down (more than 24 binades below the wave's
// top) add m to the workgroup's LDS bin of their sign and e, folded into
// wave 0's limbs at the end (only if any exist).  NaN and infinities only
// set flags.  Then wave 0 adds the waves' limbs (lane 16 s + i takes limb i
// of sign s) and carries them into 32-bit digits.
//
// Bounds (nb <= 2^36, at most 2^28 values per workgroup): a wave's limb
// takes at most one piece per round and sign, so all 16 waves' limbs of
// one index add up to below 2^20 * 2^33 (2^20 wave rounds of 256 values),
// plus at most 256 bin pieces; a bin stays below 2^28 * 2^24.  A
// workgroup's sum is below 2^28 * 2^277, so its carried digits fit the 10
// low limbs and each is below 2^32; launch 2 adds at most 256 of them per
// limb.
//
// The record is word-major: word k of workgroup b at ws[k * groups + b],
// so that launch 2 reads each word of all records with contiguous loads.
__global__ __launch_bounds__(kBinThreads) void nested_bins_kernel(const float* __restrict__ a, int64_t nb,
                                                                  uint32_t* __restrict__ ws) {
    __shared__ unsigned long long bins[2][256];
    __shared__ unsigned long long wlimbs[kBinWaves][2][kLimbWords];
    __shared__ uint32_t flags, any_slow;
    const int wave = threadIdx.x / kWave;
    const int lane = __lane_id();
    uint32_t my_flags = 0;
    // Values past nb (and a tail not in whole vectors) read as 0, which adds
    // nothing; the round loop is uniform over the wave (the sums use every
    // lane).
    const int64_t nvec = nb / 4, nvec_all = (nb + 3) / 4;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBinThreads;
    const u32x4* av = reinterpret_cast<const u32x4*>(a);
    const bool aligned16 = (reinterpret_cast<uintptr_t>(a) & 15u) == 0;
    const auto load_round = [&](int64_t wb, u32x4 (&u)[kBinVecs]) {
#pragma unroll
        for (int k = 0; k < kBinVecs; ++k) {
            const int64_t vi = wb + lane + k * stride;
            if (aligned16 && vi < nvec) {
                u[k] = av[vi];
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) u[k][c] = 4 * vi + c < nb ? __float_as_uint(a[4 * vi + c]) : 0u;
            }
        }
    };
    // the first round's loads are in flight while the LDS is cleared
    const int64_t wb0 = static_cast<int64_t>(blockIdx.x) * kBinThreads + wave * kWave;
    int64_t wb = wb0;
    u32x4 u[kBinVecs];
    load_round(wb, u);
    for (int i = threadIdx.x; i < 2 * 256; i += kBinThreads) (&bins[0][0])[i] = 0;
    for (int i = threadIdx.x; i < kBinWaves * 2 * kLimbWords; i += kBinThreads) (&wlimbs[0][0][0])[i] = 0;
    if (threadIdx.x == 0) flags = any_slow = 0;
    __syncthreads();
    unsigned long long* my_limbs = &wlimbs[wave][0][0];
    for (; wb < nvec_all; wb += kBinVecs * stride) {
        if (wb != wb0) load_round(wb, u);
        uint32_t top = 0;
#pragma unroll
        for (int k = 0; k < kBinVecs; ++k) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t e = (u[k][c] >> 23) & 0xFFu;
                if (e != 0xFFu && (u[k][c] & 0x7FFFFFFFu) != 0) top = max(top, max(e, 1u));
            }
        }
        top = wave_max_u32(top);
        const uint32_t e0 = top > kWindowBits + 1 ? top - kWindowBits : 1u;
        // branch-free for the values in the window; the rest (rare) after
        uint64_t sum_pos = 0, sum_neg = 0;
        uint32_t slow = 0;
#pragma unroll
        for (int k = 0; k < kBinVecs; ++k) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t x = u[k][c];
                const uint32_t e = (x >> 23) & 0xFFu, f = x & 0x7FFFFFu;
                const bool neg = (x >> 31) != 0, special = e == 0xFFu;
                my_flags |= special ? (f ? kFlagNan : (neg ? kFlagNegInf : kFlagPosInf)) : 0u;
                const uint32_t ee = max(e, 1u), m = e ? (f | 0x800000u) : f;  // m = 0 for zeros
                const bool fast = !special && ee >= e0;
                const uint64_t t = static_cast<uint64_t>(fast ? m : 0u) << (fast ? ee - e0 : 0u);
                sum_neg += neg ? t : 0ull;
                sum_pos += neg ? 0ull : t;
                slow |= (!special && !fast && m != 0) ? (1u << (4 * k + c)) : 0u;
            }
        }
        if (slow != 0) {
            atomicOr(&any_slow, 1u);
#pragma unroll
            for (int k = 0; k < kBinVecs; ++k) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    if (slow & (1u << (4 * k + c))) {
                        const uint32_t x = u[k][c];
                        const uint32_t e = (x >> 23) & 0xFFu, f = x & 0x7FFFFFu;
                        atomicAdd(&bins[x >> 31][e], static_cast<unsigned long long>(e ? (f | 0x800000u) : f));
                    }
                }
            }
        }
        sum_pos = wave_sum_u64(sum_pos);
        sum_neg = wave_sum_u64(sum_neg);
        if (lane == 0) {
#pragma unroll
            for (int sg = 0; sg < 2; ++sg) {
                const uint64_t v = sg ? sum_neg : sum_pos;
                if (v != 0) {
                    const WidePieces q = wide_pieces(v, static_cast<int>(e0) - 1);
                    unsigned long long* l = my_limbs + sg * kLimbWords + q.w;
                    l[0] += q.p0;
                    l[1] += q.p1;
                    l[2] += q.p2;
                }
            }
        }
    }
    if (my_flags) atomicOr(&flags, my_flags);
    __syncthreads();
    if (any_slow != 0) {  // workgroup-uniform: bins -> wave 0's limbs
        for (int i = threadIdx.x; i < 2 * 256; i += kBinThreads) {
            const uint64_t sum = (&bins[0][0])[i];
            const int sg = i >> 8, e = i & 255;
            if (sum != 0) {
                const WidePieces q = wide_pieces(sum, (e > 0 ? e : 1) - 1);
                atomicAdd(&wlimbs[0][sg][q.w], static_cast<unsigned long long>(q.p0));
                atomicAdd(&wlimbs[0][sg][q.w + 1], static_cast<unsigned long long>(q.p1));
                atomicAdd(&wlimbs[0][sg][q.w + 2], static_cast<unsigned long long>(q.p2));
            }
        }
        __syncthreads();
    }
    if (wave == 0) {
        // Lane 16 s + i (i < 12) adds limb i of sign s over all waves
        // (t < 2^54), then the digits: each limb keeps its low 32 bits plus
        // the high part of the limb below (one DPP row shift: each sign's
        // limbs sit in one row of 16 lanes), which leaves sums below 2^33,
        // i.e. carries of 0 or 1.  Those resolve as in a carry-lookahead
        // adder: G marks the lanes whose sum reached 2^32, P those whose low
        // 32 bits are all ones (they pass a carry on), and the carry into
        // each lane is bit i of ((G | P) + G) ^ (G | P) ^ G.  Limbs 10 and 11
        // never receive pieces (the top piece lands at limb 9), so no carry
        // leaves a sign's row.
        const int sg = lane >> 4, li = lane & 15;
        const bool mine = lane < 32 && li < kLimbWords;
        uint64_t t = 0;
        if (mine) {
#pragma unroll
            for (int w = 0; w < kBinWaves; ++w) t += wlimbs[w][sg][li];
        }
        const uint32_t hi_below = row_shr1_or_zero(static_cast<uint32_t>(t >> 32));
        const uint64_t sum = (t & 0xFFFFFFFFull) + hi_below;
        const uint32_t low = static_cast<uint32_t>(sum);
        const uint64_t G = __ballot(mine && (sum >> 32) != 0);
        const uint64_t P = __ballot(mine && low == 0xFFFFFFFFu);
        const uint64_t carries = ((G | P) + G) ^ (G | P) ^ G;
        const uint32_t digit = low + static_cast<uint32_t>((carries >> lane) & 1ull);
        const int64_t groups = gridDim.x;
        if (mine) ws[(sg * kLimbWords + li) * groups + blockIdx.x] = digit;
        if (lane == 0) ws[2 * kLimbWords * groups + blockIdx.x] = flags;
    }
}

// The records of launch 1 for the mean: half wave h of the workgroup
// (kOffsetParts = 32 lanes) takes record word h (a digit of one sign, or
// the flags) of every record, eight per lane, widened to 64 bits; halves
// past the last word load nothing.
__device__ __forceinline__ void load_records(const uint32_t* __restrict__ ws, int groups,
                                             uint64_t (&v)[kOffsetLoads]) {
    const int k = threadIdx.x / kOffsetParts, part = threadIdx.x % kOffsetParts;
#pragma unroll
    for (int j = 0; j < kOffsetLoads; ++j) {
        const int g = part + j * kOffsetParts;
        v[j] = (k < kRecordWords && g < groups) ? ws[static_cast<int64_t>(k) * groups + g] : 0;
    }
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_or_u64(uint64_t v) {
    return v | dpp_u64<CTRL>(v);
}

// The mean offset from the loaded records: each half wave sums (ORs, for
// the flags) its word; thread 0 rounds the mean from the limb totals (each
// below 2^40).  Every thread gets the offset (through LDS).  All threads of
// the workgroup call it.
__device__ inline float mean_offset(const uint64_t (&v)[kOffsetLoads], const NbDivider& div) {
    __shared__ unsigned long long total[kRecordWords];
    __shared__ float off;
    uint64_t sum = 0, any = 0;
#pragma unroll
    for (int j = 0; j < kOffsetLoads; ++j) {
        sum += v[j];
        any |= v[j];
    }
    sum += dpp_u64<kDppXor1>(sum);
    sum += dpp_u64<kDppXor2>(sum);
    sum += dpp_u64<kDppHalfMirror>(sum);
    sum += dpp_u64<kDppMirror>(sum);
    any = dpp_or_u64<kDppXor1>(any);
    any = dpp_or_u64<kDppXor2>(any);
    any = dpp_or_u64<kDppHalfMirror>(any);
    any = dpp_or_u64<kDppMirror>(any);
    const auto row = [](uint64_t x, int lane) {
        return (static_cast<uint64_t>(readlane_u32(static_cast<uint32_t>(x >> 32), lane)) << 32) |
               readlane_u32(static_cast<uint32_t>(x), lane);
    };
    // The read-outs stay in uniform control flow (a cross-lane read inside
    // a lane-0 branch lets the compiler move the sums' last step into that
    // branch, where the other lanes do not run it).
    const int k0 = 2 * (threadIdx.x / kWave);  // word of the wave's first half; k0 + 1 is odd: never the flags
    const uint64_t t0 = k0 == 2 * kLimbWords ? (row(any, 0) | row(any, 16)) : row(sum, 0) + row(sum, 16);
    const uint64_t t1 = row(sum, 32) + row(sum, 48);
    if (__lane_id() == 0) {
        if (k0 < kRecordWords) total[k0] = t0;
        if (k0 + 1 < kRecordWords) total[k0 + 1] = t1;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t fl = static_cast<uint32_t>(total[2 * kLimbWords]);
        uint32_t bits;
        if ((fl & kFlagNan) || ((fl & kFlagPosInf) && (fl & kFlagNegInf))) {
            bits = 0x7FC00000u;
        } else if (fl & kFlagPosInf) {
            bits = 0x7F800000u;
        } else if (fl & kFlagNegInf) {
            bits = 0xFF800000u;
        } else {
            uint64_t pos[kLimbWords], neg[kLimbWords];
#pragma unroll
            for (int i = 0; i < kLimbWords; ++i) {
                pos[i] = total[i];
                neg[i] = total[kLimbWords + i];
            }
            bits = mean_from_limbs(pos, neg, div);
        }
        off = __uint_as_float(bits);
    }
    __syncthreads();
    return off;
}

// Lowest index with the smallest |RN(v - c_i)| for four values at once, in
// a non-decreasing map c (LDS) whose entries 16t + 15 (t < 15) are also in
// sep[t] (uniform registers).  The number j of entries <= v among the
// first 255 (the binary search's result) is 16 times the count of
// separators <= v plus a binary search inside that block of 16 (the four
// values step together, so each step's LDS reads share one wait).  Then the
// neighbours: rounded distances only grow away from v on either side, so
// the winner is entry j if it is strictly closer than entry j - 1, else the
// lowest index left of v with entry j - 1's rounded distance.  NaN gives 0.
__device__ __forceinline__ void nearest_sorted4(const float* c, const float (&sep)[15], const float (&v)[4],
                                                uint32_t (&q)[4]) {
    int j[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        int t = 0;
#pragma unroll
        for (int u = 0; u < 15; ++u) t += sep[u] <= v[k] ? 1 : 0;
        j[k] = 16 * t;
    }
#pragma unroll
    for (int step = 8; step >= 1; step >>= 1) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (c[j[k] + step - 1] <= v[k]) j[k] += step;
        }
    }
    float dlo[4], dup[4], dleft[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {  // one batch of reads: entries j - 2, j - 1, j (clamped)
        const int i = j[k] > 0 ? j[k] - 1 : 0;
        dlo[k] = fabsf(v[k] - c[i]);
        dup[k] = fabsf(v[k] - c[j[k]]);  // j <= 255
        dleft[k] = fabsf(v[k] - c[i > 0 ? i - 1 : 0]);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        int i = j[k] - 1;
        if (j[k] == 0) {
            i = 0;
        } else if (dup[k] < dlo[k]) {
            i = j[k];
        } else if (i > 0 && dleft[k] == dlo[k]) {  // equal rounded distances further left (rare)
            --i;
#pragma unroll 1
            while (i > 0 && fabsf(v[k] - c[i - 1]) == dlo[k]) --i;
        }
        q[k] = static_cast<uint32_t>(i);
    }
}

// The definition's scan (strict <, from index 0): any map.
__device__ __forceinline__ uint32_t nearest_scan256(const float* c, float v) {
    uint32_t best = 0;
    float bd = fabsf(v - c[0]);
#pragma unroll 1
    for (int i = 1; i < 256; ++i) {
        const float d = fabsf(v - c[i]);
        if (d < bd) {
            bd = d;
            best = static_cast<uint32_t>(i);
        }
    }
    return best;
}

// Order-preserving integer key of a float (larger value, larger key; -0
// below +0): the float bits with the magnitude bits flipped for negatives.
__device__ __forceinline__ int32_t order_key(float x) {
    const int32_t b = static_cast<int32_t>(__float_as_uint(x));
    return b ^ ((b >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float from_order_key(int32_t k) {
    return __uint_as_float(static_cast<uint32_t>(k ^ ((k >> 31) & 0x7FFFFFFF)));
}

// Largest and smallest key of a group's values over the wave (every lane
// active), returned uniform.
struct GroupRange {
    int32_t hi, lo;
};
__device__ __forceinline__ GroupRange group_range(const float (&x)[4], int64_t b0, int64_t nb) {
    int32_t hi = INT32_MIN, lo = INT32_MAX;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (b0 + k < nb) {
            const int32_t key = order_key(x[k]);
            hi = max(hi, key);
            lo = min(lo, key);
        }
    }
    hi = max(hi, dpp_i32<kDppXor1>(hi));
    lo = min(lo, dpp_i32<kDppXor1>(lo));
    hi = max(hi, dpp_i32<kDppXor2>(hi));
    lo = min(lo, dpp_i32<kDppXor2>(lo));
    hi = max(hi, dpp_i32<kDppHalfMirror>(hi));
    lo = min(lo, dpp_i32<kDppHalfMirror>(lo));
    hi = max(hi, dpp_i32<kDppMirror>(hi));
    lo = min(lo, dpp_i32<kDppMirror>(lo));
    const auto rd = [](int32_t v, int l) { return static_cast<int32_t>(readlane_u32(static_cast<uint32_t>(v), l)); };
    return GroupRange{max(max(rd(hi, 0), rd(hi, 16)), max(rd(hi, 32), rd(hi, 48))),
                      min(min(rd(lo, 0), rd(lo, 16)), min(rd(lo, 32), rd(lo, 48)))};
}

// Four blocks per lane of group g (zeros past nb).
__device__ __forceinline__ void load_group(const float* __restrict__ a, int64_t nb, int64_t g, bool aligned16,
                                           float (&x)[4]) {
    const int64_t b0 = g * kGroup2 + __lane_id() * 4;
    if (aligned16 && b0 + 3 < nb) {
        const u32x4 u = *reinterpret_cast<const u32x4*>(a + b0);
#pragma unroll
        for (int k = 0; k < 4; ++k) x[k] = __uint_as_float(u[k]);
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) x[k] = b0 + k < nb ? a[b0 + k] : 0.0f;
    }
}

__global__ __launch_bounds__(kEncThreads) void nested_encode_kernel(const float* __restrict__ a, int64_t nb,
                                                                    const float* __restrict__ qmap2,
                                                                    const uint32_t* __restrict__ ws, int groups,
                                                                    float* __restrict__ offset_out,
                                                                    uint8_t* __restrict__ code,
                                                                    float* __restrict__ absmax2, NbDivider div) {
    __shared__ float c[256];
    __shared__ int unsorted;
    uint64_t rec[kOffsetLoads];
    load_records(ws, groups, rec);  // first: the mean waits on these
    if (threadIdx.x == 0) unsorted = 0;
    __syncthreads();
    if (threadIdx.x < 256) {
        c[threadIdx.x] = qmap2[threadIdx.x];
        // non-decreasing and NaN-free, else the full scan
        if (threadIdx.x > 0 && !(qmap2[threadIdx.x - 1] <= qmap2[threadIdx.x])) unsorted = 1;
        if (threadIdx.x == 0 && qmap2[0] != qmap2[0]) unsorted = 1;
    }
    // One group per wave per pass, groups g, g + step, ...; the first
    // group's values are loaded, and their range taken, before the mean, so
    // that this overlaps the wait for the records and the mean; each pass
    // loads the next group before working on this one.
    const int lane = __lane_id();
    const int64_t ngroups = (nb + kGroup2 - 1) / kGroup2;
    const int64_t step = static_cast<int64_t>(gridDim.x) * kEncWaves;
    int64_t g = static_cast<int64_t>(blockIdx.x) * kEncWaves + threadIdx.x / kWave;  // wave-uniform
    const bool aligned16 = (reinterpret_cast<uintptr_t>(a) & 15u) == 0;
    const bool code4 = (reinterpret_cast<uintptr_t>(code) & 3u) == 0;
    float x[4];
    load_group(a, nb, g, aligned16, x);
    float sep[15];
#pragma unroll
    for (int t = 0; t < 15; ++t) sep[t] = qmap2[16 * t + 15];
    GroupRange range = group_range(x, g * kGroup2 + lane * 4, nb);
    const float offset = mean_offset(rec, div);  // has barriers: c[] and unsorted are set
    const bool sorted = unsorted == 0;
    if (blockIdx.x == 0 && threadIdx.x == 0) *offset_out = offset;
    for (; g < ngroups; g += step) {
        float y[4];
        load_group(a, nb, g + step, aligned16, y);  // zeros past the end: no load
        const int64_t b0 = g * kGroup2 + lane * 4;
        // Group max of |RN(x - offset)|: RN(x - offset) does not decrease as
        // x grows, so the max is at the group's largest or smallest value.
        // A NaN anywhere makes the offset NaN, and then every |r| and this
        // max are NaN; an infinite offset gives NaN exactly for the groups
        // that hold the same infinity (inf - inf), as it does per value.
        const float amax2 = __builtin_elementwise_maximum(fabsf(from_order_key(range.hi) - offset),
                                                          fabsf(from_order_key(range.lo) - offset));
        if (lane == 0) absmax2[g] = amax2;
        const float s = __builtin_elementwise_maximum(amax2, kEps2);
        float v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = (x[k] - offset) / s;
        uint32_t q[4];
        if (sorted) {
            nearest_sorted4(c, sep, v, q);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) q[k] = nearest_scan256(c, v[k]);
        }
        if (code4 && b0 + 3 < nb) {
            *reinterpret_cast<uint32_t*>(code + b0) = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (b0 + k < nb) code[b0 + k] = static_cast<uint8_t>(q[k]);
            }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) x[k] = y[k];
        range = group_range(x, (g + step) * kGroup2 + lane * 4, nb);
    }
}

}  // namespace

int64_t nested_workspace_bytes(int64_t nb) {
    return static_cast<int64_t>(bin_groups(nb)) * kRecordWords * 4;
}

int launch_nested_encode(const float* absmax, int64_t nb, const float* qmap2, uint8_t* code, float* absmax2,
                         float* offset, void* workspace, void* stream) {
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const int groups = bin_groups(nb);
    uint32_t* ws = static_cast<uint32_t*>(workspace);
    hipLaunchKernelGGL(nested_bins_kernel, dim3(groups), dim3(kBinThreads), 0, st, absmax, nb, ws);
    const int64_t ngroups = (nb + kGroup2 - 1) / kGroup2;
    const int64_t want = (ngroups + kEncWaves - 1) / kEncWaves;
    const int64_t grid = want < kEncMaxGrid ? want : kEncMaxGrid;
    hipLaunchKernelGGL(nested_encode_kernel, dim3(static_cast<unsigned>(grid)), dim3(kEncThreads), 0, st, absmax, nb,
                       qmap2, ws, groups, offset, code, absmax2, make_nb_divider(static_cast<uint64_t>(nb)));
    return static_cast<int>(hipGetLastError());
}

// The encoder's workspace in device memory of this library, for callers
// that cannot allocate: one copy per GPU, kept until the process ends.  Its
// contents are scratch, so nothing needs clearing between calls.  Host code
// must not pass the array's name to a kernel (it is a host-side stand-in);
// it uses the device address from hipGetSymbolAddress, looked up once per
// device.
constexpr int64_t kScratchBytes = static_cast<int64_t>(kMaxBinGroups) * kRecordWords * 4;
static __device__ __align__(256) uint32_t scratch[kScratchBytes / 4];

namespace {
std::atomic<void*> g_scratch[kMaxDevices];
}  // namespace

int64_t nested_scratch_bytes() { return kScratchBytes; }

void* nested_scratch_ptr() {
    const int dev = current_device_index();
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        void* q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return nullptr;
        g_scratch[dev].store(q, std::memory_order_release);
        p = q;
    }
    return p;
}

}  // namespace kbit
