// Exact per-workgroup sums of fp32 values, the first half of the nested
// state's mean offset (the mean of every block absmax, rounded once; the
// rounding is exact_mean.h).  Used by the encoder's first launch over an
// absmax array and by the quantize kernel that produces the absmax itself.
//
// A finite nonzero value with biased exponent e and integer significand m
// is m * 2^(e' - 1) in units of 2^-149, e' = max(e, 1).  Per round a wave
// holds 4 values per lane.  With E the wave's largest e' and
// e0 = max(E - 24, 1), every value with e' >= e0 adds m << (e' - e0) (below
// 2^48) to the register sum of its sign, in units of 2^(e0 - 1); the wave's
// two sums (below 2^56) go into the wave's own limb accumulators in LDS once
// per round, as three pieces below 2^33 (lane 0 alone writes them, so no
// atomics).  Values further down (more than 24 binades below the wave's
// top) add m to the workgroup's LDS bin of their sign and e, folded into
// wave 0's limbs at the end (only if any exist).  NaN and infinities only
// set flags.  Then wave 0 adds the waves' limbs (lane 16 s + i takes limb i
// of sign s) and carries them into 32-bit digits: the workgroup's record,
// 25 words (10 + 2 digits per sign, then the flags).  The quantize kernel's
// variant puts every block maximum into the bins (any_slow set from the
// start) and uses only the record step.
//
// Bounds, for at most 2^28 values per workgroup: a wave's limb takes at
// most one piece per round and sign, so all waves' limbs of one index add
// up to below 2^20 * 2^33 (2^20 wave rounds of 256 values), plus at most
// 256 bin pieces; a bin stays below 2^28 * 2^24.  A workgroup's sum is
// below 2^28 * 2^277, so its carried digits fit the 10 low limbs and each
// is below 2^32.
//
// The record is word-major: word k of workgroup b at ws[k * groups + b], so
// that the second launch reads each word of all records with contiguous
// loads.
#pragma once

#include "device.h"
#include "exact_mean.h"

namespace kbit {

constexpr int kLimbWords = kWideLimbs + 2;
constexpr int kRecordWords = 2 * kLimbWords + 1;  // uint32: digits[sign][i], then the flags
constexpr uint32_t kFlagNan = 1, kFlagPosInf = 2, kFlagNegInf = 4;
constexpr int kWindowBits = 24;  // binades below the wave's top one that the register sums take
// Most records the encoder's second launch reads: those of the quantize
// kernel's nested-state variant (one per resident workgroup, two per CU);
// the encoder's own first launch writes at most 256.
constexpr int kMaxSumGroups = 512;

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

// The workgroup's LDS state: bins by (sign, exponent) and each wave's limbs.
template <int WAVES>
struct SumsShared {
    unsigned long long bins[2][256];
    unsigned long long wlimbs[WAVES][2][kLimbWords];
    uint32_t flags, any_slow;
};

// All threads; a barrier must follow before the first round.
template <int WAVES, int THREADS>
__device__ __forceinline__ void sums_clear(SumsShared<WAVES>& sh) {
    for (int i = threadIdx.x; i < 2 * 256; i += THREADS) (&sh.bins[0][0])[i] = 0;
    for (int i = threadIdx.x; i < WAVES * 2 * kLimbWords; i += THREADS) (&sh.wlimbs[0][0][0])[i] = 0;
    if (threadIdx.x == 0) sh.flags = sh.any_slow = 0;
}

// One round of the wave (all lanes, uniform control flow): the lane's 4
// values (fp32 bits) into the wave's limbs, the bins or the lane's flags.
template <int WAVES>
__device__ __forceinline__ void sums_round(SumsShared<WAVES>& sh, int wave, int lane, const u32x4& u,
                                           uint32_t& my_flags) {
    uint32_t top = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint32_t e = (u[c] >> 23) & 0xFFu;
        if (e != 0xFFu && (u[c] & 0x7FFFFFFFu) != 0) top = max(top, max(e, 1u));
    }
    top = wave_max_u32(top);
    const uint32_t e0 = top > kWindowBits + 1 ? top - kWindowBits : 1u;
    // branch-free for the values in the window; the rest (rare) after
    uint64_t sum_pos = 0, sum_neg = 0;
    uint32_t slow = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint32_t x = u[c];
        const uint32_t e = (x >> 23) & 0xFFu, f = x & 0x7FFFFFu;
        const bool neg = (x >> 31) != 0, special = e == 0xFFu;
        my_flags |= special ? (f ? kFlagNan : (neg ? kFlagNegInf : kFlagPosInf)) : 0u;
        const uint32_t ee = max(e, 1u), m = e ? (f | 0x800000u) : f;  // m = 0 for zeros
        const bool fast = !special && ee >= e0;
        const uint64_t t = static_cast<uint64_t>(fast ? m : 0u) << (fast ? ee - e0 : 0u);
        sum_neg += neg ? t : 0ull;
        sum_pos += neg ? 0ull : t;
        slow |= (!special && !fast && m != 0) ? (1u << c) : 0u;
    }
    if (slow != 0) {
        atomicOr(&sh.any_slow, 1u);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (slow & (1u << c)) {
                const uint32_t x = u[c];
                const uint32_t e = (x >> 23) & 0xFFu, f = x & 0x7FFFFFu;
                atomicAdd(&sh.bins[x >> 31][e], static_cast<unsigned long long>(e ? (f | 0x800000u) : f));
            }
        }
    }
    sum_pos = wave_sum_u64(sum_pos);
    sum_neg = wave_sum_u64(sum_neg);
    if (lane == 0) {
        unsigned long long* my_limbs = &sh.wlimbs[wave][0][0];
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

// The workgroup's record from its waves' rounds, stored as workgroup g of
// `groups` (all threads call it, after their last round).
template <int WAVES, int THREADS>
__device__ __forceinline__ void sums_record(SumsShared<WAVES>& sh, uint32_t my_flags, uint32_t* __restrict__ ws,
                                            int64_t groups, int64_t g) {
    if (my_flags) atomicOr(&sh.flags, my_flags);
    __syncthreads();
    if (sh.any_slow != 0) {  // workgroup-uniform: bins -> wave 0's limbs
        for (int i = threadIdx.x; i < 2 * 256; i += THREADS) {
            const uint64_t sum = (&sh.bins[0][0])[i];
            const int sg = i >> 8, e = i & 255;
            if (sum != 0) {
                const WidePieces q = wide_pieces(sum, (e > 0 ? e : 1) - 1);
                atomicAdd(&sh.wlimbs[0][sg][q.w], static_cast<unsigned long long>(q.p0));
                atomicAdd(&sh.wlimbs[0][sg][q.w + 1], static_cast<unsigned long long>(q.p1));
                atomicAdd(&sh.wlimbs[0][sg][q.w + 2], static_cast<unsigned long long>(q.p2));
            }
        }
        __syncthreads();
    }
    if (threadIdx.x < kWave) {
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
        const int lane = __lane_id();
        const int sg = lane >> 4, li = lane & 15;
        const bool mine = lane < 32 && li < kLimbWords;
        uint64_t t = 0;
        if (mine) {
#pragma unroll
            for (int w = 0; w < WAVES; ++w) t += sh.wlimbs[w][sg][li];
        }
        const uint32_t hi_below = row_shr1_or_zero(static_cast<uint32_t>(t >> 32));
        const uint64_t sum = (t & 0xFFFFFFFFull) + hi_below;
        const uint32_t low = static_cast<uint32_t>(sum);
        const uint64_t G = __ballot(mine && (sum >> 32) != 0);
        const uint64_t P = __ballot(mine && low == 0xFFFFFFFFu);
        const uint64_t carries = ((G | P) + G) ^ (G | P) ^ G;
        const uint32_t digit = low + static_cast<uint32_t>((carries >> lane) & 1ull);
        if (mine) ws[(sg * kLimbWords + li) * groups + g] = digit;
        if (lane == 0) ws[2 * kLimbWords * groups + g] = sh.flags;
    }
}

}  // namespace kbit
