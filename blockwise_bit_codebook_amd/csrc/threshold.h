// Exact nearest-code decisions without a per-element division, shared by
// the blockwise quantizer and the activation assignment.
//
// For a sorted codebook whose distinct neighbours are far apart compared
// with the rounding of the distances involved, the first-index argmin of
// |RN(v - c_i)| picks, between neighbouring codes lo < hi, the upper one
// exactly when v >= u for one fp32 value u (the rule is monotone in v).
// With v = RN(x/s), s > 0:  v >= u  <=>  x - M*s > 0,  where M is the
// midpoint of u and its fp32 predecessor (nudged by a few fp64 ulps for the
// round-to-even direction of an exact tie).  M*s has at most 49 significant
// bits, so one fp64 fma gives the sign exactly.
//
// Which threshold applies is found from q = fma(x, slope*rcp(s), base), an
// approximation of base + slope*v inside [2, 4): bits 16..22 of q pick one
// of 128 buckets, and a bucket's 16-byte entry holds the M of the one
// threshold whose window [t - 2^-18, t + 2^-18] meets it (t = base +
// slope*midpoint; the error of q is far below 2^-18) and the plane bytes of
// the indices on either side of it.  Each bucket row is replicated 16 times
// in LDS and lane l reads copy l mod 16, so the 16 lanes served per LDS
// cycle never share a bank; one v_perm_b32 forms the address.
#pragma once

#include "device.h"

namespace kbit {

constexpr int kBuckets = 128;
constexpr int kCopies = 16;
constexpr float kDelta = 0x1p-18f;  // bucket window half-width in q
constexpr uint64_t kNoMid = ~uint64_t(0);  // marks a failed search (never an M: bits 1:0 of M are 0)

// Bucket rows, their master copy, and the per-threshold M (fp64 bits).
template <int C>
struct ThresholdTables {
    u32x4 row[kBuckets * kCopies];  // {M, planes(below), planes(above)} per copy
    u32x4 master[kBuckets];
    uint64_t mid[C];                // mid[i]: threshold between codes i-1 and i
    float code[C];                  // the codebook (exact path)
    int fail;
};

// fp32 values in the order of their keys: key(-0) + 1 = key(+0).
__device__ __forceinline__ uint32_t order_key(float v) {
    const uint32_t b = __float_as_uint(v);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float from_key(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// The definition's choice between neighbouring codes lo < hi (lower index
// wins ties).
__device__ __forceinline__ bool upper_wins(float xn, float lo, float hi) {
    return fabsf(xn - hi) < fabsf(xn - lo);
}

// fp64 bits of M for the switching point u (the smallest fp32 value for
// which the upper code wins) and its fp32 predecessor p: RN(x/s) >= u <=>
// x - M*s > 0 (s > 0).
__device__ inline uint64_t mid_bits(float u, float p) {
    const double M = (static_cast<double>(u) + static_cast<double>(p)) * 0.5;  // exact
    // An exact tie x/s == M rounds to the even one of pred(u), u: to u means
    // "upper" at equality, so M moves down by 4 fp64 ulps; otherwise it moves
    // up (or stays); bits 1:0 are then cleared.
    const bool tie_up = static_cast<float>(M) == u;
    uint64_t b = static_cast<uint64_t>(__double_as_longlong(M));
    if (M > 0.0) b = tie_up ? b - 4u : b;
    else b = tie_up ? b + 4u : b - 4u;
    return b & ~static_cast<uint64_t>(3u);
}

// The same switching point as two fp32 values {Mh, Ml'} (low word Mh): M =
// Mh + Ml exactly with Mh = p and Ml = (u - p) / 2 (a power of two), and
// Ml' = Ml nudged by one fp32 ulp the way mid_bits nudges M.  For x and s
// with at most 11 significant bits (bf16 and fp16 values) the sign of
// fma(-Ml', s, fma(-Mh, s, x)) is the sign of x - M*s: the inner fma is
// exact whenever |x - Mh*s| is small enough to matter, and otherwise that
// difference is far larger than Ml*s.  (Exact ties x/s == M cannot occur
// for such x and s, since M has 25 significant bits.)  Returns kNoMid when
// Ml would fall below 2^-100.
__device__ inline uint64_t pair_bits(float u, float p) {
    const float ml = static_cast<float>((static_cast<double>(u) - static_cast<double>(p)) * 0.5);
    if (!(ml >= 0x1p-100f)) return kNoMid;
    const double M = (static_cast<double>(u) + static_cast<double>(p)) * 0.5;
    const bool tie_up = static_cast<float>(M) == u;
    const uint32_t mlb = __float_as_uint(ml);
    const uint32_t ml2 = tie_up ? mlb - 1u : mlb + 1u;  // M down (ties up) or up (ties down)
    return static_cast<uint64_t>(__float_as_uint(p)) | (static_cast<uint64_t>(ml2) << 32);
}

// One fp32 value T for the switching point u (predecessor p) of bf16
// inputs, for the decision RN(x/s) >= u  <=>  x - T*s >= 0 (one fma, exact
// sign).  x and s (a block maximum) are bf16 values, so x/s = (mx/ms) 2^d
// with 8-bit significands mx, ms; two distinct such quotients differ by at
// least 2^-17 relative, while [p, u] is at most 2^-23 wide, so at most one
// of them, q*, lies in [p, u].  T = u classifies every quotient outside
// [p, u] correctly, and so does T = p; the one q* picks: T = p if q* lies in
// (M, u] (it must go up), or equals M = (p + u)/2 with the tie rounding to
// u; T = u otherwise (q* in [p, M) must go down).  The lanes of the group
// (G = 32 or 64) test the 128 significands ms of s: the only candidate
// numerator is mx = round(M ms 2^-d) with d putting it into [128, 255],
// checked exactly against [p, u] with fp64 products.  Returns kNoMid when
// |M| is outside [2^-100, 2] (the exact path then applies).  Every lane of
// the wave must call it.
template <int G>
__device__ inline uint64_t tform_bits_group(float u, float p) {
    const uint32_t lane = __lane_id();
    const uint32_t i = lane % G;
    const uint32_t gshift = G == 64 ? 0u : (lane / G) * 32u;
    auto group_any = [&](bool b) {
        const uint64_t m = __builtin_amdgcn_ballot_w64(b);
        return (G == 64 ? m : ((m >> gshift) & 0xFFFFFFFFull)) != 0;
    };
    const double M = (static_cast<double>(u) + static_cast<double>(p)) * 0.5;  // exact
    const bool tie_up = static_cast<float>(M) == u;
    const double A = fabs(M);
    const bool ok = A >= 0x1p-100 && A <= 2.0;
    const double au = fabs(static_cast<double>(u)), ap = fabs(static_cast<double>(p));
    const double lo_m = au < ap ? au : ap, hi_m = au < ap ? ap : au;
    const int kk = ok ? static_cast<int>((__double_as_longlong(A) >> 52) & 0x7FF) - 1023 : 0;
    bool below = false, eq = false, above = false;
#pragma unroll
    for (int h = 0; h < 128 / G; ++h) {
        const double ms = static_cast<double>(128 + i + G * h);
        const double am = A * ms;                       // exact: 25 + 8 bits
        int d = kk;
        double P = ldexp(am, -d);                       // in [128, 512)
        if (P >= 256.0) {
            d += 1;
            P *= 0.5;
        }
        double mx = floor(P + 0.5);                     // P + 0.5 is exact
        if (mx == 256.0) {
            mx = 128.0;
            d += 1;
        }
        const double num = ldexp(mx, d);                // |x/s| * ms, exact
        const bool in = ok && mx >= 128.0 && mx <= 255.0 && lo_m * ms <= num && num <= hi_m * ms;
        below = below || (in && num < am);
        eq = eq || (in && num == am);
        above = above || (in && num > am);
    }
    below = group_any(below);
    eq = group_any(eq);
    above = group_any(above);
    const bool q_above = M > 0.0 ? above : below;       // a quotient in (M, u]
    const float T = eq ? (tie_up ? p : u) : (q_above ? p : u);
    return ok ? static_cast<uint64_t>(__float_as_uint(T)) : kNoMid;
}

// Forms of a switching point in the tables (the entry's first two words):
//   kMid64  - M as fp64 (any fp32 x and s): sign of fma(-M, s, x)
//   kPair32 - {Mh, Ml'} (x, s with at most 11 significant bits: bf16, fp16):
//             sign of fma(-Ml', s, fma(-Mh, s, x))
//   kT32    - {T, 0} (bf16 x and s): sign of fma(-T, s, x)
// In every form the decision value is never zero for the inputs it serves,
// so "upper code" is exactly "sign bit clear".
constexpr int kMid64 = 0, kPair32 = 1, kT32 = 2;

// M for the threshold between codes lo < hi, found by a group of G lanes
template <int G, int FORM = kMid64>
__device__ inline bool threshold_mid_group(float lo, float hi, uint64_t& bits) {
    static_assert(G == 32 || G == 64, "lane groups of 32 or 64");
    const uint32_t lane = __lane_id();
    const uint32_t i = lane % G;
    const uint32_t gshift = G == 64 ? 0u : (lane / G) * 32u;  // the group's bits in a ballot
    auto group_bits = [&](uint64_t m) -> uint64_t {
        return G == 64 ? m : ((m >> gshift) & 0xFFFFFFFFull);
    };
    uint32_t L = order_key(lo), R = order_key(hi);
    const bool ok = !upper_wins(lo, lo, hi) && upper_wins(hi, lo, hi);
    if (!ok) L = R - 1;  // nothing to search; reported below
    // round 0: keys mid - G/2 + 1 .. mid + G/2 inside (L, R)
    {
        const uint32_t mk = order_key((lo + hi) * 0.5f);
        const uint32_t k = mk + i - (G / 2 - 1);
        const bool inside = k > L && k < R;
        const bool up = inside && upper_wins(from_key(k), lo, hi);
        const uint64_t upm = group_bits(__builtin_amdgcn_ballot_w64(up));
        const uint64_t inm = group_bits(__builtin_amdgcn_ballot_w64(inside));
        // the tested keys are consecutive: the first "up" key and the key
        // below it bracket u if that key is also inside (or is L)
        if (R - L > 1u && inm != 0) {
            const uint32_t first_in = mk - (G / 2 - 1) + static_cast<uint32_t>(__builtin_ctzll(inm));
            const uint32_t last_in = mk - (G / 2 - 1) + static_cast<uint32_t>(63 - __builtin_clzll(inm));
            if (upm != 0) {
                const uint32_t kj = mk - (G / 2 - 1) + static_cast<uint32_t>(__builtin_ctzll(upm));
                R = kj;
                if (kj > first_in) L = kj - 1;
                else L = L;  // u may still lie below the window: keep L
            } else {
                L = last_in;
            }
        }
    }
    while (__builtin_amdgcn_ballot_w64(R - L > 1u) != 0) {
        const uint64_t w = R - L;
        auto key = [&](uint32_t j) { return L + static_cast<uint32_t>((w * j) / G); };
        // i = 0 tests L itself, known to choose the lower code
        const bool up = w > 1 && i != 0 && upper_wins(from_key(key(i)), lo, hi);
        const uint64_t mask = group_bits(__builtin_amdgcn_ballot_w64(up));
        if (w > 1) {
            if (mask == 0) {
                L = key(G - 1);
            } else {
                const uint32_t j = static_cast<uint32_t>(__builtin_ctzll(mask));
                const uint32_t kj = key(j), kp = key(j - 1);
                R = kj;
                L = kp;
            }
        }
    }
    if constexpr (FORM == kT32) {
        bits = tform_bits_group<G>(from_key(R), from_key(L));  // every lane of the wave calls it
        return ok && bits != kNoMid;
    } else if constexpr (FORM == kPair32) {
        bits = pair_bits(from_key(R), from_key(L));
        return ok && bits != kNoMid;
    } else {
        bits = mid_bits(from_key(R), from_key(L));
        return ok;
    }
}

// The same with the whole wave on one threshold.
template <int FORM = kMid64>
__device__ inline bool threshold_mid_wave(float lo, float hi, uint64_t& bits) {
    return threshold_mid_group<64, FORM>(lo, hi, bits);
}

// Entry for bucket j (q in [2 + j/64, 2 + (j+1)/64)): the M of the one
// threshold whose window meets the bucket (mid[i] from threshold_mid_group)
// and the plane bytes of the indices below and above it (bit 0 of byte p =
// plane p), with PLANE4 plane 4 in bit 1 of byte 0.  Returns false if two
// windows meet the bucket.
template <int C, bool PLANE4>
__device__ bool build_entry(const float (&c)[C], const uint64_t* mid, int j, float slope, float base,
                            u32x4& e) {
    const float lo = 2.0f + static_cast<float>(j) * (2.0f / kBuckets);
    const float hi = lo + (2.0f / kBuckets);
    // The thresholds rise with i (the codebook is sorted): below = the last
    // one whose window lies under the bucket, cand = the first whose window
    // meets it (0: none).  Selects only, no branches.
    int below = 0, cand = 0, meets = 0;
#pragma unroll
    for (int i = 1; i < C; ++i) {
        const bool distinct = c[i] != c[i - 1];
        const float t = base + ((c[i - 1] + c[i]) * 0.5f) * slope;
        const bool under = distinct && t + kDelta <= lo;
        const bool meet = distinct && !under && t - kDelta < hi;
        below = under ? i : below;
        cand = (meet && cand == 0) ? i : cand;
        meets += meet ? 1 : 0;
    }
    const uint32_t above = cand == 0 ? static_cast<uint32_t>(below) : static_cast<uint32_t>(cand);
    const uint64_t m = cand == 0 ? 0u : mid[cand];
    auto planes = [](uint32_t i) { return spread4(i & 15u) | (PLANE4 ? ((i >> 4) & 1u) << 1 : 0u); };
    e = u32x4{static_cast<uint32_t>(m), static_cast<uint32_t>(m >> 32), planes(static_cast<uint32_t>(below)),
              planes(above)};
    return meets <= 1;
}

// build_entry for all buckets at once, by every thread of a workgroup of
// THREADS (512 or 1024) threads: THREADS / 128 consecutive lanes share a
// bucket, each tests its slice of the thresholds, the slices combine with
// DPP (below = max, cand = min, meets = sum), and each lane writes its share
// of the kCopies copies of the entry into rows.  code and mid are the
// codebook and the switching points in LDS (written before a barrier that
// precedes this call).  Returns false in every lane of a bucket whose entry
// is ambiguous (two windows meet it) or whose threshold search failed; the
// caller folds that into the table's fail flag.
template <int C, bool PLANE4, int THREADS>
__device__ inline bool build_entries_parallel(const float* code, const uint64_t* mid, float slope, float base,
                                              u32x4* rows) {
    constexpr int kTpb = THREADS / kBuckets;                // threads per bucket
    static_assert(kTpb == 4 || kTpb == 8, "512 or 1024 threads");
    constexpr int kTpt = (C - 1 + kTpb - 1) / kTpb;          // thresholds per thread
    const int j = threadIdx.x / kTpb, part = threadIdx.x % kTpb;
    const float lo = 2.0f + static_cast<float>(j) * (2.0f / kBuckets);
    const float hi = lo + (2.0f / kBuckets);
    int below = 0, cand = C, meets = 0;
    bool failed = false;
#pragma unroll
    for (int t = 0; t < kTpt; ++t) {
        const int i = 1 + part * kTpt + t;
        if (i < C) {
            const float cl = code[i - 1], ch = code[i];
            const bool distinct = ch != cl;
            const float tp = base + ((cl + ch) * 0.5f) * slope;
            const bool under = distinct && tp + kDelta <= lo;
            const bool meet = distinct && !under && tp - kDelta < hi;
            below = under ? i : below;                         // thresholds rise with i
            cand = (meet && i < cand) ? i : cand;
            meets += meet ? 1 : 0;
            failed = failed || (distinct && mid[i] == kNoMid);
        }
    }
    below = max(below, static_cast<int>(dpp_u32<kDppXor1>(below)));
    below = max(below, static_cast<int>(dpp_u32<kDppXor2>(below)));
    cand = min(cand, static_cast<int>(dpp_u32<kDppXor1>(cand)));
    cand = min(cand, static_cast<int>(dpp_u32<kDppXor2>(cand)));
    meets += static_cast<int>(dpp_u32<kDppXor1>(meets));
    meets += static_cast<int>(dpp_u32<kDppXor2>(meets));
    uint32_t f = failed ? 1u : 0u;
    f |= dpp_u32<kDppXor1>(f);
    f |= dpp_u32<kDppXor2>(f);
    if constexpr (kTpb == 8) {
        below = max(below, static_cast<int>(dpp_u32<kDppHalfMirror>(below)));
        cand = min(cand, static_cast<int>(dpp_u32<kDppHalfMirror>(cand)));
        meets += static_cast<int>(dpp_u32<kDppHalfMirror>(meets));
        f |= dpp_u32<kDppHalfMirror>(f);
    }
    const uint32_t above = cand == C ? static_cast<uint32_t>(below) : static_cast<uint32_t>(cand);
    const uint64_t m = cand == C ? 0u : mid[cand];
    auto planes = [](uint32_t ix) { return spread4(ix & 15u) | (PLANE4 ? ((ix >> 4) & 1u) << 1 : 0u); };
    const u32x4 e = u32x4{static_cast<uint32_t>(m), static_cast<uint32_t>(m >> 32),
                          planes(static_cast<uint32_t>(below)), planes(above)};
    constexpr int kCpt = kCopies / kTpb;                    // copies written per thread
#pragma unroll
    for (int k = 0; k < kCpt; ++k) rows[j * kCopies + kCpt * part + k] = e;
    return meets <= 1 && f == 0;
}

// Byte address of the lane's copy of q's bucket entry: byte 1 <- bits
// 16..23 of q (bucket; bit 23 is 0 for q in [2, 4)), byte 0 <- lane offset.
__device__ __forceinline__ uint32_t entry_addr(float q, uint32_t lane_off) {
    return __builtin_amdgcn_perm(lane_off, __float_as_uint(q), 0x0C0C0204u);
}

// The entry for q and the exact decision "upper code" for x against scale
// s64 (= s as fp64).
struct Decision {
    u32x4 e;
    bool up;
};
__device__ __forceinline__ Decision decide(float x, float q, double s64, const char* tab, uint32_t lane_off) {
    Decision d;
    d.e = *reinterpret_cast<const u32x4*>(tab + entry_addr(q, lane_off));
    const double M = __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(d.e[1]) << 32) | d.e[0]));
    d.up = __builtin_fma(-M, s64, static_cast<double>(x)) > 0.0;
    return d;
}

// The same with entries in the pair form (pair_bits), for x and s of at
// most 11 significant bits: two fp32 fmas instead of a conversion, an fp64
// fma and an fp64 compare.
__device__ __forceinline__ Decision decide32(float x, float q, float s, const char* tab, uint32_t lane_off) {
    Decision d;
    d.e = *reinterpret_cast<const u32x4*>(tab + entry_addr(q, lane_off));
    const float t1 = __builtin_fmaf(-__uint_as_float(d.e[0]), s, x);
    d.up = __builtin_fmaf(-__uint_as_float(d.e[1]), s, t1) > 0.0f;
    return d;
}

}  // namespace kbit
