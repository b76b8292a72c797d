// Exact mean of fp32 values, rounded once to fp32 (round to nearest, ties
// to even, gradual underflow).  Host and device code: the reduction kernels
// produce per-(sign, exponent) sums of the values' integer significands;
// this header turns them into the rounded mean.
//
// A finite fp32 value with biased exponent e and fraction f is m * 2^-149
// times 2^(max(e, 1) - 1), with m = f + 2^23 for e > 0 and m = f for e = 0.
// So the exact sum of a set of values is X * 2^-149 with the integer
//   X = sum over signs and e of (+-)S[sign][e] * 2^(max(e, 1) - 1),
// S[sign][e] being the plain integer sum of the m's of that sign and e
// (below 2^24 * count, so a uint64 holds it for up to 2^40 values).  X fits
// in 320 bits.  The mean X * 2^-149 / nb is then rounded to fp32 from its
// exact quotient and remainder.
#pragma once

#include <stdint.h>

#ifndef KBIT_HD
#define KBIT_HD __host__ __device__
#endif

namespace kbit {

constexpr int kWideLimbs = 10;  // 320 bits as 32-bit limbs (little-endian)

// v * 2^shift (v < 2^64, 0 <= shift <= 253) as three 32-bit-limb pieces
// added at limbs w, w + 1, w + 2 (each piece below 2^33).
struct WidePieces {
    int w;
    uint64_t p0, p1, p2;
};
KBIT_HD inline WidePieces wide_pieces(uint64_t v, int shift) {
    const int b = shift & 31;
    const uint64_t lo = (v & 0xFFFFFFFFull) << b;  // < 2^63
    const uint64_t hi = (v >> 32) << b;            // < 2^63
    return WidePieces{shift >> 5, lo & 0xFFFFFFFFull, (lo >> 32) + (hi & 0xFFFFFFFFull), hi >> 32};
}

// X += v * 2^shift into uint64 limb accumulators (carries resolved later).
KBIT_HD inline void wide_add_shifted(uint64_t (&acc)[kWideLimbs + 2], uint64_t v, int shift) {
    const WidePieces q = wide_pieces(v, shift);
    acc[q.w] += q.p0;
    acc[q.w + 1] += q.p1;
    acc[q.w + 2] += q.p2;
}

// All loops below have constant trip counts and constant limb indices, so
// device code keeps the limbs in registers.

// Propagates carries so that every limb is below 2^32.
KBIT_HD inline void wide_normalize(uint64_t (&acc)[kWideLimbs + 2]) {
    uint64_t carry = 0;
#pragma unroll
    for (int i = 0; i < kWideLimbs + 2; ++i) {
        const uint64_t t = acc[i] + carry;
        acc[i] = t & 0xFFFFFFFFull;
        carry = t >> 32;
    }
}

// a - b for a >= b (normalized limbs).
KBIT_HD inline void wide_sub(uint64_t (&a)[kWideLimbs + 2], const uint64_t (&b)[kWideLimbs + 2]) {
    int64_t borrow = 0;
#pragma unroll
    for (int i = 0; i < kWideLimbs + 2; ++i) {
        const int64_t t = static_cast<int64_t>(a[i]) - static_cast<int64_t>(b[i]) - borrow;
        borrow = t < 0 ? 1 : 0;
        a[i] = static_cast<uint64_t>(t + (borrow << 32));
    }
}

// -1, 0, +1 as a < b, a == b, a > b (normalized limbs).
KBIT_HD inline int wide_cmp(const uint64_t (&a)[kWideLimbs + 2], const uint64_t (&b)[kWideLimbs + 2]) {
    int r = 0;
#pragma unroll
    for (int i = 0; i < kWideLimbs + 2; ++i) {  // the highest differing limb decides
        if (a[i] != b[i]) r = a[i] < b[i] ? -1 : 1;
    }
    return r;
}

KBIT_HD inline int bit_length64(uint64_t v) { return v ? 64 - __builtin_clzll(v) : 0; }

// Bits [pos, pos + 64) of X (bits past the top read as 0; pos may be
// negative, then the low bits are 0).
KBIT_HD inline uint64_t wide_bits64(const uint64_t (&x)[kWideLimbs + 2], int pos) {
    uint64_t r = 0;
#pragma unroll
    for (int i = 0; i < kWideLimbs; ++i) {
        const int sh = 32 * i - pos;  // where limb i lands in the result
        if (sh >= 64 || sh <= -32) continue;
        r |= sh >= 0 ? (x[i] << sh) : (x[i] >> -sh);
    }
    return r;
}

// True if any bit of X below position pos is set.
KBIT_HD inline bool wide_any_below(const uint64_t (&x)[kWideLimbs + 2], int pos) {
    bool any = false;
#pragma unroll
    for (int i = 0; i < kWideLimbs; ++i) {
        const int below = pos - 32 * i;  // bits of limb i below pos
        if (below >= 32) any = any || x[i] != 0;
        else if (below > 0) any = any || (x[i] & ((1ull << below) - 1ull)) != 0;
    }
    return any;
}

// fp32 bits of RN32(sign * X * 2^-149 / nb), 1 <= nb <= 2^36.
KBIT_HD inline uint32_t wide_mean_bits(const uint64_t (&x)[kWideLimbs + 2], bool negative, uint64_t nb) {
    int p = 0;  // bit length of X
#pragma unroll
    for (int i = 0; i < kWideLimbs; ++i) {
        if (x[i]) p = 32 * i + bit_length64(x[i]);
    }
    const uint32_t sign = negative ? 0x80000000u : 0u;
    if (p == 0) return sign;
    // N = X * 2^-s with 63 bits; Q = N / nb then has at least 27 bits.
    const int s = p - 63;
    const uint64_t N = wide_bits64(x, s);
    bool sticky = s > 0 && wide_any_below(x, s);
    const uint64_t Q = N / nb;
    sticky = sticky || (N % nb) != 0;
    // value = (Q + fraction) * 2^(s - 149); exponent of its leading bit
    const int qb = bit_length64(Q);
    int E = qb - 1 + s - 149;
    // drop d low bits of Q: down to 24 significant bits, or to the 2^-149
    // quantum in the subnormal range
    const int d = E >= -126 ? qb - 24 : -s;
    if (E < -126) E = -127;  // subnormal (exponent field 0)
    uint64_t mant;
    bool guard;
    if (d >= 64) {
        mant = 0;
        guard = d == 64 && (Q >> 63) != 0;
        sticky = sticky || (d == 64 ? (Q & ~(1ull << 63)) != 0 : Q != 0);
    } else {
        mant = Q >> d;
        guard = d > 0 && ((Q >> (d - 1)) & 1ull);
        sticky = sticky || (d > 1 && (Q & ((1ull << (d - 1)) - 1ull)) != 0);
    }
    if (guard && (sticky || (mant & 1ull))) ++mant;
    if (E == -127) {
        // subnormal: the field is the significand; 2^23 is the smallest normal
        return sign | static_cast<uint32_t>(mant);
    }
    if (mant == (1ull << 24)) {
        mant >>= 1;
        ++E;
    }
    if (E > 127) return sign | 0x7F800000u;
    return sign | (static_cast<uint32_t>(E + 127) << 23) | (static_cast<uint32_t>(mant) & 0x7FFFFFu);
}

// Rounded mean from the limb accumulators of the positive and the negative
// values (carries not yet resolved) and the count nb.
KBIT_HD inline uint32_t mean_from_limbs(uint64_t (&pos)[kWideLimbs + 2], uint64_t (&neg)[kWideLimbs + 2],
                                        uint64_t nb) {
    wide_normalize(pos);
    wide_normalize(neg);
    if (wide_cmp(pos, neg) >= 0) {
        wide_sub(pos, neg);
        return wide_mean_bits(pos, false, nb);
    }
    wide_sub(neg, pos);
    return wide_mean_bits(neg, true, nb);
}

// The same from per-(sign, exponent) significand sums S[2][256] (sign 0
// positive, 1 negative; exponent 255 unused).
KBIT_HD inline uint32_t mean_from_sums(const uint64_t (&S)[2][256], uint64_t nb) {
    uint64_t pos[kWideLimbs + 2] = {}, neg[kWideLimbs + 2] = {};
    for (int e = 0; e < 255; ++e) {
        const int shift = (e > 0 ? e : 1) - 1;
        if (S[0][e]) wide_add_shifted(pos, S[0][e], shift);
        if (S[1][e]) wide_add_shifted(neg, S[1][e], shift);
    }
    return mean_from_limbs(pos, neg, nb);
}

}  // namespace kbit
