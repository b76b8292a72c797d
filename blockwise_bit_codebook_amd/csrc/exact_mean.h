// Exact mean of fp32 values, rounded once to fp32 (round to nearest, ties
// to even, gradual underflow).  Host and device code: the reduction kernels
// add the values' integer significands, shifted by their exponents, into
// 32-bit-limb accumulators of the positive and the negative values; this
// header turns those into the rounded mean.
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

KBIT_HD inline int bit_length64(uint64_t v) { return v ? 64 - __builtin_clzll(v) : 0; }

// Division by the block count nb (1 <= nb <= 2^36) of any n below 2^63,
// without a divide instruction: with l = ceil(log2 nb) and
// m = ceil(2^(63 + l) / nb), floor(n / nb) = floor(n * m / 2^(63 + l)).
// (Division by an invariant integer through a multiply-high, after Granlund
// and Montgomery, "Division by invariant integers using multiplication",
// 1994.)  Why: n * m / 2^(63 + l) = n / nb + n * e / 2^(63 + l) with
// m = 2^(63 + l) / nb + e, 0 <= e < 1, and the second term is below
// 2^-l <= 1 / nb, while the fraction of n / nb is at most 1 - 1 / nb; so
// the floor does not change.  m is below 2^64 (2^(l - 1) < nb unless nb is
// 1, where m = 2^63).  The host builds it once per call.
struct NbDivider {
    uint64_t nb, m;
    int l;
};
inline NbDivider make_nb_divider(uint64_t nb) {
    int l = 0;
    while ((1ull << l) < nb) ++l;
    const unsigned __int128 num = (static_cast<unsigned __int128>(1) << (63 + l)) + (nb - 1);
    return NbDivider{nb, static_cast<uint64_t>(num / nb), l};
}
KBIT_HD inline uint64_t div_nb(const NbDivider& d, uint64_t n) {  // n < 2^63
    const unsigned __int128 p = static_cast<unsigned __int128>(n) * d.m;  // below 2^127
    return static_cast<uint64_t>(p >> 63) >> d.l;
}

// fp32 bits of RN32((P - N) * 2^-149 / nb), 1 <= nb <= 2^36 (the divider
// of nb), from the limb accumulators of P (positive values) and N (negative
// values): limb i weighs 2^(32 i), each limb is below 2^61 (carries not yet
// resolved), and |P - N| < 2^320.  Straight-line code for one thread: every
// array index is a constant after unrolling.
KBIT_HD inline uint32_t mean_from_limbs(const uint64_t (&pos)[kWideLimbs + 2], const uint64_t (&neg)[kWideLimbs + 2],
                                        const NbDivider& div) {
    const uint64_t nb = div.nb;
    constexpr int L = kWideLimbs + 2;
    // D = P - N as 32-bit digits plus a final carry (floor division by 2^32
    // at each limb keeps every intermediate within int64).
    uint32_t d[L];
    int64_t carry = 0;
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const int64_t t = static_cast<int64_t>(pos[i]) - static_cast<int64_t>(neg[i]) + carry;
        d[i] = static_cast<uint32_t>(t);
        carry = t >> 32;  // arithmetic shift: floor
    }
    // |D| < 2^320, so the carry is -1 exactly when D < 0; then the digits
    // hold 2^(32 L) + D and their two's complement is |D|.
    const bool negative = carry < 0;
    if (negative) {
        uint64_t c = 1;
#pragma unroll
        for (int i = 0; i < L; ++i) {
            const uint64_t t = static_cast<uint64_t>(~d[i]) + c;
            d[i] = static_cast<uint32_t>(t);
            c = t >> 32;
        }
    }
    const uint32_t sign = negative ? 0x80000000u : 0u;
    // Highest nonzero digit `top`, the two below it, and whether any digit
    // further down is nonzero.
    int top = -1;
    uint32_t h0 = 0, h1 = 0, h2 = 0;
    bool low = false;
    uint32_t below = 0;  // OR of the digits under the current i - 2
#pragma unroll
    for (int i = 0; i < kWideLimbs; ++i) {
        if (d[i] != 0) {
            top = i;
            h0 = d[i];
            h1 = i >= 1 ? d[i - 1] : 0u;
            h2 = i >= 2 ? d[i - 2] : 0u;
            low = below != 0;
        }
        if (i >= 2) below |= d[i - 2];
    }
    if (top < 0) return sign;
    // |D| = W * 2^(32 (top - 2)) + (the lower digits), W = h0:h1:h2 (96
    // bits, 64 + b of them significant).  Its leading 63 bits are
    // Nq = W >> (b + 1), scaled by 2^s with s = 32 (top - 2) + b + 1; the
    // bits shifted out and the lower digits only decide the sticky bit.
    const int b = bit_length64(h0);  // 1..32
    const uint64_t mid = (static_cast<uint64_t>(h1) << 32) | h2;
    const uint64_t Nq = (static_cast<uint64_t>(h0) << (63 - b)) | (mid >> (b + 1));
    const int s = 32 * (top - 2) + b + 1;
    bool sticky = low || (mid & ((1ull << (b + 1)) - 1ull)) != 0;
    // Q = Nq / nb has at least 27 bits; the value is (Q + fraction) * 2^s.
    // Nq < 2^63 (its top bit is bit 62).
    const uint64_t Q = div_nb(div, Nq);
    sticky = sticky || Nq - Q * nb != 0;
    const int qb = bit_length64(Q);
    int E = qb - 1 + s - 149;  // exponent of the leading bit
    // drop dq low bits of Q: down to 24 significant bits, or to the 2^-149
    // quantum in the subnormal range
    const int dq = E >= -126 ? qb - 24 : -s;
    if (E < -126) E = -127;  // subnormal (exponent field 0)
    uint64_t mant;
    bool guard;
    if (dq >= 64) {
        mant = 0;
        guard = dq == 64 && (Q >> 63) != 0;
        sticky = sticky || (dq == 64 ? (Q & ~(1ull << 63)) != 0 : Q != 0);
    } else {
        mant = Q >> dq;
        guard = dq > 0 && ((Q >> (dq - 1)) & 1ull);
        sticky = sticky || (dq > 1 && (Q & ((1ull << (dq - 1)) - 1ull)) != 0);
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

}  // namespace kbit
