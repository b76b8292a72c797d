// E4M4 one-byte block scales ([QLORA-2] PATCH 005 "Add vectorized dequant
// kernel and E4M4 uint8 absmax": functional.py encode_absmax_e4m4 /
// decode_absmax_e4m4 and the kernel-side decoder).
//
// Byte = e << 4 | m, exponent bias 11:
//   e > 0: 2^(e - 11) * (1 + m/16)        e = 0: m * 2^-14 (0x00 is zero)
// Encoding of a float32 scale a:
//   a <= 0 or NaN        -> 0
//   a = +inf             -> 0xF0 (exponent above the range, fraction 0)
//   a < 2^-10            -> m = RNE(a * 2^14), clamped to 15
//   otherwise            -> e = min(E + 11, 15) with E the binary exponent
//                           of a, m = the 23 fraction bits of a rounded to 4
//                           (half to even), clamped to 15 (no carry into e)
// The page computes the exponent as floor(log2 a) and the mantissa as
// round((a / 2^E - 1) * 16); for a normal a both are exact functions of a's
// bits, which is what is evaluated here.  Both directions are integer and
// power-of-two arithmetic, so encode and decode are exact.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kbit {

__device__ __forceinline__ uint32_t e4m4_encode(float a) {
    const uint32_t u = __float_as_uint(a);
    // normal E4M4 range [2^-10, +inf]: fp32 exponent field ex >= 117.  The
    // 23 fraction bits are rounded to 4, half to even; fractions that would
    // round up to 16 are first lowered to the largest one that rounds to 15,
    // which is the clamp.  +inf has fraction 0 and lands on 0xF0.
    const uint32_t ex = u >> 23;
    const uint32_t f = min(u & 0x7FFFFFu, 0x7BFFFFu);
    const uint32_t q = (f + 0x3FFFFu + ((f >> 19) & 1u)) >> 19;
    const uint32_t normal = ((min(ex, 131u) - 116u) << 4) + q;
    // subnormal E4M4 range [+0, 2^-10): a * 2^14 is exact and below 16, so
    // adding 2^23 in one rounding (fma) leaves RNE(a * 2^14) in the low bits
    const uint32_t sub = min(__float_as_uint(__builtin_fmaf(a, 0x1p14f, 0x1p23f)) & 0x1Fu, 15u);
    // anything else (negative, NaN) encodes as 0
    const uint32_t code = u <= 0x7F800000u ? normal : 0u;
    return u < 0x3A800000u ? sub : code;
}

__device__ __forceinline__ float e4m4_decode(uint32_t code) {
    const uint32_t e = code >> 4, m = code & 15u;
    const float sub = static_cast<float>(m) * 0x1p-14f;
    const float normal = __uint_as_float(((e + 116u) << 23) | (m << 19));
    return e != 0 ? normal : sub;
}

}  // namespace kbit
