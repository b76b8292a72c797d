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
    const int ex = static_cast<int>((u >> 23) & 0xFFu);  // biased fp32 exponent
    // normal E4M4 range: round the fraction to 4 bits, half to even
    const uint32_t frac = u & 0x7FFFFFu;
    uint32_t q = frac >> 19;
    const uint32_t r = frac & 0x7FFFFu;
    q += (r > 0x40000u || (r == 0x40000u && (q & 1u))) ? 1u : 0u;
    q = min(q, 15u);
    const uint32_t eb = static_cast<uint32_t>(min(ex - 127 + 11, 15));
    const uint32_t normal = (eb << 4) | q;
    // subnormal E4M4 range (a < 2^-10, including fp32 subnormals)
    const uint32_t sub = static_cast<uint32_t>(__builtin_rintf(__builtin_amdgcn_fmed3f(a * 0x1p14f, 0.0f, 15.0f)));
    uint32_t code = ex - 127 + 11 <= 0 ? sub : normal;
    if (ex == 0xFF) code = 0xF0u;  // +inf (NaN is caught below)
    return a > 0.0f ? code : 0u;
}

__device__ __forceinline__ float e4m4_decode(uint32_t code) {
    const uint32_t e = code >> 4, m = code & 15u;
    const float sub = static_cast<float>(m) * 0x1p-14f;
    const float normal = __uint_as_float(((e + 116u) << 23) | (m << 19));
    return e != 0 ? normal : sub;
}

}  // namespace kbit
