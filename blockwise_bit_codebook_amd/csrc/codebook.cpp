// Codebook generators (host only, no device access).
//
// All values are computed in x87 extended precision (long double) and
// rounded once to float32.
//
// * NF_K ([QLORA-2] PATCH 001 tests/test_kbit_quantization.py and PATCH 003
//   bitsandbytes/functional.py create_normal_float_codebook): levels at the
//   N(0,1) quantiles of the bin midpoints (2i+1)/(2n).  The hot path's NF
//   codebook needs an exact zero: the negative levels come from that rule at
//   n = 2^K - 1 (odd, centred on 0), the positive levels from n = 2^K, each
//   side divided by its own outermost magnitude, plus 0.
// * The inverse normal CDF: a starting value from the rational approximation
//   26.2.23 of Abramowitz & Stegun (Handbook of Mathematical Functions),
//   refined by Newton steps on Phi(x) = erfc(-x/sqrt 2)/2 with the C
//   library's long-double erfcl until the step vanishes.
// * FP4 ([PR2051] Summary names NF4/FP4): E2M1 magnitudes with both signs,
//   divided by 6 in float32.
// * Lloyd-Max N(0,1) levels ([ORBIT] methodology audit, converged Lloyd-Max
//   codebook): the fixed-point iteration of centroid and midpoint conditions
//   with closed-form Gaussian cell moments.
// * Dynamic tree 8-bit map for nested absmax codes ([PR2051] Summary names
//   the 8-bit General8 scale code): sign, decimal exponent 10^-z, linear
//   fraction in (0.1, 1) at the midpoints of 2^(6-z) slots, plus 0 and 1.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

#include "kbit.h"

namespace {

using ld = long double;

constexpr ld kSqrt2 = 1.41421356237309504880168872420969808L;
constexpr ld kInvSqrt2Pi = 0.398942280401432677939946059934381868L;

ld phi(ld x) { return kInvSqrt2Pi * expl(-0.5L * x * x); }
ld Phi(ld x) { return 0.5L * erfcl(-x / kSqrt2); }
// Upper tail 1 - Phi(x), accurate for large x.
ld Phic(ld x) { return 0.5L * erfcl(x / kSqrt2); }

// Quantile of N(0,1) for p in (0, 1/2]; negative or zero.
ld lower_quantile(ld p) {
    if (p == 0.5L) return 0.0L;
    // Abramowitz & Stegun 26.2.23 start (|error| < 4.5e-4)
    const ld t = sqrtl(-2.0L * logl(p));
    ld x = -(t - (2.515517L + 0.802853L * t + 0.010328L * t * t) /
                     (1.0L + 1.432788L * t + 0.189269L * t * t + 0.001308L * t * t * t));
    for (int it = 0; it < 50; ++it) {
        const ld step = (Phi(x) - p) / phi(x);
        x -= step;
        if (fabsl(step) <= 1e-19L * (1.0L + fabsl(x))) break;
    }
    return x;
}

// N(0,1) quantile at the midpoint (2i+1)/(2n) of bin i of n equiprobable bins.
ld midpoint_quantile(int i, int n) {
    const long num = 2L * i + 1, den = 2L * n;
    if (2 * num <= den) return lower_quantile(static_cast<ld>(num) / static_cast<ld>(den));
    return -lower_quantile(static_cast<ld>(den - num) / static_cast<ld>(den));
}

}  // namespace

extern "C" {

int kbit_codebook_nf(int K, float* out_host) {
    if (K < 2 || K > 5 || out_host == nullptr) return KBIT_EINVAL;
    const int n_odd = (1 << K) - 1, n_even = 1 << K;
    const int n_neg = (n_odd - 1) / 2;
    const ld neg_extreme = -midpoint_quantile(0, n_odd);
    int w = 0;
    for (int i = 0; i < n_neg; ++i) out_host[w++] = static_cast<float>(midpoint_quantile(i, n_odd) / neg_extreme);
    out_host[w++] = 0.0f;
    const ld pos_extreme = midpoint_quantile(n_even - 1, n_even);
    for (int i = n_even / 2; i < n_even; ++i)
        out_host[w++] = static_cast<float>(midpoint_quantile(i, n_even) / pos_extreme);
    return KBIT_OK;
}

int kbit_codebook_fp4(float* out_host) {
    if (out_host == nullptr) return KBIT_EINVAL;
    static const float mags[8] = {6.0f, 4.0f, 3.0f, 2.0f, 1.5f, 1.0f, 0.5f, 0.0f};
    for (int i = 0; i < 8; ++i) out_host[i] = -mags[i] / 6.0f;
    for (int i = 0; i < 8; ++i) out_host[8 + i] = mags[7 - i] / 6.0f;
    return KBIT_OK;
}

int kbit_codebook_lloyd_max_normal(int levels, float* out_host) {
    if (levels < 2 || levels > 256 || (levels & 1) || out_host == nullptr) return KBIT_EINVAL;
    const int L = levels;
    std::vector<ld> c(L), nc(L), edge(L + 1);
    for (int i = 0; i < L; ++i) c[i] = midpoint_quantile(i, L);
    for (int it = 0; it < 400000; ++it) {
        for (int i = 1; i < L; ++i) edge[i] = 0.5L * (c[i - 1] + c[i]);
        for (int i = 0; i < L; ++i) {
            const bool first = (i == 0), last = (i == L - 1);
            const ld lo = edge[i], hi = edge[i + 1];
            ld p;
            if (!first && lo >= 0.0L)
                p = Phic(lo) - (last ? 0.0L : Phic(hi));
            else
                p = (last ? 1.0L : Phi(hi)) - (first ? 0.0L : Phi(lo));
            const ld m = (first ? 0.0L : phi(lo)) - (last ? 0.0L : phi(hi));
            nc[i] = m / p;
        }
        ld delta = 0.0L;
        for (int i = 0; i < L; ++i) {
            const ld v = 0.5L * (nc[i] - nc[L - 1 - i]);
            delta = std::max(delta, fabsl(v - c[i]));
            c[i] = v;
        }
        if (delta < 1e-18L) break;
    }
    for (int i = 0; i < L; ++i) out_host[i] = static_cast<float>(c[i]);
    return KBIT_OK;
}

int kbit_dynamic_map8(float* out_host) {
    if (out_host == nullptr) return KBIT_EINVAL;
    std::vector<float> v;
    v.reserve(256);
    long pow10 = 1;
    for (int z = 0; z < 7; ++z, pow10 *= 10) {
        const long slots = 1L << (6 - z);
        for (long f = 0; f < slots; ++f) {
            // 10^-z * (0.1 + 0.9 (2f+1) / (2 slots)) as one exact rational
            const long num = 2 * slots + 9 * (2 * f + 1);
            const long den = 20 * slots * pow10;
            const float val = static_cast<float>(static_cast<double>(num) / static_cast<double>(den));
            v.push_back(val);
            v.push_back(-val);
        }
    }
    v.push_back(0.0f);
    v.push_back(1.0f);
    std::sort(v.begin(), v.end());
    for (int i = 0; i < 256; ++i) out_host[i] = v[i];
    return KBIT_OK;
}

}  // extern "C"
