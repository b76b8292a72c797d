// Exhaustive host check of the quantize kernel's fp32 threshold decisions
// for 16-bit inputs (threshold.h).  With u the switching point between two
// neighbouring codes, p its fp32 predecessor and M = (u + p) / 2:
//   * pair form (fp16 inputs): Mh = p, Ml = (u - p) / 2, Ml' = Ml nudged by
//     one ulp; the sign of fma(-Ml', s, fma(-Mh, s, x)) must equal
//     [RN(x / s) >= u] for every fp16 (and bf16) x in [-s, s] and every
//     fp16 (bf16) significand of s;
//   * T form (bf16 inputs): one value T in {p, u}, "upper" when
//     fma(-T, s, x) is not negative.  Here T is derived by brute force: the
//     quotients of two 8-bit significands times a power of two that fall in
//     [p, u] (at most one value) are found exactly, and T = p when that
//     value lies above M, or on M with the tie rounding to u; T = u
//     otherwise.  Every bf16 x in [-s, s] against every bf16 significand of
//     s must then decide as [RN(x / s) >= u].
// Scaling x and s by a power of two changes nothing, so s runs over [1, 2)
// plus a few binades near the ends of the range.  Exit status 0 when no case
// differs.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>
#include <thread>
#include <atomic>
#include <random>
#include <algorithm>
#include "kbit.h"
static uint32_t fb(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bf(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t key(float v) { uint32_t b = fb(v); return (b & 0x80000000u) ? ~b : (b | 0x80000000u); }
static float from_key(uint32_t k) { return bf((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k); }
static bool upper_wins(float xn, float lo, float hi) { return std::fabs(xn - hi) < std::fabs(xn - lo); }
static float half_to_float(uint16_t h) {
    uint32_t s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
    float v;
    if (e == 0) v = std::ldexp((float)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = std::ldexp((float)(m | 1024), (int)e - 25);
    return s ? -v : v;
}
struct Thr { float u, p, Mh, Ml2; bool ok; };
static Thr make_thr(float lo, float hi) {
    uint32_t L = key(lo), R = key(hi);  // L chooses lower, R chooses upper
    while (R - L > 1) { uint32_t m = L + (R - L) / 2; if (upper_wins(from_key(m), lo, hi)) R = m; else L = m; }
    Thr t; t.u = from_key(R); t.p = from_key(L);
    const double M = ((double)t.u + (double)t.p) * 0.5;
    const bool tie_up = (float)M == t.u;
    t.Mh = t.p;
    const float Ml = (float)((double)t.u - (double)t.p) * 0.5f;
    t.ok = ((double)t.Mh + (double)Ml == M) && Ml >= 0x1p-100f;
    const uint32_t b = fb(Ml);
    t.Ml2 = bf(tie_up ? b - 1 : b + 1);  // M nudged down (ties up) or up (ties down)
    return t;
}
// T of the T form for bf16 inputs (see the header), or NAN if two distinct
// quotients fell into [p, u] (the form would not apply).
static float make_T(float u, float p) {
    const double M = ((double)u + (double)p) * 0.5;
    const bool tie_up = (float)M == u;
    const double ref = std::fabs(p) > 0.0 ? std::fabs((double)p) : std::fabs((double)u);
    bool found = false, above = false, conflict = false;
    double n_seen = 0.0;
    int ms_seen = 1;
    for (int sign = -1; sign <= 1; sign += 2) {
        for (int ms = 128; ms <= 255; ++ms) {
            for (int mx = 1; mx <= 255; ++mx) {
                int e;
                std::frexp(ref * (double)ms / (double)mx, &e);  // (mx / ms) 2^e lands next to |p|
                for (int de = -2; de <= 2; ++de) {
                    const double num = sign * std::ldexp((double)mx, e + de);  // exact
                    // q = num / ms in [p, u]  <=>  p * ms <= num <= u * ms (exact products)
                    if (!((double)p * ms <= num && num <= (double)u * ms)) continue;
                    if (found && num * ms_seen != n_seen * ms) conflict = true;  // a second value
                    found = true;
                    n_seen = num;
                    ms_seen = ms;
                    const double mms = M * ms;  // exact: M has 25 significant bits, ms 8
                    above = num > mms || (num == mms && tie_up);
                }
            }
        }
    }
    if (conflict) return NAN;
#ifdef PLANT_T_FLIP
    if (found) above = !above;  // the other choice: must be caught
#endif
    return found && above ? p : u;
}
static long long check_T(float T, float u, const std::vector<float>& svals) {
    long long bad = 0;
    for (float s : svals) {
        for (uint32_t h = 0; h < 65536; ++h) {
            const float x = bf(h << 16);
            if (!(std::fabs(x) <= s)) continue;
            const bool dec = !std::signbit(std::fmaf(-T, s, x));
            const bool ref = key(x / s) >= key(u);
            if (dec != ref) {
                if (bad < 5) std::printf("  T mismatch x=%a s=%a u=%a T=%a dec=%d ref=%d\n", x, s, u, T, dec, ref);
                ++bad;
            }
        }
    }
    return bad;
}
static long long check(const Thr& t, bool half, const std::vector<float>& svals) {
    long long bad = 0, n = 0;
    for (float s : svals) {
        auto test = [&](float x) {
            if (!(std::fabs(x) <= s)) return;
            ++n;
            const float t1 = std::fmaf(-t.Mh, s, x);
#ifdef PLANT_ONE_ULP_SHIFT
            const bool dec = std::fmaf(-3.0f * t.Ml2, s, t1) > 0.0f;  // the threshold moved by one ulp
#else
            const bool dec = std::fmaf(-t.Ml2, s, t1) > 0.0f;
#endif
            const float xn = x / s;
            const bool ref = key(xn) >= key(t.u);
            if (dec != ref) { if (bad < 5) std::printf("  mismatch x=%a s=%a u=%a dec=%d ref=%d\n", x, s, t.u, dec, ref); ++bad; }
        };
        if (!half) { for (uint32_t h = 0; h < 65536; ++h) test(bf(h << 16)); }
        else { for (uint32_t h = 0; h < 65536; ++h) test(half_to_float((uint16_t)h)); }
    }
    return bad;
}
int main(int argc, char** argv) {
    const bool quick = argc > 1 && std::strcmp(argv[1], "quick") == 0;  // the random codebooks only
    std::vector<std::vector<float>> books;
    for (int K = 2; K <= 5; ++K) { std::vector<float> c(1 << K); kbit_codebook_nf(K, c.data()); books.push_back(c); }
    { std::vector<float> c(16); kbit_codebook_fp4(c.data()); books.push_back(c); }
    { std::vector<float> c(16); kbit_codebook_lloyd_max_normal(16, c.data()); for (auto& v : c) v /= 2.7326f; books.push_back(c); }
    const size_t fixed = books.size();
    std::mt19937 rng(1);
    for (int r = 0; r < 6; ++r) {
        std::vector<float> c(r < 4 ? 16 : 32);
        std::uniform_real_distribution<float> U(-1.f, 1.f);
        for (auto& v : c) v = U(rng);
        std::sort(c.begin(), c.end());
        books.push_back(c);
    }
    // s: every bf16 / fp16 significand in [1, 2) and a few other binades
    std::vector<float> sb, sh;
    for (int m = 0; m < 128; ++m) sb.push_back(1.0f + m / 128.0f);
    for (int m = 0; m < 128; m += 7) { sb.push_back(std::ldexp(1.0f + m / 128.0f, -26)); sb.push_back(std::ldexp(1.0f + m / 128.0f, 100)); }
    for (int m = 0; m < 1024; ++m) sh.push_back(1.0f + m / 1024.0f);
    for (int m = 0; m < 1024; m += 37) { sh.push_back(std::ldexp(1.0f + m / 1024.0f, -14)); sh.push_back(std::ldexp(1.0f + m / 1024.0f, 15)); }
    if (quick) books.erase(books.begin(), books.begin() + fixed);  // drop NF2..5, FP4, Lloyd-Max
    std::vector<Thr> thr;
    int notok = 0;
    for (auto& c : books) {
        for (size_t i = 1; i < c.size(); ++i) {
            if (c[i] == c[i - 1]) continue;
            const Thr t = make_thr(c[i - 1], c[i]);
            if (!t.ok) { ++notok; continue; }
            thr.push_back(t);
        }
    }
    std::atomic<long long> bad{0};
    std::atomic<size_t> next{0};
    std::vector<std::thread> pool;
    const unsigned nt = std::max(1u, std::min(8u, std::thread::hardware_concurrency()));
    for (unsigned w = 0; w < nt; ++w)
        pool.emplace_back([&] {
            for (size_t i = next++; i < thr.size(); i = next++) {
                bad += check(thr[i], false, sb) + check(thr[i], true, sh);
                const float T = make_T(thr[i].u, thr[i].p);
                if (T != T) {
                    std::printf("  T form not applicable at u=%a\n", thr[i].u);
                    ++bad;
                } else {
                    bad += check_T(T, thr[i].u, sb);
                }
            }
        });
    for (auto& th : pool) th.join();
    const int nthr = static_cast<int>(thr.size());
    printf("thresholds checked %d (not representable: %d), mismatches %lld\n", nthr, notok, bad.load());
    return bad.load() != 0 || nthr == 0;
}
