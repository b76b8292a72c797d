// Host check of the encoder's division by the block count (exact_mean.h,
// NbDivider / div_nb): floor(n / nb) by a multiply-high, against the
// integer division, for every nb up to 4096, the powers of two and their
// neighbours up to 2^36, and random nb, each with edge and random n < 2^63.
// PLANT_FLOOR_MAGIC rounds the multiplier down instead of up (a plausible
// slip) and must be caught.
#define KBIT_HD
#include "exact_mean.h"

#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

using kbit::NbDivider;

static NbDivider divider(uint64_t nb) {
#ifdef PLANT_FLOOR_MAGIC
    NbDivider d = kbit::make_nb_divider(nb);
    int l = d.l;
    d.m = static_cast<uint64_t>((static_cast<unsigned __int128>(1) << (63 + l)) / nb);
    return d;
#else
    return kbit::make_nb_divider(nb);
#endif
}

int main() {
    std::mt19937_64 rng(12345);
    std::vector<uint64_t> nbs;
    for (uint64_t nb = 1; nb <= 4096; ++nb) nbs.push_back(nb);
    for (int p = 12; p <= 36; ++p) {
        const uint64_t q = 1ull << p;
        nbs.push_back(q - 1);
        nbs.push_back(q);
        if (p < 36) nbs.push_back(q + 1);
    }
    for (int i = 0; i < 20000; ++i) nbs.push_back(1 + rng() % (1ull << 36));
    const uint64_t top = (1ull << 63) - 1;
    long long checks = 0, bad = 0;
    for (uint64_t nb : nbs) {
        const NbDivider d = divider(nb);
        // the multiplier must fit 64 bits: ceil(2^(63+l)/nb) < 2^64
        const unsigned __int128 m_exact =
            ((static_cast<unsigned __int128>(1) << (63 + d.l)) + nb - 1) / nb;
        if (m_exact >> 64) {
            std::printf("multiplier overflow nb=%llu\n", (unsigned long long)nb);
            return 1;
        }
        std::vector<uint64_t> ns = {0, 1, nb - 1, nb, nb + 1, 2 * nb - 1, 2 * nb, 1ull << 62, top, top - 1};
        const uint64_t kmax = top / nb;
        for (uint64_t k : {kmax, kmax - 1, kmax / 2, kmax / 3 + 1}) {
            const unsigned __int128 base = static_cast<unsigned __int128>(k) * nb;
            for (int dlt = -1; dlt <= 1; ++dlt) {
                const unsigned __int128 n = base + dlt;
                if (n <= top) ns.push_back(static_cast<uint64_t>(n));
            }
        }
        for (int i = 0; i < 24; ++i) ns.push_back(rng() >> 1);
        for (int i = 0; i < 8; ++i) ns.push_back((rng() >> 1) / nb * nb);  // exact multiples
        for (uint64_t n : ns) {
            if (n > top) continue;
            ++checks;
            const uint64_t want = n / nb, got = kbit::div_nb(d, n);
            if (got != want) {
                if (bad < 5)
                    std::printf("mismatch nb=%llu n=%llu want %llu got %llu\n", (unsigned long long)nb,
                                (unsigned long long)n, (unsigned long long)want, (unsigned long long)got);
                ++bad;
            }
        }
    }
    std::printf("checks %lld mismatches %lld\n", checks, bad);
    return bad == 0 ? 0 : 1;
}
