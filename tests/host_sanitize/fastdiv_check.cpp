// Checks the invariant-divisor division of fastdiv.h against the hardware division:
// every divisor up to 2^16 and 200000 random ones, each on edge values, values around the
// largest multiples and random values; and every 32-bit dividend for a few divisors of the
// token decode's kind.  Exit status 0 when nothing differs.
#include <cstdio>
#include <random>

#include "fastdiv.h"

using ltx3drope::FastDiv;
using ltx3drope::fast_div;
using ltx3drope::fast_mod;
using ltx3drope::make_fastdiv;

int main() {
    std::mt19937_64 rng(7);
    unsigned long long bad = 0, checks = 0;
    auto check = [&](uint32_t n, const FastDiv& f) {
        ++checks;
        if (fast_div(n, f) != n / f.d || fast_mod(n, f) != n % f.d) ++bad;
    };
    auto sample = [&](uint32_t d) {
        const FastDiv f = make_fastdiv(d);
        const uint32_t edge[] = {0u, 1u, d - 1, d, d + 1, 2 * d - 1, 2 * d, 0x7fffffffu, 0x80000000u,
                                 0xfffffffeu, 0xffffffffu};
        for (uint32_t n : edge) check(n, f);
        for (int i = 0; i < 200; ++i) check(static_cast<uint32_t>(rng()), f);
        const uint64_t q = 0xffffffffull / d;
        for (uint64_t k = q > 3 ? q - 3 : 0; k <= q; ++k)
            for (int e = -1; e <= 1; ++e) {
                const int64_t x = static_cast<int64_t>(k * d) + e;
                if (x >= 0 && x <= 0xffffffffll) check(static_cast<uint32_t>(x), f);
            }
    };
    for (uint32_t d = 1; d <= (1u << 16); ++d) sample(d);
    for (int i = 0; i < 200000; ++i) {
        const uint32_t d = static_cast<uint32_t>(rng());
        if (d != 0) sample(d);
    }
    for (uint32_t d : {0x80000000u, 0x80000001u, 0xffffffffu}) sample(d);
    // every dividend for divisors of the kind the token decode uses (vectors per head and per
    // token row, grid rows and planes)
    for (uint32_t d : {12u, 138720u}) {
        const FastDiv f = make_fastdiv(d);
        uint32_t n = 0;
        do {
            check(n, f);
        } while (++n != 0);
    }
    std::printf("fastdiv: %llu checks, %llu differ\n", checks, bad);
    return bad != 0;
}
