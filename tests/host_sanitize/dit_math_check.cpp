// Host build of the DiT frequency grid's device arithmetic (dit_math.h), for comparison with the
// oracle on the CPU.  Built with the __host__ / __device__ qualifiers defined empty and with
// contraction off, so it runs the same IEEE operations as the kernel.
//
//   dit_math_check grid THETA DIM NE DOUBLE   -> one float32 bit pattern (hex) per grid value
//   dit_math_check pow                        -> reads "BASE X DOUBLE" lines (hex bit patterns of
//                                                doubles), prints the correctly rounded power's
//                                                bits (float64 or float32) per line
//   dit_math_check ln2                        -> the two halves of ln 2 as hex bit patterns
#include <cinttypes>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "dit_math.h"

using namespace ltx3drope::dit;

int main(int argc, char** argv) {
    if (argc >= 6 && !std::strcmp(argv[1], "grid")) {
        const double theta = std::strtod(argv[2], nullptr);
        const long long dim = std::atoll(argv[3]), ne = std::atoll(argv[4]);
        const int dbl = std::atoi(argv[5]);
        const uint32_t n = static_cast<uint32_t>(dim / ne);
        for (uint32_t i = 0; i < n; ++i) {
            const float v = dbl ? grid_f64(theta, i, n) : grid_f32(static_cast<float>(theta), i, n);
            std::printf("%08" PRIx32 "\n", to_bits(v));
        }
        return 0;
    }
    if (argc >= 2 && !std::strcmp(argv[1], "pow")) {
        unsigned long long bb, xb;
        int dbl;
        while (std::scanf("%llx %llx %d", &bb, &xb, &dbl) == 3) {
            const double base = f64_bits_to(bb), x = f64_bits_to(xb);
            const dd p = pow_dd(base, x);
            if (dbl)
                std::printf("%016" PRIx64 "\n", to_bits(p.hi));
            else
                std::printf("%08" PRIx32 "\n", to_bits(round_f32(p)));
        }
        return 0;
    }
    if (argc >= 2 && !std::strcmp(argv[1], "ln2")) {
        std::printf("%016" PRIx64 " %016" PRIx64 "\n", to_bits(kLn2Hi), to_bits(kLn2Lo));
        return 0;
    }
    std::fprintf(stderr, "usage: %s grid THETA DIM NE DOUBLE | pow | ln2\n", argv[0]);
    return 2;
}
