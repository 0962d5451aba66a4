// Division of 32-bit unsigned integers by a run-time invariant divisor with a
// precomputed multiplier (Granlund and Montgomery, "Division by invariant
// integers using multiplication", PLDI 1994, section 4, the round-up variant
// with a 32-bit multiplier and one fix-up shift).  For d >= 1:
//     l  = ceil(log2 d)
//     m  = floor(2^32 * (2^l - d) / d) + 1          (fits in 32 bits)
//     t  = floor(m * n / 2^32)
//     n / d = (t + ((n - t) >> min(l, 1))) >> max(l - 1, 0)
// exact for every 32-bit n.  The kernels use it for their per-wavefront token
// decode: a multiply-high, a subtract, two shifts and an add, instead of the
// generic division sequence.  Plain C++ (constexpr functions compile for the
// host and, under hipcc, for the device).
#pragma once

#include <cstdint>

namespace ltx3drope {

struct FastDiv {
    uint32_t d;   // the divisor
    uint32_t m;   // multiplier
    uint32_t s1;  // min(l, 1)
    uint32_t s2;  // max(l - 1, 0)
};

constexpr FastDiv make_fastdiv(uint32_t d) {
    uint32_t l = 0;
    while (l < 32 && (uint64_t(1) << l) < d) ++l;
    const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
    return FastDiv{d, static_cast<uint32_t>(m), l > 0 ? 1u : 0u, l > 0 ? l - 1 : 0u};
}

constexpr uint32_t fast_div(uint32_t n, const FastDiv& f) {
    const uint32_t t = static_cast<uint32_t>((uint64_t(f.m) * n) >> 32);
    return (t + ((n - t) >> f.s1)) >> f.s2;
}

constexpr uint32_t fast_mod(uint32_t n, const FastDiv& f) { return n - fast_div(n, f) * f.d; }

}  // namespace ltx3drope
