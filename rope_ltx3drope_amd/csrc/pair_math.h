// Per-pair arithmetic shared by the 3D RoPE kernels (device code only).
//
// sglang PR #35698 page, "Key source snippets" (the CUDA kernel's pair-rotation
// helper) and "Implementation breakdown", step 2: an (even, odd) pair widened to
// fp32 is turned by the angle whose cosine and sine are (c, s) with four
// separately rounded products, one rounded difference and one rounded sum, no
// fused multiply-add; the result is cast back with round-to-nearest-even.  A
// NaN result is written as the canonical quiet NaN (0x7FC00000 fp32, 0x7FC0
// bf16).  Files including this header are compiled with -ffp-contract=off.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ltx3drope {

typedef float pm_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 pm_bf16x2 __attribute__((ext_vector_type(2)));

// The pair (e, o) turned by the angle whose cosine and sine are (c, s): four
// products, each rounded to fp32, then one rounded difference (even result)
// and one rounded sum (odd result); nothing is fused.
__device__ __forceinline__ void rotate(float e, float o, float c, float s, float& ye, float& yo) {
    const float m0 = __fmul_rn(e, c), m1 = __fmul_rn(o, s);
    const float m2 = __fmul_rn(e, s), m3 = __fmul_rn(o, c);
    ye = __fsub_rn(m0, m1);
    yo = __fadd_rn(m2, m3);
}

// bf16 <-> fp32.  A 32-bit word holds one pair: the even element in the low half.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Integer round-to-nearest-even (plain path): add 0x7fff plus the lowest kept bit, keep the top half.
__device__ __forceinline__ uint32_t bf16_rne_int(float y) {
    const uint32_t u = __float_as_uint(y);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;  // NaN
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// fp32 bits with any NaN replaced by the canonical quiet NaN.
__device__ __forceinline__ uint32_t f32_canon(float y) { return y != y ? 0x7fc00000u : __float_as_uint(y); }

// Hardware conversion of two floats to a packed bf16 pair (round to nearest
// even), then any NaN half replaced by the canonical quiet NaN 0x7FC0.
__device__ __forceinline__ uint32_t bf16_pack_hw(float lo, float hi) {
    const pm_f32x2 v = {lo, hi};
    const pm_bf16x2 r = __builtin_convertvector(v, pm_bf16x2);
    uint32_t w = __builtin_bit_cast(uint32_t, r);
    if (lo != lo) w = (w & 0xffff0000u) | 0x7fc0u;
    if (hi != hi) w = (w & 0x0000ffffu) | 0x7fc00000u;
    return w;
}

}  // namespace ltx3drope
