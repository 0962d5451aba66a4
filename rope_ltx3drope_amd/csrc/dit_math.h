// Arithmetic of the LTX DiT RoPE frequency grid, one value per call.
//
// sglang PR #24660 page, "Key source snippets" (the LTX DiT frequency
// generation) and "Implementation breakdown", step 2: the grid
//     theta ** linspace(0, 1, n)  * pi / 2,  cast to float32
// is generated in the requested precision (float64 or float32) along the
// official rounding trajectory.  Steps, each rounded to nearest even in the
// working precision:
//   * linspace as torch.linspace computes it: a rounded step s = 1 / (n - 1);
//     value i is s*i for i < n/2 and 1 - s*(n-1-i) with one rounding (a fused
//     multiply-add) for the rest;
//   * the power, correctly rounded: ln(theta) and exp(x ln theta) are
//     evaluated in double-double arithmetic (about 100 bits) and rounded once,
//     so the result differs from the correctly rounded power only when the
//     exact value lies within about 2^-95 (relative) of a rounding boundary;
//   * the product with pi rounded to the working precision, an exact halving,
//     and (float64 recipe) one rounding to float32.
//
// Only IEEE additions, multiplications, divisions and explicit fused
// multiply-adds are used, with contraction off, so the host and the device
// produce the same bits.  Functions are __host__ __device__; the library
// builds them for gfx950, a host program may build them with the two
// qualifiers defined empty.
#pragma once

#include <stdint.h>

namespace ltx3drope {
namespace dit {

struct dd {
    double hi, lo;
};

__host__ __device__ inline double f64_bits_to(uint64_t u) { return __builtin_bit_cast(double, u); }
__host__ __device__ inline uint64_t to_bits(double d) { return __builtin_bit_cast(uint64_t, d); }
__host__ __device__ inline float f32_from_bits(uint32_t u) { return __builtin_bit_cast(float, u); }
__host__ __device__ inline uint32_t to_bits(float f) { return __builtin_bit_cast(uint32_t, f); }

// exact sum and product of two doubles as an unevaluated pair
__host__ __device__ inline dd two_sum(double a, double b) {
    const double s = a + b;
    const double bv = s - a;
    const double av = s - bv;
    return {s, (a - av) + (b - bv)};
}
__host__ __device__ inline dd quick_two_sum(double a, double b) {  // |a| >= |b| or a == 0
    const double s = a + b;
    return {s, b - (s - a)};
}
__host__ __device__ inline dd two_prod(double a, double b) {
    const double p = a * b;
    return {p, __builtin_fma(a, b, -p)};
}

__host__ __device__ inline dd add(dd x, dd y) {
    dd s = two_sum(x.hi, y.hi);
    const dd t = two_sum(x.lo, y.lo);
    s.lo += t.hi;
    s = quick_two_sum(s.hi, s.lo);
    s.lo += t.lo;
    return quick_two_sum(s.hi, s.lo);
}
__host__ __device__ inline dd add(dd x, double y) { return add(x, dd{y, 0.0}); }
__host__ __device__ inline dd neg(dd x) { return {-x.hi, -x.lo}; }
__host__ __device__ inline dd mul(dd x, dd y) {
    dd p = two_prod(x.hi, y.hi);
    p.lo += x.hi * y.lo + x.lo * y.hi;
    return quick_two_sum(p.hi, p.lo);
}
__host__ __device__ inline dd mul(dd x, double y) {
    dd p = two_prod(x.hi, y);
    p.lo += x.lo * y;
    return quick_two_sum(p.hi, p.lo);
}
// x / y: a first quotient, then two corrections from the exact remainder
__host__ __device__ inline dd div(dd x, dd y) {
    const double q1 = x.hi / y.hi;
    dd r = add(x, neg(mul(y, q1)));
    const double q2 = r.hi / y.hi;
    r = add(r, neg(mul(y, q2)));
    const double q3 = r.hi / y.hi;
    return add(quick_two_sum(q1, q2), q3);
}
__host__ __device__ inline dd div(dd x, double y) { return div(x, dd{y, 0.0}); }
__host__ __device__ inline dd scale2(dd x, int k) { return {__builtin_ldexp(x.hi, k), __builtin_ldexp(x.lo, k)}; }

// ln 2 = 0.693147180559945309417232121458176568..., split into a double and the double nearest the rest
constexpr double kLn2Hi = 0x1.62e42fefa39efp-1;
constexpr double kLn2Lo = 0x1.abc9e3b39803fp-56;

// ln(a) for a positive normal double: a = m * 2^e with m in [sqrt(1/2), sqrt(2)),
// ln m = 2 atanh(u) with u = (m - 1) / (m + 1), |u| < 0.172, summed to 24 odd powers.
__host__ __device__ inline dd log_dd(double a) {
    const uint64_t bits = to_bits(a);
    int e = static_cast<int>((bits >> 52) & 0x7ff) - 1023;
    double m = f64_bits_to((bits & 0x000fffffffffffffull) | 0x3ff0000000000000ull);  // [1, 2)
    if (m >= 1.4142135623730951) {
        m *= 0.5;  // exact
        e += 1;
    }
    const dd num = two_sum(m, -1.0);
    const dd den = two_sum(m, 1.0);
    const dd u = div(num, den);
    const dd u2 = mul(u, u);
    dd s = div(dd{1.0, 0.0}, 49.0);
    // Unrolled, the reciprocals 1/(2k+1) are constant expressions that the compiler evaluates
    // with the same IEEE operations, so the series' chain holds only multiplications and additions.
#pragma unroll
    for (int k = 23; k >= 0; --k) s = add(mul(s, u2), div(dd{1.0, 0.0}, static_cast<double>(2 * k + 1)));
    const dd lnm = scale2(mul(s, u), 1);
    const dd eln2 = add(two_prod(static_cast<double>(e), kLn2Hi), static_cast<double>(e) * kLn2Lo);
    return add(eln2, lnm);
}

// exp(z) for |z| below about 709: z = k ln 2 + r, |r| <= ln2/2; expm1(r / 2^10) by Taylor
// series (terms to the 11th power: below 2^-120), squared back ten times as e(2 + e).  Each
// Horner step multiplies by the double-double reciprocal of j (a constant once unrolled) instead
// of dividing by j: one rounding of about 2^-105 more per step, and no division on the chain.
__host__ __device__ inline dd exp_dd(dd z) {
    const double k = __builtin_rint(z.hi / kLn2Hi);
    const dd kln2 = add(two_prod(k, kLn2Hi), k * kLn2Lo);
    const dd r = add(z, neg(kln2));
    const dd s = scale2(r, -10);
    dd t = {1.0, 0.0};
#pragma unroll
    for (int j = 11; j >= 2; --j) t = add(mul(mul(s, t), div(dd{1.0, 0.0}, static_cast<double>(j))), 1.0);
    dd e = mul(s, t);  // expm1(s)
    for (int i = 0; i < 10; ++i) e = mul(e, add(e, 2.0));
    return scale2(add(e, 1.0), static_cast<int>(k));
}

// base ** x as a normalized double-double (base a positive normal double, x finite)
__host__ __device__ inline dd pow_dd(double base, double x) {
    if (x == 0.0) return {1.0, 0.0};
    return exp_dd(mul(log_dd(base), x));
}

// a normalized double-double rounded to the nearest float32 (ties to even), for a positive
// normal result: hi is already the double nearest to hi + lo, so only a hi lying exactly
// halfway between two float32 values needs lo to break the tie
__host__ __device__ inline float round_f32(dd v) {
    float r = static_cast<float>(v.hi);
    const uint64_t below = to_bits(v.hi) & ((uint64_t(1) << 29) - 1);  // bits under float32 precision
    if (below == (uint64_t(1) << 28) && v.lo != 0.0) {
        const double rd = static_cast<double>(r);
        if (v.lo > 0.0 && rd < v.hi) r = f32_from_bits(to_bits(r) + 1u);
        if (v.lo < 0.0 && rd > v.hi) r = f32_from_bits(to_bits(r) - 1u);
    }
    return r;
}

// value i of torch.linspace(0, 1, n) (n >= 1)
__host__ __device__ inline double linspace01_f64(uint32_t i, uint32_t n) {
    if (n == 1) return 0.0;
    const double step = 1.0 / static_cast<double>(n - 1);
    if (i < n / 2) return step * static_cast<double>(i);
    return __builtin_fma(-step, static_cast<double>(n - 1 - i), 1.0);
}
__host__ __device__ inline float linspace01_f32(uint32_t i, uint32_t n) {
    if (n == 1) return 0.0f;
    const float step = 1.0f / static_cast<float>(n - 1);
    if (i < n / 2) return step * static_cast<float>(i);
    return __builtin_fmaf(-step, static_cast<float>(n - 1 - i), 1.0f);
}

constexpr double kPi = 3.141592653589793;  // pi rounded to double
constexpr float kPiF = 3.14159274f;        // pi rounded to float

// grid value i of n, float64 recipe
__host__ __device__ inline float grid_f64(double theta, uint32_t i, uint32_t n) {
    const double p = pow_dd(theta, linspace01_f64(i, n)).hi;
    const double prod = p * kPi;
    return static_cast<float>(prod * 0.5);
}
// grid value i of n, float32 recipe (theta already rounded to float32)
__host__ __device__ inline float grid_f32(float theta, uint32_t i, uint32_t n) {
    const float p = round_f32(pow_dd(static_cast<double>(theta), static_cast<double>(linspace01_f32(i, n))));
    const float prod = p * kPiF;
    return prod * 0.5f;
}

}  // namespace dit
}  // namespace ltx3drope
