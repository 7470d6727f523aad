// expf_cr.hpp — correctly rounded binary32 exp and the gated SiLU built on it
// (device code, gfx950).
#pragma once

#include "device.hpp"

namespace pf {

// Correctly rounded binary32 exp.  exp(x) is evaluated in double-double
// arithmetic (about 95 correct bits after the squarings below), far more than
// the roughly 24 + 40 bits that any binary32 argument needs to decide its
// rounding, and the double-double value is then rounded to binary32 exactly.
//   x = k ln2 + r, |r| <= ln2/2 (k = rint(x / ln2); k ln2 in double-double);
//   s = r / 2^10;  e^s - 1 by its Taylor series to s^10 (|s| < 3.4e-4);
//   (1 + m)^(2^10) by ten squarings m <- 2m + m^2;  e^x = 2^k (1 + m).
struct dd {
    double hi, lo;
};

__device__ __forceinline__ dd two_sum(double a, double b)
{
    const double s = a + b;
    const double bb = s - a;
    const double e = (a - (s - bb)) + (b - bb);
    return {s, e};
}
__device__ __forceinline__ dd fast_two_sum(double a, double b)
{
    const double s = a + b;
    const double e = b - (s - a);
    return {s, e};
}
__device__ __forceinline__ dd two_prod(double a, double b)
{
    const double p = a * b;
    const double e = fma(a, b, -p);
    return {p, e};
}
__device__ __forceinline__ dd dd_add(dd a, dd b)
{
    dd s = two_sum(a.hi, b.hi);
    const dd t = two_sum(a.lo, b.lo);
    s.lo = s.lo + t.hi;
    s = fast_two_sum(s.hi, s.lo);
    s.lo = s.lo + t.lo;
    return fast_two_sum(s.hi, s.lo);
}
__device__ __forceinline__ dd dd_mul(dd a, dd b)
{
    dd p = two_prod(a.hi, b.hi);
    const double c = a.hi * b.lo;
    const double d = a.lo * b.hi;
    p.lo = p.lo + (c + d);
    return fast_two_sum(p.hi, p.lo);
}
__device__ __forceinline__ dd dd_mul_d(dd a, double b)
{
    dd p = two_prod(a.hi, b);
    p.lo = p.lo + a.lo * b;
    return fast_two_sum(p.hi, p.lo);
}
__device__ __forceinline__ dd dd_div_d(dd a, double b)
{
    const double q1 = a.hi / b;
    const dd p = two_prod(q1, b);
    const double r = ((a.hi - p.hi) - p.lo + a.lo) / b;
    return fast_two_sum(q1, r);
}

// ln 2 split into double-double: the nearest double and the nearest double to
// the remainder.
__device__ constexpr double kLn2Hi = 0x1.62e42fefa39efp-1;
__device__ constexpr double kLn2Lo = 0x1.abc9e3b39803fp-56;

// The double-double evaluation (the rare arguments the double one below
// cannot round with certainty).  -104 <= x <= 89, x != 0.
static __device__ __noinline__ float expf_cr_dd(float xf)
{
    const double x = (double)xf;
    const double k = rint(x * (1.0 / kLn2Hi));
    const dd kl = dd_mul_d(dd{kLn2Hi, kLn2Lo}, k);
    const dd r = dd_add(dd{x, 0.0}, dd{-kl.hi, -kl.lo});
    const dd s{ldexp(r.hi, -10), ldexp(r.lo, -10)};
    // m = e^s - 1 = s (1 + s/2 (1 + s/3 (1 + ... (1 + s/10))))
    dd m{1.0, 0.0};
    for (int n = 10; n >= 2; --n) m = dd_add(dd{1.0, 0.0}, dd_mul(dd_div_d(s, (double)n), m));
    m = dd_mul(s, m);
    for (int i = 0; i < 10; ++i) m = dd_add(dd_mul_d(m, 2.0), dd_mul(m, m));
    dd y = dd_add(dd{1.0, 0.0}, m);
    const int ki = (int)k;
    y.hi = ldexp(y.hi, ki);
    y.lo = ldexp(y.lo, ki);
    // Round hi + lo to binary32.  f = RN(hi); the exact value lies on the far
    // side of the midpoint between f and its neighbour only if hi is that
    // midpoint and lo points away from f.
    float f = (float)y.hi;
    if (__builtin_isinf(f)) {
        // hi is at or past the overflow midpoint (2 - 2^-24) 2^127 between the
        // largest finite binary32 and 2^128: the exact value rounds to +inf
        // unless it lies just below that midpoint (hi on it, lo negative)
        return (y.hi == 0x1.ffffffp127 && y.lo < 0.0) ? 0x1.fffffep127f : f;
    }
    const double d = y.hi - (double)f;   // exact
    if (d != 0.0) {
        const float g = d > 0.0 ? nextafterf(f, __builtin_huge_valf()) : nextafterf(f, 0.0f);
        const double half = ((double)g - (double)f) * 0.5;
        if (d == half && ((d > 0.0 && y.lo > 0.0) || (d < 0.0 && y.lo < 0.0))) f = g;
    } else if (y.lo != 0.0) {
        // hi is a binary32 value: the exact value differs by |lo| << half a unit
    }
    return f;
}

// Correctly rounded binary32 exp.  Most arguments take one double evaluation:
//   x = k ln2 + r with ln2 split Cody-Waite style (k ln2_hi exact, |r| <= ln2/2),
//   e^r by its Taylor polynomial of degree 13 in Horner form with fused
//   multiply-adds (truncation below 2^-56, rounding below 2^-52 relative),
//   e^x = 2^k e^r: relative error below 2^-51.
// Its binary32 rounding f is the correct one unless the double lies within
// 2^-45 (relative) of the midpoint between f and its neighbour on its side, a
// margin of 64 times the error bound; those arguments, and those whose value
// overflows binary32, go to the double-double evaluation.
__device__ constexpr double kLn2CwHi = 0x1.62e42fee00000p-1;   // 32 significant bits
__device__ constexpr double kLn2CwLo = 0x1.a39ef35793c76p-33;  // ln 2 - kLn2CwHi, rounded

__device__ __forceinline__ float expf_cr(float xf)
{
    if (xf != xf) return xf;
    if (xf < -104.0f) return 0.0f;    // exp(x) < 2^-150: rounds to +0
    if (xf > 89.0f) return __builtin_huge_valf();
    if (xf == 0.0f) return 1.0f;
    const double x = (double)xf;
    const double k = rint(x * 0x1.71547652b82fep0);      // x / ln 2, nearest integer
    const double r = (x - k * kLn2CwHi) - k * kLn2CwLo;  // first difference exact
    double p = 1.0 / 6227020800.0;                        // 1/13!
    p = fma(p, r, 1.0 / 479001600.0);
    p = fma(p, r, 1.0 / 39916800.0);
    p = fma(p, r, 1.0 / 3628800.0);
    p = fma(p, r, 1.0 / 362880.0);
    p = fma(p, r, 1.0 / 40320.0);
    p = fma(p, r, 1.0 / 5040.0);
    p = fma(p, r, 1.0 / 720.0);
    p = fma(p, r, 1.0 / 120.0);
    p = fma(p, r, 1.0 / 24.0);
    p = fma(p, r, 1.0 / 6.0);
    p = fma(p, r, 0.5);
    p = fma(p, r, 1.0);
    p = fma(p, r, 1.0);
    const double y = ldexp(p, (int)k);
    const float f = (float)y;
    if (!__builtin_isinf(f)) {
        const double dy = y - (double)f;                  // exact
        if (dy == 0.0) return f;
        const float nb = dy > 0.0 ? nextafterf(f, __builtin_huge_valf()) : nextafterf(f, -__builtin_huge_valf());
        const double mid = ((double)f + (double)nb) * 0.5; // exact
        if (fabs(y - mid) > fabs(y) * 0x1p-45) return f;
    }
    return expf_cr_dd(xf);
}

// silu(g) = fl(g / fl(1 + expf_cr(-g))), each operation rounded on its own;
// past g = -88.72 exp(-g) is +inf and the quotient -0.  Out of line: it sits
// in the epilogues of fully unrolled product loops.
static __device__ __noinline__ float silu_cr(float g)
{
    const float e = expf_cr(-g);
    const float d = 1.0f + e;
    return g / d;
}

}  // namespace pf
