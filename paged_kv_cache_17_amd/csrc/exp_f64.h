// fp64 exponential for the sampling masses, by the table-driven method of
// P. T. P. Tang, "Table-driven implementation of the exponential function
// in IEEE floating-point arithmetic", ACM Trans. Math. Softw. 15(2), 1989.
//
// x = n * ln2/32 + r with n = rint(x * 32/ln2), so |r| <= ln2/64 (plus
// rounding); n = 32 m + j with 0 <= j < 32; exp(x) = 2^m * 2^(j/32) * exp(r).
//  * r: x - n * hi is exact in one fma (hi = ln2/32 rounded to a double,
//    whose last bit is 2^-58; x is a multiple of 2^-59 whenever n != 0 and
//    |r| < 2^-6, so the difference fits in 53 bits), then - n * lo with
//    lo = ln2/32 - hi;
//  * exp(r) - 1 = r + r^2 (1/2 + r/6 + r^2/24 + r^3/120 + r^4/720): the
//    Taylor polynomial to r^6, whose remainder is below r^7/7! < 4e-18;
//  * 2^(j/32): a 32-entry table of correctly rounded doubles, read from the
//    caller's copy (a kernel keeps one in LDS);
//  * result: fma(t, p, t), then the exact power-of-two scaling by m.
// Error: the table's half ulp plus the last fma's half ulp, so a little over
// one ulp at most; results below the normal range lose precision as
// subnormals do. exp(NaN) = NaN, exp(-inf) and arguments at or below -746
// give 0, arguments above 709.8 give +inf.
//
// The same source compiles for the device (kernels) and the host (the
// accuracy test, which includes this header directly).
#pragma once

#ifndef PKV_HOST_DEVICE
#define PKV_HOST_DEVICE __host__ __device__
#endif

namespace pkv {

// 2^(j / 32), j = 0 .. 31, each the double nearest to its value
constexpr double kExp2Frac[32] = {
    0x1.0000000000000p+0, 0x1.059b0d3158574p+0, 0x1.0b5586cf9890fp+0, 0x1.11301d0125b51p+0,
    0x1.172b83c7d517bp+0, 0x1.1d4873168b9aap+0, 0x1.2387a6e756238p+0, 0x1.29e9df51fdee1p+0,
    0x1.306fe0a31b715p+0, 0x1.371a7373aa9cbp+0, 0x1.3dea64c123422p+0, 0x1.44e086061892dp+0,
    0x1.4bfdad5362a27p+0, 0x1.5342b569d4f82p+0, 0x1.5ab07dd485429p+0, 0x1.6247eb03a5585p+0,
    0x1.6a09e667f3bcdp+0, 0x1.71f75e8ec5f74p+0, 0x1.7a11473eb0187p+0, 0x1.82589994cce13p+0,
    0x1.8ace5422aa0dbp+0, 0x1.93737b0cdc5e5p+0, 0x1.9c49182a3f090p+0, 0x1.a5503b23e255dp+0,
    0x1.ae89f995ad3adp+0, 0x1.b7f76f2fb5e47p+0, 0x1.c199bdd85529cp+0, 0x1.cb720dcef9069p+0,
    0x1.d5818dcfba487p+0, 0x1.dfc97337b9b5fp+0, 0x1.ea4afa2a490dap+0, 0x1.f50765b6e4540p+0,
};
constexpr double kExpInvStep = 0x1.71547652b82fep+5;    // 32 / ln2
constexpr double kExpStepHi = 0x1.62e42fefa39efp-6;     // ln2 / 32, rounded
constexpr double kExpStepLo = 0x1.abc9e3b39803fp-61;    // ln2 / 32 - kExpStepHi

// Three of the Taylor coefficients (1/120, 1/24, 1/6), the ones that enter
// the polynomial as addends. A kernel evaluating many exponentials may pass
// copies it keeps in registers, so that the compiler does not rebuild them
// for every evaluation; the values are the same.
struct ExpCoef {
    double c5, c4, c3;
};
constexpr ExpCoef kExpCoef{1.0 / 120.0, 1.0 / 24.0, 1.0 / 6.0};

// exp(x) with the table of 2^(j/32) at `tab` (kExp2Frac or a copy of it).
// Branch-free (the argument is clamped and the special results selected at
// the end), so that a caller's independent evaluations can interleave.
PKV_HOST_DEVICE inline double exp_tab(double x, const double* tab) {
    const double xc = __builtin_fmin(__builtin_fmax(x, -746.0), 710.0);   // NaN becomes -746
    const double n = __builtin_rint(xc * kExpInvStep);
    double r = __builtin_fma(-n, kExpStepHi, xc);
    r = __builtin_fma(-n, kExpStepLo, r);
    const int ni = static_cast<int>(n);
    double q = __builtin_fma(r, 1.0 / 720.0, 1.0 / 120.0);
    q = __builtin_fma(q, r, 1.0 / 24.0);
    q = __builtin_fma(q, r, 1.0 / 6.0);
    q = __builtin_fma(q, r, 0.5);
    const double p = __builtin_fma(q, r * r, r);   // exp(r) - 1
    const double t = tab[ni & 31];
    double y = __builtin_ldexp(__builtin_fma(t, p, t), ni >> 5);
    y = x > 709.8 ? __builtin_inf() : y;
    y = x > -746.0 ? y : 0.0;
    return x != x ? x : y;
}

// exp(x) for x <= 0 (or NaN), as exp_tab: every mass exp(z - max z) has
// such an argument. Nothing can overflow, and below -746 the scaled result
// rounds to 0 by itself (2^(j/32) (1 + p) 2^m with m <= -1077 lies below
// half the least subnormal), so only the lower clamp and NaN remain.
PKV_HOST_DEVICE inline double exp_nonpos(double x, const double* tab, const ExpCoef& k = kExpCoef) {
    const double xc = __builtin_fmax(x, -746.0);   // NaN becomes -746; -inf as well
    const double n = __builtin_rint(xc * kExpInvStep);
    double r = __builtin_fma(-n, kExpStepHi, xc);
    r = __builtin_fma(-n, kExpStepLo, r);
    const int ni = static_cast<int>(n);
    double q = __builtin_fma(r, 1.0 / 720.0, k.c5);
    q = __builtin_fma(q, r, k.c4);
    q = __builtin_fma(q, r, k.c3);
    q = __builtin_fma(q, r, 0.5);
    const double p = __builtin_fma(q, r * r, r);
    const double t = tab[ni & 31];
    const double y = __builtin_ldexp(__builtin_fma(t, p, t), ni >> 5);
    return x != x ? x : y;
}

}  // namespace pkv
