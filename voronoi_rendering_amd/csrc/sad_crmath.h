// sad_crmath.h -- correctly rounded float32 exp, cos and sin for the site
// preparation step (the prepared record of a site must be a pure function of
// its float32 parameters, so every value is the float32 nearest to the exact
// real result).
//
// Two stages.  A plain double evaluation (relative error below 2^-50) settles
// almost every argument: its float32 rounding is taken when the whole
// interval y (1 -+ 2^-46) around the double result y rounds to one float32
// (rounding is monotone, so the exact value, which lies inside, rounds to the
// same float32).  Otherwise (about one argument in 2^21, and NaN) the
// double-double evaluation below decides.
//
// Double-double stage: evaluate in double-double arithmetic (an unevaluated sum hi + lo of
// two doubles, about 106 significant bits; Dekker 1971, with the exact
// product from a fused multiply-add), then round hi + lo to float32 once.
//   exp:  x = k ln2 + r, |r| <= ln2/2 (Cody-Waite with a two-part ln2),
//         e^r from its Taylor series to degree 20 (remainder < 2^-97) in
//         Horner form with double-double coefficients 1/n!, then scale by 2^k.
//   sin/cos: x = k pi/2 + r, |r| <= pi/4 (three-part pi/2, exact products for
//         |k| < 2^21), Taylor series of sin r and cos r to degree 29/28
//         (remainder < 2^-110), Horner form in r^2, then the quadrant k mod 4
//         picks the result.
// Each double-double step has a relative error near 2^-104 and each
// coefficient is within 2^-106 of its value (gen_crmath_coeffs.py computes
// them in 300-bit arithmetic), so the relative error of hi + lo stays far
// below 2^-80, while a float32 result is only ambiguous when the exact value
// lies within 2^-80 of a rounding boundary, which no float32 argument in the
// supported range produces.
//
// All double operations are plain IEEE operations; the file is compiled
// without floating-point contraction, and fused multiply-adds appear only
// where written (two_prod).
#pragma once

#include <stdint.h>

#ifndef SAD_HD
#define SAD_HD __host__ __device__
#endif

namespace sad {

struct dd {
    double hi, lo;
};

SAD_HD inline dd two_sum(double a, double b) {
    double s = a + b;
    double bb = s - a;
    double e = (a - (s - bb)) + (b - bb);
    return {s, e};
}

SAD_HD inline dd fast_two_sum(double a, double b) {  // requires |a| >= |b| or a == 0
    double s = a + b;
    double e = b - (s - a);
    return {s, e};
}

SAD_HD inline dd two_prod(double a, double b) {
    double p = a * b;
    double e = __builtin_fma(a, b, -p);
    return {p, e};
}

SAD_HD inline dd dd_add(dd a, dd b) {
    dd s = two_sum(a.hi, b.hi);
    dd t = two_sum(a.lo, b.lo);
    s.lo += t.hi;
    s = fast_two_sum(s.hi, s.lo);
    s.lo += t.lo;
    return fast_two_sum(s.hi, s.lo);
}

SAD_HD inline dd dd_neg(dd a) { return {-a.hi, -a.lo}; }

SAD_HD inline dd dd_mul(dd a, dd b) {
    dd p = two_prod(a.hi, b.hi);
    p.lo += a.hi * b.lo + a.lo * b.hi;
    return fast_two_sum(p.hi, p.lo);
}

// Taylor coefficients as double-doubles (printed by gen_crmath_coeffs.py)
// 1/n!, n = 0..20
constexpr dd EXP_C[21] = {
    {0x1.0000000000000p+0, 0x0.0p+0},
    {0x1.0000000000000p+0, 0x0.0p+0},
    {0x1.0000000000000p-1, 0x0.0p+0},
    {0x1.5555555555555p-3, 0x1.5555555555555p-57},
    {0x1.5555555555555p-5, 0x1.5555555555555p-59},
    {0x1.1111111111111p-7, 0x1.1111111111111p-63},
    {0x1.6c16c16c16c17p-10, -0x1.f49f49f49f49fp-65},
    {0x1.a01a01a01a01ap-13, 0x1.a01a01a01a01ap-73},
    {0x1.a01a01a01a01ap-16, 0x1.a01a01a01a01ap-76},
    {0x1.71de3a556c734p-19, -0x1.c154f8ddc6c00p-73},
    {0x1.27e4fb7789f5cp-22, 0x1.cbbc05b4fa99ap-76},
    {0x1.ae64567f544e4p-26, -0x1.c062e06d1f209p-80},
    {0x1.1eed8eff8d898p-29, -0x1.2aec959e14c06p-83},
    {0x1.6124613a86d09p-33, 0x1.f28e0cc748ebep-87},
    {0x1.93974a8c07c9dp-37, 0x1.05d6f8a2efd1fp-92},
    {0x1.ae7f3e733b81fp-41, 0x1.1d8656b0ee8cbp-97},
    {0x1.ae7f3e733b81fp-45, 0x1.1d8656b0ee8cbp-101},
    {0x1.952c77030ad4ap-49, 0x1.ac981465ddc6cp-103},
    {0x1.6827863b97d97p-53, 0x1.eec01221a8b0bp-107},
    {0x1.2f49b46814157p-57, 0x1.2650f61dbdcb4p-112},
    {0x1.e542ba4020225p-62, 0x1.ea72b4afe3c2fp-120}};

// (-1)^n/(2n+1)!, n = 0..14
constexpr dd SIN_C[15] = {
    {0x1.0000000000000p+0, 0x0.0p+0},
    {-0x1.5555555555555p-3, -0x1.5555555555555p-57},
    {0x1.1111111111111p-7, 0x1.1111111111111p-63},
    {-0x1.a01a01a01a01ap-13, -0x1.a01a01a01a01ap-73},
    {0x1.71de3a556c734p-19, -0x1.c154f8ddc6c00p-73},
    {-0x1.ae64567f544e4p-26, 0x1.c062e06d1f209p-80},
    {0x1.6124613a86d09p-33, 0x1.f28e0cc748ebep-87},
    {-0x1.ae7f3e733b81fp-41, -0x1.1d8656b0ee8cbp-97},
    {0x1.952c77030ad4ap-49, 0x1.ac981465ddc6cp-103},
    {-0x1.2f49b46814157p-57, -0x1.2650f61dbdcb4p-112},
    {0x1.71b8ef6dcf572p-66, -0x1.d043ae40c4647p-120},
    {-0x1.761b41316381ap-75, 0x1.3423c7d91404fp-130},
    {0x1.3f3ccdd165fa9p-84, -0x1.58ddadf344487p-139},
    {-0x1.d1ab1c2dccea3p-94, -0x1.054d0c78aea14p-149},
    {0x1.259f98b4358adp-103, 0x1.eaf8c39dd9bc5p-157}};

// (-1)^n/(2n)!, n = 0..14
constexpr dd COS_C[15] = {
    {0x1.0000000000000p+0, 0x0.0p+0},
    {-0x1.0000000000000p-1, 0x0.0p+0},
    {0x1.5555555555555p-5, 0x1.5555555555555p-59},
    {-0x1.6c16c16c16c17p-10, 0x1.f49f49f49f49fp-65},
    {0x1.a01a01a01a01ap-16, 0x1.a01a01a01a01ap-76},
    {-0x1.27e4fb7789f5cp-22, -0x1.cbbc05b4fa99ap-76},
    {0x1.1eed8eff8d898p-29, -0x1.2aec959e14c06p-83},
    {-0x1.93974a8c07c9dp-37, -0x1.05d6f8a2efd1fp-92},
    {0x1.ae7f3e733b81fp-45, 0x1.1d8656b0ee8cbp-101},
    {-0x1.6827863b97d97p-53, -0x1.eec01221a8b0bp-107},
    {0x1.e542ba4020225p-62, 0x1.ea72b4afe3c2fp-120},
    {-0x1.0ce396db7f853p-70, 0x1.aebcdbd20331cp-124},
    {0x1.f2cf01972f578p-80, -0x1.9ada5fcc1ab14p-135},
    {-0x1.88e85fc6a4e5ap-89, 0x1.71c37ebd16540p-143},
    {0x1.0a18a2635085dp-98, 0x1.b9e2e28e1aa54p-153}};


SAD_HD inline uint32_t f32_bits(float f) {
    union { float f; uint32_t u; } c;
    c.f = f;
    return c.u;
}

SAD_HD inline float f32_from_bits(uint32_t u) {
    union { float f; uint32_t u; } c;
    c.u = u;
    return c.f;
}

// Round the real number hi + lo (|lo| <= ulp(hi)/2) to the nearest float32,
// ties to even.  Only hi can sit exactly on a float32 midpoint; then the sign
// of lo decides.
SAD_HD inline float round_dd_to_f32(double hi, double lo) {
    if (hi != hi) return (float)hi;
    bool neg = hi < 0.0;
    if (neg) {
        hi = -hi;
        lo = -lo;
    }
    float f = (float)hi;  // round to nearest even of hi alone
    double fd = (double)f;
    float out = f;
    if (fd != hi) {
        // the two float32 neighbours of hi are f and g
        uint32_t fb = f32_bits(f);
        float g;
        if (hi > fd) {
            g = f32_from_bits(fb + 1u);  // also steps FLT_MAX to +inf
        } else {
            g = (fb == 0u) ? 0.0f : f32_from_bits(fb - 1u);
        }
        if (f == __builtin_inff()) {
            // hi rounded up to infinity: the neighbours are FLT_MAX and "2^128"
            g = f32_from_bits(0x7f7fffffu);
            double mid = (double)g + 0x1p103;
            if (hi == mid && lo < 0.0) out = g;
        } else {
            double mid = 0.5 * (fd + (double)g);
            if (hi == mid && lo != 0.0) {
                float lower = f < g ? f : g, upper = f < g ? g : f;
                out = lo > 0.0 ? upper : lower;
            }
        }
    }
    return neg ? -out : out;
}

// ln 2 as a double-double (hi = ln 2 rounded to double)
#define SAD_LN2_HI 0x1.62e42fefa39efp-1
#define SAD_LN2_LO 0x1.abc9e3b39803fp-56
// pi/2 as a sum of three doubles
#define SAD_PIO2_1 0x1.921fb54442d18p+0
#define SAD_PIO2_2 0x1.1a62633145c07p-54
#define SAD_PIO2_3 -0x1.f1976b7ed8fbcp-110

// e^x as a double-double, for a float32 x in [-104, 89]
SAD_HD inline dd exp_dd(double x) {
    double k = __builtin_rint(x * 1.4426950408889634);
    dd kl = two_prod(k, SAD_LN2_HI);
    dd kl2 = two_prod(k, SAD_LN2_LO);
    dd r = dd_add(dd{x, 0.0}, dd_neg(kl));
    r = dd_add(r, dd_neg(kl2));
    dd s = EXP_C[20];
#pragma unroll
    for (int n = 19; n >= 0; --n) s = dd_add(dd_mul(s, r), EXP_C[n]);
    int ki = (int)k;
    double scale = __builtin_ldexp(1.0, ki);
    return {s.hi * scale, s.lo * scale};
}

SAD_HD inline float exp_cr_dd(float xf) {
    double x = (double)xf;
    if (xf != xf) return xf;
    if (x > 89.0) return __builtin_inff();
    if (x < -104.0) return 0.0f;
    const dd v = exp_dd(x);
    return round_dd_to_f32(v.hi, v.lo);
}

// sin and cos as double-doubles, for a float32 x with |x| < 2^20
SAD_HD inline void sincos_dd(double x, dd* s_out, dd* c_out) {
    double k = __builtin_rint(x * 0.63661977236758138);  // x * 2/pi
    dd t1 = two_prod(k, SAD_PIO2_1);
    dd t2 = two_prod(k, SAD_PIO2_2);
    dd r = dd_add(dd{x, 0.0}, dd_neg(t1));
    r = dd_add(r, dd_neg(t2));
    r = dd_add(r, dd{-k * SAD_PIO2_3, 0.0});
    dd r2 = dd_mul(r, r);
    dd sn = SIN_C[14], cs = COS_C[14];
#pragma unroll
    for (int n = 13; n >= 0; --n) {
        sn = dd_add(dd_mul(sn, r2), SIN_C[n]);
        cs = dd_add(dd_mul(cs, r2), COS_C[n]);
    }
    sn = dd_mul(r, sn);
    long long q = (long long)k & 3;
    dd so, co;
    if (q == 0) {
        so = sn;
        co = cs;
    } else if (q == 1) {
        so = cs;
        co = dd_neg(sn);
    } else if (q == 2) {
        so = dd_neg(sn);
        co = dd_neg(cs);
    } else {
        so = dd_neg(cs);
        co = sn;
    }
    *s_out = so;
    *c_out = co;
}

SAD_HD inline void sincos_cr_dd(float xf, float* s_out, float* c_out) {
    if (xf == 0.0f) {  // keeps the sign of a zero argument in sin
        *s_out = xf;
        *c_out = 1.0f;
        return;
    }
    dd so, co;
    sincos_dd((double)xf, &so, &co);
    *s_out = round_dd_to_f32(so.hi, so.lo);
    *c_out = round_dd_to_f32(co.hi, co.lo);
}

// ---- double stage ---------------------------------------------------------
//
// Split constants (printed by gen_crmath_coeffs.py): the leading parts have few
// significant bits, so k times them is exact for every k that occurs.
// ln 2 = SAD_LN2_A + SAD_LN2_B + O(2^-85); SAD_LN2_A has 32 significant bits
#define SAD_LN2_A 0x1.62e42fee00000p-1
#define SAD_LN2_B 0x1.a39ef35793c76p-33
// pi/2 = SAD_PIO2_A + SAD_PIO2_B + SAD_PIO2_C + O(2^-118); A and B have 33 significant bits
#define SAD_PIO2_A 0x1.921fb54400000p+0
#define SAD_PIO2_B 0x1.0b4611a600000p-34
#define SAD_PIO2_C 0x1.3198a2e037073p-69

// Called when the double stage leaves an argument to the double-double stage
// (a counting hook for host tests; empty otherwise).
#ifndef SAD_CR_FALLBACK_HOOK
#define SAD_CR_FALLBACK_HOOK()
#endif

constexpr double CR_BAND = 0x1p-46;  // > 16 x the double stage's error bound

// The float32 rounding of every value in y (1 -+ CR_BAND), if it is one
// float32 (then *out holds it).  A NaN y never settles.
SAD_HD inline bool settle_f32(double y, float* out) {
    const float a = (float)(y * (1.0 - CR_BAND));
    const float b = (float)(y * (1.0 + CR_BAND));
    *out = a;
    return a == b;
}

// exp in double: x = k ln2 + r with k = rint(x / ln2), |k| <= 150.  k SAD_LN2_A
// is exact (40 bits) and x - k SAD_LN2_A is exact (the two are within a
// factor of 2 when k != 0), so r carries two roundings: |dr| <= 2u|r| + 2^-77
// (u = 2^-53).  e^r for |r| <= 0.347 from its Taylor series to degree 13
// (remainder < 2^-56 relative) in Horner form with fused multiply-adds and
// double coefficients: the roundings of the steps and of the coefficients
// add at most 6u relative.  Scaling by 2^k is exact.  Total < 2^-50.
SAD_HD inline double exp_d(double x) {  // float32 x in [-104, 89]
    const double k = __builtin_rint(x * 1.4426950408889634);
    const double r = (x - k * SAD_LN2_A) - k * SAD_LN2_B;
    double p = EXP_C[13].hi;
#pragma unroll
    for (int n = 12; n >= 0; --n) p = __builtin_fma(p, r, EXP_C[n].hi);
    return __builtin_ldexp(p, (int)k);
}

SAD_HD inline float exp_cr(float xf) {
    if (xf != xf) return xf;
    const double x = (double)xf;
    if (x > 89.0) return __builtin_inff();
    if (x < -104.0) return 0.0f;
    float out;
    if (settle_f32(exp_d(x), &out)) return out;
    SAD_CR_FALLBACK_HOOK();
    return exp_cr_dd(xf);
}

// sin and cos in double for |x| < 2^20: x = k pi/2 + r, |r| <= pi/4, with
// k SAD_PIO2_A and k SAD_PIO2_B exact (|k| < 2^20) and x - k SAD_PIO2_A exact,
// so r carries two roundings plus the 2^-118 truncation of pi/2 times k:
// relative error < 2u + 2^-57 even for the |r| near 2^-30 that float32
// arguments reach.  With z = r^2 <= 0.618, sin r = r (1 + z S1 + ... + z^9 S9)
// and cos r = 1 + z C1 + ... + z^9 C9 (remainders below 2^-70), Horner form
// with fused multiply-adds: at most about 5u relative for sin and 4u for cos
// (cos r >= 0.707 on the interval).  Total < 2^-50.
SAD_HD inline void sincos_d(double x, double* s_out, double* c_out) {  // float32 x, |x| < 2^20
    const double k = __builtin_rint(x * 0.63661977236758138);
    const double r = ((x - k * SAD_PIO2_A) - k * SAD_PIO2_B) - k * SAD_PIO2_C;
    const double z = r * r;
    double ps = SIN_C[9].hi, pc = COS_C[9].hi;
#pragma unroll
    for (int n = 8; n >= 0; --n) {
        ps = __builtin_fma(ps, z, SIN_C[n].hi);
        pc = __builtin_fma(pc, z, COS_C[n].hi);
    }
    const double sr = r * ps;
    const long long q = (long long)k & 3;
    *s_out = q == 0 ? sr : q == 1 ? pc : q == 2 ? -sr : -pc;
    *c_out = q == 0 ? pc : q == 1 ? -sr : q == 2 ? -pc : sr;
}

SAD_HD inline void sincos_cr(float xf, float* s_out, float* c_out) {
    if (xf == 0.0f) {  // keeps the sign of a zero argument in sin
        *s_out = xf;
        *c_out = 1.0f;
        return;
    }
    const double x = (double)xf;
    if (__builtin_fabs(x) < 0x1p20) {  // false for NaN
        double sv, cv;
        sincos_d(x, &sv, &cv);
        float so, co;
        if (settle_f32(sv, &so) && settle_f32(cv, &co)) {
            *s_out = so;
            *c_out = co;
            return;
        }
    }
    SAD_CR_FALLBACK_HOOK();
    sincos_cr_dd(xf, s_out, c_out);
}

}  // namespace sad
