// sad_crmath.h -- correctly rounded float32 exp, cos and sin for the site
// preparation step (the prepared record of a site must be a pure function of
// its float32 parameters, so every value is the float32 nearest to the exact
// real result).
//
// Method: evaluate in double-double arithmetic (an unevaluated sum hi + lo of
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

SAD_HD inline float exp_cr(float xf) {
    double x = (double)xf;
    if (xf != xf) return xf;
    if (x > 89.0) return __builtin_inff();
    if (x < -104.0) return 0.0f;
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
    return round_dd_to_f32(s.hi * scale, s.lo * scale);
}

// sin and cos of a float32 argument with |x| < 2^20
SAD_HD inline void sincos_cr(float xf, float* s_out, float* c_out) {
    if (xf == 0.0f) {  // keeps the sign of a zero argument in sin
        *s_out = xf;
        *c_out = 1.0f;
        return;
    }
    double x = (double)xf;
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
    *s_out = round_dd_to_f32(so.hi, so.lo);
    *c_out = round_dd_to_f32(co.hi, co.lo);
}

}  // namespace sad
