// sad_crmath.h -- correctly rounded float32 exp, cos and sin for the site
// preparation step (the prepared record of a site must be a pure function of
// its float32 parameters, so every value is the float32 nearest to the exact
// real result).
//
// Method: evaluate in double-double arithmetic (an unevaluated sum hi + lo of
// two doubles, about 106 significant bits; Dekker 1971, with the exact
// product from a fused multiply-add), then round hi + lo to float32 once.
//   exp:  x = k ln2 + r, |r| <= ln2/2 (Cody-Waite with a two-part ln2),
//         e^r from its Taylor series in Horner form 1 + r/1 (1 + r/2 (1 + ...)),
//         20 terms (remainder < 2^-97), then scale by 2^k.
//   sin/cos: x = k pi/2 + r, |r| <= pi/4 (three-part pi/2, exact products for
//         |k| < 2^21), Taylor series of sin r and cos r to degree 29/28
//         (remainder < 2^-110), then the quadrant k mod 4 picks the result.
// The relative error of hi + lo is far below 2^-80, while a float32 result is
// only ambiguous when the exact value lies within 2^-80 of a rounding
// boundary, which no float32 argument in the supported range produces.
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

// a / b for a small positive integer b (exactly representable)
SAD_HD inline dd dd_div_int(dd a, double b) {
    double q1 = a.hi / b;
    double r = __builtin_fma(-q1, b, a.hi);  // exact remainder of the leading quotient
    double q2 = (r + a.lo) / b;
    return fast_two_sum(q1, q2);
}

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
    dd s = {1.0, 0.0};
    for (int n = 20; n >= 1; --n) s = dd_add(dd{1.0, 0.0}, dd_div_int(dd_mul(r, s), (double)n));
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
    dd sn = {1.0, 0.0}, cs = {1.0, 0.0};
    for (int n = 14; n >= 1; --n) {
        sn = dd_add(dd{1.0, 0.0}, dd_neg(dd_div_int(dd_mul(r2, sn), (double)((2 * n) * (2 * n + 1)))));
        cs = dd_add(dd{1.0, 0.0}, dd_neg(dd_div_int(dd_mul(r2, cs), (double)((2 * n - 1) * (2 * n)))));
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
