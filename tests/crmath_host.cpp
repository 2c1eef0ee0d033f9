// Host build of the HIP path's correctly rounded exp/sin/cos (the header is
// plain C++ apart from its __host__ __device__ markers), for CPU tests: the
// double stage with its double-double fallback must give the same float32 as
// the double-double stage alone, and the fallback must stay rare.
#include <cstdint>
#include <cstring>

static long g_fallbacks = 0;
#define SAD_HD
#define SAD_CR_FALLBACK_HOOK() (++g_fallbacks)
#include "../voronoi_rendering_amd/csrc/sad_crmath.h"

static bool same_bits(float a, float b) { return std::memcmp(&a, &b, 4) == 0; }

extern "C" {

// Every float32 with bit pattern b0, b0 + step, ... < b1 and its negation:
// exp through both paths, and sin/cos through both paths when |x| < 2^20.
// Returns the number of arguments where the paths differ; *fallbacks counts
// the double-double evaluations the double stage asked for, *count the
// evaluations.
long cr_compare_paths(uint32_t b0, uint32_t b1, uint32_t step, long* fallbacks, long* count) {
    long bad = 0, n = 0;
    g_fallbacks = 0;
    for (uint64_t b = b0; b < b1; b += step) {
        for (int sgn = 0; sgn < 2; ++sgn) {
            const uint32_t bits = (uint32_t)b | (sgn ? 0x80000000u : 0u);
            float x;
            std::memcpy(&x, &bits, 4);
            bad += !same_bits(sad::exp_cr(x), sad::exp_cr_dd(x));
            ++n;
            if (x > -1048576.0f && x < 1048576.0f) {
                float s1, c1, s2, c2;
                sad::sincos_cr(x, &s1, &c1);
                sad::sincos_cr_dd(x, &s2, &c2);
                bad += !(same_bits(s1, s2) && same_bits(c1, c2));
                n += 2;
            }
        }
    }
    *fallbacks = g_fallbacks;
    *count = n;
    return bad;
}

// Largest relative difference between the double stage and the double-double
// stage (before rounding) over the same arguments: exp for x in [-104, 89],
// sin and cos for |x| < 2^20 (zero excluded).
double cr_max_rel_error(uint32_t b0, uint32_t b1, uint32_t step) {
    double worst = 0.0;
    auto rel = [](double y, sad::dd v) {
        const double ref = v.hi + v.lo;
        const double d = (y - v.hi) - v.lo;
        return d < 0 ? -d / (ref < 0 ? -ref : ref) : d / (ref < 0 ? -ref : ref);
    };
    for (uint64_t b = b0; b < b1; b += step) {
        for (int sgn = 0; sgn < 2; ++sgn) {
            const uint32_t bits = (uint32_t)b | (sgn ? 0x80000000u : 0u);
            float xf;
            std::memcpy(&xf, &bits, 4);
            const double x = xf;
            if (x >= -104.0 && x <= 89.0) {
                const double e = rel(sad::exp_d(x), sad::exp_dd(x));
                worst = e > worst ? e : worst;
            }
            if (xf != 0.0f && x > -1048576.0 && x < 1048576.0) {
                double s, c;
                sad::dd so, co;
                sad::sincos_d(x, &s, &c);
                sad::sincos_dd(x, &so, &co);
                const double es = rel(s, so), ec = rel(c, co);
                worst = es > worst ? es : worst;
                worst = ec > worst ? ec : worst;
            }
        }
    }
    return worst;
}

double cr_band() { return sad::CR_BAND; }

void cr_eval(const float* x, long m, float* e, float* s, float* c) {
    for (long i = 0; i < m; ++i) {
        e[i] = sad::exp_cr(x[i]);
        sad::sincos_cr(x[i], &s[i], &c[i]);
    }
}
}
