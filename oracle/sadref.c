/*
 * sadref.c -- plain CPU oracle for the Soft Anisotropic Diagrams (SAD) hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call this code:
 * only the tests, the smoke check and the benchmark's CPU-baseline leg load it.
 * It shares no code, header or constant table with the HIP library; the two
 * meet only at the documented data formats (site records, top-K map).
 *
 * Source: "Soft Anisotropic Diagrams for Differentiable Image Representation"
 * (Iinbor, Dou, Matusik; arXiv 2604.21984), paper body as published on
 * paperpeel.com.  Each function names the section it follows.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math (no FMA
 * contraction, IEEE round-to-nearest, no flush-to-zero), optional -fopenmp.
 *
 * Precision.  The paper keeps training site parameters in float32
 * (Appendix B.2 "Site buffer").  The ranking score that decides the top-K
 * lists is therefore evaluated in float32, one rounding per operation in a
 * fixed order (score_at below).  Rendering, gradients and the loss are
 * evaluated in float64 from those float32 scores and parameters.  Adam works
 * on the float32 parameter buffer one float32 operation at a time.
 *
 * Layouts (row-major, little-endian):
 *   params  [n][12] f32: x, y, log_tau, r, c_r, c_g, c_b, theta, log_s1, log_s2, 0, 0
 *   derived [n][12] f32: x, y, tau, r, cos(theta), sin(theta), exp(-log_s1),
 *                        exp(-log_s2), c_r, c_g, c_b, 0
 *   topk    [h][w][8] u32: site ids, best first, 0xffffffff padding at the end
 *   images  [h][w][3]
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define K 8
#define NONE 0xffffffffu
#define REC 12

/* ------------------------------------------------------------------------ */
/* Site preparation: tau = exp(log tau) (Sec. 4.1), the rotation and the
 * inverse scales of the anisotropic metric (Sec. 4.1, eq. for G_i).
 * Each derived value is the float32 nearest to the exact real value
 * (round-to-nearest-even of the mathematical function).  The value is
 * computed in x87 extended precision and rounded once; a guard checks that the
 * extended result is far enough from a float32 rounding boundary that its few
 * ulps of library error cannot change the rounded float. */

static long sadref_ambiguous_roundings = 0;

static float round_ld_to_f32(long double v)
{
    if (!isfinite(v) || v == 0.0L) return (float)v;
    long double lo = v, hi = v;
    for (int i = 0; i < 4; ++i) {
        lo = nextafterl(lo, -INFINITY);
        hi = nextafterl(hi, INFINITY);
    }
    float f = (float)v;
    if ((float)lo != f || (float)hi != f) sadref_ambiguous_roundings++;
    return f;
}

long sadref_ambiguous_count(void) { return sadref_ambiguous_roundings; }

float sadref_exp_f32(float x) { return round_ld_to_f32(expl((long double)x)); }
float sadref_cos_f32(float x) { return round_ld_to_f32(cosl((long double)x)); }
float sadref_sin_f32(float x) { return round_ld_to_f32(sinl((long double)x)); }

/* Largest |theta| for which a site's rotation is evaluated; beyond it the
 * prepared record marks the site inactive (x = -1). */
#define THETA_LIMIT 1048576.0f

void sadref_prepare_sites(const float *params, int32_t n, float *derived)
{
    for (int32_t i = 0; i < n; ++i) {
        const float *p = params + (size_t)i * REC;
        float *d = derived + (size_t)i * REC;
        float theta = p[7];
        int active = p[0] >= 0.0f && fabsf(theta) <= THETA_LIMIT;
        d[0] = active ? p[0] : -1.0f;
        d[1] = active ? p[1] : -1.0f;
        d[2] = sadref_exp_f32(p[2]);
        d[3] = p[3];
        d[4] = active ? sadref_cos_f32(theta) : 1.0f;
        d[5] = active ? sadref_sin_f32(theta) : 0.0f;
        d[6] = sadref_exp_f32(-p[8]);
        d[7] = sadref_exp_f32(-p[9]);
        d[8] = p[4];
        d[9] = p[5];
        d[10] = p[6];
        d[11] = 0.0f;
    }
}

/* ------------------------------------------------------------------------ */
/* The per-site logit (Sec. 4.2): l = -tau * (||x - p||_G - r), with
 * G = R(theta) diag(s1^-2, s2^-2) R(theta)^T, so that
 * ||x - p||_G = sqrt(a^2 + b^2), a = ((x-p).u) / s1, b = ((x-p).v) / s2,
 * u = (cos, sin), v = (-sin, cos).  float32, one rounding per operation, in
 * exactly this order. */
static float score_at(const float *d, float px, float py)
{
    float dx = px - d[0];
    float dy = py - d[1];
    float a = (dx * d[4] + dy * d[5]) * d[6];
    float b = (dy * d[4] - dx * d[5]) * d[7];
    float q = a * a + b * b;
    float dist = sqrtf(q) - d[3];
    return -(d[2] * dist);
}

/* A site id names a usable site when it is in range and the site is active
 * (Appendix B.2: x < 0 marks an inactive site, skipped by every kernel). */
static int site_usable(const float *derived, int32_t n, uint32_t id)
{
    return id < (uint32_t)n && derived[(size_t)id * REC] >= 0.0f;
}

float sadref_score(const float *derived, int32_t n, uint32_t id, float px, float py)
{
    if (!site_usable(derived, n, id)) return NAN;
    return score_at(derived + (size_t)id * REC, px, py);
}

/* ------------------------------------------------------------------------ */
/* Ranking: (l1, i1) comes before (l2, i2) iff l1 > l2, or l1 == l2 and
 * i1 < i2.  Candidates whose score is NaN are dropped. */
typedef struct { float s; uint32_t id; } cand_t;

static int cand_cmp(const void *pa, const void *pb)
{
    const cand_t *a = (const cand_t *)pa, *b = (const cand_t *)pb;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    if (a->id < b->id) return -1;
    if (a->id > b->id) return 1;
    return 0;
}

/* topK of a candidate multiset: sort, drop repeated ids (a repeated id has the
 * same score, so repeats sit next to each other), keep the first K, pad. */
static void topk_of(cand_t *c, int nc, uint32_t *out)
{
    qsort(c, (size_t)nc, sizeof(cand_t), cand_cmp);
    int m = 0;
    for (int i = 0; i < nc && m < K; ++i) {
        if (m > 0 && out[m - 1] == c[i].id) continue;
        out[m++] = c[i].id;
    }
    for (; m < K; ++m) out[m] = NONE;
}

/* Add id to the candidate array if usable and its score is a number. */
static int add_cand(cand_t *c, int nc, const float *derived, int32_t n, uint32_t id, float px, float py)
{
    if (!site_usable(derived, n, id)) return nc;
    float s = score_at(derived + (size_t)id * REC, px, py);
    if (isnan(s)) return nc;
    c[nc].s = s;
    c[nc].id = id;
    return nc + 1;
}

/* Exact top-K over every site: the quantity the propagation approximates
 * (Sec. 4.3, "approximate K-th order diagram query"). */
void sadref_brute_topk(const float *derived, int32_t n, int32_t h, int32_t w, uint32_t *topk)
{
#pragma omp parallel
    {
        cand_t *c = (cand_t *)malloc(sizeof(cand_t) * (size_t)(n > 0 ? n : 1));
#pragma omp for schedule(dynamic, 4)
        for (int32_t j = 0; j < h; ++j) {
            for (int32_t i = 0; i < w; ++i) {
                float px = (float)i + 0.5f, py = (float)j + 0.5f;
                int nc = 0;
                for (int32_t s = 0; s < n; ++s) nc = add_cand(c, nc, derived, n, (uint32_t)s, px, py);
                topk_of(c, nc, topk + ((size_t)j * w + i) * K);
            }
        }
        free(c);
    }
}

/* The same exact top-K at chosen pixels only (flat indices j * w + i). */
void sadref_brute_topk_pixels(const float *derived, int32_t n, int32_t h, int32_t w, const int64_t *pix,
                              int64_t npix, uint32_t *out)
{
    (void)h;
#pragma omp parallel
    {
        cand_t *c = (cand_t *)malloc(sizeof(cand_t) * (size_t)(n > 0 ? n : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < npix; ++t) {
            int32_t i = (int32_t)(pix[t] % w), j = (int32_t)(pix[t] / w);
            float px = (float)i + 0.5f, py = (float)j + 0.5f;
            int nc = 0;
            for (int32_t s = 0; s < n; ++s) nc = add_cand(c, nc, derived, n, (uint32_t)s, px, py);
            topk_of(c, nc, out + (size_t)t * K);
        }
        free(c);
    }
}

/* ------------------------------------------------------------------------ */
/* Stochastic injection (Sec. 4.3, global probe set G_t): J site ids per pass
 * per 8x8 pixel tile, the same ids for every pixel of the tile.  The ids come
 * from SplitMix64 (Steele, Lea and Flood, OOPSLA 2014) used as a
 * counter-based generator: the output for counter c is the SplitMix64 mix of
 * seed + (c + 1) * golden-gamma, with c = pass << 32 | tile << 6 | j.  A
 * 64-bit output z maps to [0, n) by Lemire's multiply-shift on its high word. */
#define TILE 8

uint64_t sadref_splitmix64(uint64_t seed, uint64_t counter)
{
    uint64_t z = seed + (counter + 1u) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

uint32_t sadref_inject_id(uint64_t seed, uint32_t pass_index, uint32_t tile, uint32_t j, int32_t n)
{
    uint64_t ctr = ((uint64_t)pass_index << 32) | ((uint64_t)tile << 6) | (uint64_t)j;
    uint64_t z = sadref_splitmix64(seed, ctr);
    return (uint32_t)(((z >> 32) * (uint64_t)(uint32_t)n) >> 32);
}

/* One propagation pass for one pixel (Sec. 4.3, eq. for C~_t and Figure 5):
 * candidates = previous list of the pixel (temporal reuse) + previous lists of
 * the 4 pixels at +-stride along each axis that lie inside the image (spatial
 * propagation, read from the previous map only) + the tile's injected ids
 * (global probe); the new list is the top-K of that set under the logit. */
static void propagate_pixel(const float *derived, int32_t n, int32_t h, int32_t w,
                            const uint32_t *prev, int32_t i, int32_t j, int32_t stride,
                            uint64_t seed, uint32_t pass_index, int32_t inject,
                            cand_t *c, uint32_t *out)
{
    float px = (float)i + 0.5f, py = (float)j + 0.5f;
    int nc = 0;
    if (prev) {
        const int32_t nbr[5][2] = {{0, 0}, {stride, 0}, {-stride, 0}, {0, stride}, {0, -stride}};
        for (int q = 0; q < 5; ++q) {
            int32_t ii = i + nbr[q][0], jj = j + nbr[q][1];
            if (ii < 0 || ii >= w || jj < 0 || jj >= h) continue;
            const uint32_t *l = prev + ((size_t)jj * w + ii) * K;
            for (int k = 0; k < K; ++k) nc = add_cand(c, nc, derived, n, l[k], px, py);
        }
    }
    int32_t tiles_x = (w + TILE - 1) / TILE;
    uint32_t tile = (uint32_t)((j / TILE) * tiles_x + (i / TILE));
    for (int32_t q = 0; q < inject; ++q)
        nc = add_cand(c, nc, derived, n, sadref_inject_id(seed, pass_index, tile, (uint32_t)q, n), px, py);
    topk_of(c, nc, out);
}

void sadref_propagate(const float *derived, int32_t n, int32_t h, int32_t w, const uint32_t *prev,
                      uint32_t *next, int32_t stride, uint64_t seed, uint32_t pass_index, int32_t inject)
{
#pragma omp parallel
    {
        cand_t c[5 * K + 64];
#pragma omp for schedule(static)
        for (int32_t j = 0; j < h; ++j)
            for (int32_t i = 0; i < w; ++i)
                propagate_pixel(derived, n, h, w, prev, i, j, stride, seed, pass_index, inject, c,
                                next + ((size_t)j * w + i) * K);
    }
}

/* The same pass evaluated only at the listed pixels (index j*w + i). */
void sadref_propagate_pixels(const float *derived, int32_t n, int32_t h, int32_t w, const uint32_t *prev,
                             int32_t stride, uint64_t seed, uint32_t pass_index, int32_t inject,
                             const int64_t *pix, int64_t npix, uint32_t *out)
{
    cand_t c[5 * K + 64];
    for (int64_t t = 0; t < npix; ++t)
        propagate_pixel(derived, n, h, w, prev, (int32_t)(pix[t] % w), (int32_t)(pix[t] / w), stride,
                        seed, pass_index, inject, c, out + (size_t)t * K);
}

/* ------------------------------------------------------------------------ */
/* JFA prepass of a full refresh (Appendix B.3, "JFA prepass"; the render
 * protocol of Sec. 6.6 runs one JFA round before 16 propagation passes),
 * after the jump flooding of Rong and Tan (2006).  The prepass keeps JFA_K = 4
 * ids per pixel, ranked at the pixel centre like the top-K lists.
 *
 * Seed: a usable site whose logit at the centre of the pixel holding its
 * position (floor, clamped to the image) is a number claims that pixel; of
 * several sites on one pixel the one ranking first there stays.
 * jfa [h][w][4]: the seed id or NONE in slot 0, NONE in slots 1..3. */
#define JFA_K 4

void sadref_jfa_seed(const float *derived, int32_t n, int32_t h, int32_t w, uint32_t *jfa)
{
    size_t pix = (size_t)h * w;
    for (size_t p = 0; p < pix * JFA_K; ++p) jfa[p] = NONE;
    if (pix == 0) return;
    float *best = (float *)malloc(sizeof(float) * pix);
    for (int32_t i = 0; i < n; ++i) {
        if (!site_usable(derived, n, (uint32_t)i)) continue;
        const float *d = derived + (size_t)i * REC;
        int32_t ci = (int32_t)fminf(fmaxf(floorf(d[0]), 0.0f), (float)(w - 1));
        int32_t cj = (int32_t)fminf(fmaxf(floorf(d[1]), 0.0f), (float)(h - 1));
        if (!(d[1] == d[1])) cj = 0;  /* a NaN y: the first row (its logit is NaN anyway) */
        size_t p = (size_t)cj * w + ci;
        float s = score_at(d, (float)ci + 0.5f, (float)cj + 0.5f);
        if (isnan(s)) continue;
        uint32_t cur = jfa[p * JFA_K];
        if (cur == NONE || s > best[p] || (s == best[p] && (uint32_t)i < cur)) {
            jfa[p * JFA_K] = (uint32_t)i;
            best[p] = s;
        }
    }
    free(best);
}

/* Flood pass with jump step `step`: every pixel keeps the JFA_K best distinct
 * usable ids among the 4-lists of the pixels at (i + a step, j + b step),
 * a, b in {-1, 0, 1}, that lie inside the image (its own list included),
 * ranked at its own centre.  out_width 4 writes [h][w][4]; out_width 8 writes
 * a top-K map [h][w][8] with slots 4..7 NONE (the start of the propagation
 * passes). */
void sadref_jfa_flood(const float *derived, int32_t n, int32_t h, int32_t w, const uint32_t *prev, uint32_t *next,
                      int32_t step, int32_t out_width)
{
#pragma omp parallel for schedule(static)
    for (int32_t j = 0; j < h; ++j) {
        cand_t c[9 * JFA_K];
        uint32_t top[K];
        for (int32_t i = 0; i < w; ++i) {
            float px = (float)i + 0.5f, py = (float)j + 0.5f;
            int nc = 0;
            for (int b = -1; b <= 1; ++b) {
                for (int a = -1; a <= 1; ++a) {
                    int64_t ii = (int64_t)i + (int64_t)a * step, jj = (int64_t)j + (int64_t)b * step;
                    if (ii < 0 || ii >= w || jj < 0 || jj >= h) continue;
                    const uint32_t *l = prev + ((size_t)jj * w + (size_t)ii) * JFA_K;
                    for (int k = 0; k < JFA_K; ++k) nc = add_cand(c, nc, derived, n, l[k], px, py);
                }
            }
            topk_of(c, nc, top);  /* sorted, distinct: its first JFA_K entries are the JFA_K best */
            uint32_t *o = next + ((size_t)j * w + i) * (size_t)out_width;
            for (int k = 0; k < out_width; ++k) o[k] = k < JFA_K ? top[k] : NONE;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Soft additively weighted rendering (Sec. 4.2): softmax of the logits over
 * the pixel's list, then the weighted colour blend.  Entries that name no
 * usable site or whose float32 logit is not finite are skipped; an empty list
 * renders black.  The max logit is subtracted before exponentiation
 * (Appendix B.4). */
typedef struct {
    int n;
    uint32_t id[K];
    float l[K];       /* float32 logit, as ranked */
    double w[K];      /* softmax weight */
    double c[3];      /* blended colour */
} pix_eval_t;

static void eval_point(const float *derived, int32_t n, const uint32_t *list, float px, float py, pix_eval_t *e)
{
    e->n = 0;
    for (int k = 0; k < K; ++k) {
        uint32_t id = list[k];
        if (!site_usable(derived, n, id)) continue;
        float l = score_at(derived + (size_t)id * REC, px, py);
        if (!isfinite(l)) continue;
        e->id[e->n] = id;
        e->l[e->n] = l;
        e->n++;
    }
    e->c[0] = e->c[1] = e->c[2] = 0.0;
    if (e->n == 0) return;
    double m = -INFINITY;
    for (int k = 0; k < e->n; ++k) m = fmax(m, (double)e->l[k]);
    double z = 0.0;
    for (int k = 0; k < e->n; ++k) {
        e->w[k] = exp((double)e->l[k] - m);
        z += e->w[k];
    }
    for (int k = 0; k < e->n; ++k) {
        e->w[k] /= z;
        const float *d = derived + (size_t)e->id[k] * REC;
        for (int ch = 0; ch < 3; ++ch) e->c[ch] += e->w[k] * (double)d[8 + ch];
    }
}

void sadref_render_fwd(const float *derived, int32_t n, int32_t h, int32_t w, const uint32_t *topk, double *image)
{
#pragma omp parallel for schedule(static)
    for (int32_t j = 0; j < h; ++j) {
        for (int32_t i = 0; i < w; ++i) {
            pix_eval_t e;
            size_t p = (size_t)j * w + i;
            eval_point(derived, n, topk + p * K, (float)i + 0.5f, (float)j + 0.5f, &e);
            for (int ch = 0; ch < 3; ++ch) image[p * 3 + ch] = e.c[ch];
        }
    }
}

/* Random access (Sec. 6.6, render-only from cached lists): a point (qx, qy)
 * uses the list of the pixel that contains it, clamped into the image, and
 * the logits are evaluated at the point itself.  Non-finite points give NaN. */
void sadref_query_points(const float *derived, int32_t n, int32_t h, int32_t w, const uint32_t *topk,
                         const float *xy, int64_t m, double *rgb)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < m; ++t) {
        float qx = xy[2 * t], qy = xy[2 * t + 1];
        if (!isfinite(qx) || !isfinite(qy)) {
            rgb[3 * t] = rgb[3 * t + 1] = rgb[3 * t + 2] = NAN;
            continue;
        }
        double fx = floor((double)qx), fy = floor((double)qy);
        int32_t i = fx < 0 ? 0 : (fx > (double)(w - 1) ? w - 1 : (int32_t)fx);
        int32_t j = fy < 0 ? 0 : (fy > (double)(h - 1) ? h - 1 : (int32_t)fy);
        pix_eval_t e;
        eval_point(derived, n, topk + ((size_t)j * w + i) * K, qx, qy, &e);
        for (int ch = 0; ch < 3; ++ch) rgb[3 * t + ch] = e.c[ch];
    }
}

/* ------------------------------------------------------------------------ */
/* Loss and hand-derived gradients (Sec. 6.1 loss, Appendix B.4).
 * L = sum_x sum_ch (c(x) - I(x))^2 / P, P = H*W (the per-pixel normalisation
 * of Appendix B.4).  With g = dL/dc(x) = 2 (c - I) / P and, for list entry k
 * (site i), delta_k = dL/dl_k = w_k (g.c_i - g.c):
 *   colour  += w_k g
 *   log tau += delta_k l_k        (dl/dlog tau = l)
 *   r       += tau delta_k        (dl/dr = tau)
 *   with kappa = -tau delta_k / (2 sqrt q) when q > 0:
 *   x       += kappa * (-2) (a is1 cos - b is2 sin)
 *   y       += kappa * (-2) (a is1 sin + b is2 cos)
 *   theta   += kappa * 2 a_r b_r (is1^2 - is2^2)
 *   log s1  += kappa * (-2 a^2),  log s2 += kappa * (-2 b^2)
 * where a_r = dx cos + dy sin, b_r = dy cos - dx sin, a = a_r is1, b = b_r is2.
 * At q == 0 (pixel centre on the site) the position and metric terms are 0.
 * Everything is float64; sums run in pixel order then list order.
 * grad and grad_mag ([n][12], parameter-record layout) are accumulated into.
 * grad_mag receives, for every term, the same expression evaluated with the
 * absolute value of each input and of each intermediate sum or difference
 * (g uses |c| + |target|, delta uses |g|.|c_i| + |g|.|c|, a_r uses
 * |dx cos| + |dy sin|, and so on).  This is the classical running bound on
 * the rounding error of any evaluation of the expression in a lower
 * precision: an evaluation with unit roundoff u and m operations is off by
 * at most about m u times this magnitude, whatever cancellation occurs. */
void sadref_render_bwd(const float *derived, int32_t n, int32_t h, int32_t w, const uint32_t *topk,
                       const float *target, double *grad, double *grad_mag, double *loss, double *image)
{
    const double inv_p = 1.0 / ((double)h * (double)w);
    double lsum = 0.0;
    for (int32_t j = 0; j < h; ++j) {
        for (int32_t i = 0; i < w; ++i) {
            size_t p = (size_t)j * w + i;
            float px = (float)i + 0.5f, py = (float)j + 0.5f;
            pix_eval_t e;
            eval_point(derived, n, topk + p * K, px, py, &e);
            double g[3], gm[3];
            for (int ch = 0; ch < 3; ++ch) {
                double r = e.c[ch] - (double)target[p * 3 + ch];
                lsum += r * r;
                g[ch] = 2.0 * r * inv_p;
                gm[ch] = 2.0 * (fabs(e.c[ch]) + fabs((double)target[p * 3 + ch])) * inv_p;
                if (image) image[p * 3 + ch] = e.c[ch];
            }
            double gc = g[0] * e.c[0] + g[1] * e.c[1] + g[2] * e.c[2];
            double gcm = gm[0] * fabs(e.c[0]) + gm[1] * fabs(e.c[1]) + gm[2] * fabs(e.c[2]);
            for (int k = 0; k < e.n; ++k) {
                const float *d = derived + (size_t)e.id[k] * REC;
                double tau = d[2], cs = d[4], sn = d[5], is1 = d[6], is2 = d[7];
                double gci = g[0] * d[8] + g[1] * d[9] + g[2] * d[10];
                double gcim = gm[0] * fabs((double)d[8]) + gm[1] * fabs((double)d[9]) + gm[2] * fabs((double)d[10]);
                double delta = e.w[k] * (gci - gc);
                double deltam = e.w[k] * (gcim + gcm);
                double t[12] = {0}, tm[12] = {0};
                for (int ch = 0; ch < 3; ++ch) {
                    t[4 + ch] = e.w[k] * g[ch];
                    tm[4 + ch] = e.w[k] * gm[ch];
                }
                t[2] = delta * (double)e.l[k];
                tm[2] = deltam * fabs((double)e.l[k]);
                t[3] = tau * delta;
                tm[3] = tau * deltam;
                double dx = (double)px - (double)d[0], dy = (double)py - (double)d[1];
                double ar = dx * cs + dy * sn, br = dy * cs - dx * sn;
                double arm = fabs(dx * cs) + fabs(dy * sn), brm = fabs(dy * cs) + fabs(dx * sn);
                double a = ar * is1, b = br * is2;
                double q = a * a + b * b;
                if (q > 0.0) {
                    double kappa = -tau * delta / (2.0 * sqrt(q));
                    double kappam = tau * deltam / (2.0 * sqrt(q));
                    double am = arm * is1, bm = brm * is2;
                    t[0] = kappa * -2.0 * (a * is1 * cs - b * is2 * sn);
                    t[1] = kappa * -2.0 * (a * is1 * sn + b * is2 * cs);
                    t[7] = kappa * 2.0 * ar * br * (is1 * is1 - is2 * is2);
                    t[8] = kappa * -2.0 * a * a;
                    t[9] = kappa * -2.0 * b * b;
                    tm[0] = kappam * 2.0 * (am * is1 * fabs(cs) + bm * is2 * fabs(sn));
                    tm[1] = kappam * 2.0 * (am * is1 * fabs(sn) + bm * is2 * fabs(cs));
                    tm[7] = kappam * 2.0 * arm * brm * (is1 * is1 + is2 * is2);
                    tm[8] = kappam * 2.0 * am * am;
                    tm[9] = kappam * 2.0 * bm * bm;
                }
                double *G = grad + (size_t)e.id[k] * REC;
                double *A = grad_mag ? grad_mag + (size_t)e.id[k] * REC : NULL;
                for (int q2 = 0; q2 < 10; ++q2) {
                    G[q2] += t[q2];
                    if (A) A[q2] += tm[q2];
                }
            }
        }
    }
    if (loss) *loss += lsum * inv_p;
}

/* ------------------------------------------------------------------------ */
/* Budget statistics (Sec. 4.5, "Adaptive Budget: Densify and Prune", and
 * Appendix B.5, "Densification scores" and "Pruning").  For every site, over
 * the pixels whose usable entries include it, with the softmax weight w, the
 * rendered colour c and the target I of the pixel:
 *   [0] mass           sum w
 *   [1] energy         sum w |c - I|^2
 *   [2] removal delta  sum (|c' - I|^2 - |c - I|^2), where c' is the blend of
 *                      the pixel's other usable entries with their weights
 *                      renormalised (Sec. 4.5 writes it as (c - w c_k)/(1 - w)),
 *                      or black when the site is the pixel's only entry
 *   [3] sum w dx   [4] sum w dy   [5] sum w dx^2   [6] sum w dx dy   [7] sum w dy^2
 *                      with (dx, dy) = pixel centre - site position: the
 *                      weighted second moments of Appendix B.5 taken about the
 *                      site (their zeroth moment is the mass)
 * stats [n][8] and stats_mag [n][8] (sums of the absolute values of the same
 * terms, or NULL) are accumulated into (+=). */
void sadref_site_stats(const float *derived, int32_t n, int32_t h, int32_t w, const uint32_t *topk,
                       const float *target, double *stats, double *stats_mag)
{
    for (int32_t j = 0; j < h; ++j) {
        for (int32_t i = 0; i < w; ++i) {
            size_t p = (size_t)j * w + i;
            float px = (float)i + 0.5f, py = (float)j + 0.5f;
            pix_eval_t e;
            eval_point(derived, n, topk + p * K, px, py, &e);
            const float *I = target + p * 3;
            double err = 0.0;
            for (int ch = 0; ch < 3; ++ch) err += (e.c[ch] - I[ch]) * (e.c[ch] - I[ch]);
            for (int k = 0; k < e.n; ++k) {
                /* the blend without entry k, its weights taken from the logits
                 * relative to the largest remaining one */
                double m = -INFINITY, z = 0.0, cp[3] = {0.0, 0.0, 0.0};
                for (int q = 0; q < e.n; ++q)
                    if (q != k) m = fmax(m, (double)e.l[q]);
                for (int q = 0; q < e.n; ++q) {
                    if (q == k) continue;
                    const float *dq = derived + (size_t)e.id[q] * REC;
                    double eq = exp((double)e.l[q] - m);
                    z += eq;
                    for (int ch = 0; ch < 3; ++ch) cp[ch] += eq * (double)dq[8 + ch];
                }
                double err2 = 0.0;
                for (int ch = 0; ch < 3; ++ch) {
                    if (z > 0.0) cp[ch] /= z;
                    err2 += (cp[ch] - I[ch]) * (cp[ch] - I[ch]);
                }
                const float *d = derived + (size_t)e.id[k] * REC;
                double wk = e.w[k];
                double dx = (double)px - (double)d[0], dy = (double)py - (double)d[1];
                double t[8] = {wk, wk * err, err2 - err, wk * dx, wk * dy, wk * dx * dx, wk * dx * dy, wk * dy * dy};
                double *S = stats + (size_t)e.id[k] * 8;
                for (int q2 = 0; q2 < 8; ++q2) S[q2] += t[q2];
                if (stats_mag) {
                    /* the removal delta is a difference: its scale is the sum of the two errors */
                    double *A = stats_mag + (size_t)e.id[k] * 8;
                    for (int q2 = 0; q2 < 8; ++q2) A[q2] += q2 == 2 ? err2 + err : fabs(t[q2]);
                }
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Budget control: densify and prune (Sec. 4.5; Appendix B.5 "Densification
 * scores", "Split kernel", "Pruning").  Inputs: the sites, their Adam
 * moments and prepared records, the statistics of sadref_site_stats (as
 * float32) and the target.  The pages leave the amounts open; they are
 * arguments here.
 *  1. Prune: the n_prune active sites with the lowest removal delta (a NaN
 *     delta ranks last; ties: lower id first) are switched off, position
 *     (-1, -1).
 *  2. Split candidates: sites still active with mass >= min_mass and mass > 0,
 *     ranked by the densification score energy / mass^alpha (in double;
 *     ties: lower id first; a NaN score is not a candidate).
 *  3. The i-th candidate is split into the i-th inactive slot (ascending index)
 *     while both last and i < n_split.  Axis: the principal eigenvector of the
 *     weighted covariance about the site (from the moments), sigma the square
 *     root of its eigenvalue; when that is degenerate, the direction of the
 *     Sobel gradient of the target (channels summed) at the site's pixel, or
 *     (1, 0) when that is zero, with sigma the site's larger scale.  The two
 *     children sit at position +- offset sigma axis (the parent's slot takes
 *     +, clamped to the image), take the target colour of their pixels,
 *     log tau - logtau_shift and r * r_scale, and keep theta and the scales;
 *     both get zero Adam moments.
 *  4. The prepared records of every touched site are rewritten.
 * All geometry in float32, one rounding per operation in the written order.
 * done[0] = sites pruned, done[1] = sites split. */
typedef struct { double key; uint32_t id; } rank_t;

static int rank_asc(const void *pa, const void *pb)
{
    const rank_t *a = (const rank_t *)pa, *b = (const rank_t *)pb;
    if (a->key < b->key) return -1;
    if (a->key > b->key) return 1;
    return a->id < b->id ? -1 : (a->id > b->id);
}

static float target_sum(const float *target, int32_t h, int32_t w, int32_t i, int32_t j)
{
    i = i < 0 ? 0 : (i >= w ? w - 1 : i);
    j = j < 0 ? 0 : (j >= h ? h - 1 : j);
    const float *t = target + ((size_t)j * w + i) * 3;
    return (t[0] + t[1]) + t[2];
}

static int32_t cell_of(float v, int32_t size)
{
    return (int32_t)fminf(fmaxf(floorf(v), 0.0f), (float)(size - 1));
}

void sadref_densify_prune(float *params, float *m, float *v, float *derived, int32_t n, int32_t h, int32_t w,
                          const float *stats, const float *target, int32_t n_split, int32_t n_prune, float alpha,
                          float min_mass, float offset, float r_scale, float logtau_shift, int32_t *done)
{
    rank_t *r = (rank_t *)malloc(sizeof(rank_t) * (size_t)(n > 0 ? n : 1));
    uint32_t *slots = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)(n > 0 ? n : 1));
    int32_t nr = 0, pruned = 0, split = 0;
    /* 1. prune */
    for (int32_t i = 0; i < n; ++i) {
        if (!(params[(size_t)i * REC] >= 0.0f)) continue;
        float dl = stats[(size_t)i * 8 + 2];
        r[nr].key = isnan(dl) ? INFINITY : (double)dl;
        r[nr].id = (uint32_t)i;
        nr++;
    }
    qsort(r, (size_t)nr, sizeof(rank_t), rank_asc);
    for (int32_t k = 0; k < nr && k < n_prune; ++k) {
        float *p = params + (size_t)r[k].id * REC;
        p[0] = -1.0f;
        p[1] = -1.0f;
        sadref_prepare_sites(p, 1, derived + (size_t)r[k].id * REC);
        pruned++;
    }
    /* 2. candidates, best first (the key is the negated score) */
    nr = 0;
    for (int32_t i = 0; i < n; ++i) {
        const float *st = stats + (size_t)i * 8;
        if (!(params[(size_t)i * REC] >= 0.0f) || !(st[0] >= min_mass) || !(st[0] > 0.0f)) continue;
        double score = (double)st[1] / pow((double)st[0], (double)alpha);
        if (isnan(score)) continue;
        r[nr].key = -score;
        r[nr].id = (uint32_t)i;
        nr++;
    }
    qsort(r, (size_t)nr, sizeof(rank_t), rank_asc);
    /* 3. free slots, ascending */
    int32_t nf = 0;
    for (int32_t i = 0; i < n; ++i)
        if (!(params[(size_t)i * REC] >= 0.0f)) slots[nf++] = (uint32_t)i;
    for (int32_t k = 0; k < nr && k < nf && k < n_split; ++k) {
        uint32_t pi = r[k].id, ci = slots[k];
        float *pp = params + (size_t)pi * REC, *pc = params + (size_t)ci * REC;
        const float *st = stats + (size_t)pi * 8;
        const float *d = derived + (size_t)pi * REC;
        /* axis from the covariance about the site */
        float ms = st[0];
        float mx = st[3] / ms, my = st[4] / ms;
        float a = st[5] / ms - mx * mx, b = st[6] / ms - mx * my, c = st[7] / ms - my * my;
        float half = (a - c) * 0.5f;
        float lam = (a + c) * 0.5f + sqrtf(half * half + b * b);
        float e1x = b, e1y = lam - a, e2x = lam - c, e2y = b;
        float n1 = e1x * e1x + e1y * e1y, n2 = e2x * e2x + e2y * e2y;
        float ex = n1 >= n2 ? e1x : e2x, ey = n1 >= n2 ? e1y : e2y, nn = n1 >= n2 ? n1 : n2;
        float ux, uy, sigma;
        if (lam > 0.0f && nn > 0.0f && isfinite(lam) && isfinite(nn)) {
            float len = sqrtf(nn);
            ux = ex / len;
            uy = ey / len;
            sigma = sqrtf(lam);
        } else {
            int32_t i0 = cell_of(d[0], w), j0 = cell_of(d[1], h);
            float gx = (target_sum(target, h, w, i0 + 1, j0 - 1) + 2.0f * target_sum(target, h, w, i0 + 1, j0) +
                        target_sum(target, h, w, i0 + 1, j0 + 1)) -
                       (target_sum(target, h, w, i0 - 1, j0 - 1) + 2.0f * target_sum(target, h, w, i0 - 1, j0) +
                        target_sum(target, h, w, i0 - 1, j0 + 1));
            float gy = (target_sum(target, h, w, i0 - 1, j0 + 1) + 2.0f * target_sum(target, h, w, i0, j0 + 1) +
                        target_sum(target, h, w, i0 + 1, j0 + 1)) -
                       (target_sum(target, h, w, i0 - 1, j0 - 1) + 2.0f * target_sum(target, h, w, i0, j0 - 1) +
                        target_sum(target, h, w, i0 + 1, j0 - 1));
            float gl = sqrtf(gx * gx + gy * gy);
            ux = gl > 0.0f ? gx / gl : 1.0f;
            uy = gl > 0.0f ? gy / gl : 0.0f;
            sigma = 1.0f / fminf(d[6], d[7]);
        }
        float dx = (offset * sigma) * ux, dy = (offset * sigma) * uy;
        float x = pp[0], y = pp[1];
        float pos[2][2] = {{fminf(fmaxf(x + dx, 0.0f), (float)w), fminf(fmaxf(y + dy, 0.0f), (float)h)},
                           {fminf(fmaxf(x - dx, 0.0f), (float)w), fminf(fmaxf(y - dy, 0.0f), (float)h)}};
        float base[REC];
        for (int q = 0; q < REC; ++q) base[q] = pp[q];
        for (int ch = 0; ch < 2; ++ch) {
            float *o = ch == 0 ? pp : pc;
            uint32_t oi = ch == 0 ? pi : ci;
            for (int q = 0; q < REC; ++q) o[q] = base[q];
            o[0] = pos[ch][0];
            o[1] = pos[ch][1];
            const float *t = target + ((size_t)cell_of(pos[ch][1], h) * w + cell_of(pos[ch][0], w)) * 3;
            o[4] = t[0];
            o[5] = t[1];
            o[6] = t[2];
            o[2] = base[2] - logtau_shift;
            o[3] = base[3] * r_scale;
            for (int q = 0; q < REC; ++q) {
                m[(size_t)oi * REC + q] = 0.0f;
                v[(size_t)oi * REC + q] = 0.0f;
            }
        }
        sadref_prepare_sites(pp, 1, derived + (size_t)pi * REC);
        sadref_prepare_sites(pc, 1, derived + (size_t)ci * REC);
        split++;
    }
    done[0] = pruned;
    done[1] = split;
    free(r);
    free(slots);
}

/* ------------------------------------------------------------------------ */
/* Packed evaluation records (Appendix B.2, "Packed storage for evaluation"):
 * four 32-bit words per site,
 *   w0: x and y as 15-bit UNORM of x / W and y / H (bits 0-14, 15-29), bit 31
 *       set for a usable site (a site that is not usable packs to 0, 0, 0, 0),
 *   w1: colour r, g, b as 11/11/10-bit UNORM over the image's range per channel,
 *   w2: log tau' and r' as 16/16-bit UNORM over the image's ranges,
 *   w3: the direction as a 16-bit UNORM angle code over [-pi, pi] (low half)
 *       and the log-anisotropy a as float16 (high half).
 * The pages' metric has determinant 1 (eigenvalues e^a, e^-a along the
 * direction and across it).  The metric diag(s1^-2, s2^-2) in the rotated
 * frame is that one scaled by 1 / (s1 s2), and a scale of the distance is
 * absorbed by tau and r:
 *   a = log s2 - log s1,  hs = (log s1 + log s2) / 2,
 *   log tau' = log tau - hs,  r' = r exp(hs),
 * giving the same logit -tau' (sqrt(e^a u^2 + e^-a v^2) - r') with
 * (u, v) the offset in the rotated frame.
 * Per-image parameters qp[10] = (min, max - min) of log tau', r', c_r, c_g,
 * c_b over the usable sites (NaN values ignored, -0 taken as +0; no values:
 * 0, 0).
 * Codes: q = rint(clamp(t, 0, 1) * (2^bits - 1)), t = (v - min) / scale
 * (0 when scale is not positive), NaN t gives 0.  Arithmetic is float32 in
 * the order written; exp is the correctly rounded float32 exponential; the
 * angle is wrapped as theta - 2 pi_f rint(theta / (2 pi)_f) and coded from
 * (wrapped + pi_f) / (2 pi)_f; float16 rounding is to nearest even. */
#define TWO_PI_F 6.28318548f
#define INV_TWO_PI_F 0.159154937f
#define PI_F 3.14159274f
#define SADREF_PI 3.14159265358979323846

static uint32_t unorm_code(float t, uint32_t maxq)
{
    t = fminf(fmaxf(t, 0.0f), 1.0f); /* NaN becomes 0 */
    return (uint32_t)rintf(t * (float)maxq);
}

uint32_t sadref_half_bits(float f)
{
    uint32_t sign = signbit(f) ? 0x8000u : 0u;
    double a = fabs((double)f);
    if (isnan(f)) return 0x7E00u;
    if (a >= 65520.0) return sign | 0x7C00u; /* rounds to infinity */
    if (a < 0x1p-14) return sign | (uint32_t)nearbyint(a * 0x1p24); /* steps of 2^-24; 1024 = smallest normal */
    int e;
    frexp(a, &e); /* a in [2^(e-1), 2^e) */
    double ulp = ldexp(1.0, e - 11);
    double r = nearbyint(a / ulp) * ulp;
    frexp(r, &e);
    double mant = r / ldexp(1.0, e - 1) - 1.0;
    return sign | (uint32_t)((e - 1 + 15) << 10) | (uint32_t)nearbyint(mant * 1024.0);
}

double sadref_half_value(uint32_t hb)
{
    double sg = (hb & 0x8000u) ? -1.0 : 1.0;
    uint32_t e = (hb >> 10) & 31u, m = hb & 1023u;
    if (e == 0) return sg * ldexp((double)m, -24);
    if (e == 31) return m ? NAN : sg * INFINITY;
    return sg * ldexp((double)(1024u + m), (int)e - 25);
}

static void packed_values(const float *p, float v[5])
{
    float hs = 0.5f * (p[8] + p[9]);
    v[0] = p[2] - hs;
    v[1] = p[3] * sadref_exp_f32(hs);
    v[2] = p[4];
    v[3] = p[5];
    v[4] = p[6];
}

void sadref_pack_sites(const float *params, const float *derived, int32_t n, int32_t h, int32_t w, uint32_t *packed,
                       float *qp)
{
    float lo[5], hi[5];
    for (int k = 0; k < 5; ++k) {
        lo[k] = INFINITY;
        hi[k] = -INFINITY;
    }
    for (int32_t i = 0; i < n; ++i) {
        if (!site_usable(derived, n, (uint32_t)i)) continue;
        float v[5];
        packed_values(params + (size_t)i * REC, v);
        for (int k = 0; k < 5; ++k) {
            float x = v[k] + 0.0f; /* -0 counts as +0, so the range is unique */
            if (x < lo[k]) lo[k] = x;
            if (x > hi[k]) hi[k] = x;
        }
    }
    for (int k = 0; k < 5; ++k) {
        if (lo[k] > hi[k]) lo[k] = hi[k] = 0.0f;
        qp[2 * k] = lo[k];
        qp[2 * k + 1] = hi[k] - lo[k];
    }
    static const uint32_t maxq[5] = {65535u, 65535u, 2047u, 2047u, 1023u};
    for (int32_t i = 0; i < n; ++i) {
        uint32_t *o = packed + (size_t)i * 4;
        if (!site_usable(derived, n, (uint32_t)i)) {
            o[0] = o[1] = o[2] = o[3] = 0u;
            continue;
        }
        const float *p = params + (size_t)i * REC;
        float v[5];
        uint32_t q[5];
        packed_values(p, v);
        for (int k = 0; k < 5; ++k) {
            float sc = qp[2 * k + 1];
            q[k] = unorm_code(sc > 0.0f ? (v[k] - qp[2 * k]) / sc : 0.0f, maxq[k]);
        }
        uint32_t qx = unorm_code(p[0] / (float)w, 32767u), qy = unorm_code(p[1] / (float)h, 32767u);
        float th = p[7] - TWO_PI_F * rintf(p[7] * INV_TWO_PI_F);
        uint32_t qt = unorm_code((th + PI_F) * INV_TWO_PI_F, 65535u);
        o[0] = qx | (qy << 15) | 0x80000000u;
        o[1] = q[2] | (q[3] << 11) | (q[4] << 22);
        o[2] = q[0] | (q[1] << 16);
        o[3] = qt | (sadref_half_bits(p[9] - p[8]) << 16);
    }
}

/* The values a packed record stands for, in float64:
 * out[9] = (x, y, tau', r', c_r, c_g, c_b, theta, a); returns 0 for a record
 * without the usable bit. */
int sadref_unpack_site(const uint32_t *o, const float *qp, int32_t h, int32_t w, double *out)
{
    if (!(o[0] >> 31)) return 0;
    out[0] = (double)(o[0] & 32767u) / 32767.0 * (double)w;
    out[1] = (double)((o[0] >> 15) & 32767u) / 32767.0 * (double)h;
    out[2] = exp((double)qp[0] + (double)(o[2] & 65535u) / 65535.0 * (double)qp[1]);
    out[3] = (double)qp[2] + (double)(o[2] >> 16) / 65535.0 * (double)qp[3];
    out[4] = (double)qp[4] + (double)(o[1] & 2047u) / 2047.0 * (double)qp[5];
    out[5] = (double)qp[6] + (double)((o[1] >> 11) & 2047u) / 2047.0 * (double)qp[7];
    out[6] = (double)qp[8] + (double)(o[1] >> 22) / 1023.0 * (double)qp[9];
    out[7] = (double)(o[3] & 65535u) / 65535.0 * (2.0 * SADREF_PI) - SADREF_PI;
    out[8] = sadref_half_value(o[3] >> 16);
    return 1;
}

void sadref_unpack_sites(const uint32_t *packed, const float *qp, int32_t n, int32_t h, int32_t w, double *out,
                         int32_t *usable)
{
    for (int32_t i = 0; i < n; ++i) usable[i] = sadref_unpack_site(packed + (size_t)i * 4, qp, h, w, out + (size_t)i * 9);
}

double sadref_packed_logit(const double *v, double px, double py)
{
    double dx = px - v[0], dy = py - v[1];
    double cs = cos(v[7]), sn = sin(v[7]);
    double u = cs * dx + sn * dy, t = cs * dy - sn * dx;
    return -v[2] * (sqrt(exp(v[8]) * u * u + exp(-v[8]) * t * t) - v[3]);
}

/* Random access from packed records: as sadref_query_points, with each list
 * entry's site decoded from its packed record (float64); an id >= n or a
 * record without the usable bit is skipped, as are non-finite logits. */
void sadref_query_packed(const uint32_t *packed, const float *qp, int32_t n, int32_t h, int32_t w,
                         const uint32_t *topk, const float *xy, int64_t m, double *rgb)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < m; ++t) {
        float qx = xy[2 * t], qy = xy[2 * t + 1];
        if (!isfinite(qx) || !isfinite(qy)) {
            rgb[3 * t] = rgb[3 * t + 1] = rgb[3 * t + 2] = NAN;
            continue;
        }
        double fx = floor((double)qx), fy = floor((double)qy);
        int32_t i = fx < 0 ? 0 : (fx > (double)(w - 1) ? w - 1 : (int32_t)fx);
        int32_t j = fy < 0 ? 0 : (fy > (double)(h - 1) ? h - 1 : (int32_t)fy);
        const uint32_t *list = topk + ((size_t)j * w + i) * K;
        double l[K], col[K][3], mx = -INFINITY;
        int cnt = 0;
        for (int k = 0; k < K; ++k) {
            double v[9];
            if (list[k] >= (uint32_t)n || !sadref_unpack_site(packed + (size_t)list[k] * 4, qp, h, w, v)) continue;
            double s = sadref_packed_logit(v, (double)qx, (double)qy);
            if (!isfinite(s)) continue;
            l[cnt] = s;
            for (int ch = 0; ch < 3; ++ch) col[cnt][ch] = v[4 + ch];
            mx = fmax(mx, s);
            cnt++;
        }
        double z = 0.0, c[3] = {0.0, 0.0, 0.0};
        for (int k = 0; k < cnt; ++k) {
            l[k] = exp(l[k] - mx);
            z += l[k];
        }
        for (int k = 0; k < cnt; ++k)
            for (int ch = 0; ch < 3; ++ch) c[ch] += l[k] / z * col[k][ch];
        for (int ch = 0; ch < 3; ++ch) rgb[3 * t + ch] = c[ch];
    }
}

/* ------------------------------------------------------------------------ */
/* Gradient-weighted initialisation (Sec. 4.4): sites are drawn from
 *   P_init(x) = (1 - lambda) |grad I(x)| / sum |grad I| + lambda / (H W).
 * |grad I(x)| is the 2-norm over the 3 channels and both directions of the
 * 3x3 Sobel derivatives of the target (borders clamped), in float32:
 *   gx_c = (I(i+1,j-1) + 2 I(i+1,j) + I(i+1,j+1)) - (I(i-1,j-1) + 2 I(i-1,j) + I(i-1,j+1))
 *   gy_c = (I(i-1,j+1) + 2 I(i,j+1) + I(i+1,j+1)) - (I(i-1,j-1) + 2 I(i,j-1) + I(i+1,j-1))
 *   g = sqrt(((gx_0^2 + gy_0^2) + (gx_1^2 + gy_1^2)) + (gx_2^2 + gy_2^2))
 * To draw from the mixture exactly, g is taken in integer units of 2^-24
 * (truncated, at most 2^8, so that 2^30 pixels still sum exactly in 64 bits;
 * NaN counts 0).
 * Site i uses SplitMix64 outputs z_k at counters 4 i + k:
 *   z_0: uniform part when (z_0 >> 40) 2^-24 < lambda, or when every g is 0;
 *   z_1: uniform part: pixel ((z_1 >> 32) H W) >> 32; gradient part: the
 *        first pixel (row-major) whose inclusive prefix sum exceeds
 *        t = floor(z_1 G / 2^64), G the total;
 *   z_2, z_3: the position inside the pixel, i + (z_2 >> 40) 2^-24 and
 *        j + (z_3 >> 40) 2^-24 (float32 sums).
 * The record: that position, log tau, r, the target colour of the pixel,
 * angle 0, both log scales log_scale, zero padding.  Records are prepared
 * into derived as sadref_prepare_sites. */
static float tpx(const float *t, int32_t h, int32_t w, int32_t i, int32_t j, int c)
{
    i = i < 0 ? 0 : (i >= w ? w - 1 : i);
    j = j < 0 ? 0 : (j >= h ? h - 1 : j);
    return t[((size_t)j * w + i) * 3 + c];
}

void sadref_grad_mag(const float *target, int32_t h, int32_t w, float *g)
{
    for (int32_t j = 0; j < h; ++j)
        for (int32_t i = 0; i < w; ++i) {
            float acc = 0.0f;
            for (int c = 0; c < 3; ++c) {
                float gx = (tpx(target, h, w, i + 1, j - 1, c) + 2.0f * tpx(target, h, w, i + 1, j, c) +
                            tpx(target, h, w, i + 1, j + 1, c)) -
                           (tpx(target, h, w, i - 1, j - 1, c) + 2.0f * tpx(target, h, w, i - 1, j, c) +
                            tpx(target, h, w, i - 1, j + 1, c));
                float gy = (tpx(target, h, w, i - 1, j + 1, c) + 2.0f * tpx(target, h, w, i, j + 1, c) +
                            tpx(target, h, w, i + 1, j + 1, c)) -
                           (tpx(target, h, w, i - 1, j - 1, c) + 2.0f * tpx(target, h, w, i, j - 1, c) +
                            tpx(target, h, w, i + 1, j - 1, c));
                float e = gx * gx + gy * gy;
                acc = c == 0 ? e : acc + e;
            }
            g[(size_t)j * w + i] = sqrtf(acc);
        }
}

uint64_t sadref_grad_units(float g)
{
    if (!(g == g)) return 0;
    return (uint64_t)(fminf(g, 256.0f) * 16777216.0f);
}

void sadref_init_sites(const float *target, int32_t h, int32_t w, int32_t n, float lambda, uint64_t seed,
                       float log_tau, float r, float log_scale, float *params, float *derived)
{
    size_t pix = (size_t)h * (size_t)w;
    float *g = (float *)malloc(sizeof(float) * (pix > 0 ? pix : 1));
    uint64_t *cum = (uint64_t *)malloc(sizeof(uint64_t) * (pix > 0 ? pix : 1));
    sadref_grad_mag(target, h, w, g);
    uint64_t total = 0;
    for (size_t x = 0; x < pix; ++x) {
        total += sadref_grad_units(g[x]);
        cum[x] = total;
    }
    for (int32_t s = 0; s < n; ++s) {
        uint64_t z[4];
        for (int k = 0; k < 4; ++k) z[k] = sadref_splitmix64(seed, 4u * (uint64_t)s + (uint64_t)k);
        float u0 = (float)(z[0] >> 40) * 0x1p-24f;
        size_t x;
        if (u0 < lambda || total == 0) {
            x = (size_t)(((z[1] >> 32) * (uint64_t)pix) >> 32);
        } else {
            uint64_t t = (uint64_t)(((unsigned __int128)z[1] * total) >> 64);
            size_t lo = 0, hi = pix - 1; /* first x with cum[x] > t; cum[pix-1] = total > t */
            while (lo < hi) {
                size_t mid = lo + (hi - lo) / 2;
                if (cum[mid] > t) hi = mid; else lo = mid + 1;
            }
            x = lo;
        }
        int32_t i = (int32_t)(x % (size_t)w), j = (int32_t)(x / (size_t)w);
        float *p = params + (size_t)s * REC;
        p[0] = (float)i + (float)(z[2] >> 40) * 0x1p-24f;
        p[1] = (float)j + (float)(z[3] >> 40) * 0x1p-24f;
        p[2] = log_tau;
        p[3] = r;
        for (int c = 0; c < 3; ++c) p[4 + c] = target[x * 3 + c];
        p[7] = 0.0f;
        p[8] = log_scale;
        p[9] = log_scale;
        p[10] = 0.0f;
        p[11] = 0.0f;
    }
    sadref_prepare_sites(params, n, derived);
    free(g);
    free(cum);
}

/* ------------------------------------------------------------------------ */
/* Adam (Kingma and Ba, ICLR 2015) on the float32 site buffer (Sec. 5:
 * per-parameter base learning rates, fixed betas and epsilon), then the
 * projection of Sec. 4.1 (positions clamped to the image).  lr[5] holds the
 * rates of the groups (x, y), log tau, r, colour, (theta, log s1, log s2).
 * One float32 rounding per operation, in this order:
 *   m = b1*m + (1-b1)*g;  v = b2*v + (1-b2)*(g*g)
 *   p = p - lr * ((m / bc1) / (sqrt(v / bc2) + eps))
 * bc1 = 1 - b1^t and bc2 = 1 - b2^t come from the caller.  Inactive sites
 * (x < 0) are left as they are.  The gradient record is zeroed and the
 * derived record rewritten (as sadref_prepare_sites) for every site. */
static const int lr_group[10] = {0, 0, 1, 2, 3, 3, 3, 4, 4, 4};

void sadref_adam_step(float *params, float *grad, float *m, float *v, int32_t n, int32_t h, int32_t w,
                      const float *lr, float beta1, float beta2, float eps, float bc1, float bc2, float *derived)
{
    float omb1 = 1.0f - beta1, omb2 = 1.0f - beta2;
    for (int32_t i = 0; i < n; ++i) {
        float *p = params + (size_t)i * REC;
        float *g = grad + (size_t)i * REC;
        float *mm = m + (size_t)i * REC;
        float *vv = v + (size_t)i * REC;
        if (p[0] >= 0.0f) {
            for (int k = 0; k < 10; ++k) {
                float gk = g[k];
                mm[k] = beta1 * mm[k] + omb1 * gk;
                vv[k] = beta2 * vv[k] + omb2 * (gk * gk);
                float mhat = mm[k] / bc1;
                float vhat = vv[k] / bc2;
                float step = mhat / (sqrtf(vhat) + eps);
                p[k] = p[k] - lr[lr_group[k]] * step;
            }
            p[0] = fminf(fmaxf(p[0], 0.0f), (float)w);
            p[1] = fminf(fmaxf(p[1], 0.0f), (float)h);
        }
        for (int k = 0; k < REC; ++k) g[k] = 0.0f;
        if (derived) sadref_prepare_sites(p, 1, derived + (size_t)i * REC);
    }
}
