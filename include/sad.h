/*
 * sad.h -- C ABI of libsad.so, the MI355X (gfx950) hot path of
 * Soft Anisotropic Diagrams (SAD): per-pixel top-K site lists maintained by
 * jump-flood-style propagation with stochastic injection, and the soft
 * anisotropic additively weighted (Apollonius) softmax render, its backward
 * pass and the Adam update of the sites.
 *
 * Paper: "Soft Anisotropic Diagrams for Differentiable Image Representation"
 * (Iinbor, Dou, Matusik; arXiv 2604.21984).  Section references below are to
 * that paper.
 *
 * Conventions shared by every call
 * --------------------------------
 * - All array pointers are DEVICE pointers owned by the caller; the library
 *   allocates nothing and keeps no state between calls.  Host pointers are
 *   marked as such.
 * - Every call only enqueues work on `stream` (a hipStream_t; NULL = the
 *   legacy default stream) and returns at once.  Kernel faults surface at the
 *   caller's next synchronisation, as usual in HIP.
 * - Return value: SAD_OK, or a negative status.  Arguments are checked before
 *   anything is enqueued, so an error status means nothing ran.
 *     SAD_EINVAL       negative size, NULL pointer where data is needed,
 *                      misaligned pointer (arrays: 16 bytes), size limits
 *                      exceeded, aliasing that the call forbids
 *     SAD_EUNSUPPORTED a parameter outside what this library implements
 *                      (inject_per_tile > 64)
 *     SAD_EHIP         the HIP runtime refused the launch
 *   sad_status_string() names a status.
 * - Zero sizes are valid and enqueue nothing (except where an output must be
 *   written, noted per call).
 * - Limits: n <= 2^30 sites; h, w <= 2^15; M (query count) < 2^40.
 * - Calls that overlap on one stream in the usual way are safe; calls that
 *   write the same buffer from different streams without ordering race.
 *
 * Data formats (row-major, little-endian, float32 = IEEE binary32)
 * ----------------------------------------------------------------
 * Site parameters  params[n][12]  (Appendix B.2 "Site buffer": ten semantic
 *   float32 values per site; here the metric is a rotation and two scales)
 *     0 x, 1 y      position in pixels; x < 0 marks an inactive site
 *     2 log_tau     log temperature (Sec. 4.1)
 *     3 r           additive radius in units of the anisotropic norm
 *     4,5,6         colour r, g, b
 *     7 theta       rotation of the metric, radians, |theta| <= 2^20
 *     8 log_s1, 9 log_s2   log scales (pixels) along the rotated axes
 *     10, 11        padding (written as 0 by the library where it writes)
 *   The metric is G = R(theta) diag(s1^-2, s2^-2) R(theta)^T (Sec. 4.1).
 *
 * Prepared sites  derived[n][12]  (what every pixel kernel reads)
 *     0 x, 1 y, 2 tau, 3 r, 4 cos(theta), 5 sin(theta), 6 1/s1, 7 1/s2,
 *     8,9,10 colour, 11 zero.
 *   tau, cos, sin, 1/s1, 1/s2 are the float32 values nearest to the exact
 *   exp/cos/sin of the float32 parameters (round to nearest even), so the
 *   record is a pure function of params.  A site whose params x < 0 (or is
 *   NaN) or whose |theta| > 2^20 (or is NaN) gets x = y = -1, cos = 1, sin = 0
 *   and is skipped by every kernel.
 *
 * Top-K map  topk[h][w][8] uint32 (Sec. 4.6, Appendix B.2 "Top-K candidate
 *   list": K = 8 site ids per pixel, empty slots 0xffffffff).  Each list holds
 *   distinct ids, best first, empty slots last.
 *
 * Logit of site i at point (px, py) (Sec. 4.2, l_i = -tau_i d_i):
 *   dx = px - x; dy = py - y;
 *   a = (dx*cos + dy*sin) * (1/s1);  b = (dy*cos - dx*sin) * (1/s2);
 *   q = a*a + b*b;  l = -(tau * (sqrt(q) - r))
 *   float32, one IEEE rounding per operation in exactly this order, no fused
 *   multiply-add, correctly rounded sqrt, subnormals kept.  Pixel (i, j) is
 *   evaluated at its centre (i + 0.5, j + 0.5).
 * Ranking: entry (l1, id1) precedes (l2, id2) iff l1 > l2, or l1 == l2 and
 *   id1 < id2 (-0 == +0).  Candidates with a NaN logit are dropped.
 */
#ifndef SAD_H
#define SAD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SAD_ABI_VERSION 11
#define SAD_K 8
#define SAD_SITE_STRIDE 12
#define SAD_EMPTY 0xffffffffu
#define SAD_TILE 8
#define SAD_MAX_INJECT 64

#define SAD_OK 0
#define SAD_EINVAL (-1)
#define SAD_EUNSUPPORTED (-2)
#define SAD_EHIP (-3)

/* Version of this interface (SAD_ABI_VERSION). */
int sad_abi_version(void);

/* Static, NUL-terminated name of a status code; never NULL. */
const char *sad_status_string(int status);

/*
 * Prepare the per-site records the pixel kernels read (the "pack" step of
 * Appendix B.2 / Table B13, and the exp(log tau) of Sec. 4.1).
 *   params   [n][12] float32, read
 *   derived  [n][12] float32, written (format above); must not overlap params
 */
int sad_prepare_sites(const float *params, int32_t n, float *derived, void *stream);

/*
 * One top-K propagation pass (Sec. 4.3: C~_t(x) = C_{t-1}(x) u P_t(x) u G_t(x),
 * C_t(x) = topK of C~_t(x) under the logit; Figure 5).
 * For every pixel x the candidate set is
 *   - the ids of topk_prev at x (temporal reuse),
 *   - the ids of topk_prev at x +- (stride, 0) and x +- (0, stride) that lie
 *     inside the image (spatial propagation; only the previous map is read),
 *   - the global probe: inject_per_tile ids drawn for x's 8x8 tile, shared by
 *     all pixels of the tile,
 * of which ids >= n and inactive sites are dropped; topk_next at x receives
 * the first 8 distinct ids of that set in ranking order, padded with
 * 0xffffffff.  The result does not depend on the order candidates are visited.
 * Tile of pixel (i, j): (j / 8) * ceil(w / 8) + i / 8.
 * Probe id j of tile T in pass t: z = SplitMix64 output for counter
 *   c = t << 32 | T << 6 | j, i.e. z = mix(seed + (c + 1) * 0x9E3779B97F4A7C15)
 *   with SplitMix64's finaliser mix; id = ((z >> 32) * n) >> 32.
 *   derived      [n][12] prepared sites
 *   topk_prev    [h][w][8], or NULL for an all-empty previous map
 *   scores_prev  NULL, or [h][w][8] float32: the logits of topk_prev's entries
 *                under `derived` exactly as the logit formula gives them, as
 *                written to scores_next by the pass that produced topk_prev
 *                with the same prepared sites.  It saves recomputing them; a
 *                score map made before the sites changed gives wrong lists.
 *                Requires topk_prev.
 *   topk_next    [h][w][8], written
 *   scores_next  NULL, or [h][w][8] float32 written with the logits of
 *                topk_next's entries (-inf for empty slots)
 *   No two of the four maps may overlap.
 *   stride       jump step, >= 1 (Sec. 4.3 schedule B/2, ..., 1, then 1)
 *   seed         injection seed; pass_index: the pass counter t
 *   inject_per_tile  0..64 probe ids per tile per pass
 * Limit: ceil(h/8) * ceil(w/8) <= 2^26 tiles.
 */
int sad_propagate_topk(const float *derived, int32_t n, int32_t h, int32_t w, const uint32_t *topk_prev,
                       const float *scores_prev, uint32_t *topk_next, float *scores_next, int32_t stride,
                       uint64_t seed, uint32_t pass_index, int32_t inject_per_tile, void *stream);

/*
 * The maps a propagation pass (Sec. 4.3) reads and writes, for
 * sad_propagate_pass and sad_step_fused_pass: sad_propagate_topk's four, with
 * a choice of id width for each list map and two shorter forms of what passes
 * hand on to each other within a training step.
 *   topk_prev, scores_prev, topk_next, scores_next   as sad_propagate_topk
 *   prev_bits, next_bits   16 or 32, the width of topk_prev's and topk_next's
 *              ids.  A map of width 16 is [h][w][8] uint16 (16 bytes per
 *              pixel) with the empty slot 0xffff; it needs n <= 65535
 *              (SAD_EUNSUPPORTED otherwise), so that every usable id is below
 *              0xffff.  The lists are those of width 32, id for id (0xffff
 *              where that map holds 0xffffffff); an input id at or above n is
 *              dropped as there.
 *   thr_prev   NULL, or [h][w] float32: the logit of each previous list's 8th
 *              entry (-inf where the list is shorter), as written to thr_next
 *              by the pass that produced topk_prev with the same prepared
 *              sites (so that its lists hold usable ids in ranking order).
 *              Not together with scores_prev; requires topk_prev.  The pass
 *              then evaluates a pixel's other logits only if it inserts a
 *              candidate (on settled lists almost never) or scores_next is
 *              requested: it reads 4 instead of 32 bytes of logits per pixel.
 *              Thresholds made before the sites changed give wrong lists.
 *   thr_next   NULL, or [h][w] float32 written with the logit of each new
 *              list's 8th entry (-inf where it is shorter).
 *   probe_prev NULL, or [n][4] float32 (16-byte aligned): the sites' probe
 *              records as written to probe_next from the same prepared sites.
 *              The pass then decides which of a tile's probe ids can enter
 *              any of its lists from these 16-byte records instead of the
 *              48-byte prepared ones; the lists are the same.  Records made
 *              before the sites changed give wrong lists.
 *   probe_next NULL, or [n][4] float32 (16-byte aligned) written with every
 *              site's probe record: (x, y, tau m, tau r) of its prepared
 *              record, m the smaller inverse scale, or (x, y, 0, +inf) for a
 *              site whose bound is not kept (non-finite values, tau <= 0,
 *              scales more than 1024 apart).  Not written for an empty image.
 * No two of these buffers and derived may overlap (each measured on its own
 * size).  Within a training step the passes after the first can hand
 * their lists on at width 16 with their thresholds and read the first pass's
 * probe records: a pass then moves 20 instead of 64 bytes per pixel each way.
 */
typedef struct sad_pass_maps {
    const void *topk_prev;
    const float *scores_prev;
    const float *thr_prev;
    const float *probe_prev;
    void *topk_next;
    float *scores_next;
    float *thr_next;
    float *probe_next;
    int32_t prev_bits;
    int32_t next_bits;
} sad_pass_maps;

/*
 * sad_propagate_topk on the maps of a sad_pass_maps (maps: a HOST pointer,
 * read during the call).  Other arguments and checks as sad_propagate_topk.
 */
int sad_propagate_pass(const float *derived, int32_t n, int32_t h, int32_t w, const sad_pass_maps *maps,
                       int32_t stride, uint64_t seed, uint32_t pass_index, int32_t inject_per_tile, void *stream);

/*
 * A map of width 16 (see sad_pass_maps) as the same lists of width 32: every
 * id copied, the empty slot 0xffff written as 0xffffffff (Sec. 4.3 keeps one
 * list per pixel; this only changes how its ids are stored).
 *   topk16  [h][w][8] uint16, read;  topk  [h][w][8] uint32, written.
 * Both 16-byte aligned and not overlapping (SAD_EINVAL otherwise).
 */
int sad_widen_map(const uint16_t *topk16, int32_t h, int32_t w, uint32_t *topk, void *stream);

/*
 * Soft additively weighted render (Sec. 4.2): per pixel, the softmax of the
 * logits of the listed sites, w_k = exp(l_k - m) / sum exp(l_j - m) with m the
 * largest logit (Appendix B.4), and the blend c = sum w_k c_k.  List entries
 * that name no usable site, or whose logit is not finite, are skipped; an
 * empty list renders 0.
 *   image  [h][w][3] float32, written
 */
int sad_render_fwd(const float *derived, int32_t n, int32_t h, int32_t w, const uint32_t *topk, float *image,
                   void *stream);

/*
 * Loss and hand-derived gradients (Sec. 6.1 loss; Appendix B.4 "Per-pixel
 * gradients").
 * L = sum over pixels and channels of (c - target)^2 / (h*w).
 * With g = 2 (c - target) / (h*w) and delta_k = w_k (g.c_i - g.c) for entry k
 * (site i), the gradient record of site i receives, summed over pixels:
 *   colour += w_k g;  log_tau += delta_k l_k;  r += tau delta_k;
 *   and, when q > 0, with kappa = -tau delta_k / (2 sqrt q),
 *   a_r = dx cos + dy sin, b_r = dy cos - dx sin, a = a_r/s1, b = b_r/s2:
 *   x += -2 kappa (a cos/s1 - b sin/s2);  y += -2 kappa (a sin/s1 + b cos/s2);
 *   theta += 2 kappa a_r b_r (1/s1^2 - 1/s2^2);
 *   log_s1 += -2 kappa a^2;  log_s2 += -2 kappa b^2.
 * The logits are the float32 values of the formula above; the weights,
 * blend, residual and terms are formed in float64 from them.  The terms are
 * summed per site on chip over regions of 32 x 16 pixels (Sec. 4.8 reduces
 * gradients per tile before any global atomic), then added to grad with one
 * float atomic per (region, site, parameter).
 *   target     [h][w][3] float32, read
 *   grad       [n][12] float32, ACCUMULATED into (+=); the order of the float
 *              atomics, and so the last bits, vary from run to run; entries
 *              10, 11 are not touched
 *   loss       NULL, or one float32 accumulated into (+= L)
 *   image      NULL, or [h][w][3] float32 written with the rendered colours
 * grad, loss and image may overlap neither each other nor derived, topk or
 * target.  The call needs no scratch memory.
 */
int sad_render_bwd(const float *derived, int32_t n, int32_t h, int32_t w, const uint32_t *topk,
                   const float *target, float *grad, float *loss, float *image, void *stream);

/*
 * Per-site budget statistics over the map topk, the inputs of densification
 * and pruning (Sec. 4.5, "Adaptive Budget: Densify and Prune"; Appendix B.5).
 * For every site, summed over the pixels whose usable entries include it,
 * with w the site's softmax weight at the pixel, c the rendered colour and I
 * the target, stats[i][0..7] receive:
 *   [0] mass   sum w                [1] energy  sum w |c - I|^2
 *   [2] removal delta  sum (|c' - I|^2 - |c - I|^2): c' is the blend of the
 *       pixel's other usable entries with their weights renormalised (black
 *       when the site is the only one), so this is the change of the summed
 *       squared error if the site were switched off and the lists kept
 *   [3] sum w dx   [4] sum w dy   [5] sum w dx^2   [6] sum w dx dy
 *   [7] sum w dy^2   with (dx, dy) = pixel centre - site position (the
 *       weighted second moments about the site; their zeroth is the mass)
 *   target     [h][w][3] float32, read
 *   stats      [n][8] float32, 16-byte aligned, ACCUMULATED into (+=); the
 *              summation order, and so the last bits, may vary between runs;
 *              may not overlap derived, topk or target
 *   workspace  device scratch of at least sad_site_stats_workspace_bytes(h, w)
 *              bytes, 16-byte aligned, owned by the caller; its contents on
 *              entry do not matter; it may not overlap stats, derived, topk
 *              or target, nor be in use by another call at the same time
 * Sums per site are formed per region of 32 x 16 pixels on chip (exact
 * fixed-point sums in LDS), written to the workspace, then gathered per site
 * from the regions around the site's own.
 */
size_t sad_site_stats_workspace_bytes(int32_t h, int32_t w);
int sad_site_stats(const float *derived, int32_t n, int32_t h, int32_t w, const uint32_t *topk,
                   const float *target, float *stats, void *workspace, size_t workspace_bytes, void *stream);

/*
 * sad_site_stats without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments, outputs and checks as sad_site_stats;
 * the region tables live in a device array of the library,
 * SAD_STATS_SCRATCH_BYTES per GPU, held from the library's load until the
 * process ends (its address on a GPU is looked up on the first call made
 * with that GPU current).  The call allocates nothing.
 * Limit: sad_site_stats_workspace_bytes(h, w) <= SAD_STATS_SCRATCH_BYTES,
 * i.e. ceil(w / 32) * ceil(h / 16) <= 4551 regions (1920 x 1080 and 2048 x
 * 1024 fit; 2048 x 2048 does not); larger images return SAD_EUNSUPPORTED.
 * Calls on one GPU share the array: calls that overlap on one GPU (on
 * streams without ordering between them) race.
 */
#define SAD_STATS_SCRATCH_BYTES (40u << 20)
int sad_site_stats_noalloc(const float *derived, int32_t n, int32_t h, int32_t w, const uint32_t *topk,
                           const float *target, float *stats, void *stream);

/*
 * Budget control from the statistics of sad_site_stats (Sec. 4.5, "Adaptive
 * Budget: Densify and Prune"; Appendix B.5, "Densification scores", "Split
 * kernel", "Pruning").  In place on params, adam_m, adam_v and derived
 * ([n][12] float32 each, the Adam moments as sad_adam_step keeps them):
 *   1. the n_prune active sites with the lowest removal delta (stats[i][2];
 *      NaN ranks last; ties: lower id first) are switched off: position
 *      (-1, -1);
 *   2. the sites still active with mass stats[i][0] >= min_mass and > 0 are
 *      ranked by energy / mass^alpha (stats[i][1] / stats[i][0]^alpha in
 *      double; best first, ties: lower id; NaN scores skipped); while k <
 *      n_split and both lists last, the k-th is split into the k-th inactive
 *      slot (ascending index): its two children sit at its position
 *      +- offset sigma u (its own slot takes +; each clamped to [0, w] x
 *      [0, h]), with u and sigma^2 the major eigenvector and eigenvalue of
 *      the weighted covariance about the site (moments stats[i][3..7] over
 *      the mass), or when those are degenerate u the direction of the Sobel
 *      gradient of the target (channels summed) at the site's pixel ((1, 0)
 *      when zero) and sigma the site's larger scale; the children take the
 *      target colour at their pixels, log tau - logtau_shift, r * r_scale,
 *      the parent's theta and scales, and zero Adam moments;
 *   3. the prepared records of every changed site are rewritten.
 * The geometry is float32, one rounding per operation in that order.
 *   stats      [n][8] float32 (16-byte aligned) as sad_site_stats writes it
 *   target     [h][w][3] float32
 *   done       NULL, or a device int32[2]: the numbers of sites pruned and split
 *   workspace  device scratch of sad_budget_workspace_bytes(n) bytes,
 *              256-byte aligned, owned by the caller (the rankings' keys and
 *              the radix sorts' storage)
 */
size_t sad_budget_workspace_bytes(int32_t n);
int sad_densify_prune(float *params, float *adam_m, float *adam_v, float *derived, int32_t n, int32_t h, int32_t w,
                      const float *stats, const float *target, int32_t n_split, int32_t n_prune, float alpha,
                      float min_mass, float offset, float r_scale, float logtau_shift, int32_t *done,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * Gradient-weighted initialisation (Sec. 4.4): n sites drawn independently
 * from P_init(x) = (1 - lambda) |grad I(x)| / sum |grad I| + lambda / (h w).
 * |grad I| is the 2-norm over the 3 channels and both directions of the 3x3
 * Sobel derivatives of the target (borders repeated), float32; it is taken in
 * integer units of 2^-24 (truncated, capped at 2^8) and the inclusive prefix
 * sum of those units, exact in 64 bits, is the CDF.  Site s uses the
 * SplitMix64 outputs z_k for counters 4 s + k (same generator as the probes):
 *   z_0: the uniform part when (z_0 >> 40) * 2^-24 < lambda or every unit is 0,
 *   z_1: the pixel: ((z_1 >> 32) * h * w) >> 32 for the uniform part, else the
 *        first pixel (row-major) whose prefix sum exceeds (z_1 * G) >> 64,
 *        G the total,
 *   z_2, z_3: x = i + (z_2 >> 40) * 2^-24 and y = j + (z_3 >> 40) * 2^-24
 *        (float32 sums) inside that pixel (i, j).
 * The record: (x, y, log_tau, r, the target colour of pixel (i, j), angle 0,
 * log_scale, log_scale, 0, 0); derived is written as sad_prepare_sites would.
 *   target     [h][w][3] float32
 *   lambda     in [0, 1]
 *   params, derived  [n][12] float32, written, 16-byte aligned
 *   workspace  device scratch of sad_init_workspace_bytes(h, w) bytes, 256-byte
 *              aligned, owned by the caller (the units, their prefix sums and
 *              the scan's storage)
 * n = 0 does nothing; n > 0 needs h, w > 0.  Results depend only on the inputs.
 */
size_t sad_init_workspace_bytes(int32_t h, int32_t w);
int sad_init_sites(const float *target, int32_t h, int32_t w, int32_t n, float lambda, uint64_t seed, float log_tau,
                   float r, float log_scale, float *params, float *derived, void *workspace, size_t workspace_bytes,
                   void *stream);

/*
 * Packed 16-byte evaluation records (Appendix B.2, "Packed storage for
 * evaluation") and random access from them (Sec. 6.6).
 * sad_pack_sites: packed [n][4] uint32 (16-byte aligned) receives one record
 * per site: w0 = qx | qy << 15 | 1 << 31 with qx, qy the 15-bit UNORM codes of
 * x / w and y / h; w1 = colour codes r | g << 11 | b << 22 (11/11/10 bits);
 * w2 = log tau' code | r' code << 16; w3 = angle code | float16(a) << 16.
 * The stored site is the determinant-1 form of the same logit:
 * hs = 0.5 (log s1 + log s2), log tau' = log tau - hs, r' = r exp(hs)
 * (correctly rounded float32 exp), a = log s2 - log s1 (float16, nearest
 * even).  qparams float32[10] receives (min, max - min) of log tau', r', c_r,
 * c_g, c_b over the usable sites (NaN ignored, -0 as +0; none: 0, 0); codes
 * are rint(clamp(t, 0, 1) (2^bits - 1)) with t = (v - min) / (max - min) (0
 * when the range is not positive); the angle code is that of
 * (theta_w + pi_f) / (2 pi)_f, theta_w = theta - (2 pi)_f rint(theta / (2 pi)_f),
 * all float32 in that order.  A site that is not usable (derived x < 0) packs
 * to four zeros.  qparams is also the scratch of the range reduction, so it
 * must not be read while the call runs.  n > 0 needs h, w > 0.
 * sad_query_packed: as sad_query_points, with each list entry decoded from
 * its record (value = min + code / (2^bits - 1) (max - min); x = qx w / 32767,
 * y = qy h / 32767; angle = code 2 pi / 65535 - pi); entries with an id >= n or
 * without the usable bit are skipped.  The offsets to the point are formed in
 * float64; exp, sine and cosine use the GPU's hardware approximations, so
 * results differ from exact decoding by a few float32 roundings of the logits.
 */
int sad_pack_sites(const float *params, const float *derived, int32_t n, int32_t h, int32_t w, uint32_t *packed,
                   float *qparams, void *stream);
int sad_query_packed(const uint32_t *packed, const float *qparams, int32_t n, int32_t h, int32_t w,
                     const uint32_t *topk, const float *xy, int64_t m, float *rgb, void *stream);

/*
 * JFA prepass of a full list refresh (Appendix B.3, "JFA prepass"; the render
 * protocol of Sec. 6.6 runs one JFA round, then propagation passes starting
 * from the round's last output, then the render), after the jump flooding of
 * Rong and Tan (2006).  A 4-list holds 4 site ids ranked at the pixel centre
 * as the top-K lists are, EMPTY-padded.
 *
 * sad_jfa_seed: jfa [h][w][4] uint32 (16-byte aligned) is overwritten: the
 * pixel holding a usable site's position (floor of x and y, clamped to the
 * image) gets in slot 0 the site ranking first at its centre among the sites
 * on it; every other slot is EMPTY.
 *
 * sad_jfa_flood: one flood pass with jump step `step` >= 1: every pixel gets
 * the 4 best distinct usable ids of the 4-lists jfa_prev at (i + a step,
 * j + b step), a, b in {-1, 0, 1}, inside the image (its own included).
 * out_width 4 writes out as [h][w][4]; out_width 8 writes a top-K map
 * [h][w][8] with slots 4..7 EMPTY, the start of the propagation passes.  A
 * round runs the steps B/2, B/4, ..., 1 with B the smallest power of two
 * >= max(h, w).  out must not overlap jfa_prev or derived.
 */
int sad_jfa_seed(const float *derived, int32_t n, int32_t h, int32_t w, uint32_t *jfa, void *stream);
int sad_jfa_flood(const float *derived, int32_t n, int32_t h, int32_t w, const uint32_t *jfa_prev, uint32_t *out,
                  int32_t step, int32_t out_width, void *stream);

/*
 * One training-iteration pass in one call: a propagation pass followed by
 * the loss and gradients over the lists it produced (the one-pass update of
 * a training iteration, Sec. 6.6 / Table 9, then Sec. 4.8 / Appendix B.4).
 * Equivalent to sad_propagate_topk(derived, n, h, w, topk_prev, scores_prev,
 * topk_next, scores_next, stride, seed, pass_index, inject_per_tile) then
 * sad_render_bwd(derived, n, h, w, topk_next, target, grad, loss, image):
 * topk_next, scores_next and image are the same bits; grad and loss differ
 * only by summation order, as between two calls of sad_render_bwd.  One
 * kernel does both: each workgroup runs the pass on a region of 32 x 16
 * pixels and the backward starts from the lists and float32 logits the pass
 * left in registers (no list is read back, no logit evaluated again).  Every
 * argument is checked before any work is enqueued, so a rejected call leaves
 * all buffers untouched.
 * Arguments, formats and checks are those of the two calls; in addition
 * topk_next and scores_next must not overlap target, grad, loss, image or
 * derived.
 */
int sad_step_fused(const float *derived, int32_t n, int32_t h, int32_t w, const uint32_t *topk_prev,
                   const float *scores_prev, uint32_t *topk_next, float *scores_next, int32_t stride, uint64_t seed,
                   uint32_t pass_index, int32_t inject_per_tile, const float *target, float *grad, float *loss,
                   float *image, void *stream);

/*
 * sad_step_fused on the maps of a sad_pass_maps (maps: a HOST pointer, read
 * during the call): the last pass of a step whose earlier passes handed their
 * lists on at width 16, with thresholds or probe records.  The pass writes
 * 32-bit ids (next_bits = 32), or 16-bit ones (next_bits = 16, n <= 65535)
 * for the next step's first pass, and no thresholds or probe records
 * (thr_next and probe_next NULL; SAD_EINVAL otherwise).  With thr_prev the backward
 * evaluates the pixels' logits from the site records it stages anyway,
 * rather than taking them from the pass.  In addition to the checks of
 * sad_step_fused, grad, loss and image must not overlap topk_prev,
 * scores_prev, thr_prev or probe_prev.
 */
int sad_step_fused_pass(const float *derived, int32_t n, int32_t h, int32_t w, const sad_pass_maps *maps,
                        int32_t stride, uint64_t seed, uint32_t pass_index, int32_t inject_per_tile,
                        const float *target, float *grad, float *loss, float *image, void *stream);

/*
 * One Adam step (Kingma & Ba) on the site parameters (Sec. 5: per-parameter
 * base learning rates, fixed betas and epsilon), then the projection of
 * Sec. 4.1 (positions clamped to [0, w] x [0, h]), then the prepared records
 * rewritten.  Per parameter k < 10 of an active site (x >= 0), in float32,
 * one rounding per operation, in this order:
 *   m = b1*m + (1 - b1)*g;   v = b2*v + (1 - b2)*(g*g);
 *   p = p - lr * ((m / bc1) / (sqrt(v / bc2) + eps))
 * where (1 - b1) and (1 - b2) are float32 subtractions.  Inactive sites keep
 * params, m and v.  Every site's gradient record is zeroed.
 *   lr       HOST pointer to 5 float32 rates: (x, y), log_tau, r, colour,
 *            (theta, log_s1, log_s2); read during the call
 *   bias_corr1, bias_corr2   1 - beta1^t and 1 - beta2^t from the caller
 *   derived  [n][12] written as by sad_prepare_sites, or NULL to skip
 */
int sad_adam_step(float *params, float *grad, float *m, float *v, int32_t n, int32_t h, int32_t w, const float *lr,
                  float beta1, float beta2, float eps, float bias_corr1, float bias_corr2, float *derived,
                  void *stream);

/*
 * sad_adam_step that also rewrites the sites' probe records from the new
 * prepared records (the probe records of sad_pass_maps, bit for bit what a
 * pass writes to probe_next from these prepared sites), so that the first
 * pass after the update can cull its probes from them instead of writing
 * them (Sec. 4.3: the probes are drawn afresh every pass; Sec. 5: the sites
 * change only in the optimiser step).
 *   probe    NULL (then as sad_adam_step), or [n][4] float32, 16-byte
 *            aligned, written; requires derived.  May overlap none of the
 *            other buffers (SAD_EINVAL).
 */
int sad_adam_step_probe(float *params, float *grad, float *m, float *v, int32_t n, int32_t h, int32_t w,
                        const float *lr, float beta1, float beta2, float eps, float bias_corr1, float bias_corr2,
                        float *derived, float *probe, void *stream);

/*
 * Random access (Sec. 6.6, the render-only path from cached lists): point t
 * at (qx, qy) uses the list of pixel (clamp(floor(qx), 0, w-1),
 * clamp(floor(qy), 0, h-1)) and evaluates the logits at (qx, qy) itself, then
 * blends as sad_render_fwd.  A non-finite coordinate gives NaN colour.
 *   xy   [m][2] float32 (8-byte aligned), rgb [m][3] float32 written
 */
int sad_query_points(const float *derived, int32_t n, int32_t h, int32_t w, const uint32_t *topk, const float *xy,
                     int64_t m, float *rgb, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SAD_H */
