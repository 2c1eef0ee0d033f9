// sad_backward.hip -- the loss and the hand-derived gradients of the soft
// anisotropic render (Sec. 6.1 loss; Appendix B.4 "Per-pixel gradients"),
// summed per site on chip before they leave the workgroup (Sec. 4.8
// "Gradient Accumulation"), and the call that runs a propagation pass and
// the backward over its lists.
//
// One workgroup per region of 32 x 16 pixels (sad_region.h), in two phases:
//
//  A. Pixel-major, one lane per pixel.  Every listed site claims a slot of
//     the region's LDS table and counts its entry there; the claimed sites'
//     records are read once into LDS; the counts become bucket starts and
//     the buckets are cut into pieces of at most PIECE entries.  The pixel's
//     forward follows: float32 logits (the ranking's own values), their
//     exponentials, and then in float64 the normaliser, the blended colour,
//     the residual and dL/dc.  What the second phase needs of the pixel
//     (the largest logit, 1/Z, dL/dc and dL/dc . c) goes to LDS, and the
//     pixel's index goes to the bucket of each of its entries: a counting
//     sort of the region's entries by site.
//  B. Site-major, one piece per lane.  A lane holds one site's record and
//     runs over the piece's pixels, recomputing each entry's logit and weight
//     from the pixel's values, forming the 10 terms of Appendix B.4 in
//     float64 and summing them in registers; the piece's sums are then added
//     to the slot's float64 sums in LDS (one LDS add per term per piece,
//     rather than one per term per list entry).
// Finally every slot's 10 sums leave the workgroup as float atomics on the
// site's gradient record, once per (region, site).
//
// Precision: the residual c - I and the differences c_i - c cancel when the
// render is close to the target or the site's colour to the blend; carried
// in float64 they leave the gradients within a few float32 roundings of the
// exact sums (the per-entry float32 inputs are the logits, the hardware
// exponential of l - max l and the reciprocal square root of q).
#include "sad_propagate.h"
#include "sad_region.h"

namespace sad {

constexpr int PIECE = 10;  // entries of one site per phase-B lane
constexpr int MAX_PIECES = (REGION_PIX * K + PIECE - 1) / PIECE + SLOTS;
constexpr int BWD_THREADS = WAVE * REGION_WAVES;
static_assert(SLOTS == 4 * WAVE, "one wavefront plans the pieces, 4 slots per lane");
static_assert(REGION_PIX * K < (1 << 13) && PIECE < 16 && SLOTS <= 256, "piece table packing");

// What phase B needs of a pixel: the largest logit, 1/Z, dL/dc (float32,
// formed in float64) and dL/dc . c (float64, c the blended colour).
struct PixState {
    float m, g0, g1, g2;
    double iz, gc;
};

struct BwdArgs {
    const float* derived;
    const uint32_t* topk;
    const float* target;
    float* grad;
    float* loss;
    float* image;
    int32_t n, h, w;
    RegionGrid rg;
    double inv_p;  // 1 / (h w)
};

// Site geometry for the gradient terms, in float64.
struct SiteD {
    double x, y, tau, cs, sn, is1, is2;
};

__device__ __forceinline__ SiteD site_d(float4 g0, float4 g1) {
    return {(double)g0.x, (double)g0.y, (double)g0.z, (double)g1.x, (double)g1.y, (double)g1.z, (double)g1.w};
}

// The 10 terms of one list entry (Appendix B.4), in the gradient record's
// order (x, y, log tau, r, colour, theta, log s1, log s2): (px, py) the pixel
// centre, l the entry's float32 logit, w its weight, delta = dL/dl =
// w (g.c_i - g.c) and g = dL/dc.  With 2 kappa = -tau delta / sqrt(q):
// x: -2 kappa (a cos/s1 - b sin/s2), y: -2 kappa (a sin/s1 + b cos/s2),
// theta: 2 kappa a_r b_r (1/s1^2 - 1/s2^2), log s_k: -2 kappa a^2, -2 kappa
// b^2; at q = 0 (the pixel centre on the site) these are 0.
__device__ __forceinline__ void entry_terms(const SiteD& s, double px, double py, float l, double w, double delta,
                                            const float (&g)[3], double (&t)[NGRAD]) {
    t[4] = w * (double)g[0];
    t[5] = w * (double)g[1];
    t[6] = w * (double)g[2];
    t[2] = delta * (double)l;
    t[3] = s.tau * delta;
    const double dx = px - s.x, dy = py - s.y;
    const double ar = dx * s.cs + dy * s.sn, br = dy * s.cs - dx * s.sn;
    const double aa = ar * s.is1, bb = br * s.is2;
    const double q = aa * aa + bb * bb;
    t[0] = t[1] = t[7] = t[8] = t[9] = 0.0;
    if (q > 0.0) {
        const float qf = (float)q;
        const double rs = qf >= 0x1p-100f ? (double)__builtin_amdgcn_rsqf(qf) : 1.0 / __builtin_sqrt(q);
        const double kap2 = -s.tau * delta * rs;  // 2 kappa
        t[0] = -kap2 * (aa * s.is1 * s.cs - bb * s.is2 * s.sn);
        t[1] = -kap2 * (aa * s.is1 * s.sn + bb * s.is2 * s.cs);
        t[7] = kap2 * ar * br * ((s.is1 - s.is2) * (s.is1 + s.is2));  // 1/s1^2 - 1/s2^2 without cancellation
        t[8] = -kap2 * aa * aa;
        t[9] = -kap2 * bb * bb;
    }
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, WAVE);
    return v;
}

// One wavefront turns the per-slot entry counts into bucket starts (in
// place) and cuts every bucket into ceil(count / PIECE) pieces of nearly
// equal length; ptab receives start | length << 13 | slot << 17 per piece,
// *npieces their number.
__device__ __forceinline__ void plan_pieces(uint32_t* cnt, uint32_t* ptab, uint32_t* npieces, int lane) {
    uint32_t c[4], pcs[4], sc = 0, sp = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        c[q] = cnt[4 * lane + q];
        pcs[q] = (c[q] + PIECE - 1) / PIECE;
        sc += c[q];
        sp += pcs[q];
    }
    uint32_t isc = sc, isp = sp;  // inclusive prefix sums over the lanes
#pragma unroll
    for (int off = 1; off < WAVE; off <<= 1) {
        const uint32_t u = __shfl_up(isc, off, WAVE), v = __shfl_up(isp, off, WAVE);
        if (lane >= off) {
            isc += u;
            isp += v;
        }
    }
    uint32_t b0 = isc - sc, pb = isp - sp;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t s = 4 * lane + q;
        cnt[s] = b0;
        uint32_t st = b0;
        for (uint32_t k = 0; k < pcs[q]; ++k) {
            const uint32_t len = c[q] / pcs[q] + (k < c[q] % pcs[q] ? 1u : 0u);
            ptab[pb + k] = st | (len << 13) | (s << 17);
            st += len;
        }
        b0 += c[q];
        pb += pcs[q];
    }
    if (lane == WAVE - 1) *npieces = isp;
}

__global__ __launch_bounds__(BWD_THREADS) __attribute__((amdgpu_waves_per_eu(4))) void k_backward(BwdArgs a) {
    __shared__ uint32_t keys[SLOTS];
    __shared__ float4 recs[SLOTS * 3];       // prepared record of the site in each slot
    __shared__ uint32_t cnt[SLOTS];          // entries per slot, then the slot's first position in `order`
    __shared__ uint32_t ptab[MAX_PIECES];
    __shared__ uint16_t order[REGION_PIX * K];  // pixels of the region's entries, grouped by slot
    __shared__ PixState ps[REGION_PIX];
    __shared__ double acc[NGRAD * SLOTS];    // per term and slot
    __shared__ double wsum[REGION_WAVES];
    __shared__ uint32_t npieces;

    const uint32_t n = (uint32_t)a.n;
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), wv = tid / WAVE;
    const int reg = xcd_block(blockIdx.x, gridDim.x);
    const int rx = reg % a.rg.rgx, ry = reg / a.rg.rgx;
    int i, j;
    region_pixel(rx, ry, wv, lane, i, j);
    const bool inside = i < a.w && j < a.h;
    const size_t p = (size_t)j * a.w + i;
    const float px = (float)i + 0.5f, py = (float)j + 0.5f;

    for (int s = tid; s < SLOTS; s += BWD_THREADS) {
        keys[s] = EMPTY;
        cnt[s] = 0;
    }
    for (int s = tid; s < NGRAD * SLOTS; s += BWD_THREADS) acc[s] = 0.0;

    // The pixel's list, each lane starting at its own offset (anti-diagonal of
    // the tile) so that neighbouring pixels listing the same sites claim and
    // count different slots at each step.
    const int rot = (lane + (lane >> 3)) & (K - 1);
    uint32_t ids[K];
    float tg[3] = {0.f, 0.f, 0.f};
    {
        uint4 l0 = make_uint4(EMPTY, EMPTY, EMPTY, EMPTY), l1 = l0;
        if (inside) {
            const uint4* l = reinterpret_cast<const uint4*>(a.topk + p * K);
            l0 = l[0];
            l1 = l[1];
            tg[0] = a.target[p * 3 + 0];
            tg[1] = a.target[p * 3 + 1];
            tg[2] = a.target[p * 3 + 2];
        }
        rotate_list(l0, l1, rot);
        ids[0] = l0.x; ids[1] = l0.y; ids[2] = l0.z; ids[3] = l0.w;
        ids[4] = l1.x; ids[5] = l1.y; ids[6] = l1.z; ids[7] = l1.w;
    }
    __syncthreads();  // table cleared

    // A1. slots, and each entry's position in its slot's bucket
    int slot[K];
    claim_slots(keys, ids, n, slot);
    uint32_t pos[K];
#pragma unroll
    for (int k = 0; k < K; ++k) pos[k] = slot[k] >= 0 ? atomicAdd(&cnt[slot[k]], 1u) : 0u;
    __syncthreads();

    // A2. every claimed site's record read from memory once, into LDS; the
    //     first wavefront plans the pieces meanwhile
    for (int s = tid; s < SLOTS; s += BWD_THREADS) {
        const uint32_t id = keys[s];
        if (id == EMPTY) continue;
        const float4* r = reinterpret_cast<const float4*>(a.derived + (size_t)id * REC);
        recs[s * 3 + 0] = r[0];
        recs[s * 3 + 1] = r[1];
        recs[s * 3 + 2] = r[2];
    }
    if (wv == 0) plan_pieces(cnt, ptab, &npieces, lane);
    __syncthreads();

    // A3. the pixel's forward.  When an entry of some lane of the wavefront
    //     found no slot (its probe chain ran out), the wavefront takes a copy
    //     of this code that reads such records from memory and sends their
    //     terms to memory directly; otherwise every record read is an LDS
    //     read (one pointer that may point to either memory would make every
    //     read a slower generic load).
    bool slotted = true;
#pragma unroll
    for (int k = 0; k < K; ++k) slotted &= (ids[k] >= n) | (slot[k] >= 0);
    double lsum = 0.0;
    auto forward = [&](auto lds_only) {
        // part q (0: x y tau r, 1: cos sin 1/s1 1/s2, 2: colour) of entry k's record
        auto rec = [&](int k, int q) -> float4 {
            if constexpr (decltype(lds_only)::value)
                return recs[(slot[k] >= 0 ? slot[k] : 0) * 3 + q];
            else
                return slot[k] >= 0 ? recs[slot[k] * 3 + q]
                                    : reinterpret_cast<const float4*>(a.derived + (size_t)ids[k] * REC)[q];
        };
        float l[K], e[K];
        bool use[K];
        float mx = -__builtin_inff();
#pragma unroll
        for (int k = 0; k < K; ++k) {
            use[k] = false;
            l[k] = 0.0f;
            if (ids[k] >= n) continue;
            Geo g;
            g.g0 = rec(k, 0);
            g.g1 = rec(k, 1);
            const float s = usable_logit(g, true, px, py);
            if (!finitef(s)) continue;
            use[k] = true;
            l[k] = s;
            mx = fmaxf(mx, s);
        }
        double z = 0.0;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            e[k] = use[k] ? __expf(l[k] - mx) : 0.0f;
            z += (double)e[k];
        }
        const double iz = z > 0.0 ? 1.0 / z : 0.0;
        double c[3] = {0.0, 0.0, 0.0};
#pragma unroll
        for (int k = 0; k < K; ++k) {
            if (!use[k]) continue;
            const double wk = (double)e[k] * iz;
            const float4 col = rec(k, 2);
            c[0] += wk * (double)col.x;
            c[1] += wk * (double)col.y;
            c[2] += wk * (double)col.z;
        }
        float g[3];
        double gc = 0.0;
#pragma unroll
        for (int ch = 0; ch < 3; ++ch) {
            const double r = c[ch] - (double)tg[ch];
            lsum += r * r;
            g[ch] = (float)(2.0 * r * a.inv_p);
            gc += (double)g[ch] * c[ch];
        }
        if (inside && a.image) {
            a.image[p * 3 + 0] = (float)c[0];
            a.image[p * 3 + 1] = (float)c[1];
            a.image[p * 3 + 2] = (float)c[2];
        }
        ps[tid] = PixState{mx == -__builtin_inff() ? 0.0f : mx, g[0], g[1], g[2], iz, gc};
        if constexpr (!decltype(lds_only)::value) {
#pragma unroll
            for (int k = 0; k < K; ++k) {
                if (!use[k] || slot[k] >= 0) continue;
                const float4 g0 = rec(k, 0), g1 = rec(k, 1), col = rec(k, 2);
                const double wk = (double)e[k] * iz;
                const double delta =
                    wk * ((double)g[0] * (double)col.x + (double)g[1] * (double)col.y + (double)g[2] * (double)col.z - gc);
                double t[NGRAD];
                entry_terms(site_d(g0, g1), (double)px, (double)py, l[k], wk, delta, g, t);
#pragma unroll
                for (int q = 0; q < NGRAD; ++q) unsafeAtomicAdd(&a.grad[(size_t)ids[k] * REC + q], (float)t[q]);
            }
        }
    };
    if (__all(slotted))
        forward(std::true_type{});
    else
        forward(std::false_type{});
#pragma unroll
    for (int k = 0; k < K; ++k)
        if (slot[k] >= 0) order[cnt[slot[k]] + pos[k]] = (uint16_t)tid;
    if (a.loss) {
        const double ws = wave_sum_d(lsum);
        if (lane == 0) wsum[wv] = ws;
    }
    __syncthreads();

    // B. one piece per lane: a site's entries, pieces dealt across the
    //    wavefronts in turn
    const uint32_t np = npieces;
    for (uint32_t base = 0; base < np; base += BWD_THREADS) {
        const uint32_t pc = base + (uint32_t)(lane * REGION_WAVES + wv);
        if (pc >= np) continue;
        const uint32_t pe = ptab[pc];
        const int start = (int)(pe & 0x1FFFu), len = (int)((pe >> 13) & 0xFu), s = (int)(pe >> 17);
        Geo geo;
        geo.g0 = recs[s * 3 + 0];
        geo.g1 = recs[s * 3 + 1];
        const float4 col = recs[s * 3 + 2];
        const SiteD sd = site_d(geo.g0, geo.g1);
        const bool active = geo.g0.x >= 0.0f;  // a claimed id is < n; an inactive site has x < 0
        double sum[NGRAD];
#pragma unroll
        for (int q = 0; q < NGRAD; ++q) sum[q] = 0.0;
        for (int it = 0; it < len; ++it) {
            const int pp = order[start + it];
            const PixState st = ps[pp];
            int pi, pj;
            region_pixel(rx, ry, pp / WAVE, pp & (WAVE - 1), pi, pj);
            const float fx = (float)pi + 0.5f, fy = (float)pj + 0.5f;
            const float l = logit(geo, fx, fy);
            if (!(active & finitef(l))) continue;  // unusable entries take no part (as in the forward)
            const double wk = (double)__expf(l - st.m) * st.iz;
            const float g[3] = {st.g0, st.g1, st.g2};
            const double delta =
                wk * ((double)g[0] * (double)col.x + (double)g[1] * (double)col.y + (double)g[2] * (double)col.z - st.gc);
            double t[NGRAD];
            entry_terms(sd, (double)fx, (double)fy, l, wk, delta, g, t);
#pragma unroll
            for (int q = 0; q < NGRAD; ++q) sum[q] += t[q];
        }
#pragma unroll
        for (int q = 0; q < NGRAD; ++q) atomicAdd(&acc[q * SLOTS + s], sum[q]);
    }
    __syncthreads();

    // C. the region's per-site sums leave the workgroup: one float atomic per
    //    (site, term)
    for (int pr = tid; pr < NGRAD * SLOTS; pr += BWD_THREADS) {
        const int q = pr / SLOTS, s = pr % SLOTS;
        const uint32_t id = keys[s];
        if (id == EMPTY) continue;
        const double v = acc[pr];
        if (v != 0.0) unsafeAtomicAdd(&a.grad[(size_t)id * REC + q], (float)v);
    }
    if (a.loss && tid == 0) {
        double tot = 0.0;
        for (int k = 0; k < REGION_WAVES; ++k) tot += wsum[k];
        unsafeAtomicAdd(a.loss, (float)(tot * a.inv_p));
    }
}

// Argument checks of a backward pass over the list map topk, and its kernel
// arguments.  Returns SAD_OK with b filled in, or the error status.
inline int bwd_setup(const float* derived, int32_t n, int32_t h, int32_t w, const uint32_t* topk,
                     const float* target, float* grad, float* loss, float* image, BwdArgs& b) {
    if (!sites_ok(n) || !image_ok(h, w)) return SAD_EINVAL;
    const int64_t pix = int64_t(h) * w;
    if (!array_ok(derived, n, 16) || !array_ok(topk, pix, 16)) return SAD_EINVAL;
    if (!array_ok(target, pix, 4) || !array_ok(grad, n, 16)) return SAD_EINVAL;
    if ((loss && !aligned(loss, 4)) || (image && !aligned(image, 4))) return SAD_EINVAL;
    // the outputs may overlap neither each other nor any input
    const int64_t gbytes = int64_t(n) * REC * 4;
    const void* outs[3] = {grad, loss, image};
    const int64_t obytes[3] = {gbytes, 4, pix * 12};
    const void* ins[3] = {derived, topk, target};
    const int64_t ibytes[3] = {gbytes, pix * K * 4, pix * 12};
    for (int o = 0; o < 3; ++o) {
        for (int q = 0; q < 3; ++q)
            if (overlap(outs[o], obytes[o], ins[q], ibytes[q])) return SAD_EINVAL;
        for (int q = o + 1; q < 3; ++q)
            if (overlap(outs[o], obytes[o], outs[q], obytes[q])) return SAD_EINVAL;
    }
    b.derived = derived;
    b.topk = topk;
    b.target = target;
    b.grad = grad;
    b.loss = loss;
    b.image = image;
    b.n = n;
    b.h = h;
    b.w = w;
    b.rg = region_grid(h, w);
    b.inv_p = pix > 0 ? 1.0 / ((double)h * (double)w) : 0.0;
    return SAD_OK;
}

inline int bwd_launch(const BwdArgs& b, void* stream) {
    const size_t nreg = (size_t)b.rg.rgx * b.rg.rgy;
    clear_error();
    hipLaunchKernelGGL(k_backward, dim3((unsigned)nreg), dim3(BWD_THREADS), 0, as_stream(stream), b);
    return launch_status();
}

}  // namespace sad

using namespace sad;

extern "C" int sad_render_bwd(const float* derived, int32_t n, int32_t h, int32_t w, const uint32_t* topk,
                              const float* target, float* grad, float* loss, float* image, void* stream) {
    BwdArgs b;
    const int st = bwd_setup(derived, n, h, w, topk, target, grad, loss, image, b);
    if (st != SAD_OK) return st;
    if (int64_t(h) * w == 0) return SAD_OK;
    return bwd_launch(b, stream);
}

extern "C" int sad_step_fused(const float* derived, int32_t n, int32_t h, int32_t w, const uint32_t* topk_prev,
                              const float* scores_prev, uint32_t* topk_next, float* scores_next, int32_t stride,
                              uint64_t seed, uint32_t pass_index, int32_t inject_per_tile, const float* target,
                              float* grad, float* loss, float* image, void* stream) {
    PropArgs pa;
    int st = prop_setup(derived, n, h, w, topk_prev, scores_prev, topk_next, scores_next, stride, seed, pass_index,
                        inject_per_tile, pa);
    if (st != SAD_OK) return st;
    BwdArgs b;
    st = bwd_setup(derived, n, h, w, topk_next, target, grad, loss, image, b);
    if (st != SAD_OK) return st;
    // the pass's outputs must not share memory with anything else the step reads or writes
    const int64_t pix = int64_t(h) * w, mbytes = pix * K * 4, gbytes = int64_t(n) * REC * 4;
    const void* outs[2] = {topk_next, scores_next};
    const void* others[5] = {target, grad, loss, image, derived};
    const int64_t obytes[5] = {pix * 12, gbytes, 4, pix * 12, gbytes};
    for (int o = 0; o < 2; ++o)
        for (int q = 0; q < 5; ++q)
            if (overlap(outs[o], mbytes, others[q], obytes[q])) return SAD_EINVAL;
    if (pix == 0) return SAD_OK;
    // every check has passed: the pass, then the backward over its lists, in
    // stream order
    st = sad_propagate_topk(derived, n, h, w, topk_prev, scores_prev, topk_next, scores_next, stride, seed, pass_index,
                            inject_per_tile, stream);
    if (st != SAD_OK) return st;
    return bwd_launch(b, stream);
}
