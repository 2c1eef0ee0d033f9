// sad_render.hip -- soft anisotropic Apollonius render (Sec. 4.2), random-
// access queries (Sec. 6.6) and the per-site budget statistics (Sec. 4.5,
// Appendix B.5).
//
// The forward render uses the same mapping as the propagation pass: one
// wavefront per 8x8 tile, 4 consecutive tiles per 256-thread workgroup.  The
// statistics work on regions of 2 x 4 tiles and reduce the per-site terms in
// two stages (described before k_region_stats); queries take one thread per
// point.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "sad_propagate.h"
#include "sad_region.h"

namespace sad {

// Evaluate one point: the usable entries of its list, their logits, the
// softmax weights and the blended colour.  Returns the number of entries.
struct PointEval {
    int n;
    uint32_t id[K];
    float l[K];
    float e[K];  // exp(l - max), later normalised to weights
    float c[3];
    float4 col[K];  // colour part of each entry's record
};

__device__ __forceinline__ void eval_point(const float* __restrict__ derived, uint32_t nsites, const uint4 l0,
                                           const uint4 l1, float px, float py, PointEval& pe) {
    const uint32_t ids[K] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
    pe.n = 0;
    float mx = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < K; ++k) {
        pe.id[k] = EMPTY;
        pe.l[k] = 0.0f;
    }
    if (nsites > 0) {
        // all record loads first, colours included (clamped ids, no branches):
        // one round trip to memory for the whole record set, then the logits
        Geo g[K];
#pragma unroll
        for (int k = 0; k < K; ++k) g[k] = load_geo_clamped(derived, nsites, ids[k]);
#pragma unroll
        for (int k = 0; k < K; ++k)
            pe.col[k] = reinterpret_cast<const float4*>(derived + (size_t)(ids[k] < nsites ? ids[k] : 0u) * REC)[2];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const float s = usable_logit(g[k], ids[k] < nsites, px, py);
            const bool ok = finitef(s);  // also drops NaN: unusable entries
            pe.id[k] = ok ? ids[k] : EMPTY;
            pe.l[k] = ok ? s : 0.0f;
            mx = ok ? fmaxf(mx, s) : mx;
            pe.n += ok ? 1 : 0;
        }
    }
    float z = 0.0f;
    pe.c[0] = pe.c[1] = pe.c[2] = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const float ek = __expf(pe.l[k] - mx);
        pe.e[k] = pe.id[k] != EMPTY ? ek : 0.0f;
        z += pe.e[k];
    }
    if (pe.n == 0) return;
    float iz = 1.0f / z;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const bool on = pe.id[k] != EMPTY;
        pe.e[k] *= iz;
        const float4 col = pe.col[k];
        pe.c[0] += on ? pe.e[k] * col.x : 0.0f;
        pe.c[1] += on ? pe.e[k] * col.y : 0.0f;
        pe.c[2] += on ? pe.e[k] * col.z : 0.0f;
    }
}

struct PixArgs {
    const float* derived;
    const uint32_t* topk;
    const float* target;
    float* image;
    float* grad;
    float* loss;
    int32_t n, h, w, tiles_x, n_tiles;
    float inv_p;
};

__device__ __forceinline__ bool tile_pixel(const PixArgs& a, int& i, int& j) {
    const int lane = threadIdx.x & (WAVE - 1);
    const int tile = xcd_block(blockIdx.x, gridDim.x) * (blockDim.x / WAVE) + (threadIdx.x / WAVE);
    const int tx = tile % a.tiles_x, ty = tile / a.tiles_x;
    i = tx * TILE + (lane & (TILE - 1));
    j = ty * TILE + (lane / TILE);
    return tile < a.n_tiles && i < a.w && j < a.h;
}

__global__ __launch_bounds__(256) void k_render_fwd(PixArgs a) {
    int i, j;
    if (!tile_pixel(a, i, j)) return;
    const size_t p = (size_t)j * a.w + i;
    const uint4* l = reinterpret_cast<const uint4*>(a.topk + p * K);
    PointEval pe;
    eval_point(a.derived, (uint32_t)a.n, l[0], l[1], (float)i + 0.5f, (float)j + 0.5f, pe);
    a.image[p * 3 + 0] = pe.c[0];
    a.image[p * 3 + 1] = pe.c[1];
    a.image[p * 3 + 2] = pe.c[2];
}

// ---------------------------------------------------------------- budget statistics
//
// Per-site statistics of Sec. 4.5 / Appendix B.5 over the map.  A workgroup
// covers one region (sad_region.h), one wavefront per tile; every listed site
// claims a slot of the region's LDS table, its record is read into LDS once,
// and each pixel's 8 statistics terms per entry are summed per slot.
//
// The LDS sums are exact 64-bit fixed-point integers: a term t of column q
// becomes floor(t 2^E_q) (2^E_q chosen per column from the range of its
// terms), so the integer adds are exact and independent of their order.
// (LDS float atomics are an order of magnitude slower than integer ones on
// this GPU.)  A term with |t 2^E_q| >= 2^53 (far outside the column's range)
// goes to global memory as a float atomic instead, so a slot, which receives
// at most one term per pixel of the region, never overflows.
//
// The sums then leave the workgroup without device-wide float atomics: every
// site has a home region (the one containing its position), the workgroup
// writes its table (keys at the same slots, the summed values of the sites
// whose home is in the 3 x 3 regions around it) to a workspace, and a second
// kernel gives every site the sum of its entries in the 9 tables around its
// home (found by the same hash probing).  Sites listed by a region outside
// that neighbourhood (very wide footprints) are added with float atomics
// directly; their slot keeps a placeholder key so probe chains stay intact.
constexpr int NSTAT = 8;
constexpr double FIX_LIMIT_HI = 0x1p21;  // |t 2^E| < 2^53, i.e. |t 2^(E-32)| < 2^21, goes to the fixed-point sums
constexpr uint32_t PLACEHOLDER = 0xfffffffeu;

// home region of a site from its prepared position (same arithmetic in both kernels)
__device__ __forceinline__ void home_region(float x, float y, RegionGrid rg, int& hx, int& hy) {
    hx = min(max((int)floorf(x * (1.0f / REGION_W)), 0), rg.rgx - 1);
    hy = min(max((int)floorf(y * (1.0f / REGION_H)), 0), rg.rgy - 1);
}

struct StatArgs {
    PixArgs p;
    RegionGrid rg;
    uint32_t* tkeys;               // [regions][SLOTS] site id, EMPTY or PLACEHOLDER
    float* tvals;                  // [regions][SLOTS][NSTAT]
    float* out;                    // [n][NSTAT], accumulated into
    double fix_scale_hi[NSTAT];    // per column: 2^(E_q - 32)
    double fix_inv[NSTAT];         // per column: 2^-E_q
};

// The fixed-point value of a term t, given u = t 2^(E-32) (exact in double,
// |u| < 2^21): floor(t 2^E) as a 64-bit two's-complement integer.  With
// hi = floor(u) and f = u - hi in [0, 1), t 2^E = hi 2^32 + f 2^32 and
// 0 <= f 2^32 < 2^32: hi is the upper word and floor(f 2^32) the lower.  f is
// exact except for a tiny negative u, where f = 1 - |u| is rounded to double;
// the lower word is then off by less than one unit (2^-E), within the
// resolution of the sums.
__device__ __forceinline__ unsigned long long to_fixed(double u) {
    const double hi = floor(u);
    const double lo = (u - hi) * 4294967296.0;
    return ((unsigned long long)(uint32_t)(int32_t)hi << 32) | (unsigned long long)(uint32_t)lo;
}

__global__ __launch_bounds__(WAVE* REGION_WAVES) void k_region_stats(StatArgs b) {
    __shared__ uint32_t keys[SLOTS];
    __shared__ float4 recs[SLOTS * 3];  // prepared record of the site in each slot
    __shared__ unsigned long long acc[NSTAT * SLOTS];
    const PixArgs& a = b.p;
    const uint32_t n = (uint32_t)a.n;

    for (int s = threadIdx.x; s < SLOTS; s += blockDim.x) keys[s] = EMPTY;
    for (int s = threadIdx.x; s < NSTAT * SLOTS; s += blockDim.x) acc[s] = 0ull;

    const int lane = threadIdx.x & (WAVE - 1), wv = threadIdx.x / WAVE;
    const int reg = xcd_block(blockIdx.x, gridDim.x);
    const int rx = reg % b.rg.rgx, ry = reg / b.rg.rgx;
    int i, j;
    region_pixel(rx, ry, wv, lane, i, j);
    const bool inside = i < a.w && j < a.h;
    const size_t p = (size_t)j * a.w + i;
    const float px = (float)i + 0.5f, py = (float)j + 0.5f;

    // The pixel's list, each lane starting at its own offset (anti-diagonal of
    // the tile) so that neighbouring pixels with the same list add to different
    // sites at each step.
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
    __syncthreads();  // keys cleared

    // 1. a slot for every listed site
    int slot[K];
    claim_slots(keys, ids, n, slot);
    __syncthreads();

    // 2. every claimed site's record is read from memory once, into LDS
    for (int s = threadIdx.x; s < SLOTS; s += blockDim.x) {
        const uint32_t id = keys[s];
        if (id == EMPTY) continue;
        const float4* r = reinterpret_cast<const float4*>(a.derived + (size_t)id * REC);
        recs[s * 3 + 0] = r[0];
        recs[s * 3 + 1] = r[1];
        recs[s * 3 + 2] = r[2];
    }
    __syncthreads();

    // 3. the pixel's forward and statistics terms, records from LDS.  When an
    //    entry of some lane of the wavefront found no slot (its probe chain
    //    ran out), the wavefront takes a copy of this code that reads such
    //    records from memory; otherwise every record read is an LDS read.
    // part q (0: x y tau r, 1: cos sin 1/s1 1/s2, 2: colour) of entry k's record
    bool slotted = true;
#pragma unroll
    for (int k = 0; k < K; ++k) slotted &= (ids[k] >= n) | (slot[k] >= 0);
    auto fwd_stats = [&](auto lds_only) {
        auto rec = [&](int k, int q) -> float4 {
            if constexpr (decltype(lds_only)::value)
                return recs[(slot[k] >= 0 ? slot[k] : 0) * 3 + q];
            else
                return slot[k] >= 0 ? recs[slot[k] * 3 + q]
                                    : reinterpret_cast<const float4*>(a.derived + (size_t)ids[k] * REC)[q];
        };
        if (!inside) return;
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
        float z = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            e[k] = use[k] ? __expf(l[k] - mx) : 0.0f;
            z += e[k];
        }
        float c[3] = {0.f, 0.f, 0.f};
        float cl[K][3];  // the entries' colours
        if (z > 0.0f) {
            const float iz = 1.0f / z;
#pragma unroll
            for (int k = 0; k < K; ++k) {
                if (!use[k]) continue;
                e[k] *= iz;
                const float4 col = rec(k, 2);
                c[0] += e[k] * col.x;
                c[1] += e[k] * col.y;
                c[2] += e[k] * col.z;
                cl[k][0] = col.x;
                cl[k][1] = col.y;
                cl[k][2] = col.z;
            }
        }
        // entry k's terms go to its slot's fixed-point sums, or to memory when
        // it has no slot or a term is outside the fixed-point range
        auto add_terms = [&](int k, uint32_t id, const float (&t)[NSTAT]) {
#pragma unroll
            for (int q2 = 0; q2 < NSTAT; ++q2) {
                const double u = (double)t[q2] * b.fix_scale_hi[q2];
                if (slot[k] >= 0 && fabs(u) < FIX_LIMIT_HI)
                    atomicAdd(&acc[q2 * SLOTS + slot[k]], to_fixed(u));
                else
                    unsafeAtomicAdd(&b.out[(size_t)id * NSTAT + q2], t[q2]);
            }
        };
        // mass, energy, removal delta, moments about the site
        float err = 0.0f;
#pragma unroll
        for (int ch = 0; ch < 3; ++ch) err += (c[ch] - tg[ch]) * (c[ch] - tg[ch]);
        // c' of an entry (the blend of the other usable entries) from the
        // normalised weights, which include the largest one (>= 1/8); for
        // the entry holding the largest logit the others are re-weighted
        // relative to the largest remaining logit, so that their blend
        // survives even when their normalised weights underflow
        int top = -1;
#pragma unroll
        for (int k = 0; k < K; ++k) top = (top < 0 && use[k] && l[k] == mx) ? k : top;
        float m2 = -__builtin_inff();
#pragma unroll
        for (int k = 0; k < K; ++k) m2 = (use[k] && k != top) ? fmaxf(m2, l[k]) : m2;
        float ct[3] = {0.f, 0.f, 0.f}, zt = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            if (!use[k] || k == top) continue;
            const float ek = __expf(l[k] - m2);
            zt += ek;
            ct[0] += ek * cl[k][0];
            ct[1] += ek * cl[k][1];
            ct[2] += ek * cl[k][2];
        }
        const float izt = zt > 0.0f ? 1.0f / zt : 0.0f;  // no other entry: c' is black
#pragma unroll
        for (int k = 0; k < K; ++k) {
            if (!use[k]) continue;
            float cp[3] = {0.f, 0.f, 0.f}, zk = 0.0f;
#pragma unroll
            for (int j2 = 0; j2 < K; ++j2) {
                if (j2 == k || !use[j2]) continue;
                zk += e[j2];
                cp[0] += e[j2] * cl[j2][0];
                cp[1] += e[j2] * cl[j2][1];
                cp[2] += e[j2] * cl[j2][2];
            }
            const bool is_top = k == top;
            const float izk = is_top ? izt : 1.0f / zk;
            const float w = e[k];
            // |c' - I|^2 - |c - I|^2 = (c' - c).(c' + c - 2I) with c' - c = w (c' - c_k)
            float dl = 0.0f;
#pragma unroll
            for (int ch = 0; ch < 3; ++ch) {
                const float cpc = (is_top ? ct[ch] : cp[ch]) * izk;
                dl += (cpc - cl[k][ch]) * (cpc + c[ch] - 2.0f * tg[ch]);
            }
            const float4 g0 = rec(k, 0);
            const float dx = px - g0.x, dy = py - g0.y;
            const float wdx = w * dx, wdy = w * dy;
            const float t[NSTAT] = {w, w * err, w * dl, wdx, wdy, wdx * dx, wdx * dy, wdy * dy};
            add_terms(k, ids[k], t);
        }
    };
    if (__all(slotted))
        fwd_stats(std::true_type{});
    else
        fwd_stats(std::false_type{});
    __syncthreads();
    // 4. publish the region's table
    const int region = reg;
    for (int s = threadIdx.x; s < SLOTS; s += blockDim.x) {
        const uint32_t id = keys[s];
        uint32_t key = id;
        if (id != EMPTY) {
            float v[NSTAT];
#pragma unroll
            for (int q2 = 0; q2 < NSTAT; ++q2) v[q2] = (float)((double)(long long)acc[q2 * SLOTS + s] * b.fix_inv[q2]);
            const float4 r0 = recs[s * 3 + 0];
            int hx, hy;
            home_region(r0.x, r0.y, b.rg, hx, hy);
            if (abs(hx - rx) <= 1 && abs(hy - ry) <= 1) {
                float* dst = b.tvals + ((size_t)region * SLOTS + s) * NSTAT;
#pragma unroll
                for (int q2 = 0; q2 < NSTAT; ++q2) dst[q2] = v[q2];
            } else {
                key = PLACEHOLDER;
#pragma unroll
                for (int q2 = 0; q2 < NSTAT; ++q2) unsafeAtomicAdd(&b.out[(size_t)id * NSTAT + q2], v[q2]);
            }
        }
        b.tkeys[(size_t)region * SLOTS + s] = key;
    }
}

// Every site gets the sum of its entries in the tables of the 3 x 3 regions
// around its home region.  A workgroup takes GATHER_SITES sites with one thread
// per (site, table): the thread finds the site in its table by the probing the
// statistics pass used (stopping at an empty slot or after REGION_PROBES
// slots) and loads the entry; then one thread per site adds the 9 partial sums
// in a fixed order to the site's output record.  One writer per site, no
// atomics, and a result that does not depend on scheduling.  A site found in
// no table is not touched.
constexpr int GATHER_SITES = 28;  // 28 x 9 = 252 threads

__global__ __launch_bounds__(256) void k_stats_gather(RegionGrid rg, const uint32_t* __restrict__ tkeys,
                                                      const float* __restrict__ tvals,
                                                      const float* __restrict__ derived, float* __restrict__ out,
                                                      int32_t n) {
    __shared__ float part[GATHER_SITES][9][NSTAT];
    __shared__ int found[GATHER_SITES][9];
    const int ls = threadIdx.x / 9, t = threadIdx.x % 9;
    const int site = blockIdx.x * GATHER_SITES + ls;
    if (ls < GATHER_SITES) {
        float v[NSTAT];
#pragma unroll
        for (int q2 = 0; q2 < NSTAT; ++q2) v[q2] = 0.0f;
        int hit = 0;
        if (site < n) {
            int hx, hy;
            home_region(derived[(size_t)site * REC], derived[(size_t)site * REC + 1], rg, hx, hy);
            const int tx = hx + (t % 3) - 1, ty = hy + (t / 3) - 1;
            if (tx >= 0 && tx < rg.rgx && ty >= 0 && ty < rg.rgy) {
                const size_t base = (size_t)(ty * rg.rgx + tx) * SLOTS;
                uint32_t pos = slot_hash((uint32_t)site);
                for (int pr = 0; pr < REGION_PROBES; ++pr) {
                    const uint32_t key = tkeys[base + pos];
                    if (key == (uint32_t)site) {
                        const float* src = tvals + (base + pos) * NSTAT;
#pragma unroll
                        for (int q2 = 0; q2 < NSTAT; ++q2) v[q2] = src[q2];
                        hit = 1;
                        break;
                    }
                    if (key == EMPTY) break;
                    pos = (pos + slot_step((uint32_t)site)) & (SLOTS - 1);
                }
            }
        }
#pragma unroll
        for (int q2 = 0; q2 < NSTAT; ++q2) part[ls][t][q2] = v[q2];
        found[ls][t] = hit;
    }
    __syncthreads();
    const int s2 = blockIdx.x * GATHER_SITES + (int)threadIdx.x;
    if (threadIdx.x < GATHER_SITES && s2 < n) {
        int any = 0;
        float sum[NSTAT];
#pragma unroll
        for (int q2 = 0; q2 < NSTAT; ++q2) sum[q2] = 0.0f;
        for (int t2 = 0; t2 < 9; ++t2) {
            any |= found[threadIdx.x][t2];
#pragma unroll
            for (int q2 = 0; q2 < NSTAT; ++q2) sum[q2] += part[threadIdx.x][t2][q2];
        }
        if (any) {
            float* gr = out + (size_t)s2 * NSTAT;
#pragma unroll
            for (int q2 = 0; q2 < NSTAT; ++q2) gr[q2] += sum[q2];
        }
    }
}

struct QueryArgs {
    const float* derived;
    const uint32_t* topk;
    const float* xy;
    float* rgb;
    int64_t m, base;  // points base .. m - 1 in this launch
    int32_t n, h, w;
};

__global__ __launch_bounds__(256) void k_query(QueryArgs a) {
    const int64_t t = a.base + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= a.m) return;
    const float2 q = reinterpret_cast<const float2*>(a.xy)[t];
    float* o = a.rgb + t * 3;
    if (!finitef(q.x) || !finitef(q.y)) {
        o[0] = o[1] = o[2] = __builtin_nanf("");
        return;
    }
    const int i = (int)fminf(fmaxf(floorf(q.x), 0.0f), (float)(a.w - 1));
    const int j = (int)fminf(fmaxf(floorf(q.y), 0.0f), (float)(a.h - 1));
    const uint4* l = reinterpret_cast<const uint4*>(a.topk + ((size_t)j * a.w + i) * K);
    PointEval pe;
    eval_point(a.derived, (uint32_t)a.n, l[0], l[1], q.x, q.y, pe);
    o[0] = pe.c[0];
    o[1] = pe.c[1];
    o[2] = pe.c[2];
}

inline int pix_common(const float* derived, int32_t n, int32_t h, int32_t w, const uint32_t* topk) {
    if (!sites_ok(n) || !image_ok(h, w)) return SAD_EINVAL;
    const int64_t pix = int64_t(h) * w;
    if (!array_ok(derived, n, 16) || !array_ok(topk, pix, 16)) return SAD_EINVAL;
    return SAD_OK;
}

inline PixArgs pix_args(const float* derived, int32_t n, int32_t h, int32_t w, const uint32_t* topk) {
    PixArgs a{};
    a.derived = derived;
    a.topk = topk;
    a.n = n;
    a.h = h;
    a.w = w;
    a.tiles_x = tiles_x(w);
    a.n_tiles = tiles_x(w) * tiles_y(h);
    a.inv_p = (h > 0 && w > 0) ? (float)(1.0 / ((double)h * (double)w)) : 0.0f;
    return a;
}

}  // namespace sad

using namespace sad;

extern "C" int sad_render_fwd(const float* derived, int32_t n, int32_t h, int32_t w, const uint32_t* topk,
                              float* image, void* stream) {
    int st = pix_common(derived, n, h, w, topk);
    if (st != SAD_OK) return st;
    const int64_t pix = int64_t(h) * w;
    if (!array_ok(image, pix, 4)) return SAD_EINVAL;
    if (pix == 0) return SAD_OK;
    PixArgs a = pix_args(derived, n, h, w, topk);
    a.image = image;
    clear_error();
    hipLaunchKernelGGL(k_render_fwd, dim3((a.n_tiles + 3) / 4), dim3(256), 0, as_stream(stream), a);
    return launch_status();
}

extern "C" size_t sad_site_stats_workspace_bytes(int32_t h, int32_t w) {
    if (!image_ok(h, w)) return 0;
    const RegionGrid rg = region_grid(h, w);
    return (size_t)rg.rgx * rg.rgy * SLOTS * (sizeof(uint32_t) + NSTAT * sizeof(float));
}

extern "C" int sad_site_stats(const float* derived, int32_t n, int32_t h, int32_t w, const uint32_t* topk,
                              const float* target, float* stats, void* workspace, size_t workspace_bytes,
                              void* stream) {
    int st = pix_common(derived, n, h, w, topk);
    if (st != SAD_OK) return st;
    const int64_t pix = int64_t(h) * w;
    if (!array_ok(target, pix, 4) || !array_ok(stats, n, 16)) return SAD_EINVAL;
    const int64_t sbytes = int64_t(n) * NSTAT * 4;
    if (overlap(stats, sbytes, derived, int64_t(n) * REC * 4) || overlap(stats, sbytes, topk, pix * K * 4) ||
        overlap(stats, sbytes, target, pix * 12))
        return SAD_EINVAL;
    const size_t need = sad_site_stats_workspace_bytes(h, w);
    if (pix > 0 && (workspace == nullptr || !aligned(workspace, 16) || workspace_bytes < need)) return SAD_EINVAL;
    const void* reads[4] = {stats, target, topk, derived};
    const int64_t rbytes[4] = {sbytes, pix * 12, pix * K * 4, int64_t(n) * REC * 4};
    for (int q = 0; q < 4; ++q)
        if (overlap(workspace, (int64_t)need, reads[q], rbytes[q])) return SAD_EINVAL;
    if (pix == 0) return SAD_OK;
    StatArgs b;
    b.p = pix_args(derived, n, h, w, topk);
    b.p.target = target;
    b.out = stats;
    b.rg = region_grid(h, w);
    const size_t nreg = (size_t)b.rg.rgx * b.rg.rgy;
    b.tkeys = reinterpret_cast<uint32_t*>(workspace);
    b.tvals = reinterpret_cast<float*>(b.tkeys + nreg * SLOTS);
    // per-column fixed-point scales 2^E_q with |t| 2^E_q < 2^52 for the usual
    // range of each term: weights <= 1, errors of colours in [0, 1] <= 3 (the
    // removal delta <= 6), offsets from a site inside the image <= D (the
    // smallest power of two >= max(h, w)); other terms go to float atomics
    int lg = 0;
    while ((int64_t(1) << lg) < std::max(h, w)) ++lg;
    const int eq[NSTAT] = {52, 50, 49, 52 - lg, 52 - lg, 52 - 2 * lg, 52 - 2 * lg, 52 - 2 * lg};
    for (int q = 0; q < NSTAT; ++q) {
        b.fix_scale_hi[q] = ldexp(1.0, eq[q] - 32);
        b.fix_inv[q] = ldexp(1.0, -eq[q]);
    }
    clear_error();
    hipLaunchKernelGGL(k_region_stats, dim3((unsigned)nreg), dim3(WAVE * REGION_WAVES), 0, as_stream(stream), b);
    if (n > 0)
        hipLaunchKernelGGL(k_stats_gather, dim3((unsigned)((n + GATHER_SITES - 1) / GATHER_SITES)),
                           dim3(GATHER_SITES * 9), 0, as_stream(stream), b.rg, b.tkeys, b.tvals, derived, stats, n);
    return launch_status();
}

// ---------------------------------------------------------------- statistics without allocation
//
// sad_site_stats_noalloc: the statistics with their region tables in a
// file-scope device array instead of a caller's workspace, for callers that
// cannot allocate.  Every GPU the library runs on holds its own copy of the
// array (SAD_STATS_SCRATCH_BYTES) from the library's load until the process
// ends.  In host code `stats_scratch` names a host-side stand-in, not device
// memory: its device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and only that address is
// passed to kernels.  Calls on one GPU share the array, so calls that overlap
// on one GPU (different streams, no ordering) race.
namespace {

static __device__ __align__(256) unsigned char stats_scratch[SAD_STATS_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mutex;
void* scratch_addr[MAX_DEVICES];  // device address of stats_scratch per device, once resolved

// The current device's address of stats_scratch, resolved on its first use.
int scratch_for_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return SAD_EHIP;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_addr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(stats_scratch)) != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return SAD_EHIP;
        }
        scratch_addr[dev] = p;
    }
    *out = scratch_addr[dev];
    return SAD_OK;
}

}  // namespace

extern "C" int sad_site_stats_noalloc(const float* derived, int32_t n, int32_t h, int32_t w, const uint32_t* topk,
                                      const float* target, float* stats, void* stream) {
    if (!image_ok(h, w)) return SAD_EINVAL;
    if (sad_site_stats_workspace_bytes(h, w) > (size_t)SAD_STATS_SCRATCH_BYTES) return SAD_EUNSUPPORTED;
    if (int64_t(h) * w == 0) return sad_site_stats(derived, n, h, w, topk, target, stats, nullptr, 0, stream);
    void* scratch = nullptr;
    const int st = scratch_for_current_device(&scratch);
    if (st != SAD_OK) return st;
    return sad_site_stats(derived, n, h, w, topk, target, stats, scratch, SAD_STATS_SCRATCH_BYTES, stream);
}

extern "C" int sad_query_points(const float* derived, int32_t n, int32_t h, int32_t w, const uint32_t* topk,
                                const float* xy, int64_t m, float* rgb, void* stream) {
    int st = pix_common(derived, n, h, w, topk);
    if (st != SAD_OK) return st;
    if (m < 0 || m > MAX_QUERIES) return SAD_EINVAL;
    if (!array_ok(xy, m, 8) || !array_ok(rgb, m, 4)) return SAD_EINVAL;
    if (m > 0 && int64_t(h) * w == 0) return SAD_EINVAL;  // queries need a list to read
    if (m == 0) return SAD_OK;
    QueryArgs a;
    a.derived = derived;
    a.topk = topk;
    a.xy = xy;
    a.rgb = rgb;
    a.m = m;
    a.n = n;
    a.h = h;
    a.w = w;
    clear_error();
    for (a.base = 0; a.base < m; a.base += QUERY_CHUNK)  // a dispatch holds fewer than 2^32 work-items
        hipLaunchKernelGGL(k_query, dim3((unsigned)((std::min(QUERY_CHUNK, m - a.base) + 255) / 256)), dim3(256), 0,
                           as_stream(stream), a);
    return launch_status();
}
