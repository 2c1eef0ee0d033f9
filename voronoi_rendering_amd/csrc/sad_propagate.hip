// sad_propagate.hip -- one top-K propagation pass (Sec. 4.3, Figure 5).
//
// Mapping: one wavefront (64 lanes) per 8x8 pixel tile, one lane per pixel;
// a 256-thread workgroup holds 4 consecutive tiles.  The tile is also the unit
// of the global probe: its 64 injected ids are drawn once per wavefront, one
// per lane, and shared by all pixels of the tile.
//
// Per lane the list is a sorted register array (TopK).  Candidates come from
// the pixel's own previous list, the previous lists of the 4 pixels at
// +-stride (read-only map, so the pass is a Jacobi update and the result does
// not depend on scheduling) and the tile's probe ids.
//
// Culling of probe ids: each lane bounds its probe site's logit over the
// whole tile (distance from the site to the tile's box of pixel centres times
// the smaller inverse scale, see probe_may_enter) and the wavefront keeps only
// the sites whose bound can beat the weakest current 8th-best logit of the
// tile.  The bound includes the float32 rounding of the exact logit
// evaluation, so a culled site can never enter any list: the culling changes
// the work, not the result.
#include "sad_device.h"
#include "sad_host.h"

namespace sad {

struct PropArgs {
    const float* derived;
    const uint32_t* prev;
    uint32_t* next;
    uint64_t seed;
    int32_t n, h, w, stride, inject, tiles_x, n_tiles;
    uint32_t pass_index;
};

__device__ __forceinline__ void consider(TopK& t, const float* __restrict__ derived, uint32_t n, uint32_t id,
                                         float px, float py) {
    if (id >= n) return;  // also drops the EMPTY sentinel
    Geo g = load_geo(derived, id);
    if (!(g.g0.x >= 0.0f)) return;  // inactive site
    float s = logit(g, px, py);
    if (s != s) return;  // NaN logits are dropped
    t.insert(s, id);
}

// Can the probe site (geometry g) rank among the 8 best of any pixel of the
// tile whose pixel centres span [bx0, bx1] x [by0, by1], given that every
// pixel of the tile already holds 8 entries of logit >= thr?
//
// For every pixel centre P of the box, ||P - p||_G >= m ||P - p||_2 >= m D,
// with m the smaller inverse scale and D the distance from p to the box, so
// the exact logit is at most -tau (m D - r).  The float32 evaluation of the
// logit differs from the exact one by at most tau u ((8.5 kappa + 4) sqrt(q)
// + 2 |r|), u = 2^-24, kappa = M/m the anisotropy ratio; for kappa <= 1024
// this is below 2^-8 (tau sqrt(q) + tau |r|).  The bound therefore keeps a
// 2^-8 relative margin on both terms, which also covers the rounding of the
// bound's own evaluation.  Sites with non-finite values or extreme anisotropy
// are never culled.
__device__ __forceinline__ bool probe_may_enter(const Geo& g, float thr, float bx0, float bx1, float by0,
                                                float by1) {
    float tau = g.g0.z, r = g.g0.w, is1 = g.g1.z, is2 = g.g1.w;
    float m = fminf(is1, is2), M = fmaxf(is1, is2);
    bool boundable = finitef(g.g0.x) && finitef(g.g0.y) && finitef(tau) && finitef(r) && finitef(M) && m > 0.0f &&
                     M <= 1024.0f * m;
    if (!boundable) return true;
    float ex = fmaxf(fmaxf(bx0 - g.g0.x, g.g0.x - bx1), 0.0f);
    float ey = fmaxf(fmaxf(by0 - g.g0.y, g.g0.y - by1), 0.0f);
    float dist = __builtin_sqrtf(ex * ex + ey * ey);
    float A = tau * (m * dist);
    float C = tau * r;
    float ub = (C - A * (1.0f - 0x1p-8f)) + 0x1p-8f * (tau * fabsf(r));
    return !(ub < thr);
}

__global__ __launch_bounds__(256) void k_propagate(PropArgs a) {
    const int lane = threadIdx.x & (WAVE - 1);
    const int tile = blockIdx.x * (blockDim.x / WAVE) + (threadIdx.x / WAVE);
    if (tile >= a.n_tiles) return;  // uniform per wavefront
    const int tx = tile % a.tiles_x, ty = tile / a.tiles_x;
    const int i = tx * TILE + (lane & (TILE - 1));
    const int j = ty * TILE + (lane / TILE);
    const bool inside = i < a.w && j < a.h;
    const float px = (float)i + 0.5f, py = (float)j + 0.5f;
    const uint32_t n = (uint32_t)a.n;

    TopK t;
    t.clear();
    if (inside && a.prev) {
        const int nb[5][2] = {{0, 0}, {a.stride, 0}, {-a.stride, 0}, {0, a.stride}, {0, -a.stride}};
#pragma unroll
        for (int q = 0; q < 5; ++q) {
            int ii = i + nb[q][0], jj = j + nb[q][1];
            if (ii < 0 || ii >= a.w || jj < 0 || jj >= a.h) continue;
            const uint4* l = reinterpret_cast<const uint4*>(a.prev + ((size_t)jj * a.w + ii) * K);
            uint4 l0 = l[0], l1 = l[1];
            consider(t, a.derived, n, l0.x, px, py);
            consider(t, a.derived, n, l0.y, px, py);
            consider(t, a.derived, n, l0.z, px, py);
            consider(t, a.derived, n, l0.w, px, py);
            consider(t, a.derived, n, l1.x, px, py);
            consider(t, a.derived, n, l1.y, px, py);
            consider(t, a.derived, n, l1.z, px, py);
            consider(t, a.derived, n, l1.w, px, py);
        }
    }

    if (a.inject > 0) {
        // the weakest 8th-best logit of the tile (+inf for lanes outside the image)
        float thr = wave_min(inside ? t.s[K - 1] : __builtin_inff());
        uint32_t pid = EMPTY;
        bool keep = false;
        if (lane < a.inject) {
            pid = probe_id(a.seed, a.pass_index, (uint32_t)tile, (uint32_t)lane, n);
            Geo g = load_geo(a.derived, pid);
            if (g.g0.x >= 0.0f) {
                float bx0 = (float)(tx * TILE) + 0.5f, by0 = (float)(ty * TILE) + 0.5f;
                float bx1 = (float)min(tx * TILE + TILE - 1, a.w - 1) + 0.5f;
                float by1 = (float)min(ty * TILE + TILE - 1, a.h - 1) + 0.5f;
                keep = probe_may_enter(g, thr, bx0, bx1, by0, by1);
            }
        }
        uint64_t mask = __ballot(keep);
        while (mask) {
            int q = __builtin_ctzll(mask);
            mask &= mask - 1;
            uint32_t id = (uint32_t)__builtin_amdgcn_readlane((int)pid, q);
            if (inside) consider(t, a.derived, n, id, px, py);
        }
    }

    if (inside) {
        uint4* o = reinterpret_cast<uint4*>(a.next + ((size_t)j * a.w + i) * K);
        o[0] = make_uint4(t.id[0], t.id[1], t.id[2], t.id[3]);
        o[1] = make_uint4(t.id[4], t.id[5], t.id[6], t.id[7]);
    }
}

}  // namespace sad

using namespace sad;

extern "C" int sad_propagate_topk(const float* derived, int32_t n, int32_t h, int32_t w, const uint32_t* topk_prev,
                                  uint32_t* topk_next, int32_t stride, uint64_t seed, uint32_t pass_index,
                                  int32_t inject_per_tile, void* stream) {
    if (!sites_ok(n) || !image_ok(h, w) || stride < 1 || inject_per_tile < 0) return SAD_EINVAL;
    if (inject_per_tile > SAD_MAX_INJECT) return SAD_EUNSUPPORTED;
    const int64_t pix = int64_t(h) * w;
    if (!array_ok(derived, n, 16) || !array_ok(topk_next, pix, 16)) return SAD_EINVAL;
    if (topk_prev && !aligned(topk_prev, 16)) return SAD_EINVAL;
    if (overlap(topk_prev, pix * K * 4, topk_next, pix * K * 4)) return SAD_EINVAL;
    const int64_t ntiles = int64_t(tiles_x(w)) * tiles_y(h);
    if (ntiles > MAX_TILES) return SAD_EINVAL;
    if (pix == 0) return SAD_OK;
    PropArgs a;
    a.derived = derived;
    a.prev = topk_prev;
    a.next = topk_next;
    a.seed = seed;
    a.n = n;
    a.h = h;
    a.w = w;
    a.stride = stride;
    a.inject = n > 0 ? inject_per_tile : 0;
    a.tiles_x = tiles_x(w);
    a.n_tiles = (int32_t)ntiles;
    a.pass_index = pass_index;
    clear_error();
    hipLaunchKernelGGL(k_propagate, dim3((unsigned)((ntiles + 3) / 4)), dim3(256), 0, as_stream(stream), a);
    return launch_status();
}
