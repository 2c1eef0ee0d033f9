// sad_render.hip -- soft anisotropic Apollonius render (Sec. 4.2), its
// backward pass with the per-site gradient reduction (Sec. 4.8, Appendix
// B.4), and random-access queries (Sec. 6.6).
//
// Pixel kernels use the same mapping as the propagation pass: one wavefront
// per 8x8 tile, 4 consecutive tiles per 256-thread workgroup, so a workgroup
// covers a 32x8 pixel strip.
//
// Gradient reduction: many pixels of a strip share sites, so the per-pixel
// contributions are first summed in LDS, in an open-addressing table keyed by
// site id (multiplicative hash, linear probing, bounded probe count; keys
// claimed by compare-and-swap), then each occupied slot is flushed with one
// global float atomic per parameter.  A contribution whose site finds no slot
// within the probe bound goes straight to global memory.
#include "sad_device.h"
#include "sad_host.h"

namespace sad {

// Evaluate one point: the usable entries of its list, their logits, the
// softmax weights and the blended colour.  Returns the number of entries.
struct PointEval {
    int n;
    uint32_t id[K];
    float l[K];
    float e[K];  // exp(l - max), later normalised to weights
    float c[3];
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
        uint32_t id = ids[k];
        if (id >= nsites) continue;
        Geo g = load_geo(derived, id);
        if (!(g.g0.x >= 0.0f)) continue;
        float s = logit(g, px, py);
        if (!finitef(s)) continue;
        pe.id[k] = id;
        pe.l[k] = s;
        mx = fmaxf(mx, s);
        pe.n++;
    }
    float z = 0.0f;
    pe.c[0] = pe.c[1] = pe.c[2] = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        pe.e[k] = 0.0f;
        if (pe.id[k] == EMPTY) continue;
        pe.e[k] = __expf(pe.l[k] - mx);
        z += pe.e[k];
    }
    if (pe.n == 0) return;
    float iz = 1.0f / z;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        if (pe.id[k] == EMPTY) continue;
        pe.e[k] *= iz;
        const float4 col = reinterpret_cast<const float4*>(derived + (size_t)pe.id[k] * REC)[2];
        pe.c[0] += pe.e[k] * col.x;
        pe.c[1] += pe.e[k] * col.y;
        pe.c[2] += pe.e[k] * col.z;
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
    const int tile = blockIdx.x * (blockDim.x / WAVE) + (threadIdx.x / WAVE);
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

constexpr int HASH_SLOTS = 512;
constexpr int HASH_PROBES = 16;
constexpr int NGRAD = 10;

__global__ __launch_bounds__(256) void k_render_bwd(PixArgs a) {
    __shared__ uint32_t keys[HASH_SLOTS];
    __shared__ float acc[HASH_SLOTS * NGRAD];
    __shared__ float wsum[256 / WAVE];

    for (int s = threadIdx.x; s < HASH_SLOTS; s += blockDim.x) keys[s] = EMPTY;
    for (int s = threadIdx.x; s < HASH_SLOTS * NGRAD; s += blockDim.x) acc[s] = 0.0f;
    __syncthreads();

    int i, j;
    const bool inside = tile_pixel(a, i, j);
    float lsum = 0.0f;
    if (inside) {
        const size_t p = (size_t)j * a.w + i;
        const float px = (float)i + 0.5f, py = (float)j + 0.5f;
        const uint4* l = reinterpret_cast<const uint4*>(a.topk + p * K);
        PointEval pe;
        eval_point(a.derived, (uint32_t)a.n, l[0], l[1], px, py, pe);
        float g[3];
#pragma unroll
        for (int ch = 0; ch < 3; ++ch) {
            float r = pe.c[ch] - a.target[p * 3 + ch];
            lsum += r * r;
            g[ch] = 2.0f * r * a.inv_p;
            if (a.image) a.image[p * 3 + ch] = pe.c[ch];
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const uint32_t id = pe.id[k];
            if (id == EMPTY) continue;
            const float4* rec = reinterpret_cast<const float4*>(a.derived + (size_t)id * REC);
            const float4 g0 = rec[0], g1 = rec[1], col = rec[2];
            const float w = pe.e[k];
            const float tau = g0.z, cs = g1.x, sn = g1.y, is1 = g1.z, is2 = g1.w;
            // g.(c_i - c): differences first, so a site coloured like the pixel
            // does not lose its gradient to cancellation
            const float delta = w * (g[0] * (col.x - pe.c[0]) + g[1] * (col.y - pe.c[1]) + g[2] * (col.z - pe.c[2]));
            float t[NGRAD];
            t[4] = w * g[0];
            t[5] = w * g[1];
            t[6] = w * g[2];
            t[2] = delta * pe.l[k];
            t[3] = tau * delta;
            const float dx = px - g0.x, dy = py - g0.y;
            const float ar = dx * cs + dy * sn, br = dy * cs - dx * sn;
            const float aa = ar * is1, bb = br * is2;
            const float q = aa * aa + bb * bb;
            t[0] = t[1] = t[7] = t[8] = t[9] = 0.0f;
            if (q > 0.0f) {
                const float kap2 = -tau * delta * __builtin_amdgcn_rsqf(q);  // 2 kappa
                t[0] = -kap2 * (aa * is1 * cs - bb * is2 * sn);
                t[1] = -kap2 * (aa * is1 * sn + bb * is2 * cs);
                t[7] = kap2 * ar * br * ((is1 - is2) * (is1 + is2));  // 1/s1^2 - 1/s2^2 without cancellation
                t[8] = -kap2 * aa * aa;
                t[9] = -kap2 * bb * bb;
            }
            // find or claim the site's slot
            uint32_t h = (id * 2654435761u) >> 23;  // 9-bit multiplicative hash
            int slot = -1;
            for (int pr = 0; pr < HASH_PROBES; ++pr) {
                const uint32_t s = (h + pr) & (HASH_SLOTS - 1);
                uint32_t cur = keys[s];
                if (cur == EMPTY) cur = atomicCAS(&keys[s], EMPTY, id);
                if (cur == EMPTY || cur == id) {
                    slot = (int)s;
                    break;
                }
            }
            if (slot >= 0) {
#pragma unroll
                for (int q2 = 0; q2 < NGRAD; ++q2) atomicAdd(&acc[slot * NGRAD + q2], t[q2]);
            } else {
#pragma unroll
                for (int q2 = 0; q2 < NGRAD; ++q2) unsafeAtomicAdd(&a.grad[(size_t)id * REC + q2], t[q2]);
            }
        }
    }
    if (a.loss) {
        float ws = wave_sum(lsum);
        if ((threadIdx.x & (WAVE - 1)) == 0) wsum[threadIdx.x / WAVE] = ws;
    }
    __syncthreads();
    for (int s = threadIdx.x; s < HASH_SLOTS; s += blockDim.x) {
        const uint32_t id = keys[s];
        if (id == EMPTY) continue;
#pragma unroll
        for (int q2 = 0; q2 < NGRAD; ++q2) unsafeAtomicAdd(&a.grad[(size_t)id * REC + q2], acc[s * NGRAD + q2]);
    }
    if (a.loss && threadIdx.x == 0) {
        float tot = 0.0f;
        for (int k = 0; k < (int)(blockDim.x / WAVE); ++k) tot += wsum[k];
        unsafeAtomicAdd(a.loss, tot * a.inv_p);
    }
}

struct QueryArgs {
    const float* derived;
    const uint32_t* topk;
    const float* xy;
    float* rgb;
    int64_t m;
    int32_t n, h, w;
};

__global__ __launch_bounds__(256) void k_query(QueryArgs a) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
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

extern "C" int sad_render_bwd(const float* derived, int32_t n, int32_t h, int32_t w, const uint32_t* topk,
                              const float* target, float* grad, float* loss, float* image, void* stream) {
    int st = pix_common(derived, n, h, w, topk);
    if (st != SAD_OK) return st;
    const int64_t pix = int64_t(h) * w;
    if (!array_ok(target, pix, 4) || !array_ok(grad, n, 16)) return SAD_EINVAL;
    if ((loss && !aligned(loss, 4)) || (image && !aligned(image, 4))) return SAD_EINVAL;
    if (overlap(grad, int64_t(n) * REC * 4, derived, int64_t(n) * REC * 4)) return SAD_EINVAL;
    if (pix == 0) return SAD_OK;
    PixArgs a = pix_args(derived, n, h, w, topk);
    a.target = target;
    a.grad = grad;
    a.loss = loss;
    a.image = image;
    clear_error();
    hipLaunchKernelGGL(k_render_bwd, dim3((a.n_tiles + 3) / 4), dim3(256), 0, as_stream(stream), a);
    return launch_status();
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
    hipLaunchKernelGGL(k_query, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, as_stream(stream), a);
    return launch_status();
}
