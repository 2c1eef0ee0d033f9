// sad_packed.hip -- packed 16-byte evaluation records (Appendix B.2,
// "Packed storage for evaluation") and random access from them (Sec. 6.6).
//
// A record is four 32-bit words: w0 = x/W and y/H as 15-bit UNORM (bits 0-14,
// 15-29) and the usable flag (bit 31); w1 = colour as 11/11/10-bit UNORM;
// w2 = log tau' and r' as 16/16-bit UNORM; w3 = the direction as a 16-bit
// angle code over [-pi, pi] and the log-anisotropy a as float16.  The pages'
// metric has determinant 1; a site with two scales is stored as the same
// logit's determinant-1 site: a = log s2 - log s1, hs = (log s1 + log s2) / 2,
// log tau' = log tau - hs, r' = r exp(hs).  Colour, log tau' and r' are coded
// over per-image ranges (min, max - min over the usable sites), ten floats
// kept beside the array.  Packing is float32 in a fixed order with the
// correctly rounded exp, so the codes are exact functions of the sites.
//
// The query decodes each list entry from its record: positions in float64
// (the offset to the point is the only quantity that cancels), the rest in
// float32 with the hardware exp, sine and cosine (angle code in turns).
#include <algorithm>

#include "sad_crmath.h"
#include "sad_device.h"
#include "sad_host.h"

namespace sad {

constexpr int NPACK = 5;  // log tau', r', c_r, c_g, c_b

__device__ __forceinline__ uint32_t ordered_key(float v) {
    const uint32_t u = __float_as_uint(v + 0.0f);  // -0 as +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ bool usable_site(const float* derived, int32_t n, int i) {
    return i < n && derived[(size_t)i * REC] >= 0.0f;
}

__device__ __forceinline__ void packed_values(const float* p, float v[NPACK]) {
    const float hs = 0.5f * (p[8] + p[9]);
    v[0] = p[2] - hs;
    v[1] = p[3] * exp_cr(hs);
    v[2] = p[4];
    v[3] = p[5];
    v[4] = p[6];
}

__device__ __forceinline__ uint32_t unorm_code(float t, uint32_t maxq) {
    t = fminf(fmaxf(t, 0.0f), 1.0f);  // NaN becomes 0
    return (uint32_t)rintf(t * (float)maxq);
}

// keys[2k] = min key (all ones when empty), keys[2k + 1] = max key (0 when empty)
__global__ void k_pack_clear(uint32_t* keys) {
    const int t = threadIdx.x;
    if (t < 2 * NPACK) keys[t] = (t & 1) ? 0u : 0xFFFFFFFFu;
}

constexpr int PACK_WG = 256;

__global__ __launch_bounds__(PACK_WG) void k_pack_range(const float* __restrict__ params,
                                                        const float* __restrict__ derived, int32_t n,
                                                        uint32_t* keys) {
    __shared__ uint32_t lo[PACK_WG / WAVE][NPACK], hi[PACK_WG / WAVE][NPACK];
    const int i = blockIdx.x * PACK_WG + threadIdx.x;
    uint32_t kl[NPACK], kh[NPACK];
#pragma unroll
    for (int k = 0; k < NPACK; ++k) {
        kl[k] = 0xFFFFFFFFu;
        kh[k] = 0u;
    }
    if (usable_site(derived, n, i)) {
        float v[NPACK];
        packed_values(params + (size_t)i * REC, v);
#pragma unroll
        for (int k = 0; k < NPACK; ++k)
            if (v[k] == v[k]) kl[k] = kh[k] = ordered_key(v[k]);
    }
    // wavefront minimum and maximum, then one atomic per workgroup and value
#pragma unroll
    for (int k = 0; k < NPACK; ++k)
#pragma unroll
        for (int off = 1; off < WAVE; off <<= 1) {
            kl[k] = min(kl[k], (uint32_t)__shfl_xor((int)kl[k], off));
            kh[k] = max(kh[k], (uint32_t)__shfl_xor((int)kh[k], off));
        }
    const int wv = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
    if (lane == 0)
#pragma unroll
        for (int k = 0; k < NPACK; ++k) {
            lo[wv][k] = kl[k];
            hi[wv][k] = kh[k];
        }
    __syncthreads();
    if (threadIdx.x < NPACK) {
        const int k = threadIdx.x;
        uint32_t a = lo[0][k], b = hi[0][k];
        for (int x = 1; x < PACK_WG / WAVE; ++x) {
            a = min(a, lo[x][k]);
            b = max(b, hi[x][k]);
        }
        if (a != 0xFFFFFFFFu) atomicMin(keys + 2 * k, a);
        if (b != 0u) atomicMax(keys + 2 * k + 1, b);
    }
}

// keys -> (min, max - min) in place; no values gives 0, 0
__global__ void k_pack_finish(float* qp) {
    const int k = threadIdx.x;
    if (k >= NPACK) return;
    uint32_t* keys = reinterpret_cast<uint32_t*>(qp);
    const uint32_t a = keys[2 * k], b = keys[2 * k + 1];
    const bool empty = a == 0xFFFFFFFFu;
    const float lo = empty ? 0.0f : key_value(a), hi = empty ? 0.0f : key_value(b);
    qp[2 * k] = lo;
    qp[2 * k + 1] = hi - lo;
}

__global__ __launch_bounds__(256) void k_pack(const float* __restrict__ params, const float* __restrict__ derived,
                                              int32_t n, int32_t h, int32_t w, const float* __restrict__ qp,
                                              uint4* __restrict__ packed) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    if (!usable_site(derived, n, i)) {
        packed[i] = make_uint4(0u, 0u, 0u, 0u);
        return;
    }
    const float* p = params + (size_t)i * REC;
    float v[NPACK];
    packed_values(p, v);
    constexpr uint32_t maxq[NPACK] = {65535u, 65535u, 2047u, 2047u, 1023u};
    uint32_t q[NPACK];
#pragma unroll
    for (int k = 0; k < NPACK; ++k) {
        const float sc = qp[2 * k + 1];
        q[k] = unorm_code(sc > 0.0f ? (v[k] - qp[2 * k]) / sc : 0.0f, maxq[k]);
    }
    const uint32_t qx = unorm_code(p[0] / (float)w, 32767u), qy = unorm_code(p[1] / (float)h, 32767u);
    const float th = p[7] - 6.28318548f * rintf(p[7] * 0.159154937f);
    const uint32_t qt = unorm_code((th + 3.14159274f) * 0.159154937f, 65535u);
    const _Float16 a = (_Float16)(p[9] - p[8]);  // round to nearest even
    const uint32_t ab = (uint32_t)__builtin_bit_cast(uint16_t, a);
    packed[i] = make_uint4(qx | (qy << 15) | 0x80000000u, q[2] | (q[3] << 11) | (q[4] << 22), q[0] | (q[1] << 16),
                           qt | (ab << 16));
}

struct QPArgs {
    const uint4* packed;
    const float* qp;
    const uint32_t* topk;
    const float* xy;
    float* rgb;
    int64_t m, base;  // points base .. m - 1 in this launch
    int32_t n, h, w;
};

__global__ __launch_bounds__(256) void k_query_packed(QPArgs a) {
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
    const uint4* lp = reinterpret_cast<const uint4*>(a.topk + ((size_t)j * a.w + i) * K);
    const uint4 l0 = lp[0], l1 = lp[1];
    const uint32_t ids[K] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
    const uint32_t n = (uint32_t)a.n;
    float l[K], c[K][3];
    bool ok[K];
    float mx = -__builtin_inff();
    if (n > 0) {
        uint4 r[K];
#pragma unroll
        for (int k = 0; k < K; ++k) r[k] = a.packed[ids[k] < n ? ids[k] : 0u];  // all loads first
        // per-image ranges and steps (uniform across the wavefront)
        float lo[2 * NPACK];
#pragma unroll
        for (int k = 0; k < 2 * NPACK; ++k) lo[k] = a.qp[k];
        const float st_lt = lo[1] / 65535.0f, st_r = lo[3] / 65535.0f;
        const float st_c[3] = {lo[5] / 2047.0f, lo[7] / 2047.0f, lo[9] / 1023.0f};
        const double sx = (double)a.w / 32767.0, sy = (double)a.h / 32767.0;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const uint4 w4 = r[k];
            const float dx = (float)((double)q.x - (double)(w4.x & 32767u) * sx);
            const float dy = (float)((double)q.y - (double)((w4.x >> 15) & 32767u) * sy);
            const float tau = __expf(lo[0] + (float)(w4.z & 65535u) * st_lt);
            const float rr = lo[2] + (float)(w4.z >> 16) * st_r;
            const float turn = (float)(w4.w & 65535u) * (1.0f / 65535.0f) - 0.5f;  // angle / (2 pi)
            const float sn = __builtin_amdgcn_sinf(turn), cs = __builtin_amdgcn_cosf(turn);
            const float an = (float)__builtin_bit_cast(_Float16, (uint16_t)(w4.w >> 16));
            const float u = cs * dx + sn * dy, v = cs * dy - sn * dx;
            const float s = -tau * (__builtin_sqrtf(__expf(an) * (u * u) + __expf(-an) * (v * v)) - rr);
            ok[k] = (ids[k] < n) & ((w4.x >> 31) != 0u) & finitef(s);
            l[k] = ok[k] ? s : 0.0f;
            mx = ok[k] ? fmaxf(mx, s) : mx;
            c[k][0] = lo[4] + (float)(w4.y & 2047u) * st_c[0];
            c[k][1] = lo[6] + (float)((w4.y >> 11) & 2047u) * st_c[1];
            c[k][2] = lo[8] + (float)(w4.y >> 22) * st_c[2];
        }
    } else {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            ok[k] = false;
            l[k] = 0.0f;
            c[k][0] = c[k][1] = c[k][2] = 0.0f;
        }
    }
    float e[K], z = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        e[k] = ok[k] ? __expf(l[k] - mx) : 0.0f;
        z += e[k];
    }
    float out[3] = {0.0f, 0.0f, 0.0f};
    if (z > 0.0f) {
        const float iz = 1.0f / z;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const float wk = e[k] * iz;
#pragma unroll
            for (int ch = 0; ch < 3; ++ch) out[ch] += ok[k] ? wk * c[k][ch] : 0.0f;
        }
    }
    o[0] = out[0];
    o[1] = out[1];
    o[2] = out[2];
}

}  // namespace sad

using namespace sad;

extern "C" int sad_pack_sites(const float* params, const float* derived, int32_t n, int32_t h, int32_t w,
                              uint32_t* packed, float* qparams, void* stream) {
    if (!sites_ok(n) || !image_ok(h, w)) return SAD_EINVAL;
    if (n > 0 && (h == 0 || w == 0)) return SAD_EINVAL;  // positions are coded relative to the image
    if (!array_ok(params, n, 16) || !array_ok(derived, n, 16) || !array_ok(packed, n, 16) ||
        !array_ok(qparams, 2 * NPACK, 4) || qparams == nullptr)
        return SAD_EINVAL;
    const int64_t rb = int64_t(n) * REC * 4, pb = int64_t(n) * 16, qb = 2 * NPACK * 4;
    if (overlap(packed, pb, params, rb) || overlap(packed, pb, derived, rb) || overlap(qparams, qb, params, rb) ||
        overlap(qparams, qb, derived, rb) || overlap(qparams, qb, packed, pb))
        return SAD_EINVAL;
    hipStream_t s = as_stream(stream);
    clear_error();
    uint32_t* keys = reinterpret_cast<uint32_t*>(qparams);  // the reduction's keys, then the ranges
    hipLaunchKernelGGL(k_pack_clear, dim3(1), dim3(64), 0, s, keys);
    if (n > 0)
        hipLaunchKernelGGL(k_pack_range, dim3((unsigned)((n + PACK_WG - 1) / PACK_WG)), dim3(PACK_WG), 0, s, params,
                           derived, n, keys);
    hipLaunchKernelGGL(k_pack_finish, dim3(1), dim3(64), 0, s, qparams);
    if (n > 0)
        hipLaunchKernelGGL(k_pack, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, params, derived, n, h, w,
                           qparams, reinterpret_cast<uint4*>(packed));
    return launch_status();
}

extern "C" int sad_query_packed(const uint32_t* packed, const float* qparams, int32_t n, int32_t h, int32_t w,
                                const uint32_t* topk, const float* xy, int64_t m, float* rgb, void* stream) {
    if (!sites_ok(n) || !image_ok(h, w) || m < 0 || m > MAX_QUERIES) return SAD_EINVAL;
    const int64_t pix = int64_t(h) * w;
    if (m > 0 && pix == 0) return SAD_EINVAL;  // a point needs a list
    if (!array_ok(packed, n, 16) || !array_ok(qparams, 2 * NPACK, 4) || qparams == nullptr ||
        !array_ok(topk, m > 0 ? pix : 0, 16) || !array_ok(xy, m, 8) || !array_ok(rgb, m, 4))
        return SAD_EINVAL;
    const int64_t ob = m * 12;
    if (overlap(rgb, ob, packed, int64_t(n) * 16) || overlap(rgb, ob, qparams, 2 * NPACK * 4) ||
        overlap(rgb, ob, topk, pix * K * 4) || overlap(rgb, ob, xy, m * 8))
        return SAD_EINVAL;
    if (m == 0) return SAD_OK;
    QPArgs a;
    a.packed = reinterpret_cast<const uint4*>(packed);
    a.qp = qparams;
    a.topk = topk;
    a.xy = xy;
    a.rgb = rgb;
    a.m = m;
    a.n = n;
    a.h = h;
    a.w = w;
    clear_error();
    for (a.base = 0; a.base < m; a.base += QUERY_CHUNK)  // a dispatch holds fewer than 2^32 work-items
        hipLaunchKernelGGL(k_query_packed, dim3((unsigned)((std::min(QUERY_CHUNK, m - a.base) + 255) / 256)),
                           dim3(256), 0, as_stream(stream), a);
    return launch_status();
}
