// sad_sites.hip -- per-site kernels: site preparation and the Adam step.
//
// One thread per site, 256-thread workgroups (the per-site dispatch shape of
// the paper's Table B13).  Both kernels are small next to the pixel kernels:
// they touch 48-byte records of N sites, while a pixel pass touches 32 bytes
// of every pixel's list.
#include "sad_device.h"
#include "sad_host.h"
#include "sad_prepare.h"

namespace sad {

__global__ __launch_bounds__(256) void k_prepare(const float* __restrict__ params, int32_t n,
                                                  float* __restrict__ derived) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const float4* p = reinterpret_cast<const float4*>(params + (size_t)i * REC);
    prepare_one(p[0], p[1], p[2], reinterpret_cast<float4*>(derived + (size_t)i * REC));
}

struct AdamArgs {
    float lr[5];
    float beta1, beta2, eps, bc1, bc2;
    float w, h;
};

// One Adam update of one parameter, one float32 rounding per operation.
__device__ __forceinline__ float adam_one(float p, float g, float& m, float& v, float lr, const AdamArgs& a,
                                          float omb1, float omb2) {
    m = a.beta1 * m + omb1 * g;
    v = a.beta2 * v + omb2 * (g * g);
    float mhat = m / a.bc1;
    float vhat = v / a.bc2;
    float step = mhat / (__builtin_sqrtf(vhat) + a.eps);
    return p - lr * step;
}

__global__ __launch_bounds__(256) void k_adam(float* __restrict__ params, float* __restrict__ grad,
                                               float* __restrict__ mom1, float* __restrict__ mom2, int32_t n,
                                               AdamArgs a, float* __restrict__ derived,
                                               float4* __restrict__ probe) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float4* P = reinterpret_cast<float4*>(params + (size_t)i * REC);
    float4* G = reinterpret_cast<float4*>(grad + (size_t)i * REC);
    float4* M = reinterpret_cast<float4*>(mom1 + (size_t)i * REC);
    float4* V = reinterpret_cast<float4*>(mom2 + (size_t)i * REC);
    float4 p0 = P[0], p1 = P[1], p2 = P[2];
    if (p0.x >= 0.0f) {
        float4 g0 = G[0], g1 = G[1], g2 = G[2];
        float4 m0 = M[0], m1 = M[1], m2 = M[2];
        float4 v0 = V[0], v1 = V[1], v2 = V[2];
        float omb1 = 1.0f - a.beta1, omb2 = 1.0f - a.beta2;
        // parameter order: x, y, log_tau, r | c_r, c_g, c_b, theta | log_s1, log_s2
        p0.x = adam_one(p0.x, g0.x, m0.x, v0.x, a.lr[0], a, omb1, omb2);
        p0.y = adam_one(p0.y, g0.y, m0.y, v0.y, a.lr[0], a, omb1, omb2);
        p0.z = adam_one(p0.z, g0.z, m0.z, v0.z, a.lr[1], a, omb1, omb2);
        p0.w = adam_one(p0.w, g0.w, m0.w, v0.w, a.lr[2], a, omb1, omb2);
        p1.x = adam_one(p1.x, g1.x, m1.x, v1.x, a.lr[3], a, omb1, omb2);
        p1.y = adam_one(p1.y, g1.y, m1.y, v1.y, a.lr[3], a, omb1, omb2);
        p1.z = adam_one(p1.z, g1.z, m1.z, v1.z, a.lr[3], a, omb1, omb2);
        p1.w = adam_one(p1.w, g1.w, m1.w, v1.w, a.lr[4], a, omb1, omb2);
        p2.x = adam_one(p2.x, g2.x, m2.x, v2.x, a.lr[4], a, omb1, omb2);
        p2.y = adam_one(p2.y, g2.y, m2.y, v2.y, a.lr[4], a, omb1, omb2);
        // projection of Sec. 4.1: positions stay inside the image
        p0.x = fminf(fmaxf(p0.x, 0.0f), a.w);
        p0.y = fminf(fmaxf(p0.y, 0.0f), a.h);
        P[0] = p0;
        P[1] = p1;
        P[2] = p2;
        M[0] = m0;
        M[1] = m1;
        M[2] = m2;
        V[0] = v0;
        V[1] = v1;
        V[2] = v2;
    }
    float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    G[0] = z;
    G[1] = z;
    G[2] = z;
    if (derived) {
        const Geo g = prepare_one(p0, p1, p2, reinterpret_cast<float4*>(derived + (size_t)i * REC));
        if (probe) probe[i] = probe_record(g);
    }
}

}  // namespace sad

using namespace sad;

extern "C" int sad_prepare_sites(const float* params, int32_t n, float* derived, void* stream) {
    if (!sites_ok(n) || !array_ok(params, n, 16) || !array_ok(derived, n, 16)) return SAD_EINVAL;
    if (overlap(params, int64_t(n) * REC * 4, derived, int64_t(n) * REC * 4)) return SAD_EINVAL;
    if (n == 0) return SAD_OK;
    clear_error();
    hipLaunchKernelGGL(k_prepare, dim3((n + 255) / 256), dim3(256), 0, as_stream(stream), params, n, derived);
    return launch_status();
}

extern "C" int sad_adam_step_probe(float* params, float* grad, float* m, float* v, int32_t n, int32_t h, int32_t w,
                                   const float* lr, float beta1, float beta2, float eps, float bias_corr1,
                                   float bias_corr2, float* derived, float* probe, void* stream) {
    if (!sites_ok(n) || !image_ok(h, w) || lr == nullptr) return SAD_EINVAL;
    if (!array_ok(params, n, 16) || !array_ok(grad, n, 16) || !array_ok(m, n, 16) || !array_ok(v, n, 16))
        return SAD_EINVAL;
    if (derived && !aligned(derived, 16)) return SAD_EINVAL;
    if (probe && (!derived || !aligned(probe, 16))) return SAD_EINVAL;  // records of the prepared sites
    const int64_t bytes = int64_t(n) * REC * 4;
    const void* bufs[6] = {params, grad, m, v, derived, probe};
    const int64_t sizes[6] = {bytes, bytes, bytes, bytes, bytes, int64_t(n) * 16};
    for (int a = 0; a < 6; ++a)
        for (int b = a + 1; b < 6; ++b)
            if (overlap(bufs[a], sizes[a], bufs[b], sizes[b])) return SAD_EINVAL;
    if (n == 0) return SAD_OK;
    AdamArgs args;
    for (int k = 0; k < 5; ++k) args.lr[k] = lr[k];
    args.beta1 = beta1;
    args.beta2 = beta2;
    args.eps = eps;
    args.bc1 = bias_corr1;
    args.bc2 = bias_corr2;
    args.w = (float)w;
    args.h = (float)h;
    clear_error();
    hipLaunchKernelGGL(k_adam, dim3((n + 255) / 256), dim3(256), 0, as_stream(stream), params, grad, m, v, n, args,
                       derived, reinterpret_cast<float4*>(probe));
    return launch_status();
}

extern "C" int sad_adam_step(float* params, float* grad, float* m, float* v, int32_t n, int32_t h, int32_t w,
                             const float* lr, float beta1, float beta2, float eps, float bias_corr1,
                             float bias_corr2, float* derived, void* stream) {
    return sad_adam_step_probe(params, grad, m, v, n, h, w, lr, beta1, beta2, eps, bias_corr1, bias_corr2, derived,
                               nullptr, stream);
}
