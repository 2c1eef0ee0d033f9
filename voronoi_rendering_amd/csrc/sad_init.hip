// sad_init.hip -- gradient-weighted initialisation (Sec. 4.4): sites drawn
// from P_init = (1 - lambda) |grad I| / sum |grad I| + lambda / (H W).
//
// |grad I| is the 2-norm over the three channels and both directions of the
// 3x3 Sobel derivatives of the target (borders repeated), in float32 with one
// rounding per operation in the order written below.  The draw is exact: the
// magnitudes become integers in units of 2^-24 (truncated, capped at 2^8, so
// 2^30 pixels still sum in 64 bits), an inclusive prefix sum over them is the
// CDF, and every site picks its pixel from SplitMix64 outputs at counters
// 4 i + k: k = 0 chooses the uniform part ((z >> 40) 2^-24 < lambda, or a flat
// image), k = 1 the pixel (multiply-shift for the uniform part; the first
// prefix sum above floor(z G / 2^64) for the gradient part), k = 2, 3 the
// offsets inside the pixel.  A site starts there with the target colour of
// its pixel, the given log tau, r and log scale (both axes) and angle 0.
#include <rocprim/device/device_scan.hpp>

#include "sad_device.h"
#include "sad_host.h"
#include "sad_prepare.h"

namespace sad {

__device__ __forceinline__ float tpx(const float* t, int h, int w, int i, int j, int c) {
    i = min(max(i, 0), w - 1);
    j = min(max(j, 0), h - 1);
    return t[((size_t)j * w + i) * 3 + c];
}

constexpr int INIT_BX = 32, INIT_BY = 8;

__global__ __launch_bounds__(INIT_BX* INIT_BY) void k_init_units(const float* __restrict__ target, int32_t h,
                                                                  int32_t w, uint64_t* __restrict__ units) {
    const int i = blockIdx.x * INIT_BX + threadIdx.x % INIT_BX;
    const int j = blockIdx.y * INIT_BY + threadIdx.x / INIT_BX;
    if (i >= w || j >= h) return;
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        const float gx = (tpx(target, h, w, i + 1, j - 1, c) + 2.0f * tpx(target, h, w, i + 1, j, c) +
                          tpx(target, h, w, i + 1, j + 1, c)) -
                         (tpx(target, h, w, i - 1, j - 1, c) + 2.0f * tpx(target, h, w, i - 1, j, c) +
                          tpx(target, h, w, i - 1, j + 1, c));
        const float gy = (tpx(target, h, w, i - 1, j + 1, c) + 2.0f * tpx(target, h, w, i, j + 1, c) +
                          tpx(target, h, w, i + 1, j + 1, c)) -
                         (tpx(target, h, w, i - 1, j - 1, c) + 2.0f * tpx(target, h, w, i, j - 1, c) +
                          tpx(target, h, w, i + 1, j - 1, c));
        const float e = gx * gx + gy * gy;
        acc = c == 0 ? e : acc + e;
    }
    const float g = __builtin_sqrtf(acc);
    units[(size_t)j * w + i] = (g == g) ? (uint64_t)(fminf(g, 256.0f) * 16777216.0f) : 0ull;
}

struct InitArgs {
    const float* target;
    const uint64_t* cdf;  // inclusive prefix sums of the units, [h * w]
    float* params;
    float* derived;
    int32_t n, w;
    uint32_t pix;
    float lambda, log_tau, r, log_scale;
    uint64_t seed;
};

__global__ __launch_bounds__(256) void k_init_sample(InitArgs a) {
    const int s = blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= a.n) return;
    uint64_t z[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) z[k] = splitmix64(a.seed, 4ull * (uint64_t)s + (uint64_t)k);
    const uint64_t total = a.cdf[a.pix - 1];
    const float u0 = (float)(uint32_t)(z[0] >> 40) * 0x1p-24f;
    uint32_t x;
    if (u0 < a.lambda || total == 0) {
        x = (uint32_t)(((z[1] >> 32) * (uint64_t)a.pix) >> 32);
    } else {
        const uint64_t t = __umul64hi(z[1], total);
        uint32_t lo = 0, hi = a.pix - 1;  // the first x with cdf[x] > t; cdf[pix - 1] = total > t
        while (lo < hi) {
            const uint32_t mid = lo + (hi - lo) / 2;
            if (a.cdf[mid] > t)
                hi = mid;
            else
                lo = mid + 1;
        }
        x = lo;
    }
    const uint32_t i = x % (uint32_t)a.w, j = x / (uint32_t)a.w;
    const float* c = a.target + (size_t)x * 3;
    const float4 p0 = make_float4((float)i + (float)(uint32_t)(z[2] >> 40) * 0x1p-24f,
                                  (float)j + (float)(uint32_t)(z[3] >> 40) * 0x1p-24f, a.log_tau, a.r);
    const float4 p1 = make_float4(c[0], c[1], c[2], 0.0f);
    const float4 p2 = make_float4(a.log_scale, a.log_scale, 0.0f, 0.0f);
    float4* o = reinterpret_cast<float4*>(a.params + (size_t)s * REC);
    o[0] = p0;
    o[1] = p1;
    o[2] = p2;
    prepare_one(p0, p1, p2, reinterpret_cast<float4*>(a.derived + (size_t)s * REC));
}

// Workspace: units [pix] u64, cdf [pix] u64, the scan's temporary storage.
inline size_t init_layout(int64_t pix, char* base, uint64_t** units, uint64_t** cdf, void** tmp, size_t* tmp_bytes) {
    size_t tb = 0;
    (void)rocprim::inclusive_scan(nullptr, tb, (const uint64_t*)nullptr, (uint64_t*)nullptr, (size_t)pix,
                                  rocprim::plus<uint64_t>());
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char* p = base ? base + off : nullptr;
        off += (bytes + 255) & ~(size_t)255;
        return p;
    };
    char* u = take((size_t)pix * 8);
    char* c = take((size_t)pix * 8);
    char* t = take(tb);
    if (units) *units = reinterpret_cast<uint64_t*>(u);
    if (cdf) *cdf = reinterpret_cast<uint64_t*>(c);
    if (tmp) *tmp = t;
    if (tmp_bytes) *tmp_bytes = tb;
    return off;
}

}  // namespace sad

using namespace sad;

extern "C" size_t sad_init_workspace_bytes(int32_t h, int32_t w) {
    if (!image_ok(h, w)) return 0;
    return init_layout(int64_t(h) * w, nullptr, nullptr, nullptr, nullptr, nullptr);
}

extern "C" int sad_init_sites(const float* target, int32_t h, int32_t w, int32_t n, float lambda, uint64_t seed,
                              float log_tau, float r, float log_scale, float* params, float* derived, void* workspace,
                              size_t workspace_bytes, void* stream) {
    if (!sites_ok(n) || !image_ok(h, w) || !(lambda >= 0.0f && lambda <= 1.0f)) return SAD_EINVAL;
    const int64_t pix = int64_t(h) * w;
    if (n == 0) return SAD_OK;
    if (pix == 0) return SAD_EINVAL;  // sites need pixels to be drawn from
    if (!array_ok(target, pix, 4) || !array_ok(params, n, 16) || !array_ok(derived, n, 16)) return SAD_EINVAL;
    const size_t need = sad_init_workspace_bytes(h, w);
    if (workspace == nullptr || !aligned(workspace, 256) || workspace_bytes < need) return SAD_EINVAL;
    const int64_t rb = int64_t(n) * REC * 4;
    const void* bufs[4] = {target, params, derived, workspace};
    const int64_t bytes[4] = {pix * 12, rb, rb, (int64_t)need};
    for (int x = 0; x < 4; ++x)
        for (int y = x + 1; y < 4; ++y)
            if (overlap(bufs[x], bytes[x], bufs[y], bytes[y])) return SAD_EINVAL;
    uint64_t *units = nullptr, *cdf = nullptr;
    void* tmp = nullptr;
    size_t tb = 0;
    init_layout(pix, static_cast<char*>(workspace), &units, &cdf, &tmp, &tb);
    hipStream_t s = as_stream(stream);
    clear_error();
    hipLaunchKernelGGL(k_init_units, dim3((unsigned)((w + INIT_BX - 1) / INIT_BX), (unsigned)((h + INIT_BY - 1) / INIT_BY)),
                       dim3(INIT_BX * INIT_BY), 0, s, target, h, w, units);
    if (rocprim::inclusive_scan(tmp, tb, units, cdf, (size_t)pix, rocprim::plus<uint64_t>(), s) != hipSuccess)
        return SAD_EHIP;
    InitArgs a;
    a.target = target;
    a.cdf = cdf;
    a.params = params;
    a.derived = derived;
    a.n = n;
    a.w = w;
    a.pix = (uint32_t)pix;
    a.lambda = lambda;
    a.log_tau = log_tau;
    a.r = r;
    a.log_scale = log_scale;
    a.seed = seed;
    hipLaunchKernelGGL(k_init_sample, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
    return launch_status();
}
