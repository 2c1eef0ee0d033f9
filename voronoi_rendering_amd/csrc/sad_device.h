// sad_device.h -- device helpers shared by the SAD kernels: the float32 logit
// in its fixed operation order, the ranking order, the register top-K list,
// the wavefront reductions and the injection generator.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sad.h"

namespace sad {

constexpr int K = SAD_K;
constexpr int REC = SAD_SITE_STRIDE;
constexpr uint32_t EMPTY = SAD_EMPTY;
constexpr int TILE = SAD_TILE;
constexpr int WAVE = 64;

// Site geometry as the logit needs it: g0 = (x, y, tau, r), g1 = (cos, sin, 1/s1, 1/s2).
struct Geo {
    float4 g0, g1;
};

__device__ __forceinline__ Geo load_geo(const float* __restrict__ derived, uint32_t id) {
    const float4* p = reinterpret_cast<const float4*>(derived + (size_t)id * REC);
    Geo g;
    g.g0 = p[0];
    g.g1 = p[1];
    return g;
}

// Logit of Sec. 4.2, l = -tau (||x - p||_G - r), evaluated in float32 in the
// documented order (the file is built without contraction; sqrtf is the
// correctly rounded square root).
__device__ __forceinline__ float logit(const Geo& g, float px, float py) {
    float dx = px - g.g0.x;
    float dy = py - g.g0.y;
    float a = (dx * g.g1.x + dy * g.g1.y) * g.g1.z;
    float b = (dy * g.g1.x - dx * g.g1.y) * g.g1.w;
    float q = a * a + b * b;
    float d = __builtin_sqrtf(q) - g.g0.w;
    return -(g.g0.z * d);
}

// (s1, i1) ranks before (s2, i2)
__device__ __forceinline__ bool ranks_before(float s1, uint32_t i1, float s2, uint32_t i2) {
    return s1 > s2 || (s1 == s2 && i1 < i2);
}

// Sorted list of the best K (logit, id) pairs seen so far, in registers.
// Empty slots hold (-inf, EMPTY), which every real candidate ranks before.
struct TopK {
    float s[K];
    uint32_t id[K];

    __device__ __forceinline__ void clear() {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            s[k] = -__builtin_inff();
            id[k] = EMPTY;
        }
    }

    // Insert a candidate with a non-NaN logit.  An id already in the list
    // carries the same logit, so it is recognised and skipped.
    __device__ __forceinline__ void insert(float sc, uint32_t cid) {
        if (!ranks_before(sc, cid, s[K - 1], id[K - 1])) return;
        bool dup = false;
#pragma unroll
        for (int k = 0; k < K; ++k) dup |= (id[k] == cid);
        if (dup) return;
        bool b[K];
#pragma unroll
        for (int k = 0; k < K; ++k) b[k] = ranks_before(sc, cid, s[k], id[k]);
#pragma unroll
        for (int k = K - 1; k >= 1; --k) {
            float ns = b[k - 1] ? s[k - 1] : (b[k] ? sc : s[k]);
            uint32_t ni = b[k - 1] ? id[k - 1] : (b[k] ? cid : id[k]);
            s[k] = ns;
            id[k] = ni;
        }
        if (b[0]) {
            s[0] = sc;
            id[0] = cid;
        }
    }
};

// SplitMix64 (Steele, Lea, Flood 2014) evaluated at a counter: the output
// of the generator whose state is seed after counter + 1 increments.
__device__ __forceinline__ uint64_t splitmix64(uint64_t seed, uint64_t counter) {
    uint64_t z = seed + (counter + 1ull) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ __forceinline__ uint32_t probe_id(uint64_t seed, uint32_t pass_index, uint32_t tile, uint32_t j,
                                             uint32_t n) {
    uint64_t c = ((uint64_t)pass_index << 32) | ((uint64_t)tile << 6) | (uint64_t)j;
    uint64_t z = splitmix64(seed, c);
    return (uint32_t)(((z >> 32) * (uint64_t)n) >> 32);
}

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fminf(v, __shfl_xor(v, off, WAVE));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, WAVE);
    return v;
}

__device__ __forceinline__ bool finitef(float v) { return __builtin_isfinite(v); }

}  // namespace sad
