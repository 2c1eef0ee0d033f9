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

// Workgroups are dealt to the chip's 8 XCDs in turn (workgroup b runs on XCD
// b mod 8), each XCD with its own L2.  xcd_block renumbers them so that each
// XCD receives one contiguous range of logical indices out of g: with
// row-major tiles that is a band of the image, whose neighbour lists and
// site records then stay within one L2.  A bijection on [0, g).
__device__ __forceinline__ int xcd_block(int b, int g) {
    const int q = g >> 3, r = g & 7;
    const int x = b & 7, k = b >> 3;
    return x < r ? x * (q + 1) + k : r * (q + 1) + (x - r) * q + k;
}

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

// Geometry of site id, or of site 0 when id is out of range (the caller then
// discards the result); requires n >= 1.  The load does not depend on any
// branch, so a batch of these can be in flight together.
__device__ __forceinline__ Geo load_geo_clamped(const float* __restrict__ derived, uint32_t n, uint32_t id) {
    return load_geo(derived, id < n ? id : 0u);
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

// The logit of a loaded site, or NaN when the id was out of range or the site
// is inactive (x < 0 or NaN).
__device__ __forceinline__ float usable_logit(const Geo& g, bool in_range, float px, float py) {
    const float s = logit(g, px, py);
    return (in_range && g.g0.x >= 0.0f) ? s : __builtin_nanf("");
}

// (s1, i1) ranks before (s2, i2).  Bitwise operators: the three compares are
// independent and no branch is formed around them.
__device__ __forceinline__ bool ranks_before(float s1, uint32_t i1, float s2, uint32_t i2) {
    return (s1 > s2) | ((s1 == s2) & (i1 < i2));
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

    // Is v one of the listed ids?  Written as a minimum of differences (one
    // vector compare at the end) rather than 8 compares whose lane masks are
    // combined on the scalar unit: the chain of vector-to-scalar dependencies
    // costs more than the few extra vector instructions.
    __device__ __forceinline__ bool has(uint32_t v) const {
        uint32_t mn = v ^ id[0];
#pragma unroll
        for (int k = 1; k < K; ++k) mn = min(mn, v ^ id[k]);
        return mn == 0u;
    }

    // Insert (sc, cid) when ok; ok must be false for a NaN logit.  An id
    // already in the list carries the same logit, so it is recognised and
    // skipped.  Branch-free: every lane runs the same selects, and the list
    // stays in the same registers whatever the outcome.
    __device__ __forceinline__ void insert_if(float sc, uint32_t cid, bool ok) {
        ok = ok & !has(cid);
        // b[k]: the candidate ranks before entry k (b[k - 1] implies b[k])
        bool b[K];
#pragma unroll
        for (int k = 0; k < K; ++k) b[k] = ok & ranks_before(sc, cid, s[k], id[k]);
#pragma unroll
        for (int k = K - 1; k >= 1; --k) {
            s[k] = b[k - 1] ? s[k - 1] : (b[k] ? sc : s[k]);
            id[k] = b[k - 1] ? id[k - 1] : (b[k] ? cid : id[k]);
        }
        s[0] = b[0] ? sc : s[0];
        id[0] = b[0] ? cid : id[0];
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

// Minimum over the wavefront with DPP lane moves (no LDS round trips):
// quad swaps, half-row and row mirrors, then the row broadcasts 15 and 31
// fold rows together; lane 63 ends with the minimum of all 64 lanes.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}

__device__ __forceinline__ float wave_min(float v) {
    v = fminf(v, dpp_f32<0xb1, 0xf>(v));   // quad_perm [1,0,3,2]
    v = fminf(v, dpp_f32<0x4e, 0xf>(v));   // quad_perm [2,3,0,1]
    v = fminf(v, dpp_f32<0x141, 0xf>(v));  // row_half_mirror
    v = fminf(v, dpp_f32<0x140, 0xf>(v));  // row_mirror
    v = fminf(v, dpp_f32<0x142, 0xa>(v));  // row_bcast:15 into rows 1 and 3
    v = fminf(v, dpp_f32<0x143, 0xc>(v));  // row_bcast:31 into rows 2 and 3
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, WAVE);
    return v;
}

__device__ __forceinline__ bool finitef(float v) { return __builtin_isfinite(v); }

// The probe record of a site: what the tile cull of a propagation pass
// (probe_may_enter) needs of it in 16 bytes, (x, y, tau m, tau r) with m the
// smaller inverse scale, so that a pass that probes sites it has no other
// use for gathers 16 instead of 32 bytes per probe (and the records of all
// sites, 16 bytes each, stay in each XCD's L2).  A site the bound cannot
// cover gets (x, y, 0, +inf): never culled.  Written by a pass or, with the
// prepared records, by the Adam step.
__device__ __forceinline__ float4 probe_record(const Geo& g) {
    const float tau = g.g0.z, r = g.g0.w, is1 = g.g1.z, is2 = g.g1.w;
    const float m = fminf(is1, is2), M = fmaxf(is1, is2);
    const bool boundable = finitef(g.g0.x) & finitef(g.g0.y) & finitef(tau) & finitef(r) & finitef(M) & (tau > 0.0f) &
                           (m > 0.0f) & (M <= 1024.0f * m);
    return make_float4(g.g0.x, g.g0.y, boundable ? tau * m : 0.0f, boundable ? tau * r : __builtin_inff());
}

}  // namespace sad
