// sad_region.h -- the per-region site table shared by the kernels that sum
// per-pixel terms per site (the backward pass of Sec. 4.8 / Appendix B.4 and
// the budget statistics of Sec. 4.5 / Appendix B.5).
//
// A workgroup covers one region of RT_X x RT_Y tiles (32 x 16 pixels), one
// wavefront per 8x8 tile.  Every site listed by a pixel of the region gets a
// slot of an LDS table of SLOTS entries, keyed by site id with open
// addressing: a multiplicative hash (the pages' 2654435761 multiplier) picks
// the first slot and a second hash an odd step, so the probe sequence visits
// every slot and sequences of different sites do not run together as linear
// probing's do; at most REGION_PROBES slots are tried, keys are claimed by
// compare-and-swap.
#pragma once

#include "sad_device.h"

namespace sad {

constexpr int RT_X = 4, RT_Y = 2;  // tiles per region
constexpr int REGION_W = RT_X * TILE, REGION_H = RT_Y * TILE;
constexpr int REGION_WAVES = RT_X * RT_Y;
constexpr int REGION_PIX = REGION_W * REGION_H;
constexpr int SLOTS = 256;
constexpr int REGION_PROBES = 32;
constexpr int NGRAD = 10;

struct RegionGrid {
    int32_t rgx, rgy;
};

__host__ __device__ inline RegionGrid region_grid(int32_t h, int32_t w) {
    return {(w + REGION_W - 1) / REGION_W, (h + REGION_H - 1) / REGION_H};
}

__device__ __forceinline__ uint32_t slot_hash(uint32_t id) { return (id * 2654435761u) >> 24; }  // 8 bits
__device__ __forceinline__ uint32_t slot_step(uint32_t id) { return ((id * 0x85ebca6bu) >> 24) | 1u; }  // odd

// Rotate the 8 list entries left by r (0..7): entry k moves to (k - r) mod 8.
__device__ __forceinline__ void rotate_list(uint4& l0, uint4& l1, int r) {
    uint32_t v[K] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
#pragma unroll
    for (int bit = 0; bit < 3; ++bit) {
        const int sh = 1 << bit;
        const bool on = (r >> bit) & 1;
        uint32_t u[K];
#pragma unroll
        for (int k = 0; k < K; ++k) u[k] = on ? v[(k + sh) & (K - 1)] : v[k];
#pragma unroll
        for (int k = 0; k < K; ++k) v[k] = u[k];
    }
    l0 = make_uint4(v[0], v[1], v[2], v[3]);
    l1 = make_uint4(v[4], v[5], v[6], v[7]);
}

// The pixel of lane `lane` of wavefront `wv` in region (rx, ry).
__device__ __forceinline__ void region_pixel(int rx, int ry, int wv, int lane, int& i, int& j) {
    i = (rx * RT_X + (wv % RT_X)) * TILE + (lane & (TILE - 1));
    j = (ry * RT_Y + (wv / RT_X)) * TILE + (lane / TILE);
}

// Claim a slot of the table `keys` (EMPTY where free) for every id < n of
// the lane's list: all 8 probes of a lane go out together, round by round,
// instead of one chain per entry.  slot[k] is the slot, or -1 when the id is
// not a site or its probe chain ran out.  Called by every lane of the
// wavefront (the loop condition is wavefront-wide).
__device__ __forceinline__ void claim_slots(uint32_t* keys, const uint32_t (&ids)[K], uint32_t n, int (&slot)[K]) {
    int pos[K];
    uint32_t pend = 0;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        slot[k] = -1;
        pos[k] = (int)slot_hash(ids[k]);
        if (ids[k] < n) pend |= 1u << k;
    }
    for (int round = 0; round < REGION_PROBES && __any(pend != 0); ++round) {
        uint32_t cur[K];
#pragma unroll
        for (int k = 0; k < K; ++k) cur[k] = ((pend >> k) & 1) ? keys[pos[k]] : 0u;
#pragma unroll
        for (int k = 0; k < K; ++k)
            if (((pend >> k) & 1) && cur[k] == EMPTY) cur[k] = atomicCAS(&keys[pos[k]], EMPTY, ids[k]);
#pragma unroll
        for (int k = 0; k < K; ++k) {
            if (!((pend >> k) & 1)) continue;
            if (cur[k] == EMPTY || cur[k] == ids[k]) {
                slot[k] = pos[k];
                pend &= ~(1u << k);
            } else {
                pos[k] = (pos[k] + (int)slot_step(ids[k])) & (SLOTS - 1);
            }
        }
    }
}

}  // namespace sad
