// sad_jfa.hip -- the JFA prepass of a full list refresh (Appendix B.3, "JFA
// prepass"; the render protocol of Sec. 6.6 runs one JFA round, then 16
// propagation passes, then the render), after the jump flooding of Rong and
// Tan (2006).  Each pixel keeps 4 ids ranked at its centre like the top-K
// lists (logit descending, lower id first on ties).
//
// Seed: every usable site claims the pixel holding its position; of several
// sites on one pixel the one ranking first there stays.  A per-site pass
// takes the maximum of a 64-bit key per pixel (the logit, mapped to an
// unsigned integer of the same order, above the complement of the id), which
// selects exactly that site whatever order the atomics land in.
//
// Flood pass with step s: every pixel keeps the 4 best distinct usable ids of
// the 4-lists at (i + a s, j + b s), a, b in {-1, 0, 1}, inside the image.
// One wavefront per 8x8 tile.  An id is not scored again when it is in the
// pixel's list or in one of the two lists visited just before (in the order
// centre, right, bottom-right, bottom, bottom-left, left, top-left, top,
// top-right): such an id is in the list or has been beaten by 4 better ones,
// and the 4th entry only improves.  About half of a pixel's 36 candidates
// repeat; most repeats sit in those two lists.  A wavefront skips a
// neighbour's scoring when no lane has a new id in it.
#include "sad_device.h"
#include "sad_host.h"

namespace sad {

constexpr int JFA_K = 4;

// The 4 best (logit, id) pairs so far, in ranking order; empty slots hold
// (-inf, EMPTY).
struct Top4 {
    float s[JFA_K];
    uint32_t id[JFA_K];

    __device__ __forceinline__ void clear() {
#pragma unroll
        for (int k = 0; k < JFA_K; ++k) {
            s[k] = -__builtin_inff();
            id[k] = EMPTY;
        }
    }

    __device__ __forceinline__ bool has(uint32_t v) const {
        return (v == id[0]) | (v == id[1]) | (v == id[2]) | (v == id[3]);
    }

    // insert (sc, cid) when ok (ok must be false for a NaN logit or a listed id)
    __device__ __forceinline__ void insert_if(float sc, uint32_t cid, bool ok) {
        bool b[JFA_K];
#pragma unroll
        for (int k = 0; k < JFA_K; ++k) b[k] = ok & ranks_before(sc, cid, s[k], id[k]);
#pragma unroll
        for (int k = JFA_K - 1; k >= 1; --k) {
            s[k] = b[k - 1] ? s[k - 1] : (b[k] ? sc : s[k]);
            id[k] = b[k - 1] ? id[k - 1] : (b[k] ? cid : id[k]);
        }
        s[0] = b[0] ? sc : s[0];
        id[0] = b[0] ? cid : id[0];
    }
};

// An unsigned integer with the order of the float32 logit (-0 counts as +0).
__device__ __forceinline__ uint32_t ordered_bits(float s) {
    const uint32_t u = __float_as_uint(s + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int clamp_cell(float v, int size) {
    return (int)fminf(fmaxf(floorf(v), 0.0f), (float)(size - 1));  // a NaN becomes 0
}

// jfa[p] = {0, 0, EMPTY, EMPTY}: an empty 64-bit key in slots 0-1
__global__ __launch_bounds__(256) void k_jfa_clear(uint4* jfa, int64_t pix) {
    const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (p < pix) jfa[p] = make_uint4(0u, 0u, EMPTY, EMPTY);
}

__global__ __launch_bounds__(256) void k_jfa_seed(const float* __restrict__ derived, int32_t n, int32_t h, int32_t w,
                                                  unsigned long long* jfa64) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const Geo g = load_geo(derived, (uint32_t)i);
    if (!(g.g0.x >= 0.0f)) return;  // inactive (or NaN)
    const int ci = clamp_cell(g.g0.x, w), cj = clamp_cell(g.g0.y, h);
    const float s = logit(g, (float)ci + 0.5f, (float)cj + 0.5f);
    if (s != s) return;
    const unsigned long long key = ((unsigned long long)ordered_bits(s) << 32) | (unsigned long long)~(uint32_t)i;
    atomicMax(jfa64 + ((size_t)cj * w + ci) * 2, key);
}

__global__ __launch_bounds__(256) void k_jfa_finish(uint4* jfa, int64_t pix) {
    const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= pix) return;
    const uint4 v = jfa[p];
    const uint32_t id = (v.x | v.y) ? ~v.x : EMPTY;  // key = (order << 32) | ~id, 0 when empty
    jfa[p] = make_uint4(id, EMPTY, EMPTY, EMPTY);
}

struct JfaArgs {
    const float* derived;
    const uint4* prev;  // [h][w] 4-lists
    uint32_t* next;     // [h][w][out_width]
    int32_t n, h, w, step, out_width, tiles_x, n_tiles;
};

constexpr int JFA_WAVES = 4;

__global__ __launch_bounds__(WAVE* JFA_WAVES) void k_jfa_flood(JfaArgs a) {
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
    const int tile = xcd_block(blockIdx.x, gridDim.x) * JFA_WAVES + wv;
    if (tile >= a.n_tiles) return;  // uniform per wavefront
    const int lane = threadIdx.x & (WAVE - 1);
    const int tx = tile % a.tiles_x, ty = tile / a.tiles_x;
    const int i = tx * TILE + (lane & (TILE - 1)), j = ty * TILE + lane / TILE;
    const bool inside = (i < a.w) & (j < a.h);
    const float px = (float)i + 0.5f, py = (float)j + 0.5f;
    const uint32_t n = (uint32_t)a.n;

    // the 9 lists, read from clamped in-image addresses (ok marks the real ones)
    uint4 nl[9];
    bool ok[9];
#pragma unroll
    for (int q = 0; q < 9; ++q) {
        const int ii = i + (q % 3 - 1) * a.step, jj = j + (q / 3 - 1) * a.step;
        ok[q] = inside & (ii >= 0) & (ii < a.w) & (jj >= 0) & (jj < a.h);
        nl[q] = a.prev[(size_t)min(max(jj, 0), a.h - 1) * a.w + min(max(ii, 0), a.w - 1)];
    }
    Top4 t;
    t.clear();
    if (n > 0) {
        constexpr int ORDER[9] = {4, 5, 8, 7, 6, 3, 0, 1, 2};  // q = (a + 1) + 3 (b + 1)
        uint32_t seen1[JFA_K], seen2[JFA_K];  // the ids of the last two lists visited
#pragma unroll
        for (int k = 0; k < JFA_K; ++k) seen1[k] = seen2[k] = EMPTY;
#pragma unroll
        for (int q0 = 0; q0 < 9; ++q0) {
            const int q = ORDER[q0];
            const uint32_t v[JFA_K] = {nl[q].x, nl[q].y, nl[q].z, nl[q].w};
            bool fresh[JFA_K];
            bool any = false;
#pragma unroll
            for (int k = 0; k < JFA_K; ++k) {
                const bool seen = (v[k] == seen1[0]) | (v[k] == seen1[1]) | (v[k] == seen1[2]) | (v[k] == seen1[3]) |
                                  (v[k] == seen2[0]) | (v[k] == seen2[1]) | (v[k] == seen2[2]) | (v[k] == seen2[3]);
                fresh[k] = ok[q] & (v[k] < n) & !t.has(v[k]) & !seen;
                any |= fresh[k];
            }
#pragma unroll
            for (int k = 0; k < JFA_K; ++k) {
                seen2[k] = seen1[k];
                seen1[k] = ok[q] ? v[k] : EMPTY;  // a list outside the image was not considered
            }
            if (!__any(any)) continue;
            Geo g[JFA_K];  // only lanes with a new id fetch its record
#pragma unroll
            for (int k = 0; k < JFA_K; ++k) {
                g[k].g0 = make_float4(-1.0f, -1.0f, 0.0f, 0.0f);
                g[k].g1 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                if (fresh[k]) g[k] = load_geo(a.derived, v[k]);  // fresh implies v[k] < n
            }
#pragma unroll
            for (int k = 0; k < JFA_K; ++k) {
                const float s = usable_logit(g[k], v[k] < n, px, py);
                t.insert_if(s, v[k], fresh[k] & (s == s) & !t.has(v[k]));
            }
        }
    }
    if (inside) {
        uint4* o = reinterpret_cast<uint4*>(a.next + ((size_t)j * a.w + i) * a.out_width);
        o[0] = make_uint4(t.id[0], t.id[1], t.id[2], t.id[3]);
        if (a.out_width == 8) o[1] = make_uint4(EMPTY, EMPTY, EMPTY, EMPTY);
    }
}

}  // namespace sad

using namespace sad;

extern "C" int sad_jfa_seed(const float* derived, int32_t n, int32_t h, int32_t w, uint32_t* jfa, void* stream) {
    if (!sites_ok(n) || !image_ok(h, w)) return SAD_EINVAL;
    const int64_t pix = int64_t(h) * w;
    if (!array_ok(derived, n, 16) || !array_ok(jfa, pix, 16)) return SAD_EINVAL;
    if (overlap(jfa, pix * JFA_K * 4, derived, int64_t(n) * REC * 4)) return SAD_EINVAL;
    if (pix == 0) return SAD_OK;
    clear_error();
    const unsigned gp = (unsigned)((pix + 255) / 256);
    hipLaunchKernelGGL(k_jfa_clear, dim3(gp), dim3(256), 0, as_stream(stream), reinterpret_cast<uint4*>(jfa), pix);
    if (n > 0)
        hipLaunchKernelGGL(k_jfa_seed, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, as_stream(stream), derived, n,
                           h, w, reinterpret_cast<unsigned long long*>(jfa));
    hipLaunchKernelGGL(k_jfa_finish, dim3(gp), dim3(256), 0, as_stream(stream), reinterpret_cast<uint4*>(jfa), pix);
    return launch_status();
}

extern "C" int sad_jfa_flood(const float* derived, int32_t n, int32_t h, int32_t w, const uint32_t* jfa_prev,
                             uint32_t* out, int32_t step, int32_t out_width, void* stream) {
    if (!sites_ok(n) || !image_ok(h, w) || step < 1 || (out_width != 4 && out_width != 8)) return SAD_EINVAL;
    const int64_t pix = int64_t(h) * w;
    if (!array_ok(derived, n, 16) || !array_ok(jfa_prev, pix, 16) || !array_ok(out, pix, 16)) return SAD_EINVAL;
    const int64_t ibytes = pix * JFA_K * 4, obytes = pix * out_width * 4, dbytes = int64_t(n) * REC * 4;
    if (overlap(out, obytes, jfa_prev, ibytes) || overlap(out, obytes, derived, dbytes)) return SAD_EINVAL;
    const int64_t ntiles = int64_t(tiles_x(w)) * tiles_y(h);
    if (ntiles > MAX_TILES) return SAD_EINVAL;
    if (pix == 0) return SAD_OK;
    JfaArgs a;
    a.derived = derived;
    a.prev = reinterpret_cast<const uint4*>(jfa_prev);
    a.next = out;
    a.n = n;
    a.h = h;
    a.w = w;
    a.step = step;
    a.out_width = out_width;
    a.tiles_x = tiles_x(w);
    a.n_tiles = (int32_t)ntiles;
    clear_error();
    hipLaunchKernelGGL(k_jfa_flood, dim3((unsigned)((ntiles + JFA_WAVES - 1) / JFA_WAVES)), dim3(WAVE * JFA_WAVES), 0,
                       as_stream(stream), a);
    return launch_status();
}
