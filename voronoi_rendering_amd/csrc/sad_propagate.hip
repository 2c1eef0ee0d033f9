// sad_propagate.hip -- the propagation kernel and its C ABI entry points: one
// wavefront per 8x8 tile, 4 consecutive tiles per 256-thread workgroup (the
// per-tile work is propagate_tile).
#include "sad_host.h"
#include "sad_propagate.h"

namespace sad {

constexpr int WAVES_PER_WG = 4;

template <bool SMALL_IDS, bool PREV16, bool NEXT16, bool THR_IN>
__global__ __launch_bounds__(WAVE* WAVES_PER_WG) __attribute__((amdgpu_waves_per_eu(SMALL_IDS ? 6 : 1)))
void k_propagate(PropArgs a) {
    __shared__ QueueId<SMALL_IDS> queue[WAVES_PER_WG][QCAP][WAVE];  // queued ids, then survivors' ids
    __shared__ float qscore[WAVES_PER_WG][QCAP][WAVE];    // survivors' logits
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);  // uniform: tile arithmetic stays scalar
    const int tile = xcd_block(blockIdx.x, gridDim.x) * WAVES_PER_WG + wv;
    if (tile >= a.n_tiles) return;  // uniform per wavefront
    TopK t;
    propagate_tile<SMALL_IDS, PREV16, NEXT16, THR_IN>(a, tile, queue[wv], qscore[wv], t);
}

// A 16-bit-id map widened to 32-bit ids, one thread per pixel (one 16-byte
// load, two 16-byte stores); the empty slot 0xffff becomes 0xffffffff.
__global__ __launch_bounds__(256) void k_widen(const uint4* __restrict__ in, int64_t pix, uint4* __restrict__ out) {
    const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= pix) return;
    const uint4 v = in[p];
    const uint32_t h[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t lo = h[k] & 0xFFFFu, hi = h[k] >> 16;
        o[2 * k] = lo == 0xFFFFu ? 0xFFFFFFFFu : lo;
        o[2 * k + 1] = hi == 0xFFFFu ? 0xFFFFFFFFu : hi;
    }
    out[2 * p] = make_uint4(o[0], o[1], o[2], o[3]);
    out[2 * p + 1] = make_uint4(o[4], o[5], o[6], o[7]);
}

// Launch the pass on checked arguments.
inline int prop_launch(const PropArgs& a, void* stream) {
    if (a.n_tiles == 0) return SAD_OK;
    clear_error();
    const dim3 grid((unsigned)((a.n_tiles + WAVES_PER_WG - 1) / WAVES_PER_WG)), block(WAVE * WAVES_PER_WG);
    const hipStream_t s = as_stream(stream);
    const bool p16 = a.prev16 != nullptr, n16 = a.next16 != nullptr, thr = a.prev_thr != nullptr;
    if (a.n > SMALL_IDS_MAX) {
        if (thr)
            hipLaunchKernelGGL((k_propagate<false, false, false, true>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((k_propagate<false, false, false, false>), grid, block, 0, s, a);
    } else if (thr) {
        if (p16 && n16)
            hipLaunchKernelGGL((k_propagate<true, true, true, true>), grid, block, 0, s, a);
        else if (p16)
            hipLaunchKernelGGL((k_propagate<true, true, false, true>), grid, block, 0, s, a);
        else if (n16)
            hipLaunchKernelGGL((k_propagate<true, false, true, true>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((k_propagate<true, false, false, true>), grid, block, 0, s, a);
    } else {
        if (p16 && n16)
            hipLaunchKernelGGL((k_propagate<true, true, true, false>), grid, block, 0, s, a);
        else if (p16)
            hipLaunchKernelGGL((k_propagate<true, true, false, false>), grid, block, 0, s, a);
        else if (n16)
            hipLaunchKernelGGL((k_propagate<true, false, true, false>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((k_propagate<true, false, false, false>), grid, block, 0, s, a);
    }
    return launch_status();
}

}  // namespace sad

using namespace sad;

extern "C" int sad_propagate_topk(const float* derived, int32_t n, int32_t h, int32_t w, const uint32_t* topk_prev,
                                  const float* scores_prev, uint32_t* topk_next, float* scores_next, int32_t stride,
                                  uint64_t seed, uint32_t pass_index, int32_t inject_per_tile, void* stream) {
    PropArgs a;
    const int st = prop_setup(derived, n, h, w, maps32(topk_prev, scores_prev, topk_next, scores_next), stride, seed,
                              pass_index, inject_per_tile, a);
    if (st != SAD_OK) return st;
    return prop_launch(a, stream);
}

extern "C" int sad_propagate_pass(const float* derived, int32_t n, int32_t h, int32_t w, const sad_pass_maps* maps,
                                  int32_t stride, uint64_t seed, uint32_t pass_index, int32_t inject_per_tile,
                                  void* stream) {
    if (!maps) return SAD_EINVAL;
    PropArgs a;
    const int st = prop_setup(derived, n, h, w, *maps, stride, seed, pass_index, inject_per_tile, a);
    if (st != SAD_OK) return st;
    return prop_launch(a, stream);
}

extern "C" int sad_widen_map(const uint16_t* topk16, int32_t h, int32_t w, uint32_t* topk, void* stream) {
    if (!image_ok(h, w)) return SAD_EINVAL;
    const int64_t pix = int64_t(h) * w;
    if (!array_ok(topk16, pix, 16) || !array_ok(topk, pix, 16)) return SAD_EINVAL;
    if (overlap(topk16, pix * K * 2, topk, pix * K * 4)) return SAD_EINVAL;
    if (pix == 0) return SAD_OK;
    clear_error();
    hipLaunchKernelGGL(k_widen, dim3((unsigned)((pix + 255) / 256)), dim3(256), 0, as_stream(stream),
                       reinterpret_cast<const uint4*>(topk16), pix, reinterpret_cast<uint4*>(topk));
    return launch_status();
}
