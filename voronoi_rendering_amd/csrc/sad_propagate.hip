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
