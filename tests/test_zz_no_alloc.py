"""sad_site_stats_noalloc, the statistics entry point that allocates nothing
(its region tables live in the library's own device array), against
sad_site_stats with a caller's workspace: two calls in a row through the C
ABI, the second with a smaller image and fewer sites, each also against the
oracle."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import assert_stats_close, dev, map_to_np, say, to_gpu, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sad():
    from voronoi_rendering_amd import ops

    say("[gpu] device: " + torch.cuda.get_device_name(0))
    return ops


def gpu_map(sad, dg, h, w, strides, seed):
    cur = sad.empty_map(h, w, dev())
    nxt = torch.empty_like(cur)
    for t, s in enumerate(strides):
        sad.propagate_topk(dg, h, w, cur, nxt, stride=int(s), seed=seed, pass_index=t, inject=64)
        cur, nxt = nxt, cur
    return cur


def one_case(sad, ref, wl, strides, label):
    from voronoi_rendering_amd import _native

    p = wl.make_sites()
    d = ref.prepare_sites(p)
    tgt = wl.make_target()
    dg = sad.prepare_sites(to_gpu(p))
    topk = gpu_map(sad, dg, wl.h, wl.w, strides, wl.inject_seed)
    m_np = map_to_np(topk)
    tg = to_gpu(tgt)
    want = torch.zeros((wl.n, sad.NSTAT), dtype=torch.float32, device=dev())
    sad.site_stats(dg, wl.h, wl.w, topk, tg, want)
    got = torch.zeros_like(want)
    st = _native.lib().sad_site_stats_noalloc(dg.data_ptr(), wl.n, wl.h, wl.w, topk.data_ptr(), tg.data_ptr(),
                                              got.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0, _native.status_string(st)
    torch.cuda.synchronize()
    st_ref, mag = ref.site_stats(d, wl.h, wl.w, m_np, tgt)
    g, w_ = to_np(got), to_np(want)
    assert_stats_close(w_, st_ref, mag, m_np, (wl.h, wl.w), f"{label}: workspace entry point")
    assert_stats_close(g, st_ref, mag, m_np, (wl.h, wl.w), f"{label}: allocation-free entry point")
    # the same kernels over the same tables: within the statistics bar of each other
    assert_stats_close(g, w_.astype(np.float64), mag, m_np, (wl.h, wl.w), f"{label}: allocation-free vs workspace")
    say(f"[gpu] {label}: allocation-free statistics equal the workspace call's in "
        f"{(g.view(np.uint32) == w_.view(np.uint32)).mean():.4f} of the values")


def test_noalloc_stats_two_calls_smaller_second(sad, ref):
    one_case(sad, ref, synth.C2, synth.jfa_strides(synth.C2.h, synth.C2.w, 16), "768x512 / 50k sites")
    one_case(sad, ref, synth.C1, synth.C1.strides, "64x64 / 256 sites")
