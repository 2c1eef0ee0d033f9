"""The C-ABI library loads, exports every symbol include/sad.h declares, and
rejects invalid arguments before enqueueing any work (no GPU needed: every
call here fails its argument checks, which run on the host)."""
import ctypes as C
import re
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]


@pytest.fixture(scope="module")
def lib():
    from voronoi_rendering_amd import _native

    if not _native.LIB_PATH.exists():
        pytest.fail("libsad.so is not built (run __graft_entry__.build())")
    return _native.lib()


def declared_symbols():
    text = (ROOT / "include" / "sad.h").read_text()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char \*)\s*(sad_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    syms = declared_symbols()
    for name in ("sad_prepare_sites", "sad_propagate_topk", "sad_render_fwd", "sad_render_bwd",
                 "sad_site_stats_workspace_bytes", "sad_step_fused", "sad_site_stats", "sad_jfa_seed",
                 "sad_jfa_flood", "sad_budget_workspace_bytes", "sad_densify_prune", "sad_init_workspace_bytes",
                 "sad_init_sites", "sad_pack_sites", "sad_query_packed",
                 "sad_adam_step", "sad_query_points", "sad_status_string", "sad_abi_version",
                 "sad_propagate_pass", "sad_step_fused_pass", "sad_adam_step_probe", "sad_widen_map"):
        assert name in syms


def test_every_declared_symbol_is_exported(lib):
    from voronoi_rendering_amd import _native

    for name in declared_symbols():
        assert hasattr(lib, name), name
        assert name in _native.symbols(), name


def test_version_and_status_strings(lib):
    assert lib.sad_abi_version() == 11
    for st in (0, -1, -2, -3, 7):
        assert lib.sad_status_string(st)


EINVAL, EUNSUP = -1, -2
P = 0x10000  # a 16-byte aligned stand-in address: never dereferenced, the checks fail first


def test_prepare_rejects(lib):
    assert lib.sad_prepare_sites(None, -1, None, None) == EINVAL
    assert lib.sad_prepare_sites(None, 4, P, None) == EINVAL  # NULL params
    assert lib.sad_prepare_sites(P + 4, 4, P + 4096, None) == EINVAL  # misaligned
    assert lib.sad_prepare_sites(P, 4, P + 16, None) == EINVAL  # overlapping buffers
    assert lib.sad_prepare_sites(P, (1 << 30) + 1, P + (1 << 40), None) == EINVAL
    assert lib.sad_prepare_sites(None, 0, None, None) == 0  # empty: nothing to do


def test_propagate_rejects(lib):
    f = lib.sad_propagate_topk
    ok = dict(derived=P, n=10, h=8, w=8, prev=None, sprev=None, nxt=P + 4096, snext=None, stride=1, seed=0, pi=0,
              inj=64)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["derived"], a["n"], a["h"], a["w"], a["prev"], a["sprev"], a["nxt"], a["snext"], a["stride"],
                 a["seed"], a["pi"], a["inj"], None)

    assert call(stride=0) == EINVAL
    assert call(n=-1) == EINVAL
    assert call(h=-2) == EINVAL
    assert call(w=(1 << 15) + 1) == EINVAL
    assert call(inj=-1) == EINVAL
    assert call(inj=65) == EUNSUP
    assert call(nxt=None) == EINVAL
    assert call(derived=None) == EINVAL
    assert call(prev=P + 4096) == EINVAL  # in place
    assert call(prev=P + 4096 + 32 * 8) == EINVAL  # overlapping
    assert call(nxt=P + 4100) == EINVAL  # misaligned
    assert call(sprev=P + 65536) == EINVAL  # scores without a previous map
    assert call(prev=P + 65536, sprev=P + 65536) == EINVAL  # scores alias the map
    assert call(snext=P + 4096) == EINVAL  # the two outputs alias
    assert call(snext=P + 65540) == EINVAL  # misaligned scores
    assert call(h=0, nxt=None) == 0  # empty image


def test_propagate_pass_rejects(lib):
    """The pass on a sad_pass_maps: widths other than 16 and 32, 16-bit maps
    with more than 65,535 sites, threshold maps without a previous map or
    together with a score map, misaligned probe records, and overlaps
    measured on each buffer's own size (for 8x8 pixels a 16-bit map is 1 KiB,
    a threshold map 256 bytes; 10 sites' probe records are 160 bytes, their
    prepared records 480)."""
    from voronoi_rendering_amd._native import PassMaps

    f = lib.sad_propagate_pass
    base = dict(topk_prev=P + 65536, prev_bits=16, topk_next=P + 4096, next_bits=16)

    def call(n=10, **kw):
        m = PassMaps(**dict(base, **kw))
        return f(P, n, 8, 8, C.byref(m), 1, 0, 0, 64, None)

    assert f(P, 10, 8, 8, None, 1, 0, 0, 64, None) == EINVAL  # no maps
    assert call(prev_bits=8) == EINVAL
    assert call(next_bits=64) == EINVAL
    assert call(prev_bits=0, topk_prev=None) == EINVAL  # the width is checked even without a previous map
    assert call(n=65536) == EUNSUP  # 16-bit ids need n <= 65535
    assert call(n=65536, next_bits=32) == EUNSUP
    assert call(topk_prev=P + 4096 + 1008) == EINVAL  # 16-bit maps overlap in their last 16 bytes
    assert call(topk_next=P + 4100) == EINVAL  # misaligned
    assert call(topk_next=None) == EINVAL
    assert call(scores_prev=P + 8192, scores_next=P + 8192 + 2032) == EINVAL  # score maps overlap (2 KiB each)
    assert call(scores_next=P + 4096 + 512) == EINVAL  # next scores inside the next map
    assert call(thr_prev=P + 8192, topk_prev=None) == EINVAL  # thresholds without a previous map
    assert call(scores_prev=P + 8192, topk_prev=None) == EINVAL  # scores without a previous map
    assert call(thr_prev=P + 8192, scores_prev=P + 12288) == EINVAL  # thresholds and scores together
    assert call(thr_prev=P + 8194) == EINVAL  # misaligned thresholds
    assert call(thr_prev=P + 8192, thr_next=P + 8192 + 252) == EINVAL  # threshold maps overlap (256 bytes each)
    assert call(thr_next=P + 65536 + 1020) == EINVAL  # next thresholds over the previous map
    assert call(thr_prev=P + 4096 + 1000) == EINVAL  # previous thresholds over the next map
    assert call(probe_prev=P + 8200) == EINVAL  # misaligned probe records
    assert call(probe_next=P + 8200) == EINVAL
    assert call(probe_next=P + 464) == EINVAL  # probe records over the prepared records
    assert call(probe_prev=P + 8192, probe_next=P + 8192 + 144) == EINVAL  # the two record arrays overlap
    assert call(probe_next=P + 65536 + 1008) == EINVAL  # records over the previous map
    assert call(probe_next=P + 4096 + 1008) == EINVAL  # records over the next map
    assert call(probe_prev=P + 4096 + 1008) == EINVAL  # previous records over the next map
    assert call(probe_prev=P + 320) == EINVAL  # previous records over the prepared records
    assert call(probe_prev=P + 65536 + 512) == EINVAL  # previous records over the previous map
    g = lib.sad_step_fused_pass
    G, T = P + (1 << 20), P + (2 << 20)  # grad and target, apart from everything
    fbase = dict(topk_prev=P + 65536, prev_bits=16, topk_next=P + 4096, next_bits=32)

    def fused(n=10, grad=G, loss=None, image=None, **kw):
        m = PassMaps(**dict(fbase, **kw))
        return g(P, n, 8, 8, C.byref(m), 1, 0, 0, 64, T, grad, loss, image, None)

    assert g(P, 10, 8, 8, None, 1, 0, 0, 64, T, G, None, None, None) == EINVAL  # no maps
    assert fused(n=65536) == EUNSUP
    assert fused(prev_bits=24) == EINVAL
    assert fused(next_bits=8) == EINVAL  # the fused pass writes 32- or 16-bit lists
    assert fused(next_bits=16, n=65536) == EUNSUP  # 16-bit lists need n <= 65535
    assert fused(next_bits=16, grad=P + 4096 + 1008) == EINVAL  # gradients over the 16-bit map's last 16 bytes
    assert fused(next_bits=16, scores_next=P + 4096 + 1008) == EINVAL  # logits over the 16-bit map
    assert fused(thr_next=P + 8192) == EINVAL  # and no thresholds
    assert fused(probe_next=P + 8192) == EINVAL  # or probe records
    assert fused(grad=None) == EINVAL
    assert fused(grad=P + 65536) == EINVAL  # gradients over the previous map
    assert fused(thr_prev=P + 8192, loss=P + 8192 + 8) == EINVAL  # loss inside the thresholds
    assert fused(image=P + 65536 + 512) == EINVAL  # image over the previous map
    assert fused(probe_prev=P + 8192, loss=P + 8192 + 152) == EINVAL  # loss inside the probe records
    assert fused(probe_prev=G + 48) == EINVAL  # gradients over the probe records


def test_widen_map_rejects(lib):
    """Widening a 16-bit map (8x8 pixels: 1 KiB in, 2 KiB out): misaligned or
    missing maps, overlapping maps, bad sizes; an empty image does nothing."""
    wm = lib.sad_widen_map
    assert wm(P, 8, 8, None, None) == EINVAL
    assert wm(None, 8, 8, P + 4096, None) == EINVAL
    assert wm(P + 8, 8, 8, P + 4096, None) == EINVAL  # misaligned input
    assert wm(P, 8, 8, P + 4104, None) == EINVAL  # misaligned output
    assert wm(P, 8, 8, P + 1008, None) == EINVAL  # output over the input's last 16 bytes
    assert wm(P + 2032, 8, 8, P, None) == EINVAL  # input over the output's last 16 bytes
    assert wm(P, -1, 8, P + 4096, None) == EINVAL
    assert wm(P, 8, 1 << 20, P + 4096, None) == EINVAL
    assert wm(None, 0, 8, None, None) == 0  # empty image: nothing to do


def test_render_query_adam_reject(lib):
    assert lib.sad_render_fwd(P, 10, 8, 8, P + 4096, None, None) == EINVAL
    assert lib.sad_render_fwd(P, 10, -8, 8, P + 4096, P + 8192, None) == EINVAL
    bwd = lib.sad_render_bwd
    G, T, L = P + 65536, P + 8192, P + 131072  # grad, target, loss: apart
    assert bwd(P, 10, 8, 8, P + 4096, T, None, None, None, None) == EINVAL  # no grad
    assert bwd(P, 10, 8, 8, P + 4096, None, G, None, None, None) == EINVAL  # no target
    assert bwd(P, 10, 8, 8, P + 4096, T, P, None, None, None) == EINVAL  # grad aliases derived
    assert bwd(P, 10, 8, 8, P + 4096, T, P + 4096, None, None, None) == EINVAL  # grad over the lists
    assert bwd(P, 10, 8, 8, P + 4096, T, T, None, None, None) == EINVAL  # grad over the target
    assert bwd(P, 10, 8, 8, P + 4096, T, G, P + 2, None, None) == EINVAL  # loss misaligned
    assert bwd(P, 10, 8, 8, P + 4096, T, G, T + 16, None, None) == EINVAL  # loss inside the target
    assert bwd(P, 10, 8, 8, P + 4096, T, G, G + 64, None, None) == EINVAL  # loss inside grad
    assert bwd(P, 10, 8, 8, P + 4096, T, G, None, P + 4096 + 32, None) == EINVAL  # image over the lists
    assert bwd(P, 10, 8, 8, P + 4096, T, G, None, G + 16, None) == EINVAL  # image over grad
    assert bwd(P, 10, 8, 8, P + 4096, T, G, L, L, None) == EINVAL  # image over the loss
    assert bwd(P, 10, 8, 8, P + 4096, T, G, None, P + 2, None) == EINVAL  # image misaligned, over derived
    assert bwd(P, -1, 8, 8, P + 4096, T, G, None, None, None) == EINVAL
    assert bwd(P, 10, 0, 8, None, None, G, None, None, None) == 0  # empty image: nothing to do
    assert lib.sad_query_points(P, 10, 8, 8, P + 4096, P + 8192, -1, P + 65536, None) == EINVAL
    assert lib.sad_query_points(P, 10, 8, 8, P + 4096, P + 8196, 5, P + 65536, None) == EINVAL  # xy misaligned
    assert lib.sad_query_points(P, 10, 0, 8, P + 4096, P + 8192, 5, P + 65536, None) == EINVAL  # no lists
    assert lib.sad_query_points(P, 10, 8, 8, P + 4096, None, 0, None, None) == 0
    lr = (C.c_float * 5)(*([1e-3] * 5))
    assert lib.sad_adam_step(P, P + 4096, P + 8192, P + 12288, 10, 8, 8, None, .9, .999, 1e-8, .1, .001, None,
                             None) == EINVAL  # no rates
    assert lib.sad_adam_step(P, P, P + 8192, P + 12288, 10, 8, 8, lr, .9, .999, 1e-8, .1, .001, None,
                             None) == EINVAL  # params aliases grad
    assert lib.sad_adam_step(P, P + 4096, P + 8192, P + 12288, -3, 8, 8, lr, .9, .999, 1e-8, .1, .001, None,
                             None) == EINVAL
    # the Adam step that also writes probe records (10 sites: 480-byte records, 160-byte probe records)
    adam_p = lib.sad_adam_step_probe
    D = P + 16384
    assert adam_p(P, P + 4096, P + 8192, P + 12288, 10, 8, 8, lr, .9, .999, 1e-8, .1, .001, None, P + 20480,
                  None) == EINVAL  # probe records without prepared records
    assert adam_p(P, P + 4096, P + 8192, P + 12288, 10, 8, 8, lr, .9, .999, 1e-8, .1, .001, D, P + 20488,
                  None) == EINVAL  # misaligned probe records
    assert adam_p(P, P + 4096, P + 8192, P + 12288, 10, 8, 8, lr, .9, .999, 1e-8, .1, .001, D, D + 464,
                  None) == EINVAL  # probe records over the prepared records
    assert adam_p(P, P + 4096, P + 8192, P + 12288, 10, 8, 8, lr, .9, .999, 1e-8, .1, .001, D, P + 4096 + 320,
                  None) == EINVAL  # probe records over the gradients
    assert adam_p(P, P + 4096, P + 8192, P + 12288, 10, 8, 8, lr, .9, .999, 1e-8, .1, .001, D, P - 144,
                  None) == EINVAL  # probe records reaching into params
    assert adam_p(P, P + 4096, P + 8192, P + 12288, 0, 8, 8, lr, .9, .999, 1e-8, .1, .001, D, P + 20480,
                  None) == 0  # no sites: nothing to do


def test_step_fused_rejects(lib):
    f = lib.sad_step_fused
    ok = dict(derived=P, n=10, h=8, w=8, prev=None, sprev=None, nxt=P + 4096, snext=None, stride=1, seed=0, pi=0,
              inj=64, tgt=P + 8192, grad=P + 65536, loss=None, img=None)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["derived"], a["n"], a["h"], a["w"], a["prev"], a["sprev"], a["nxt"], a["snext"], a["stride"],
                 a["seed"], a["pi"], a["inj"], a["tgt"], a["grad"], a["loss"], a["img"], None)

    # the checks of the propagation pass
    assert call(stride=0) == EINVAL
    assert call(inj=65) == EUNSUP
    assert call(nxt=None) == EINVAL
    assert call(prev=P + 4096) == EINVAL
    # the checks of the backward pass
    assert call(tgt=None) == EINVAL
    assert call(grad=None) == EINVAL
    assert call(grad=P) == EINVAL  # aliases derived
    assert call(loss=P + 2) == EINVAL
    assert call(loss=P + 8192 + 4) == EINVAL  # loss inside the target
    # the pass's outputs against everything else the step touches
    assert call(nxt=P + 8192) == EINVAL  # over the target
    assert call(snext=P + 65536) == EINVAL  # over the gradients
    assert call(snext=P + 12288, img=P + 12288) == EINVAL  # image over the scores
    assert call(nxt=P + 16384, loss=P + 16384 + 64) == EINVAL  # loss inside the list map
    assert call(h=0, nxt=None, tgt=None) == 0  # empty image: nothing to do


def test_site_stats_rejects(lib):
    f = lib.sad_site_stats
    WS = 1 << 30
    wsb = lib.sad_site_stats_workspace_bytes(8, 8)
    assert wsb > 0 and lib.sad_site_stats_workspace_bytes(-1, 8) == 0
    ok = dict(derived=P, n=10, h=8, w=8, topk=P + 4096, tgt=P + 8192, stats=P + 65536, ws=WS, wsb=wsb)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["derived"], a["n"], a["h"], a["w"], a["topk"], a["tgt"], a["stats"], a["ws"], a["wsb"], None)

    assert call(n=-1) == EINVAL
    assert call(topk=None) == EINVAL
    assert call(tgt=None) == EINVAL
    assert call(stats=None) == EINVAL
    assert call(stats=P + 65536 + 4) == EINVAL  # misaligned
    assert call(stats=P + 16) == EINVAL  # overlaps the site records
    assert call(ws=None) == EINVAL
    assert call(wsb=wsb - 1) == EINVAL
    assert call(stats=WS + 64) == EINVAL  # inside the workspace
    assert call(ws=P + 8192 + 64) == EINVAL  # workspace over the target
    assert call(ws=P + 4096) == EINVAL  # workspace over the lists
    assert call(ws=P) == EINVAL  # workspace over the site records
    assert call(stats=P + 4096) == EINVAL  # statistics over the lists
    assert call(stats=P + 8192) == EINVAL  # statistics over the target
    assert call(h=0, topk=None, tgt=None, ws=None) == 0  # empty image: nothing to do


def test_site_stats_noalloc_rejects(lib):
    """The allocation-free statistics refuse what sad_site_stats refuses, and
    images whose region tables exceed the library's array (checked before any
    GPU call)."""
    f = lib.sad_site_stats_noalloc
    assert f(P, 10, 2048, 2048, P + 4096, P + 8192, P + 65536, None) == EUNSUP
    assert f(P, 10, 1 << 15, 1 << 15, P + 4096, P + 8192, P + 65536, None) == EUNSUP
    assert f(P, 10, -1, 8, P + 4096, P + 8192, P + 65536, None) == EINVAL
    assert lib.sad_site_stats_workspace_bytes(1080, 1920) <= 40 << 20 < lib.sad_site_stats_workspace_bytes(2048, 2048)


def test_jfa_rejects(lib):
    assert lib.sad_jfa_seed(P, -1, 8, 8, P + 4096, None) == EINVAL
    assert lib.sad_jfa_seed(P, 10, 8, 8, None, None) == EINVAL
    assert lib.sad_jfa_seed(P, 10, 8, 8, P + 4100, None) == EINVAL  # misaligned
    assert lib.sad_jfa_seed(P, 10, 8, 8, P + 64, None) == EINVAL  # over the site records
    assert lib.sad_jfa_seed(P, 10, 0, 8, None, None) == 0  # empty image
    f = lib.sad_jfa_flood
    assert f(P, 10, 8, 8, P + 4096, P + 8192, 0, 4, None) == EINVAL  # step 0
    assert f(P, 10, 8, 8, P + 4096, P + 8192, 1, 5, None) == EINVAL  # width
    assert f(P, 10, 8, 8, None, P + 8192, 1, 4, None) == EINVAL
    assert f(P, 10, 8, 8, P + 4096, P + 4096 + 512, 1, 8, None) == EINVAL  # out over the input
    assert f(P, 10, 8, 8, P + 4096, P + 16, 1, 4, None) == EINVAL  # out over the site records
    assert f(P, 10, 0, 8, None, None, 1, 4, None) == 0


def test_densify_prune_rejects(lib):
    f = lib.sad_densify_prune
    n = 10
    wsb = lib.sad_budget_workspace_bytes(n)
    WS = 1 << 30
    ok = dict(p=P, m=P + 4096, v=P + 8192, d=P + 12288, n=n, h=8, w=8, st=P + 16384, t=P + 20480, ns=2, npr=1,
              done=None, ws=WS, wsb=wsb)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["p"], a["m"], a["v"], a["d"], a["n"], a["h"], a["w"], a["st"], a["t"], a["ns"], a["npr"], 1.0,
                 1.0, 0.5, 0.85, 0.1, a["done"], a["ws"], a["wsb"], None)

    assert call(ns=-1) == EINVAL
    assert call(npr=-1) == EINVAL
    assert call(m=None) == EINVAL
    assert call(st=P + 16384 + 4) == EINVAL  # misaligned
    assert call(v=P + 4096 + 64) == EINVAL  # the moments overlap
    assert call(h=0, t=None) == EINVAL  # sites but no target image
    assert call(ws=None) == EINVAL
    assert call(ws=WS + 16) == EINVAL  # workspace not 256-byte aligned
    assert call(wsb=wsb - 1) == EINVAL
    assert call(done=P + 2) == EINVAL
    assert call(done=P + 8) == EINVAL  # inside the sites
    assert call(n=0, ws=None, done=None) == 0  # no sites and no counts: nothing to launch


def test_init_sites_rejects(lib):
    f = lib.sad_init_sites
    h, w, n = 8, 8, 10
    wsb = lib.sad_init_workspace_bytes(h, w)
    assert wsb >= 2 * 8 * h * w
    WS = 1 << 30
    ok = dict(t=P, h=h, w=w, n=n, lam=0.5, p=P + 4096, d=P + 8192, ws=WS, wsb=wsb)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["t"], a["h"], a["w"], a["n"], a["lam"], 7, 0.0, 0.0, 0.0, a["p"], a["d"], a["ws"], a["wsb"], None)

    assert call(lam=-0.1) == EINVAL
    assert call(lam=1.5) == EINVAL
    assert call(lam=float("nan")) == EINVAL
    assert call(n=-1) == EINVAL
    assert call(h=0) == EINVAL  # sites need pixels
    assert call(t=None) == EINVAL
    assert call(p=P + 4096 + 4) == EINVAL  # misaligned
    assert call(d=P + 4096 + 16) == EINVAL  # overlaps params
    assert call(p=P + 64) == EINVAL  # overlaps the target
    assert call(ws=None) == EINVAL
    assert call(ws=WS + 64) == EINVAL
    assert call(wsb=wsb - 1) == EINVAL
    assert call(n=0, t=None, ws=None) == 0  # nothing to draw


def test_packed_rejects(lib):
    pk, q, m_ = lib.sad_pack_sites, lib.sad_query_packed, P + 65536
    assert pk(P, P + 4096, -1, 8, 8, P + 8192, P + 12288, None) == EINVAL
    assert pk(P, P + 4096, 10, 0, 8, P + 8192, P + 12288, None) == EINVAL  # positions need an image
    assert pk(P, P + 4096, 10, 8, 8, P + 8, P + 12288, None) == EINVAL  # misaligned records
    assert pk(P, P + 4096, 10, 8, 8, P + 4096 + 64, P + 12288, None) == EINVAL  # records over derived
    assert pk(P, P + 4096, 10, 8, 8, P + 8192, None, None) == EINVAL
    assert pk(P, P + 4096, 10, 8, 8, P + 8192, P + 8192 + 32, None) == EINVAL  # ranges inside the records
    assert q(P, P + 4096, 10, 8, 8, P + 8192, m_, -1, m_ + 4096, None) == EINVAL
    assert q(P, P + 4096, 10, 0, 8, P + 8192, m_, 5, m_ + 4096, None) == EINVAL  # points without lists
    assert q(P, None, 10, 8, 8, P + 8192, m_, 5, m_ + 4096, None) == EINVAL
    assert q(P, P + 4096, 10, 8, 8, P + 8192, m_ + 4, 5, m_ + 4096, None) == EINVAL  # misaligned points
    assert q(P, P + 4096, 10, 8, 8, P + 8192, m_, 5, m_ + 8, None) == EINVAL  # colours over the points
    assert q(P, P + 4096, 10, 8, 8, P + 8192, m_, 0, m_ + 4096, None) == 0  # no points
