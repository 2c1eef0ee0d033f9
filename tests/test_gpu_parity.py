"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Top-K maps, prepared records and Adam updates are compared bit for bit;
colours, gradients and the loss within the tolerances of gpu_util.  Inputs
come from the seeded generators in ``synth``; expected values only from the
oracle.
"""
import math

import numpy as np
import pytest
import torch

import synth
from gpu_util import (assert_colour_close, assert_grad_close, assert_stats_close, dev, map_to_np, say, to_gpu,
                      to_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sad():
    from voronoi_rendering_amd import ops

    say("[gpu] device: " + torch.cuda.get_device_name(0))
    return ops


def gpu_schedule(ops, d_gpu, h, w, strides, seed, inject=64, first_pass=0, prev=None):
    cur = prev if prev is not None else ops.empty_map(h, w, dev())
    nxt = torch.empty_like(cur)
    for t, s in enumerate(strides):
        ops.propagate_topk(d_gpu, h, w, cur, nxt, stride=int(s), seed=seed, pass_index=first_pass + t, inject=inject)
        cur, nxt = nxt, cur
    return cur


# ---------------------------------------------------------------- prepare

def test_prepare_bit_exact(sad, ref):
    p = np.concatenate([synth.C2.make_sites(), synth.C4.make_sites()[:100_000], synth.C3.make_sites()[:1000]])
    extra = synth.sites(9, 16, 32, 32)
    extra[0, 0] = -1.0  # inactive
    extra[1, 7] = 2.0e6  # beyond the rotation range
    extra[2, 7] = np.nan
    extra[3, 7] = -0.0
    extra[4, 8:10] = [90.0, -90.0]  # subnormal and infinite inverse scales
    extra[5, 2] = 88.7  # tau near the float32 limit
    extra[6, 7] = 1048575.9
    extra[7, 7] = -3.0e5
    extra[8, 0] = np.nan
    p = np.concatenate([p, extra])
    want = ref.prepare_sites(p)
    got = to_np(sad.prepare_sites(to_gpu(p)))
    assert ref.ambiguous_count() == 0
    same = (got.view(np.uint32) == want.view(np.uint32)) | (np.isnan(got) & np.isnan(want))
    assert same.all(), np.argwhere(~same)[:5]


# ---------------------------------------------------------------- propagation

def test_propagate_c1_every_pass(sad, ref):
    """64x64, 256 sites, 20 passes from an empty map: every intermediate map
    equals the oracle's, and the result is the exact top-8 at >= 99% of pixels."""
    wl = synth.C1
    p = wl.make_sites()
    d = ref.prepare_sites(p)
    dg = sad.prepare_sites(to_gpu(p))
    cur_ref, cur_gpu = None, sad.empty_map(wl.h, wl.w, dev())
    nxt = torch.empty_like(cur_gpu)
    for t, s in enumerate(wl.strides):
        cur_ref = ref.propagate(d, wl.h, wl.w, cur_ref, s, wl.inject_seed, t, wl.inject)
        sad.propagate_topk(dg, wl.h, wl.w, cur_gpu, nxt, stride=s, seed=wl.inject_seed, pass_index=t,
                           inject=wl.inject)
        cur_gpu, nxt = nxt, cur_gpu
        got = map_to_np(cur_gpu)
        assert np.array_equal(got, cur_ref), f"pass {t}: {np.argwhere(got != cur_ref)[:3]}"
    exact = ref.brute_topk(d, wl.h, wl.w)
    frac = (map_to_np(cur_gpu) == exact).all(-1).mean()
    say(f"[gpu] C1 exact top-8 fraction after 20 passes: {frac:.4f}")
    assert frac >= 0.99


@pytest.mark.parametrize("h,w,n,strides,inject", [
    (1, 1, 3, (1, 1), 64),
    (1, 37, 20, (16, 4, 1), 64),
    (45, 1, 20, (32, 2, 1), 5),
    (13, 29, 300, (8, 4, 2, 1, 1), 64),
    (67, 72, 1000, (64, 32, 16, 8, 4, 2, 1), 17),
    (40, 40, 0, (1, 1), 64),  # no sites: lists stay empty
    (24, 31, 50, (100, 1), 0),  # no injection: the map stays empty
    (24, 31, 5, (1, 3), 1),
])
def test_propagate_ragged_and_edge_cases(sad, ref, h, w, n, strides, inject):
    p = synth.sites(60 + h + n, n, h, w)
    if n >= 10:
        p[3, 0] = -1.0  # an inactive site
        p[7] = p[5]  # identical sites: ties broken by index
    d = ref.prepare_sites(p)
    dg = sad.prepare_sites(to_gpu(p)) if n > 0 else torch.zeros((0, 12), dtype=torch.float32, device=dev())
    want = ref.propagate_schedule(d, h, w, None, strides, 77, 3, inject)
    got = map_to_np(gpu_schedule(sad, dg, h, w, strides, 77, inject, first_pass=3))
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]


@pytest.mark.parametrize("h,w,n,strides,inject", [
    (1, 1, 3, (1, 1, 1), 64),
    (13, 29, 300, (8, 4, 2, 1), 64),
    (40, 40, 0, (1, 1), 64),  # no sites: no probe records, lists stay empty
    (24, 31, 5, (1, 3, 1), 1),
    (67, 9, 70, (16, 4, 1), 64),
    (1, 1, 150, (1, 1, 1), 64),  # 150 sites, one tile of 64 lanes: each lane writes up to 3 probe records
])
def test_propagate_step_forms_edge_cases(sad, ref, h, w, n, strides, inject):
    """The forms a training step hands on (16-bit maps, 8th logits, probe
    records written by the first pass and culled from by the later ones) on
    ragged and degenerate images and site counts: the oracle's lists."""
    p = synth.sites(90 + h + n, n, h, w)
    if n >= 10:
        p[3, 0] = -1.0  # an inactive site
    d = ref.prepare_sites(p)
    dg = sad.prepare_sites(to_gpu(p)) if n > 0 else torch.zeros((0, 12), dtype=torch.float32, device=dev())
    m = ref.propagate_schedule(d, h, w, None, (8, 4, 2, 1), 13, 0, inject)
    prev, thr = to_gpu(m), None
    probe = torch.empty((n, 4), dtype=torch.float32, device=dev())
    for t, s_ in enumerate(strides):
        want = ref.propagate(d, h, w, m, s_, 13, 4 + t, inject)
        out = torch.empty((h, w, 8), dtype=torch.int16, device=dev())
        out_thr = torch.empty((h, w), dtype=torch.float32, device=dev())
        sad.propagate_topk(dg, h, w, prev, out, stride=s_, seed=13, pass_index=4 + t, inject=inject, prev_thr=thr,
                           out_thr=out_thr, prev_probe=probe if t > 0 else None, out_probe=probe if t == 0 else None)
        got = map16_to_np(out)
        assert np.array_equal(got, want), f"pass {t}: {np.argwhere(got != want)[:4]}"
        m, prev, thr = want, out, out_thr


def test_propagate_from_given_map_with_stale_ids(sad, ref):
    """A previous map with out-of-range ids, inactive sites and duplicates."""
    h, w, n = 30, 42, 200
    p = synth.sites(70, n, h, w)
    p[11, 0] = -2.0
    d = ref.prepare_sites(p)
    rng = np.random.default_rng(5)
    prev = rng.integers(0, n + 40, (h, w, 8)).astype(np.uint32)
    prev[rng.random((h, w, 8)) < 0.2] = 0xFFFFFFFF
    prev[..., 3] = prev[..., 2]  # duplicates inside a list
    prev[0, 0, :] = 11  # only an inactive site
    want = ref.propagate(d, h, w, prev, 2, 5, 9, 64)
    got = map_to_np(sad.propagate_topk(sad.prepare_sites(to_gpu(p)), h, w, to_gpu(prev), stride=2, seed=5,
                                       pass_index=9, inject=64))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("n", [5000, 70000])
def test_propagate_full_neighbour_queue(sad, ref, n):
    """Every queued neighbour id survives: pixels with an empty list between
    pixels holding 8 distinct ids each, so the 16 ids of a pair of
    neighbour lists are all fresh and all beat the empty 8th entry (the
    scoring batches then reach the end of the queue); both id widths."""
    h, w = 37, 70
    p = synth.sites(90 + n % 7, n, h, w)
    d = ref.prepare_sites(p)
    rng = np.random.default_rng(n)
    prev = np.full((h, w, 8), 0xFFFFFFFF, dtype=np.uint32)
    ys, xs = np.mgrid[0:h, 0:w]
    full = (xs + ys) % 2 == 0
    prev[full] = np.stack([rng.choice(n, 8, replace=False) for _ in range(int(full.sum()))]).astype(np.uint32)
    dg = sad.prepare_sites(to_gpu(p))
    for stride in (1, 3):
        want = ref.propagate(d, h, w, prev, stride, 6, 21, 64)
        got = map_to_np(sad.propagate_topk(dg, h, w, to_gpu(prev), stride=stride, seed=6, pass_index=21, inject=64))
        assert np.array_equal(got, want), f"stride {stride}: {np.argwhere(got != want)[:5]}"


@pytest.mark.parametrize("n", [1500, 70000])
def test_propagate_extreme_sites(sad, ref, n):
    """Sites far outside the workloads' ranges, where the screen of queued
    ids (an approximate logit and an error bound) has the least room: scales
    from e^-6 to e^8 px per axis (anisotropy up to e^14), tau from e^-6 to
    e^6, r from -5 to 20, a tenth of the sites a thousand image widths away,
    some at the pixel centres.  Eight passes from the oracle's warm map, each
    bit for bit; both id widths."""
    h, w = 60, 90
    rec = synth.SiteRecipe(ls_lo=-6.0, ls_hi=8.0, r_lo=-5.0, r_hi=20.0, logtau_lo=-6.0, logtau_hi=6.0)
    p = synth.sites(4242 + n, n, h, w, rec)
    rng = np.random.default_rng(n)
    far = rng.random(n) < 0.1
    p[far, 0] *= np.float32(1000.0)
    p[far, 1] *= np.float32(1000.0)
    centred = rng.random(n) < 0.05
    p[centred, 0] = np.floor(p[centred, 0] % w) + np.float32(0.5)
    p[centred, 1] = np.floor(p[centred, 1] % h) + np.float32(0.5)
    d = ref.prepare_sites(p)
    dg = sad.prepare_sites(to_gpu(p))
    m = ref.propagate_schedule(d, h, w, None, synth.jfa_strides(h, w, 12), 31, 0, 64)
    cur = to_gpu(m)
    for t, stride in enumerate((8, 4, 2, 1, 1, 3, 2, 1)):
        want = ref.propagate(d, h, w, m, stride, 31, 12 + t, 64)
        got_t = sad.propagate_topk(dg, h, w, cur, stride=stride, seed=31, pass_index=12 + t, inject=64)
        got = map_to_np(got_t)
        assert np.array_equal(got, want), f"pass {t} stride {stride}: {np.argwhere(got != want)[:5]}"
        m, cur = want, got_t


@pytest.mark.parametrize("n", [65535, 65536])
def test_propagate_at_the_16_bit_id_boundary(sad, ref, n):
    """Site counts on both sides of the packed 16-bit membership test, with
    previous lists holding ids whose low 16 bits equal those of listed ids
    (v + 2^16, 2^16 - 1, EMPTY): out-of-range ids must be dropped and never
    mistaken for listed ones."""
    h, w = 45, 58
    p = synth.sites(80 + n, n, h, w)
    d = ref.prepare_sites(p)
    base = ref.propagate_schedule(d, h, w, None, (32, 16, 8, 4, 2, 1), 9, 0, 64).astype(np.int64)
    rng = np.random.default_rng(n)
    prev = base.copy()
    r = rng.random(prev.shape)
    prev[r < 0.25] = (base[r < 0.25] % 65536) + 65536  # aliases of listed ids, all >= n
    prev[(r >= 0.25) & (r < 0.3)] = 65535  # in range only when n = 65536
    prev[(r >= 0.3) & (r < 0.35)] = 0xFFFFFFFF
    prev = prev.astype(np.uint32)
    dg = sad.prepare_sites(to_gpu(p))
    for stride in (1, 3):
        want = ref.propagate(d, h, w, prev, stride, 4, 12, 64)
        got = map_to_np(sad.propagate_topk(dg, h, w, to_gpu(prev), stride=stride, seed=4, pass_index=12, inject=64))
        assert np.array_equal(got, want), f"stride {stride}: {np.argwhere(got != want)[:5]}"


@pytest.fixture(scope="module")
def c2_state(sad, ref):
    """The 768x512, 50k-site workload: 16 warm-up passes, then one step's
    strides 8, 4, 2, 1, on both sides."""
    wl = synth.C2
    p = wl.make_sites()
    d = ref.prepare_sites(p)
    strides = synth.jfa_strides(wl.h, wl.w, wl.warm_passes) + list(wl.strides)
    say(f"[gpu] C2 oracle: {len(strides)} passes at {wl.w}x{wl.h}, n={wl.n}")
    m_ref = ref.propagate_schedule(d, wl.h, wl.w, None, strides, wl.inject_seed, 0, wl.inject)
    dg = sad.prepare_sites(to_gpu(p))
    m_gpu = gpu_schedule(sad, dg, wl.h, wl.w, strides, wl.inject_seed, wl.inject)
    return wl, p, d, dg, m_ref, m_gpu


def test_propagate_c2_full_map(c2_state):
    wl, p, d, dg, m_ref, m_gpu = c2_state
    got = map_to_np(m_gpu)
    assert np.array_equal(got, m_ref), f"{(got != m_ref).any(-1).sum()} pixels differ"


def test_c2_map_quality(sad, ref):
    """Quality of the 768x512 / 50k-site map (top-8 sets against brute force
    on 1,024 random pixels): 16 passes from an empty map find few sites (a
    site enters the lists only when a probe lands on it), the full refresh
    about two thirds of the lists, and steps on the static sites settle the
    lists to the exact top-8."""
    from voronoi_rendering_amd.pipeline import SadField

    wl = synth.C2
    p = wl.make_sites()
    d = ref.prepare_sites(p)
    tgt = to_gpu(wl.make_target())
    pix = np.random.default_rng(70).integers(0, wl.h * wl.w, 1024)
    exact = np.sort(ref.brute_topk_pixels(d, wl.h, wl.w, pix), axis=1)
    sel = torch.from_numpy(pix).to(dev())

    def match(f):
        got = np.sort(to_np(f.topk.view(-1, 8)[sel]).view(np.uint32), axis=1)
        return float((got == exact).all(1).mean())

    f = SadField(to_gpu(p), wl.h, wl.w, wl.inject_seed, inject=wl.inject)
    f.warm(wl.warm_passes)
    from_empty = match(f)
    f.refresh(16)
    refreshed = match(f)
    for _ in range(500):
        f.sites_changed()
        f.step(list(wl.strides), tgt, fused=True)
    settled = match(f)
    say(f"[gpu] C2 exact match: 16 passes from empty {from_empty:.3f}, full refresh {refreshed:.3f}, "
        f"+500 steps {settled:.3f}")
    assert refreshed >= 0.5 and settled >= 0.99


def test_pipeline_step_with_32bit_ids(sad, ref):
    """SadField.step with more than 65,535 sites (512x512, 70,000 sites): the
    passes hand on 32-bit maps with only their 8th logits and cull probes from
    the probe records; from the GPU's map after a full refresh and two steps,
    a further step's lists are the oracle's chain bit for bit and its loss
    and gradients the oracle's backward's."""
    from voronoi_rendering_amd.pipeline import SadField

    h, w, n = 512, 512, 70_000
    p = synth.sites(1717, n, h, w)
    p[::97, 0] = -1.0  # inactive sites
    d = ref.prepare_sites(p)
    tgt_np = synth.target_noise_edges(1718, h, w)
    tgt = to_gpu(tgt_np)
    strides = [8, 4, 2, 1]
    f = SadField(to_gpu(p), h, w, 29, inject=64)
    f.refresh(16)
    for _ in range(2):
        f.sites_changed()
        f.step(strides, tgt, fused=True)
    assert f.inter is not None and f.inter[0].dtype == torch.int32
    f.sites_changed()
    prev = map_to_np(f.topk)
    first = f.pass_index
    f.grad.zero_()
    f.loss.zero_()
    f.step(strides, tgt, fused=True)
    for k, s in enumerate(strides):
        prev = ref.propagate(d, h, w, prev, s, 29, first + k, 64)
    got = map_to_np(f.topk)
    assert np.array_equal(got, prev), f"{(got != prev).any(-1).sum()} pixels differ"
    g_ref, _, loss_ref, _ = ref.render_bwd(d, h, w, prev, tgt_np)
    assert abs(f.loss.item() - loss_ref) <= 1e-5 * loss_ref
    assert_grad_close(to_np(f.grad), g_ref, "32-bit step gradients")


def test_bench_map_step(sad, ref):
    """The launch configuration the bench times: the 768x512 / 50k-site map
    built by the full refresh and settled by 500 steps, then one more step
    as the bench runs it, then one pass by pass (stride-8 pass with the logits
    recomputed, passes with score maps, the backward): the lists and the
    gradients against the oracle run on the GPU's map."""
    from voronoi_rendering_amd.pipeline import SadField

    wl = synth.C2
    p = wl.make_sites()
    d = ref.prepare_sites(p)
    tgt_np = wl.make_target()
    tgt = to_gpu(tgt_np)
    f = SadField(to_gpu(p), wl.h, wl.w, wl.inject_seed, inject=wl.inject)
    f.refresh(16)
    for _ in range(500):
        f.sites_changed()
        f.step(list(wl.strides), tgt, fused=True)
    # the step as the bench runs it (the previous step's 16-bit map, thresholds,
    # probe records current with the sites, the fused last pass writing the
    # next 16-bit map): each pass's lists are the oracle's, so the last map
    # must be the oracle's chain, and the gradients its backward's
    f.sites_changed(probe_records_current=True)
    assert f.cur16 and f.probe_valid
    prev = field_lists(f)
    first = f.pass_index
    f.grad.zero_()
    f.loss.zero_()
    f.step(list(wl.strides), tgt, fused=True)
    for k, s in enumerate(wl.strides):
        prev = ref.propagate(d, wl.h, wl.w, prev, s, wl.inject_seed, first + k, wl.inject)
    assert f.cur16
    got = field_lists(f)
    assert np.array_equal(got, prev), f"step: {(got != prev).any(-1).sum()} pixels differ"
    assert np.array_equal(map_to_np(f.topk), prev)  # widened on request
    g_ref, _, loss_ref, _ = ref.render_bwd(d, wl.h, wl.w, prev, tgt_np)
    assert abs(f.loss.item() - loss_ref) <= 1e-5 * loss_ref
    assert_grad_close(to_np(f.grad), g_ref, "step gradients")
    # then pass by pass on 32-bit maps with score maps
    f.sites_changed()
    for s in wl.strides:
        first = f.pass_index
        f.propagate([s])
        want = ref.propagate(d, wl.h, wl.w, prev, s, wl.inject_seed, first, wl.inject)
        got = map_to_np(f.topk)
        assert np.array_equal(got, want), f"stride {s}: {(got != want).any(-1).sum()} pixels differ"
        prev = want
    g_ref, g_abs, loss_ref, _ = ref.render_bwd(d, wl.h, wl.w, prev, tgt_np)
    grad = torch.zeros((wl.n, 12), dtype=torch.float32, device=dev())
    loss = torch.zeros(1, dtype=torch.float32, device=dev())
    sad.render_bwd(f.derived, wl.h, wl.w, f.topk, tgt, grad, loss, None)
    assert abs(loss.item() - loss_ref) <= 1e-5 * loss_ref
    assert_grad_close(to_np(grad), g_ref, "settled-map gradients")


def test_propagate_with_score_maps(sad, ref, c2_state):
    """Passes chained through score maps (the previous pass's logits reused)
    give the oracle's lists bit for bit, and the score map holds exactly the
    float32 logits of the listed sites."""
    wl, p, d, dg, m_ref, m_gpu = c2_state
    strides = (8, 4, 2, 1, 1)
    cur = m_gpu
    sc = None
    for t, s in enumerate(strides):
        out_s = torch.empty((wl.h, wl.w, 8), dtype=torch.float32, device=dev())
        cur = sad.propagate_topk(dg, wl.h, wl.w, cur, stride=s, seed=7, pass_index=500 + t, inject=64,
                                 prev_scores=sc, out_scores=out_s)
        sc = out_s
    want = ref.propagate_schedule(d, wl.h, wl.w, m_ref, strides, 7, 500, 64)
    got = map_to_np(cur)
    assert np.array_equal(got, want), f"{(got != want).any(-1).sum()} pixels differ"
    scores = to_np(sc)
    rng = np.random.default_rng(2)
    for pix in rng.choice(wl.h * wl.w, 300, replace=False):
        j, i = divmod(int(pix), wl.w)
        for k in range(8):
            sid = int(got[j, i, k])
            if sid == 0xFFFFFFFF:
                assert scores[j, i, k] == -np.inf
            else:
                assert np.float32(ref.score(d, sid, i + 0.5, j + 0.5)).view(np.uint32) == \
                    scores[j, i, k].view(np.uint32)


def test_propagate_is_deterministic(sad, c2_state):
    wl, p, d, dg, m_ref, m_gpu = c2_state
    a = sad.propagate_topk(dg, wl.h, wl.w, m_gpu, stride=1, seed=1, pass_index=99, inject=64)
    b = sad.propagate_topk(dg, wl.h, wl.w, m_gpu, stride=1, seed=1, pass_index=99, inject=64)
    assert torch.equal(a, b)


@pytest.fixture(scope="module")
def c4_state(sad, ref):
    """2048x2048, 400k sites: 16 warm-up passes and the step strides
    16, 8, 4, 2, 1 on both sides."""
    wl = synth.C4
    p = wl.make_sites()
    d = ref.prepare_sites(p)
    strides = synth.jfa_strides(wl.h, wl.w, wl.warm_passes) + list(wl.strides)
    dg = sad.prepare_sites(to_gpu(p))
    m_gpu = gpu_schedule(sad, dg, wl.h, wl.w, strides, wl.inject_seed, wl.inject)
    cur = None
    for t, s in enumerate(strides):
        cur = ref.propagate(d, wl.h, wl.w, cur, s, wl.inject_seed, t, wl.inject)
        say(f"[gpu] C4 oracle pass {t + 1}/{len(strides)} (stride {s})")
    return wl, d, dg, cur, m_gpu


def test_propagate_c4_full_map(c4_state):
    """The 2048x2048 map after warm-up and one step equals the oracle's bit for bit."""
    wl, d, dg, m_ref, m_gpu = c4_state
    got = map_to_np(m_gpu)
    assert np.array_equal(got, m_ref), f"{(got != m_ref).any(-1).sum()} pixels differ"


def test_render_c4(sad, ref, c4_state):
    """Forward, loss and gradients at 2048x2048 / 400k sites (the densest
    gradient scatter of the workloads)."""
    wl, d, dg, m_ref, m_gpu = c4_state
    tgt = wl.make_target()
    g_ref, g_abs, loss_ref, img_ref = ref.render_bwd(d, wl.h, wl.w, m_ref, tgt)
    grad = torch.zeros((wl.n, 12), dtype=torch.float32, device=dev())
    loss = torch.zeros(1, dtype=torch.float32, device=dev())
    img = torch.empty((wl.h, wl.w, 3), dtype=torch.float32, device=dev())
    sad.render_bwd(dg, wl.h, wl.w, m_gpu, to_gpu(tgt), grad, loss, img)
    assert_colour_close(to_np(img), img_ref, "C4 image")
    assert abs(loss.item() - loss_ref) <= 1e-5 * loss_ref
    assert_grad_close(to_np(grad), g_ref, "C4 gradients")


def test_propagate_and_render_8192_sampled(sad, ref):
    """8192x8192 (2^20 tiles) with 2M sites, some inactive: two passes from
    the empty map (strides 64 and 1), 4,000 sampled pixels and the image's
    corners and edges of each pass against the oracle run on the GPU's
    previous map, then the render at those pixels."""
    h = w = 8192
    n = 2_000_000
    p = synth.sites(77, n, h, w, synth.WIDE_SCALES)
    p[::97, 0] = -1.0
    say(f"[gpu] {w}x{h}, n={n}: preparing sites")
    d = ref.prepare_sites(p)
    dg = sad.prepare_sites(to_gpu(p))
    assert np.array_equal(to_np(dg).view(np.uint32), d.view(np.uint32))
    rng = np.random.default_rng(5)
    edge = [0, w - 1, (h - 1) * w, h * w - 1, 5 * w, 5 * w + w - 1, (h - 1) * w + 77]
    pix = np.concatenate([rng.integers(0, h * w, 4000), edge]).astype(np.int64)
    sel = torch.from_numpy(pix).to(dev())
    cur = sad.empty_map(h, w, dev())
    nxt = torch.empty_like(cur)
    prev_np = None
    for t, s in enumerate((64, 1)):
        sad.propagate_topk(dg, h, w, cur, nxt, stride=s, seed=91, pass_index=t, inject=64)
        got = to_np(nxt.view(-1, 8)[sel]).view(np.uint32)
        want = ref.propagate_pixels(d, h, w, prev_np, s, 91, t, 64, pix)
        assert np.array_equal(got, want), f"pass {t}: {(got != want).any(-1).sum()} sampled pixels differ"
        say(f"[gpu] pass {t} (stride {s}) matches at {len(pix)} pixels")
        prev_np = map_to_np(nxt)
        cur, nxt = nxt, cur
    xy = np.stack([pix % w + 0.5, pix // w + 0.5], 1).astype(np.float32)
    got = to_np(sad.query_points(dg, h, w, cur, to_gpu(xy)))
    assert np.abs(got - ref.query_points(d, h, w, prev_np, xy)).max() <= 1e-5


def test_calls_follow_the_current_stream(sad, ref):
    """Every call enqueues on the caller's current stream: each C-ABI call made
    inside `with torch.cuda.stream(side)` receives that stream's handle (a
    recorder stands between the binding and the library), and the side stream
    gives the same map and image as the default stream, bit for bit, and the
    same loss and gradients up to the order of their float atomics."""
    from voronoi_rendering_amd import _native

    wl = synth.C1
    p = to_gpu(wl.make_sites())
    tgt = to_gpu(wl.make_target())

    def run():
        d = sad.prepare_sites(p)
        cur = sad.empty_map(wl.h, wl.w, dev())
        nxt = torch.empty_like(cur)
        for t, st in enumerate(wl.strides):
            sad.propagate_topk(d, wl.h, wl.w, cur, nxt, stride=st, seed=wl.inject_seed, pass_index=t,
                               inject=wl.inject)
            cur, nxt = nxt, cur
        grad = torch.zeros((wl.n, 12), dtype=torch.float32, device=dev())
        loss = torch.zeros(1, dtype=torch.float32, device=dev())
        img = torch.empty((wl.h, wl.w, 3), dtype=torch.float32, device=dev())
        sad.render_bwd(d, wl.h, wl.w, cur, tgt, grad, loss, img)
        stats = sad.site_stats(d, wl.h, wl.w, cur, tgt)
        return cur, img, loss, grad, stats

    class Recorder:
        """Forwards to the library; notes the stream (last argument) of every call."""

        def __init__(self, lib):
            self.lib, self.calls = lib, []

        def __getattr__(self, name):
            fn = getattr(self.lib, name)
            if not name.startswith("sad_") or name.endswith("_bytes") or name in ("sad_status_string",
                                                                                 "sad_abi_version"):
                return fn

            def call(*args):
                self.calls.append((name, args[-1]))
                return fn(*args)

            return call

    base = [to_np(x) for x in run()]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    real = _native.lib()
    rec = Recorder(real)
    _native._lib = rec
    try:
        with torch.cuda.stream(side):
            out = run()
    finally:
        _native._lib = real
    side.synchronize()
    names = {c[0] for c in rec.calls}
    assert {"sad_prepare_sites", "sad_propagate_topk", "sad_render_bwd", "sad_site_stats"} <= names
    assert side.cuda_stream != torch.cuda.default_stream().cuda_stream
    assert all(stream == side.cuda_stream for _, stream in rec.calls), rec.calls
    got = [to_np(x) for x in out]
    for a, b in zip(base[:2], got[:2]):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    np.testing.assert_allclose(got[2], base[2], rtol=1e-6)
    np.testing.assert_allclose(got[3], base[3], rtol=1e-5, atol=1e-7 * np.abs(base[3]).max())
    np.testing.assert_allclose(got[4], base[4], rtol=1e-5, atol=1e-7 * np.abs(base[4]).max())


# ---------------------------------------------------------------- render / backward

def test_render_fwd_c1_c2(sad, ref, c2_state):
    wl1 = synth.C1
    p1 = wl1.make_sites()
    d1 = ref.prepare_sites(p1)
    m1 = ref.brute_topk(d1, wl1.h, wl1.w)
    got = to_np(sad.render_fwd(sad.prepare_sites(to_gpu(p1)), wl1.h, wl1.w, to_gpu(m1)))
    assert_colour_close(got, ref.render_fwd(d1, wl1.h, wl1.w, m1), "C1 image")
    wl, p, d, dg, m_ref, m_gpu = c2_state
    got = to_np(sad.render_fwd(dg, wl.h, wl.w, to_gpu(m_ref)))
    assert_colour_close(got, ref.render_fwd(d, wl.h, wl.w, m_ref), "C2 image")


def test_render_bwd_c1(sad, ref):
    wl = synth.C1
    p = wl.make_sites()
    p[9, 0] = -1.0  # an inactive site listed nowhere, and a stale list entry below
    d = ref.prepare_sites(p)
    m = ref.propagate_schedule(d, wl.h, wl.w, None, wl.strides, wl.inject_seed, 0, wl.inject)
    m[5, 5, 7] = 9
    m[6, 6, 7] = 100000
    tgt = wl.make_target()
    g_ref, g_abs, loss_ref, img_ref = ref.render_bwd(d, wl.h, wl.w, m, tgt)
    dg = sad.prepare_sites(to_gpu(p))
    grad = torch.zeros((wl.n, 12), dtype=torch.float32, device=dev())
    loss = torch.zeros(1, dtype=torch.float32, device=dev())
    img = torch.empty((wl.h, wl.w, 3), dtype=torch.float32, device=dev())
    sad.render_bwd(dg, wl.h, wl.w, to_gpu(m), to_gpu(tgt), grad, loss, img)
    assert_colour_close(to_np(img), img_ref, "C1 image from backward")
    assert abs(loss.item() - loss_ref) <= 1e-5 * loss_ref
    g = to_np(grad)
    assert_grad_close(g, g_ref, "C1 gradients")
    assert np.all(g[:, 10:] == 0)
    # accumulation: a second call adds the same again
    sad.render_bwd(dg, wl.h, wl.w, to_gpu(m), to_gpu(tgt), grad, loss, None)
    assert_grad_close(to_np(grad), 2 * g_ref, "C1 gradients, accumulated twice")


def test_render_bwd_c2(sad, ref, c2_state):
    wl, p, d, dg, m_ref, m_gpu = c2_state
    tgt = wl.make_target()
    g_ref, g_abs, loss_ref, _ = ref.render_bwd(d, wl.h, wl.w, m_ref, tgt)
    grad = torch.zeros((wl.n, 12), dtype=torch.float32, device=dev())
    loss = torch.zeros(1, dtype=torch.float32, device=dev())
    sad.render_bwd(dg, wl.h, wl.w, m_gpu, to_gpu(tgt), grad, loss, None)
    assert abs(loss.item() - loss_ref) <= 1e-5 * loss_ref
    assert_grad_close(to_np(grad), g_ref, "C2 gradients")


# ---------------------------------------------------------------- budget statistics

def stats_vs_oracle(sad, ref, d, dg, h, w, m_np, tgt, label, stats=None, times=1):
    st_ref, mag = ref.site_stats(d, h, w, m_np, tgt)
    st = sad.site_stats(dg, h, w, to_gpu(m_np), to_gpu(tgt), stats)
    assert_stats_close(to_np(st), times * st_ref, times * mag, m_np, (h, w), label, calls=times)
    return st


def test_site_stats_c1(sad, ref):
    """64x64 / 256 sites: the exact top-8 map, then a map with empty lists,
    out-of-range ids and an inactive site."""
    wl = synth.C1
    p = wl.make_sites()
    p[5, 0] = -1.0
    d = ref.prepare_sites(p)
    dg = sad.prepare_sites(to_gpu(p))
    tgt = wl.make_target()
    m = ref.brute_topk(d, wl.h, wl.w)
    stats_vs_oracle(sad, ref, d, dg, wl.h, wl.w, m, tgt, "C1 exact map")
    rng = np.random.default_rng(3)
    m2 = m.copy()
    m2[rng.random(m2.shape[:2]) < 0.05] = 0xFFFFFFFF
    m2[..., 7][rng.random(m2.shape[:2]) < 0.2] = 5
    m2[..., 6][rng.random(m2.shape[:2]) < 0.1] = 999
    stats_vs_oracle(sad, ref, d, dg, wl.h, wl.w, m2, tgt, "C1 map with gaps")


def test_site_stats_c2_accumulates(sad, ref, c2_state):
    """The 768x512 / 50k-site map after warm-up and one step; a second call
    adds the same sums again."""
    wl, p, d, dg, m_ref, m_gpu = c2_state
    tgt = wl.make_target()
    st = stats_vs_oracle(sad, ref, d, dg, wl.h, wl.w, m_ref, tgt, "C2 statistics")
    stats_vs_oracle(sad, ref, d, dg, wl.h, wl.w, m_ref, tgt, "C2 statistics, second call", stats=st, times=2)


@pytest.mark.parametrize("h,w,n", [(13, 29, 300), (1, 37, 20), (45, 58, 1), (70, 9, 2000)])
def test_site_stats_ragged(sad, ref, h, w, n):
    p = synth.sites(40 + n, n, h, w)
    d = ref.prepare_sites(p)
    m = ref.propagate_schedule(d, h, w, None, synth.jfa_strides(h, w, 12), 8, 0, 64)
    tgt = np.random.default_rng(n).random((h, w, 3)).astype(np.float32)
    stats_vs_oracle(sad, ref, d, sad.prepare_sites(to_gpu(p)), h, w, m, tgt, f"{h}x{w}, n={n}")


# ---------------------------------------------------------------- budget control

def budget_case(ref, seed, n, h, w, stats=None, d=None, p=None):
    rng = np.random.default_rng(seed)
    if p is None:
        p = synth.sites(seed, n, h, w)
        p[rng.random(n) < 0.15, 0] = -1.0
    m = rng.normal(size=p.shape).astype(np.float32)
    v = rng.random(p.shape).astype(np.float32)
    t = rng.random((h, w, 3)).astype(np.float32)
    d = ref.prepare_sites(p) if d is None else d
    if stats is None:
        stats = np.zeros((n, 8), np.float32)
        stats[:, 0] = rng.random(n) * 10
        stats[:, 1] = rng.random(n) * 2
        stats[:, 2] = rng.normal(size=n)
        stats[:, 3:5] = rng.normal(size=(n, 2))
        stats[:, 5] = stats[:, 7] = rng.random(n) * 20 + 5
        stats[:, 6] = rng.normal(size=n)
        stats[rng.random(n) < 0.05, 5:8] = 0.0  # degenerate covariance: the target's gradient decides
    return p, m, v, d, stats, t


def budget_vs_oracle(sad, ref, p, m, v, d, stats, t, h, w, label, **kw):
    want = ref.densify_prune(p, m, v, d, h, w, stats, t, kw["n_split"], kw["n_prune"], kw["alpha"], kw["min_mass"],
                             kw["offset"], kw["r_scale"], kw["logtau_shift"])
    gp, gm, gv, gd = (to_gpu(x) for x in (p, m, v, d))
    done = sad.densify_prune(gp, gm, gv, gd, h, w, to_gpu(stats), to_gpu(t), **kw)
    for got, exp, name in zip((gp, gm, gv, gd), want[:4], ("params", "m", "v", "derived")):
        got = to_np(got)
        assert np.array_equal(got.view(np.uint32), exp.view(np.uint32)), \
            f"{label}: {name} differs at sites {np.unique(np.argwhere(got != exp)[:, 0])[:8]}"
    assert tuple(to_np(done)) == want[4], label


@pytest.mark.parametrize("alpha", [0.0, 1.0, 0.7])
def test_densify_prune_bit_exact(sad, ref, alpha):
    h, w, n = 40, 52, 600
    p, m, v, d, st, t = budget_case(ref, 31, n, h, w)
    kw = dict(n_split=40, n_prune=25, alpha=alpha, min_mass=1.0, offset=0.5, r_scale=0.85, logtau_shift=0.1)
    budget_vs_oracle(sad, ref, p, m, v, d, st, t, h, w, f"alpha {alpha}", **kw)


def test_densify_prune_400k(sad, ref):
    """400k sites on a 2048x2048 target: the sorts take their large-input path."""
    h = w = 2048
    p, m, v, d, st, t = budget_case(ref, 37, 400_000, h, w)
    kw = dict(n_split=9000, n_prune=7000, alpha=0.5, min_mass=1.0, offset=0.5, r_scale=0.85, logtau_shift=0.1)
    budget_vs_oracle(sad, ref, p, m, v, d, st, t, h, w, "400k sites", **kw)


def test_densify_prune_limits(sad, ref):
    h, w, n = 17, 23, 80
    p, m, v, d, st, t = budget_case(ref, 33, n, h, w)
    # more splits than free slots, more prunes than active sites
    for ns, npr in ((70, 0), (5, 200), (0, 0), (200, 10)):
        kw = dict(n_split=ns, n_prune=npr, alpha=1.0, min_mass=0.5, offset=0.7, r_scale=0.9, logtau_shift=0.05)
        budget_vs_oracle(sad, ref, p, m, v, d, st, t, h, w, f"split {ns} prune {npr}", **kw)


def test_densify_prune_on_real_statistics(sad, ref, c2_state):
    """The 768x512 / 50k-site map: statistics from the GPU, then the same
    float32 statistics into both sides."""
    wl, p, d, dg, m_ref, m_gpu = c2_state
    tgt = wl.make_target()
    stats = to_np(sad.site_stats(dg, wl.h, wl.w, m_gpu, to_gpu(tgt)))
    p2 = p.copy()
    p2[::50, 0] = -1.0  # free slots
    d2 = ref.prepare_sites(p2)
    _, m, v, _, _, _ = budget_case(ref, 35, wl.n, wl.h, wl.w, stats=stats, d=d2, p=p2)
    kw = dict(n_split=800, n_prune=500, alpha=1.0, min_mass=1.0, offset=0.5, r_scale=0.85, logtau_shift=0.1)
    budget_vs_oracle(sad, ref, p2, m, v, d2, stats, tgt, wl.h, wl.w, "768x512 statistics", **kw)


def test_densify_prune_without_sites(sad):
    e = torch.zeros((0, 12), dtype=torch.float32, device=dev())
    done = sad.densify_prune(e, e.clone(), e.clone(), e.clone(), 8, 8, torch.zeros((0, 8), device=dev()),
                             torch.zeros((8, 8, 3), device=dev()), n_split=3, n_prune=3)
    assert tuple(to_np(done)) == (0, 0)


def test_field_densify_prune_bookkeeping(sad, ref):
    """SadField.densify_prune: statistics from the field's own map, then the
    budget step; the active count moves by split - pruned, the prepared
    records follow the sites, and the field keeps training."""
    from voronoi_rendering_amd.pipeline import SadField

    wl = synth.C1
    p = wl.make_sites()
    p[np.random.default_rng(2).random(wl.n) < 0.2, 0] = -1.0
    f = SadField(to_gpu(p), wl.h, wl.w, wl.inject_seed, inject=wl.inject)
    f.warm(16)
    tgt = to_gpu(wl.make_target())
    before = int((f.params[:, 0] >= 0).sum())
    done = to_np(f.densify_prune(tgt, n_split=30, n_prune=12, min_mass=0.5))
    after = to_np(f.params)
    assert done[0] == 12 and 0 < done[1] <= 30
    assert int((after[:, 0] >= 0).sum()) == before - done[0] + done[1]
    assert np.array_equal(to_np(f.derived).view(np.uint32), ref.prepare_sites(after).view(np.uint32))
    prev, first = map_to_np(f.topk), f.pass_index
    f.propagate([4, 2, 1])
    want = ref.propagate_schedule(ref.prepare_sites(after), wl.h, wl.w, prev, [4, 2, 1], wl.inject_seed, first,
                                  wl.inject)
    assert np.array_equal(map_to_np(f.topk), want)


def test_fit_with_budget_schedule(sad, ref):
    """A fit from a gradient-weighted draw with scheduled budget steps: the
    site count follows the schedule, prepared records follow the sites, every
    list holds distinct usable ids only, and the error drops."""
    from voronoi_rendering_amd.pipeline import BudgetSchedule, SadField

    wl = synth.C1
    tgt = to_gpu(wl.make_target())
    f = SadField.from_target(tgt, 400, lam=0.3, seed=17, log_scale=0.5)
    f.warm(16)
    err0 = float(((f.render() - tgt) ** 2).mean())
    sched = BudgetSchedule(every=5, start=5, stop=20, n_split=10, n_prune=50, min_mass=0.5)
    f.fit(tgt, 25, [4, 2, 1], sched)
    assert f.active_sites() == 400 - 4 * 50 + 4 * 10
    p = to_np(f.params)
    assert np.array_equal(to_np(f.derived).view(np.uint32), ref.prepare_sites(p).view(np.uint32))
    m = map_to_np(f.topk)
    usable = p[:, 0] >= 0
    for row in m.reshape(-1, 8):
        ids = row[row != 0xFFFFFFFF]
        assert len(set(ids.tolist())) == len(ids) and usable[ids].all()
    assert float(((f.render() - tgt) ** 2).mean()) < err0


# ---------------------------------------------------------------- initialisation

def init_vs_oracle(sad, ref, t, n, lam, seed, label, **kw):
    h, w = t.shape[:2]
    want_p, want_d = ref.init_sites(t, h, w, n, lam, seed, **kw)
    gp, gd = sad.init_sites(to_gpu(t), n, lam=lam, seed=seed, **kw)
    for got, exp, name in ((gp, want_p, "params"), (gd, want_d, "derived")):
        got = to_np(got)
        assert np.array_equal(got.view(np.uint32), exp.view(np.uint32)), \
            f"{label}: {name} differs at sites {np.unique(np.argwhere(got != exp)[:, 0])[:8]}"


@pytest.mark.parametrize("lam", [0.0, 0.25, 1.0])
def test_init_sites_bit_exact(sad, ref, lam):
    t = synth.target_polygons(5, 37, 53, n_poly=5).astype(np.float32)
    init_vs_oracle(sad, ref, t, 3000, lam, 77, f"37x53 lambda {lam}", log_tau=0.5, r=0.25, log_scale=-0.3)


def test_init_sites_768x512(sad, ref):
    wl = synth.C3
    say(f"[gpu] init {wl.w}x{wl.h}, n={wl.n}")
    init_vs_oracle(sad, ref, wl.make_target(), wl.n, 0.3, wl.param_seed, "768x512 / 50k", log_scale=0.7)


def test_init_sites_edge_cases(sad, ref):
    init_vs_oracle(sad, ref, np.full((1, 1, 3), 0.2, np.float32), 5, 0.0, 1, "1x1")
    init_vs_oracle(sad, ref, np.full((7, 11, 3), 0.4, np.float32), 500, 0.0, 2, "flat image")
    t = np.zeros((10, 12, 3), np.float32)
    t[4, 6, 0] = 2.0 ** -22
    t[7, 2, 1] = 2.0 ** -23
    init_vs_oracle(sad, ref, t, 2000, 0.0, 5, "a few gradient units")
    t = np.random.default_rng(3).random((1, 300, 3)).astype(np.float32)
    init_vs_oracle(sad, ref, t, 700, 0.5, 6, "one row")
    t[0, 5, 2] = np.nan
    t[0, 9, 0] = 1e6  # capped weight
    init_vs_oracle(sad, ref, t, 700, 0.1, 8, "NaN and huge values")


def test_init_sites_without_sites(sad):
    p, d = sad.init_sites(torch.zeros((4, 4, 3), device=dev()), 0, lam=0.5, seed=1)
    assert p.shape == (0, 12) and d.shape == (0, 12)


# ---------------------------------------------------------------- packed records

def pack_vs_oracle(sad, ref, p, h, w, label):
    d = ref.prepare_sites(p)
    want_pk, want_qp = ref.pack_sites(p, d, h, w)
    gpk, gqp = sad.pack_sites(to_gpu(p), to_gpu(d), h, w)
    got_pk = to_np(gpk).view(np.uint32)
    assert np.array_equal(to_np(gqp).view(np.uint32), want_qp.view(np.uint32)), f"{label}: ranges {to_np(gqp)} {want_qp}"
    bad = np.argwhere(got_pk != want_pk)
    assert len(bad) == 0, f"{label}: {len(bad)} words differ, first {bad[:4].tolist()}"
    return d, want_pk, want_qp, gpk, gqp


def packed_query_bound(ref, pk, qp, h, w, topk, xy):
    """Per point, what float32 decoding may change in the colour: with the
    float64 decode of each usable entry (tau, r, a, offset d, distance, logit),
    dl_k = 2^-19 (|l_k| (1 + |log tau_k|) + tau_k (dist_k + |r_k| + e^(|a_k|/2) |d_k|))
    covers the roundings of the offset, the range decode and the hardware exp,
    sine and cosine; the softmax moves the colour by at most
    2 max_k dl_k max_k |c_k - c|, plus the colour decode's rounding."""
    v, ok = ref.unpack_sites(pk, qp, h, w)
    n = len(ok)
    xy = np.nan_to_num(xy, nan=0.0, posinf=0.0, neginf=0.0)  # non-finite points are NaN on both sides
    i = np.clip(np.floor(xy[:, 0]), 0, w - 1).astype(int)
    j = np.clip(np.floor(xy[:, 1]), 0, h - 1).astype(int)
    ids = topk[j, i].astype(np.int64)  # [m][8]
    use = (ids < n) & ok[np.minimum(ids, n - 1)]
    e = v[np.minimum(ids, n - 1)]  # [m][8][9]
    dx = xy[:, 0:1].astype(np.float64) - e[..., 0]
    dy = xy[:, 1:2].astype(np.float64) - e[..., 1]
    cs, sn = np.cos(e[..., 7]), np.sin(e[..., 7])
    u, t = cs * dx + sn * dy, cs * dy - sn * dx
    dist = np.sqrt(np.exp(e[..., 8]) * u * u + np.exp(-e[..., 8]) * t * t)
    lg = -e[..., 2] * (dist - e[..., 3])
    use &= np.isfinite(lg)
    dl = 2.0 ** -19 * (np.abs(lg) * (1 + np.abs(np.log(e[..., 2]))) +
                       e[..., 2] * (dist + np.abs(e[..., 3]) + np.exp(np.abs(e[..., 8]) / 2) * np.hypot(dx, dy)))
    dl = np.where(use, dl, 0.0).max(1)
    col = e[..., 4:7]
    cmax = np.where(use[..., None], col, -np.inf).max(1)
    cmin = np.where(use[..., None], col, np.inf).min(1)
    spread = np.where(use.any(1)[:, None], cmax - cmin, 0.0)
    return 2 * dl[:, None] * spread + 2.0 ** -20 * (1 + np.abs(col).max(axis=(1, 2)))[:, None]


def query_packed_vs_oracle(sad, ref, pk, qp, gpk, gqp, h, w, topk_np, topk_gpu, xy, label):
    want = ref.query_packed(pk, qp, h, w, topk_np, xy)
    got = to_np(sad.query_packed(gpk, gqp, h, w, topk_gpu, to_gpu(xy)))
    bound = packed_query_bound(ref, pk, qp, h, w, topk_np, xy)
    fin = np.isfinite(want)
    assert np.array_equal(fin, np.isfinite(got)), label
    err = np.abs(got - want)[fin]
    ratio = (np.abs(got - want) / bound)[fin]
    say(f"[gpu] {label}: max |err| {err.max():.3g}, median {np.median(err):.3g}, max err/bound {ratio.max():.3g}")
    assert (ratio <= 1.0).all(), f"{label}: {int((ratio > 1).sum())} values beyond the bound, worst {ratio.max():.3g}"
    assert err.max() <= 1e-5, label  # and the query path's bar


def test_pack_sites_bit_exact(sad, ref):
    wl = synth.C1
    p = wl.make_sites()
    p[::7, 0] = -1.0
    pack_vs_oracle(sad, ref, p, wl.h, wl.w, "64x64 / 256")
    p = synth.sites(3, 5000, 37, 53, synth.WIDE_SCALES)
    p[:, 7] = np.random.default_rng(4).uniform(-50, 50, 5000).astype(np.float32)  # wrapped angles
    p[10, 4] = -0.0
    p[11, 2] = np.nan  # ignored by the ranges, coded 0
    pack_vs_oracle(sad, ref, p, 37, 53, "37x53 / 5000, wide angles, NaN")
    p = synth.sites(5, 40, 9, 9)
    p[:, 0] = -1.0
    pack_vs_oracle(sad, ref, p, 9, 9, "no usable site")
    pack_vs_oracle(sad, ref, np.zeros((0, 12), np.float32), 9, 9, "no sites")


def test_query_packed_c1(sad, ref):
    wl = synth.C1
    p = wl.make_sites()
    p[3, 0] = -1.0
    d, pk, qp, gpk, gqp = pack_vs_oracle(sad, ref, p, wl.h, wl.w, "C1")
    m = ref.brute_topk(d, wl.h, wl.w)
    xy = synth.queries(21, 20000, wl.h, wl.w)
    xy[:5] = [[np.nan, 1.0], [-3.0, 2.0], [70.0, 70.0], [0.0, 0.0], [64.0, 64.0]]
    query_packed_vs_oracle(sad, ref, pk, qp, gpk, gqp, wl.h, wl.w, m, to_gpu(m), xy, "C1 queries")


def test_query_packed_c5_sampled(sad, ref):
    """The 768x512 / 50k-site map and 2^24 points in one call; sampled points
    against the oracle."""
    wl = synth.C5
    p = wl.make_sites()
    d, pk, qp, gpk, gqp = pack_vs_oracle(sad, ref, p, wl.h, wl.w, "C5 records")
    dg = sad.prepare_sites(to_gpu(p))
    m_gpu = gpu_schedule(sad, dg, wl.h, wl.w, synth.jfa_strides(wl.h, wl.w, wl.warm_passes), wl.inject_seed,
                         wl.inject)
    xy = wl.make_queries()
    rgb = to_np(sad.query_packed(gpk, gqp, wl.h, wl.w, m_gpu, to_gpu(xy)))
    pick = np.random.default_rng(8).choice(len(xy), 20000, replace=False)
    mnp = map_to_np(m_gpu)
    want = ref.query_packed(pk, qp, wl.h, wl.w, mnp, xy[pick])
    bound = packed_query_bound(ref, pk, qp, wl.h, wl.w, mnp, xy[pick])
    ratio = np.abs(rgb[pick] - want) / bound
    say(f"[gpu] C5 packed: max |err| {np.abs(rgb[pick] - want).max():.3g}, max err/bound {ratio.max():.3g}")
    assert (ratio <= 1.0).all() and np.abs(rgb[pick] - want).max() <= 1e-5


def test_queries_past_one_launch(sad, ref):
    """2^30 + 777 points (more than one launch's chunk) from both query paths
    on a 64x64 map: sampled points, those around the chunk boundary and the
    last ones against the oracle."""
    wl = synth.C1
    p = wl.make_sites()
    d = ref.prepare_sites(p)
    m_np = ref.brute_topk(d, wl.h, wl.w)
    dg, mg = to_gpu(d), to_gpu(m_np)
    pk, qp = ref.pack_sites(p, d, wl.h, wl.w)
    gpk, gqp = to_gpu(pk), to_gpu(qp)
    m = (1 << 30) + 777
    say(f"[gpu] {m} points on the GPU")
    g = torch.Generator(device=dev())
    g.manual_seed(12)
    xy = torch.rand((m, 2), generator=g, device=dev())
    xy *= torch.tensor([wl.w, wl.h], dtype=torch.float32, device=dev())
    rgb = torch.empty((m, 3), dtype=torch.float32, device=dev())
    pick = np.concatenate([np.random.default_rng(3).integers(0, m, 3000), np.arange((1 << 30) - 50, m)])
    pt = to_np(xy[torch.from_numpy(pick).to(dev())])
    sad.query_points(dg, wl.h, wl.w, mg, xy, rgb)
    got = to_np(rgb[torch.from_numpy(pick).to(dev())])
    assert np.abs(got - ref.query_points(d, wl.h, wl.w, m_np, pt)).max() <= 1e-5
    rgb.fill_(-1.0)
    sad.query_packed(gpk, gqp, wl.h, wl.w, mg, xy, rgb)
    got = to_np(rgb[torch.from_numpy(pick).to(dev())])
    want = ref.query_packed(pk, qp, wl.h, wl.w, m_np, pt)
    assert (np.abs(got - want) <= packed_query_bound(ref, pk, qp, wl.h, wl.w, m_np, pt)).all()
    del xy, rgb


# ---------------------------------------------------------------- JFA prepass and full refresh

def crowded_sites(seed, n, h, w):
    """Sites with pixels shared by several sites, inactive ones and one on the far corner."""
    p = synth.sites(seed, n, h, w)
    rng = np.random.default_rng(seed)
    p[rng.random(n) < 0.1, 0] = -1.0
    k = n // 4
    p[:k, 0] = rng.integers(0, 4, k) + rng.random(k) * 0.999
    p[:k, 1] = rng.integers(0, 3, k) + rng.random(k) * 0.999
    p[k, 0], p[k, 1] = float(w), float(h)
    return p


@pytest.mark.parametrize("h,w,n", [(37, 53, 400), (1, 1, 7), (64, 64, 256), (9, 70, 3000)])
def test_jfa_seed_and_flood(sad, ref, h, w, n):
    p = crowded_sites(20 + n, n, h, w)
    d = ref.prepare_sites(p)
    dg = sad.prepare_sites(to_gpu(p))
    want = ref.jfa_seed(d, h, w)
    got = sad.jfa_seed(dg, h, w)
    assert np.array_equal(map_to_np(got), want), "seed"
    rng = np.random.default_rng(n)
    prev = rng.integers(0, n + 9, (h, w, 4)).astype(np.uint32)  # stale ids past n, repeats inside lists
    prev[rng.random((h, w, 4)) < 0.3] = 0xFFFFFFFF
    prev[..., 1] = np.where(rng.random((h, w)) < 0.1, prev[..., 0], prev[..., 1])
    for step, width in ((1, 4), (3, 8), (16, 4), (64, 8)):
        want = ref.jfa_flood(d, h, w, prev, step, width)
        got = sad.jfa_flood(dg, h, w, to_gpu(prev), step, width)
        assert np.array_equal(map_to_np(got), want), f"flood step {step} width {width}"


@pytest.mark.parametrize("h,w,n", [(64, 64, 256), (512, 512, 25_000), (45, 131, 900), (1, 1, 3),
                                   (2048, 2048, 400_000)])
def test_full_refresh_and_render(sad, ref, h, w, n):
    """One JFA round, 16 propagation passes and the render, from the sites alone."""
    from voronoi_rendering_amd.pipeline import SadField

    p = synth.sites(70 + n, n, h, w, synth.WIDE_SCALES)
    d = ref.prepare_sites(p)
    say(f"[gpu] full refresh {w}x{h}, n={n}")
    want = ref.full_refresh(d, h, w, 11)
    f = SadField(to_gpu(p), h, w, 11)
    f.refresh(16)
    got = map_to_np(f.topk)
    assert np.array_equal(got, want), f"{(got != want).any(-1).sum()} pixels differ"
    assert_colour_close(to_np(f.render()), ref.render_fwd(d, h, w, want), f"refresh render {w}x{h}")


# Top-8 exact match after a full refresh with 8, 12 and 16 passes (Table 7 of
# the pages: 256 random pixels, 4 trials; their values on another GPU).
PAGES_TABLE7 = {(1024, 16384): (0.963, 0.970, 0.970), (1024, 65536): (0.398, 0.867, 0.867),
                (1024, 131072): (0.072, 0.782, 0.782), (2048, 16384): (0.981, 0.987, 0.987),
                (2048, 65536): (0.393, 0.956, 0.956), (2048, 131072): (0.059, 0.907, 0.907)}


@pytest.mark.parametrize("side,n", list(PAGES_TABLE7))
def test_refresh_exact_match_fraction(sad, ref, side, n):
    """The refresh's lists against brute force over every site on 256 random
    pixels per trial (set equality of the top 8), 4 trials."""
    from voronoi_rendering_amd.pipeline import SadField

    frac = {8: [], 12: [], 16: []}
    for trial in range(4):
        p = synth.sites_unique_cells(900 + trial, n, side, side)
        d = ref.prepare_sites(p)
        pix = np.random.default_rng(50 + trial).integers(0, side * side, 256)
        exact = np.sort(ref.brute_topk_pixels(d, side, side, pix), axis=1)
        f = SadField(to_gpu(p), side, side, 60 + trial)
        for n_pass in frac:
            f.refresh(n_pass)
            got = np.sort(to_np(f.topk.view(-1, 8)[torch.from_numpy(pix).to(dev())]).view(np.uint32), axis=1)
            frac[n_pass].append(float((got == exact).all(1).mean()))
    mean = {k: float(np.mean(v)) for k, v in frac.items()}
    say(f"[gpu] exact match {side}^2, {n} sites: 8/12/16 passes {mean[8]:.3f} / {mean[12]:.3f} / "
        f"{mean[16]:.3f} (pages {PAGES_TABLE7[(side, n)]})")
    assert mean[16] >= mean[8] - 0.02
    assert mean[16] >= 0.7  # measured 0.73 to 0.98


# ---------------------------------------------------------------- fused pass + backward

def fused_vs_oracle(sad, ref, d, dg, h, w, prev_np, prev_gpu, stride, seed, t, inject, tgt, prev_scores=None,
                    label=""):
    """One fused call against the oracle's pass then backward, and against
    the two separate GPU calls."""
    m1 = ref.propagate(d, h, w, prev_np, stride, seed, t, inject)
    g_ref, g_abs, loss_ref, img_ref = ref.render_bwd(d, h, w, m1, tgt)
    n = d.shape[0]
    outs = []
    for fused in (True, False):
        out = torch.empty((h, w, 8), dtype=torch.int32, device=dev())
        osc = torch.empty((h, w, 8), dtype=torch.float32, device=dev())
        grad = torch.zeros((n, 12), dtype=torch.float32, device=dev())
        loss = torch.zeros(1, dtype=torch.float32, device=dev())
        img = torch.empty((h, w, 3), dtype=torch.float32, device=dev())
        if fused:
            sad.step_fused(dg, h, w, prev_gpu, out, to_gpu(tgt), grad, stride=stride, seed=seed, pass_index=t,
                           inject=inject, prev_scores=prev_scores, out_scores=osc, loss=loss, image=img)
        else:
            sad.propagate_topk(dg, h, w, prev_gpu, out, stride=stride, seed=seed, pass_index=t, inject=inject,
                               prev_scores=prev_scores, out_scores=osc)
            sad.render_bwd(dg, h, w, out, to_gpu(tgt), grad, loss, img)
        outs.append((map_to_np(out), to_np(osc), to_np(grad), loss.item(), to_np(img)))
    (lf, sf, gf, lossf, imf), (lc, sc_, gc, lossc, imc) = outs
    assert np.array_equal(lf, m1), f"{label}: {(lf != m1).any(-1).sum()} pixels differ from the oracle"
    assert np.array_equal(lf, lc)
    assert np.array_equal(sf.view(np.uint32), sc_.view(np.uint32)), f"{label}: score maps differ"
    assert np.array_equal(imf.view(np.uint32), imc.view(np.uint32)), f"{label}: images differ"
    assert_colour_close(imf, img_ref, f"{label} image")
    assert abs(lossf - loss_ref) <= 1e-5 * loss_ref
    assert_grad_close(gf, g_ref, f"{label} gradients")
    assert np.all(gf[:, 10:] == 0)
    return lf, sf


def test_step_fused_c2(sad, ref, c2_state):
    """The fused last pass + backward on the 768x512 map: first without a
    score map (as after an Adam step), then chained through the score map it
    wrote."""
    wl, p, d, dg, m_ref, m_gpu = c2_state
    tgt = wl.make_target()
    lst, sc = fused_vs_oracle(sad, ref, d, dg, wl.h, wl.w, m_ref, m_gpu, 1, wl.inject_seed, 700, wl.inject, tgt,
                              label="C2 fused")
    fused_vs_oracle(sad, ref, d, dg, wl.h, wl.w, lst, to_gpu(lst), 2, wl.inject_seed, 701, wl.inject, tgt,
                    prev_scores=to_gpu(sc), label="C2 fused, score map")


@pytest.mark.parametrize("h,w,n,stride,inject", [(37, 53, 200, 2, 64), (16, 32, 40, 1, 7), (9, 70, 64, 8, 64)])
def test_step_fused_ragged(sad, ref, h, w, n, stride, inject):
    """Images that end inside a tile and inside a backward region, an inactive
    site and a stale list entry; also the first pass from an empty map."""
    p = synth.sites(31 + h, n, h, w, synth.SMALL_SCALES)
    p[3, 0] = -1.0
    d = ref.prepare_sites(p)
    dg = sad.prepare_sites(to_gpu(p))
    rng = np.random.default_rng(h * w)
    tgt = rng.random((h, w, 3)).astype(np.float32)
    fused_vs_oracle(sad, ref, d, dg, h, w, None, None, stride, 5, 0, inject, tgt, label=f"{h}x{w} from empty")
    m = ref.propagate_schedule(d, h, w, None, synth.jfa_strides(h, w, 6), 5, 1, inject)
    m[0, 0, 7] = 3  # the inactive site, left in a list
    fused_vs_oracle(sad, ref, d, dg, h, w, m, to_gpu(m), stride, 5, 9, inject, tgt, label=f"{h}x{w}")


def test_step_fused_without_sites(sad, ref):
    """No sites: the pass leaves every list empty, the image is 0 and the
    loss is the target's mean square, as the oracle gives."""
    h, w = 9, 13
    p = np.zeros((0, 12), dtype=np.float32)
    d = ref.prepare_sites(p)
    tgt = np.random.default_rng(1).random((h, w, 3)).astype(np.float32)
    m_ref = ref.propagate(d, h, w, None, 1, 5, 0, 64)
    _, _, loss_ref, img_ref = ref.render_bwd(d, h, w, m_ref, tgt)
    dg = torch.zeros((0, 12), dtype=torch.float32, device=dev())
    out = torch.empty((h, w, 8), dtype=torch.int32, device=dev())
    grad = torch.zeros((0, 12), dtype=torch.float32, device=dev())
    loss = torch.zeros(1, dtype=torch.float32, device=dev())
    img = torch.full((h, w, 3), 7.0, dtype=torch.float32, device=dev())
    sad.step_fused(dg, h, w, None, out, to_gpu(tgt), grad, stride=1, seed=5, pass_index=0, inject=64, loss=loss,
                   image=img)
    assert np.array_equal(map_to_np(out), m_ref)
    assert np.array_equal(to_np(img), img_ref)
    assert abs(loss.item() - loss_ref) <= 1e-5 * loss_ref


def test_pipeline_step_fused_equals_separate_calls(sad, ref):
    """SadField.step with the fused call and with separate calls give the same
    lists and gradients within the tolerance, over three steps of the 64x64
    workload from an empty map (the fused step keeps no logits of its last
    pass, so the next step recomputes them; the lists do not change)."""
    from voronoi_rendering_amd.pipeline import SadField

    wl = synth.C1
    p = to_gpu(wl.make_sites())
    tgt = to_gpu(wl.make_target())
    fields = [SadField(p.clone(), wl.h, wl.w, wl.inject_seed, inject=wl.inject) for _ in range(2)]
    for _ in range(3):
        for f, fused in zip(fields, (True, False)):
            f.step([4, 2, 1], tgt, fused=fused)
    a, b = fields
    assert torch.equal(a.topk, b.topk)
    assert not a.scores_valid and b.scores_valid
    # the same kernels either way; terms that go to float atomics (very large
    # ones) may be summed in another order
    ga, gb = to_np(a.grad).astype(np.float64), to_np(b.grad).astype(np.float64)
    assert np.all(np.abs(ga - gb) <= 1e-5 * np.abs(gb) + 1e-6 * np.abs(gb).max(axis=0))


def map16_to_np(t: torch.Tensor) -> np.ndarray:
    """A 16-bit-id map read back as 32-bit ids (0xffff -> 0xffffffff)."""
    m = t.cpu().numpy().view(np.uint16).astype(np.uint32)
    m[m == 0xFFFF] = 0xFFFFFFFF
    return m


def map16_from_np(m: np.ndarray) -> torch.Tensor:
    """32-bit ids (all below 0xffff or 0xffffffff) as a 16-bit-id map on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(m.astype(np.uint16)).view(np.int16)).to(dev())


def field_lists(f) -> np.ndarray:
    """A field's current lists as 32-bit ids, read without changing its state:
    from the 16-bit map a step's last pass left (which the next step's first
    pass then reads, as in training) or from the 32-bit map."""
    return map16_to_np(f.map16) if f.cur16 else map_to_np(f.maps[f.cur])


@pytest.mark.parametrize("h,w,n", [(64, 64, 256), (13, 29, 300), (67, 72, 1000), (37, 70, 65535)])
def test_propagate_16bit_maps(sad, ref, h, w, n):
    """Passes that read and write 16-bit-id maps (every combination of the two
    widths, with and without score maps) give the oracle's lists, id for id,
    and the same score maps as the 32-bit passes; from an empty map, through
    the warm-up schedule and a step's strides, up to the 16-bit limit of
    65,535 sites (the last id 65,534 next to the empty slot 0xffff)."""
    p = synth.sites(300 + n, n, h, w)
    if n >= 10:
        p[3, 0] = -1.0  # an inactive site
    d = ref.prepare_sites(p)
    dg = sad.prepare_sites(to_gpu(p))
    strides = list(synth.jfa_strides(h, w, 6)) + [8, 4, 2, 1, 1]
    m = None
    prev32 = prev16 = None
    sc_prev = None
    for t, s_ in enumerate(strides):
        want = ref.propagate(d, h, w, m, s_, 17, t, 64)
        out16 = torch.empty((h, w, 8), dtype=torch.int16, device=dev())
        out32 = torch.empty((h, w, 8), dtype=torch.int32, device=dev())
        sc16 = torch.empty((h, w, 8), dtype=torch.float32, device=dev())
        sc32 = torch.empty((h, w, 8), dtype=torch.float32, device=dev())
        # 16 -> 16 (or empty -> 16) with score maps; 16 -> 32 without; 32 -> 16 with the 32-bit scores
        sad.propagate_topk(dg, h, w, prev16, out16, stride=s_, seed=17, pass_index=t, inject=64,
                           prev_scores=sc_prev, out_scores=sc16)
        sad.propagate_topk(dg, h, w, prev16, out32, stride=s_, seed=17, pass_index=t, inject=64)
        got16, got32 = map16_to_np(out16), map_to_np(out32)
        assert np.array_equal(got16, want), f"pass {t} 16->16: {np.argwhere(got16 != want)[:4]}"
        assert np.array_equal(got32, want), f"pass {t} 16->32"
        if prev32 is not None:
            o = torch.empty((h, w, 8), dtype=torch.int16, device=dev())
            sad.propagate_topk(dg, h, w, prev32, o, stride=s_, seed=17, pass_index=t, inject=64,
                               out_scores=sc32)
            assert np.array_equal(map16_to_np(o), want), f"pass {t} 32->16"
            assert np.array_equal(to_np(sc32).view(np.uint32), to_np(sc16).view(np.uint32)), f"pass {t} scores"
        m, prev16, prev32, sc_prev = want, out16, out32, sc16


def eighth_logits(ref, d, m):
    """The oracle's logit of each list's 8th entry (-inf where it is empty)."""
    h, w = m.shape[:2]
    out = np.full((h, w), -np.inf, dtype=np.float32)
    for j in range(h):
        for i in range(w):
            if m[j, i, 7] != 0xFFFFFFFF:
                out[j, i] = ref.score(d, int(m[j, i, 7]), i + 0.5, j + 0.5)
    return out


@pytest.mark.parametrize("h,w,n,bits", [(64, 64, 256, 16), (29, 45, 400, 32), (40, 40, 3000, 16)])
def test_propagate_thresholds(sad, ref, h, w, n, bits):
    """Passes that hand on only each list's 8th logit: from an empty map
    through the warm-up schedule (lists fill up, so most lanes insert and
    evaluate their other logits) and a step's strides, every pass gives the
    oracle's lists and 8th logits bit for bit, and asked for all logits it
    writes the score map the full pass writes."""
    p = synth.sites(500 + n, n, h, w)
    p[5, 0] = -1.0  # an inactive site
    d = ref.prepare_sites(p)
    dg = sad.prepare_sites(to_gpu(p))
    dt = torch.int16 if bits == 16 else torch.int32
    strides = list(synth.jfa_strides(h, w, 5)) + [8, 4, 2, 1, 3, 1]
    m, prev, thr = None, None, None
    for t, s_ in enumerate(strides):
        want = ref.propagate(d, h, w, m, s_, 23, t, 64)
        out = torch.empty((h, w, 8), dtype=dt, device=dev())
        out_thr = torch.empty((h, w), dtype=torch.float32, device=dev())
        sad.propagate_topk(dg, h, w, prev, out, stride=s_, seed=23, pass_index=t, inject=64, prev_thr=thr,
                           out_thr=out_thr)
        got = map16_to_np(out) if bits == 16 else map_to_np(out)
        assert np.array_equal(got, want), f"pass {t}: {np.argwhere(got != want)[:4]}"
        assert np.array_equal(to_np(out_thr).view(np.uint32), eighth_logits(ref, d, want).view(np.uint32)), t
        if thr is not None:
            # all logits asked for: the lanes that did not insert evaluate theirs too
            full = torch.empty((h, w, 8), dtype=dt, device=dev())
            sc = torch.empty((h, w, 8), dtype=torch.float32, device=dev())
            sad.propagate_topk(dg, h, w, prev, full, stride=s_, seed=23, pass_index=t, inject=64, prev_thr=thr,
                               out_scores=sc)
            ref_sc = torch.empty((h, w, 8), dtype=torch.float32, device=dev())
            sad.propagate_topk(dg, h, w, to_gpu(m), torch.empty((h, w, 8), dtype=torch.int32, device=dev()),
                               stride=s_, seed=23, pass_index=t, inject=64, out_scores=ref_sc)
            assert np.array_equal(to_np(sc).view(np.uint32), to_np(ref_sc).view(np.uint32)), f"pass {t} scores"
        m, prev, thr = want, out, out_thr


def test_step_fused_from_thresholds(sad, ref):
    """The fused last pass + backward from a 16-bit map with only its 8th
    logits, on lists still filling (64x64 workload after 6 passes from empty,
    most lanes insert) and on the settled 768x512-like density at 96x128: the
    oracle's lists, loss and gradients (the backward takes the logits from
    the site records it stages)."""
    for (h, w, n, npass) in ((64, 64, 256, 6), (96, 128, 1500, 14)):
        p = synth.sites(700 + n, n, h, w, synth.WIDE_SCALES)
        d = ref.prepare_sites(p)
        dg = sad.prepare_sites(to_gpu(p))
        strides = synth.jfa_strides(h, w, npass)
        m = ref.propagate_schedule(d, h, w, None, strides, 41, 0, 64)
        thr = torch.from_numpy(eighth_logits(ref, d, m)).to(dev())
        m1 = ref.propagate(d, h, w, m, 1, 41, npass, 64)
        tgt = synth.target_noise_edges(710 + n, h, w)
        g_ref, _, loss_ref, img_ref = ref.render_bwd(d, h, w, m1, tgt)
        out = torch.empty((h, w, 8), dtype=torch.int32, device=dev())
        grad = torch.zeros((n, 12), dtype=torch.float32, device=dev())
        loss = torch.zeros(1, dtype=torch.float32, device=dev())
        img = torch.empty((h, w, 3), dtype=torch.float32, device=dev())
        sad.step_fused(dg, h, w, map16_from_np(m), out, to_gpu(tgt), grad, stride=1, seed=41, pass_index=npass,
                       inject=64, loss=loss, image=img, prev_thr=thr)
        assert np.array_equal(map_to_np(out), m1), f"{h}x{w}: lists"
        assert_colour_close(to_np(img), img_ref, f"{h}x{w} image")
        assert abs(loss.item() - loss_ref) <= 1e-5 * loss_ref
        assert_grad_close(to_np(grad), g_ref, f"{h}x{w} gradients from thresholds")


def probe_records_np(d: np.ndarray) -> np.ndarray:
    """The probe records the pass writes, restated from the prepared records
    (x, y, tau, r, cos, sin, 1/s1, 1/s2, ...): (x, y, tau m, tau r) in
    float32 with m the smaller inverse scale, or (x, y, 0, inf) where the
    bound is not kept (non-finite values, tau <= 0, m <= 0, scales more than
    1024 apart)."""
    x, y, tau, r = d[:, 0], d[:, 1], d[:, 2], d[:, 3]
    m, M = np.minimum(d[:, 6], d[:, 7]), np.maximum(d[:, 6], d[:, 7])
    with np.errstate(all="ignore"):
        ok = (np.isfinite(x) & np.isfinite(y) & np.isfinite(tau) & np.isfinite(r) & np.isfinite(M) & (tau > 0)
              & (m > 0) & (M <= np.float32(1024) * m))
        out = np.stack([x, y, np.where(ok, tau * m, np.float32(0)), np.where(ok, tau * r, np.float32(np.inf))], 1)
    return out.astype(np.float32)


@pytest.mark.parametrize("n,bits", [(300, 16), (3000, 32), (3000, 16)])
def test_propagate_probe_records(sad, ref, n, bits):
    """Passes that cull their probes from the sites' 16-byte probe records:
    the first pass writes them (checked against their definition), and from
    there every pass of a chain through strides 8 ... 1 and back gives the
    oracle's lists bit for bit, on sites far outside the workloads' ranges
    (anisotropy up to e^14, where records carry no bound, a tenth of the sites
    far away, inactive sites); with 16-bit maps and thresholds as a step hands
    them on, or 32-bit maps."""
    h, w = 60, 90
    rec = synth.SiteRecipe(ls_lo=-6.0, ls_hi=8.0, r_lo=-5.0, r_hi=20.0, logtau_lo=-6.0, logtau_hi=6.0)
    p = synth.sites(5151 + n, n, h, w, rec)
    rng = np.random.default_rng(n + bits)
    far = rng.random(n) < 0.1
    p[far, 0] *= np.float32(1000.0)
    p[far, 1] *= np.float32(1000.0)
    p[rng.random(n) < 0.05, 0] = -1.0  # inactive
    d = ref.prepare_sites(p)
    dg = sad.prepare_sites(to_gpu(p))
    m = ref.propagate_schedule(d, h, w, None, synth.jfa_strides(h, w, 12), 37, 0, 64)
    probe = torch.empty((n, 4), dtype=torch.float32, device=dev())
    dt = torch.int16 if bits == 16 else torch.int32
    prev = map16_from_np(m) if bits == 16 else to_gpu(m)
    thr = None
    for t, stride in enumerate((8, 4, 2, 1, 1, 3, 2, 1)):
        want = ref.propagate(d, h, w, m, stride, 37, 12 + t, 64)
        out = torch.empty((h, w, 8), dtype=dt, device=dev())
        out_thr = torch.empty((h, w), dtype=torch.float32, device=dev()) if bits == 16 else None
        sad.propagate_topk(dg, h, w, prev, out, stride=stride, seed=37, pass_index=12 + t, inject=64,
                           prev_thr=thr, out_thr=out_thr, prev_probe=probe if t > 0 else None,
                           out_probe=probe if t == 0 else None)
        if t == 0:
            got_rec, want_rec = to_np(probe), probe_records_np(to_np(dg))
            assert np.array_equal(got_rec.view(np.uint32), want_rec.view(np.uint32)), \
                np.argwhere(got_rec.view(np.uint32) != want_rec.view(np.uint32))[:4]
            assert (got_rec[:, 3] == np.inf).any() and (got_rec[:, 3] < np.inf).any()
        got = map16_to_np(out) if bits == 16 else map_to_np(out)
        assert np.array_equal(got, want), f"pass {t} stride {stride}: {np.argwhere(got != want)[:4]}"
        m, prev, thr = want, out, out_thr


def test_step_fused_from_probe_records(sad, ref):
    """The fused last pass + backward culling its probes from the probe
    records a pass wrote, from a 16-bit map with thresholds and from a 32-bit
    map: the oracle's lists, loss and gradients."""
    h, w, n, npass = 96, 128, 1500, 14
    p = synth.sites(900 + n, n, h, w, synth.WIDE_SCALES)
    d = ref.prepare_sites(p)
    dg = sad.prepare_sites(to_gpu(p))
    m = ref.propagate_schedule(d, h, w, None, synth.jfa_strides(h, w, npass), 43, 0, 64)
    probe = torch.empty((n, 4), dtype=torch.float32, device=dev())
    scratch = torch.empty((h, w, 8), dtype=torch.int32, device=dev())
    sad.propagate_topk(dg, h, w, to_gpu(m), scratch, stride=2, seed=43, pass_index=99, inject=64, out_probe=probe)
    m1 = ref.propagate(d, h, w, m, 1, 43, npass, 64)
    tgt = synth.target_noise_edges(910 + n, h, w)
    g_ref, _, loss_ref, img_ref = ref.render_bwd(d, h, w, m1, tgt)
    thr = torch.from_numpy(eighth_logits(ref, d, m)).to(dev())
    for prev, prev_thr in ((map16_from_np(m), thr), (to_gpu(m), None)):
        out = torch.empty((h, w, 8), dtype=torch.int32, device=dev())
        grad = torch.zeros((n, 12), dtype=torch.float32, device=dev())
        loss = torch.zeros(1, dtype=torch.float32, device=dev())
        img = torch.empty((h, w, 3), dtype=torch.float32, device=dev())
        sad.step_fused(dg, h, w, prev, out, to_gpu(tgt), grad, stride=1, seed=43, pass_index=npass, inject=64,
                       loss=loss, image=img, prev_thr=prev_thr, prev_probe=probe)
        assert np.array_equal(map_to_np(out), m1), "lists"
        assert_colour_close(to_np(img), img_ref, "image")
        assert abs(loss.item() - loss_ref) <= 1e-5 * loss_ref
        assert_grad_close(to_np(grad), g_ref, "gradients with probe records")


def test_step_fused_from_16bit_map(sad, ref, c2_state):
    """The fused last pass + backward reading a 16-bit-id map (and its score
    map) on the 768x512 map: the oracle's lists, loss and gradients, and the
    same lists, image and score map as the call that reads the 32-bit map."""
    wl, p, d, dg, m_ref, m_gpu = c2_state
    h, w = wl.h, wl.w
    tgt = wl.make_target()
    prev16 = map16_from_np(m_ref)
    assert np.array_equal(map16_to_np(prev16), m_ref)
    m1 = ref.propagate(d, h, w, m_ref, 1, wl.inject_seed, 702, wl.inject)
    g_ref, _, loss_ref, img_ref = ref.render_bwd(d, h, w, m1, tgt)
    res = []
    for prev in (prev16, m_gpu):
        out = torch.empty((h, w, 8), dtype=torch.int32, device=dev())
        osc = torch.empty((h, w, 8), dtype=torch.float32, device=dev())
        grad = torch.zeros((wl.n, 12), dtype=torch.float32, device=dev())
        loss = torch.zeros(1, dtype=torch.float32, device=dev())
        img = torch.empty((h, w, 3), dtype=torch.float32, device=dev())
        sad.step_fused(dg, h, w, prev, out, to_gpu(tgt), grad, stride=1, seed=wl.inject_seed, pass_index=702,
                       inject=wl.inject, out_scores=osc, loss=loss, image=img)
        res.append((map_to_np(out), to_np(osc), to_np(grad), loss.item(), to_np(img)))
    (l16, s16, g16, loss16, i16), (l32, s32, _, _, i32) = res
    assert np.array_equal(l16, m1) and np.array_equal(l16, l32)
    assert np.array_equal(s16.view(np.uint32), s32.view(np.uint32))
    assert np.array_equal(i16.view(np.uint32), i32.view(np.uint32))
    assert_colour_close(i16, img_ref, "fused from 16-bit image")
    assert abs(loss16 - loss_ref) <= 1e-5 * loss_ref
    assert_grad_close(g16, g_ref, "fused from 16-bit gradients")


def test_step_fused_to_16bit_map(sad, ref, c2_state):
    """The fused last pass + backward writing 16-bit-id lists (as a training
    step hands them to the next step): the same lists, id for id, as the
    call that writes 32-bit ones (the oracle's), the same image bit for bit,
    the loss (summed across regions by float atomics, so its last bits vary
    from call to call) and the gradients within the bar; the next step's first pass
    reads that map (recomputing its logits) and gives the oracle's lists;
    widened, the map is the 32-bit one."""
    wl, p, d, dg, m_ref, m_gpu = c2_state
    h, w = wl.h, wl.w
    tgt = wl.make_target()
    m1 = ref.propagate(d, h, w, m_ref, 1, wl.inject_seed, 702, wl.inject)
    g_ref, _, loss_ref, img_ref = ref.render_bwd(d, h, w, m1, tgt)
    res = []
    for dt in (torch.int16, torch.int32):
        out = torch.empty((h, w, 8), dtype=dt, device=dev())
        grad = torch.zeros((wl.n, 12), dtype=torch.float32, device=dev())
        loss = torch.zeros(1, dtype=torch.float32, device=dev())
        img = torch.empty((h, w, 3), dtype=torch.float32, device=dev())
        sad.step_fused(dg, h, w, map16_from_np(m_ref), out, to_gpu(tgt), grad, stride=1, seed=wl.inject_seed,
                       pass_index=702, inject=wl.inject, loss=loss, image=img)
        res.append((out, to_np(grad), loss.item(), to_np(img)))
    (o16, g16, loss16, i16), (o32, _, loss32, i32) = res
    assert np.array_equal(map16_to_np(o16), m1) and np.array_equal(map_to_np(o32), m1)
    assert np.array_equal(map_to_np(sad.widen_map(o16)), m1)
    assert np.array_equal(i16.view(np.uint32), i32.view(np.uint32))
    for lv in (loss16, loss32):
        assert abs(lv - loss_ref) <= 1e-5 * loss_ref
    assert_colour_close(i16, img_ref, "fused to 16-bit image")
    assert_grad_close(g16, g_ref, "fused to 16-bit gradients")
    m2 = ref.propagate(d, h, w, m1, 8, wl.inject_seed, 703, wl.inject)
    nxt = torch.empty((h, w, 8), dtype=torch.int16, device=dev())
    sad.propagate_topk(dg, h, w, o16, nxt, stride=8, seed=wl.inject_seed, pass_index=703, inject=wl.inject)
    assert np.array_equal(map16_to_np(nxt), m2)


@pytest.mark.parametrize("h,w,n", [(1, 1, 3), (13, 29, 300), (67, 72, 1000), (45, 131, 65535)])
def test_field_steps_16bit_handoff(sad, ref, h, w, n):
    """A field's fused steps on ragged and degenerate images: the last pass
    hands its lists to the next step as a 16-bit map, and the next step's
    first pass reads it with the probe records current (as after an Adam
    step); two steps, every map and both backwards against the oracle chain
    from the same warm-up, up to 65,535 sites."""
    from voronoi_rendering_amd.pipeline import SadField

    p = synth.sites(7100 + n, n, h, w, synth.WIDE_SCALES)
    d = ref.prepare_sites(p)
    tgt_np = synth.target_noise_edges(7200 + n, h, w)
    tgt = to_gpu(tgt_np)
    f = SadField(to_gpu(p), h, w, 77, inject=64)
    warm = synth.jfa_strides(h, w, 10)
    f.warm(10)
    m = ref.propagate_schedule(d, h, w, None, warm, 77, 0, 64)
    assert np.array_equal(field_lists(f), m)
    strides = [8, 4, 2, 1]
    for step in range(2):
        first = f.pass_index
        f.grad.zero_()
        f.loss.zero_()
        f.step(strides, tgt, fused=True)
        f.sites_changed(probe_records_current=True)
        assert f.cur16 and f.probe_valid
        m = ref.propagate_schedule(d, h, w, m, strides, 77, first, 64)
        got = field_lists(f)
        assert np.array_equal(got, m), f"{h}x{w} step {step}: {(got != m).any(-1).sum()} pixels differ"
        g_ref, _, loss_ref, _ = ref.render_bwd(d, h, w, m, tgt_np)
        assert abs(f.loss.item() - loss_ref) <= 1e-5 * max(loss_ref, 1e-30)
        assert_grad_close(to_np(f.grad), g_ref, f"{h}x{w} step {step} gradients")
    assert np.array_equal(map_to_np(f.topk), m) and not f.cur16  # widened on request


@pytest.mark.parametrize("h,w", [(1, 1), (13, 29), (67, 72), (512, 768)])
def test_widen_map(sad, h, w):
    """A 16-bit-id map widened to 32-bit ids: every id kept, 0xffff (empty)
    written as 0xffffffff; ragged and single-pixel images."""
    rng = np.random.default_rng(h * 1000 + w)
    m = rng.integers(0, 0x10000, (h, w, 8), dtype=np.uint32)
    m[rng.random((h, w, 8)) < 0.2] = 0xFFFF
    m[0, 0, :2] = (0, 0xFFFE)
    want = m.copy()
    want[want == 0xFFFF] = 0xFFFFFFFF
    m16 = torch.from_numpy(np.ascontiguousarray(m.astype(np.uint16)).view(np.int16)).to(dev())
    assert np.array_equal(map_to_np(sad.widen_map(m16)), want)


# ---------------------------------------------------------------- Adam

def test_adam_bit_exact(sad, ref):
    n, h, w = 50_000, 512, 768
    p = synth.C2.make_sites()
    p[17, 0] = -1.0
    p[18, 0] = 0.0  # pushed below 0, clamped
    p[19, 1] = float(h)  # pushed above h, clamped
    rng = np.random.default_rng(3)
    m = (rng.normal(0, 1e-3, (n, 12)) * (np.arange(12) < 10)).astype(np.float32)
    v = (rng.random((n, 12)) * 1e-6 * (np.arange(12) < 10)).astype(np.float32)
    g = synth.gradients(4, n)
    g[18, 0], g[19, 1] = 1.0, -1.0
    lr = np.array([1e-2, 1e-3, 2e-3, 3e-3, 4e-3], np.float32)
    bc1, bc2 = ref.bias_corrections(0.9, 0.999, 7)
    want = ref.adam_step(p, g, m, v, h, w, lr, 0.9, 0.999, 1e-8, bc1, bc2)
    for with_probe in (False, True):
        P, G, M, V = (to_gpu(x.copy()) for x in (p, g, m, v))
        D = torch.empty_like(P)
        probe = torch.full((n, 4), np.nan, dtype=torch.float32, device=dev()) if with_probe else None
        sad.adam_step(P, G, M, V, h, w, lr.tolist(), 0.9, 0.999, 1e-8, bc1, bc2, D, probe)
        for name, gt, wt in zip(("params", "grad", "m", "v", "derived"), (P, G, M, V, D), want):
            a = to_np(gt)
            assert np.array_equal(a.view(np.uint32), wt.view(np.uint32)), (name, np.argwhere(a != wt)[:5])
        if with_probe:
            # the probe records of the new prepared sites, as a pass writes them
            got_rec, want_rec = to_np(probe), probe_records_np(want[4])
            assert np.array_equal(got_rec.view(np.uint32), want_rec.view(np.uint32)), \
                np.argwhere(got_rec.view(np.uint32) != want_rec.view(np.uint32))[:4]


# ---------------------------------------------------------------- queries

def test_query_points(sad, ref, c2_state):
    wl, p, d, dg, m_ref, m_gpu = c2_state
    xy = synth.queries(4005, 1 << 18, wl.h, wl.w)
    xy[:4] = [[-5.0, 3.0], [wl.w + 9.5, wl.h + 0.25], [np.nan, 2.0], [1.0, -np.inf]]
    got = to_np(sad.query_points(dg, wl.h, wl.w, m_gpu, to_gpu(xy)))
    assert_colour_close(got, ref.query_points(d, wl.h, wl.w, m_ref, xy), "query colours")
    # at pixel centres a query is the render itself, bit for bit
    yy, xx = np.mgrid[0:wl.h, 0:wl.w]
    centres = np.stack([xx.ravel() + 0.5, yy.ravel() + 0.5], 1).astype(np.float32)
    q = to_np(sad.query_points(dg, wl.h, wl.w, m_gpu, to_gpu(centres)))
    img = to_np(sad.render_fwd(dg, wl.h, wl.w, m_gpu)).reshape(-1, 3)
    assert np.array_equal(q, img)


def test_query_c5_full_batch_sampled(sad, ref):
    """2^24 random points on the 768x512 / 50k-site representation (site
    recipe of the small-scale workload, map warmed with 16 passes); 2^16
    sampled outputs checked against the oracle."""
    wl = synth.C5
    p = wl.make_sites()
    d = ref.prepare_sites(p)
    dg = sad.prepare_sites(to_gpu(p))
    strides = synth.jfa_strides(wl.h, wl.w, wl.warm_passes)
    m_gpu = gpu_schedule(sad, dg, wl.h, wl.w, strides, wl.inject_seed)
    m_ref = ref.propagate_schedule(d, wl.h, wl.w, None, strides, wl.inject_seed, 0, 64)
    assert np.array_equal(map_to_np(m_gpu), m_ref)
    xy = wl.make_queries()
    rgb = to_np(sad.query_points(dg, wl.h, wl.w, m_gpu, to_gpu(xy)))
    idx = np.random.default_rng(0).choice(xy.shape[0], 1 << 16, replace=False)
    assert_colour_close(rgb[idx], ref.query_points(d, wl.h, wl.w, m_ref, xy[idx]), "C5 sampled colours")


# ---------------------------------------------------------------- training loop

def test_training_first_iterations_track_oracle(sad, ref):
    """The 768x512 / 50k-site fitting loop (tau = 1 at start, lr 1e-3, betas
    0.9/0.999): 10 iterations of 4 passes + forward + backward + Adam on both
    sides, each running free.  The GPU's gradients differ from the oracle's
    in the last bits (float32 results of float64 sums, float atomics across
    regions), and Adam turns tiny differences of near-zero gradients into
    different steps, so the trajectories are compared within tolerance: PSNR
    within 0.01 dB at every iteration, nearly all lists and parameters equal.
    test_training_reanchored checks every step exactly."""
    from voronoi_rendering_amd.pipeline import SadField

    wl = synth.C3
    p = wl.make_sites()
    tgt = wl.make_target()
    warm = synth.jfa_strides(wl.h, wl.w, wl.warm_passes)
    lr = np.full(5, 1e-3, np.float32)
    # oracle trajectory
    d = ref.prepare_sites(p)
    cur = ref.propagate_schedule(d, wl.h, wl.w, None, warm, wl.inject_seed, 0, 64)
    pp, m, v = p.copy(), np.zeros_like(p), np.zeros_like(p)
    psnr_ref, pi = [], len(warm)
    for it in range(1, 11):
        cur = ref.propagate_schedule(d, wl.h, wl.w, cur, wl.strides, wl.inject_seed, pi, 64)
        pi += len(wl.strides)
        g, _, loss, _ = ref.render_bwd(d, wl.h, wl.w, cur, tgt)
        psnr_ref.append(10 * math.log10(3.0 / loss))
        bc1, bc2 = ref.bias_corrections(0.9, 0.999, it)
        pp, _, m, v, d = ref.adam_step(pp, g.astype(np.float32), m, v, wl.h, wl.w, lr, 0.9, 0.999, 1e-8, bc1, bc2)
    # GPU trajectory
    f = SadField(to_gpu(p), wl.h, wl.w, wl.inject_seed)
    f.warm(wl.warm_passes)
    target = to_gpu(tgt)
    psnr_gpu = []
    for it in range(10):
        f.loss.zero_()
        f.train_iter(wl.strides, target)
        psnr_gpu.append(10 * math.log10(3.0 / f.loss.item()))
    say("[gpu] C3 PSNR oracle " + " ".join(f"{x:.4f}" for x in psnr_ref))
    say("[gpu] C3 PSNR gpu    " + " ".join(f"{x:.4f}" for x in psnr_gpu))
    assert np.all(np.abs(np.array(psnr_gpu) - np.array(psnr_ref)) <= 0.01)
    same_lists = (map_to_np(f.topk) == cur).all(-1).mean()
    close = np.abs(to_np(f.params)[:, :10] - pp[:, :10]) <= 1e-5 * (1 + np.abs(pp[:, :10]))
    say(f"[gpu] C3 after 10 iterations: lists equal {same_lists:.5f}, params within 1e-5: {close.mean():.5f}")
    assert same_lists >= 0.999
    assert close.mean() >= 0.99
    assert np.all(np.abs(to_np(f.params)[:, :10] - pp[:, :10]) <= 10 * 2 * 1e-3 + 1e-4)


def test_training_reanchored(sad, ref):
    """The same 10 iterations of the 768x512 / 50k-site fitting loop (the
    field's own calls: score maps, the fused last pass and backward, Adam),
    each checked against the oracle started from the GPU's state before it:
    the oracle runs the iteration's 4 passes from the GPU's map and prepared
    sites (lists bit for bit), its backward over those lists (gradients at
    the bar, loss 1e-5), and Adam from the GPU's params, moments and
    gradients (params, moments, prepared records bit for bit)."""
    from voronoi_rendering_amd.pipeline import SadField, bias_corrections

    wl = synth.C3
    p = wl.make_sites()
    tgt = wl.make_target()
    target = to_gpu(tgt)
    f = SadField(to_gpu(p), wl.h, wl.w, wl.inject_seed)
    f.warm(wl.warm_passes)
    lr = np.asarray(f.adam.lr, np.float32)
    for it in range(1, 11):
        p0, m0, v0, d0 = (to_np(x).copy() for x in (f.params, f.m, f.v, f.derived))
        # the lists are read without widening the step's 16-bit map, so every
        # iteration after the first starts from it, as a fit does
        map0, pi0 = field_lists(f).copy(), f.pass_index
        assert (it == 1) or (f.cur16 and f.probe_valid)
        assert np.array_equal(d0.view(np.uint32), ref.prepare_sites(p0).view(np.uint32))
        f.loss.zero_()
        f.step(list(wl.strides), target)
        map1, g_gpu, loss_gpu = field_lists(f), to_np(f.grad).copy(), f.loss.item()
        f.adam_step()
        p1, m1, v1, d1 = (to_np(x) for x in (f.params, f.m, f.v, f.derived))
        # the oracle from the GPU's state before the iteration
        want_map = ref.propagate_schedule(d0, wl.h, wl.w, map0, wl.strides, wl.inject_seed, pi0, wl.inject)
        assert np.array_equal(map1, want_map), f"iteration {it}: {(map1 != want_map).any(-1).sum()} pixels differ"
        g_ref, _, loss_ref, _ = ref.render_bwd(d0, wl.h, wl.w, want_map, tgt)
        assert abs(loss_gpu - loss_ref) <= 1e-5 * loss_ref, (it, loss_gpu, loss_ref)
        assert_grad_close(g_gpu, g_ref, f"iteration {it} gradients")
        bc1, bc2 = bias_corrections(f.adam.beta1, f.adam.beta2, it)
        wp, wg, wm, wv, wd = ref.adam_step(p0, g_gpu, m0, v0, wl.h, wl.w, lr, f.adam.beta1, f.adam.beta2,
                                           f.adam.eps, bc1, bc2)
        for name, got, want in (("params", p1, wp), ("m", m1, wm), ("v", v1, wv), ("derived", d1, wd)):
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"iteration {it}: Adam {name} differs"
        say(f"[gpu] C3 iteration {it}: lists, Adam bit-exact; PSNR {10 * math.log10(3.0 / loss_ref):.4f} dB")
