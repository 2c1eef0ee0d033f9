"""Pins of the oracle's JFA prepass (Appendix B.3 "JFA prepass", after the
jump flooding of Rong and Tan 2006) and of the full refresh of the render
protocol (Sec. 6.6: one JFA round, 16 propagation passes, render).

The seed and a flood pass are restated with Python dictionaries and sets on
small inputs (scores from the separately pinned float32 logit); a JFA round
must carry every site to every pixel when there are at most 4 sites (nothing
is ever evicted from the 4-lists, and the steps B/2, ..., 1 reach every
offset); on an ordinary Voronoi diagram (isotropic, r = 0, one temperature)
its first entry matches the nearest site almost everywhere, and the full
refresh rebuilds the exact top-8 lists almost everywhere.
"""
import numpy as np
import pytest

import synth

NONE = 0xFFFFFFFF


def usable(d, n, i):
    return i < n and d[i, 0] >= 0


def ranked(ref, d, n, ids, px, py):
    """Distinct usable ids with a number for a logit, best first."""
    c = {}
    for i in ids:
        i = int(i)
        if not usable(d, n, i) or i in c:
            continue
        s = ref.score(d, i, px, py)
        if s == s:
            c[i] = s
    return sorted(c, key=lambda i: (-c[i], i))


def random_sites(seed, n, h, w):
    p = synth.sites(seed, n, h, w)
    rng = np.random.default_rng(seed)
    p[rng.random(n) < 0.1, 0] = -1.0  # inactive
    # crowd some sites into a few pixels and onto the borders
    k = n // 4
    p[:k, 0] = rng.integers(0, 3, k) + rng.random(k) * 0.999
    p[:k, 1] = rng.integers(0, 2, k) + rng.random(k) * 0.999
    p[k, 0], p[k, 1] = float(w), float(h)  # on the far corner: clamped into the last pixel
    return p


@pytest.mark.parametrize("h,w,n", [(5, 7, 40), (9, 4, 120), (1, 1, 6), (16, 16, 300)])
def test_seed_brute_force(ref, h, w, n):
    p = random_sites(10 + n, n, h, w)
    d = ref.prepare_sites(p).reshape(-1, 12)
    got = ref.jfa_seed(d, h, w)
    want = np.full((h, w, 4), NONE, np.uint32)
    on = {}
    for i in range(n):
        if d[i, 0] < 0:
            continue
        ci = int(min(max(np.floor(d[i, 0]), 0), w - 1))
        cj = int(min(max(np.floor(d[i, 1]), 0), h - 1))
        on.setdefault((cj, ci), []).append(i)
    for (cj, ci), ids in on.items():
        r = ranked(ref, d, n, ids, ci + 0.5, cj + 0.5)
        if r:
            want[cj, ci, 0] = r[0]
    assert np.array_equal(got, want)


@pytest.mark.parametrize("h,w,n,step,width", [(6, 9, 30, 1, 4), (6, 9, 30, 2, 8), (11, 5, 80, 4, 4),
                                              (11, 5, 80, 16, 8), (1, 13, 10, 3, 4)])
def test_flood_pass_restatement(ref, h, w, n, step, width):
    p = random_sites(30 + n + step, n, h, w)
    d = ref.prepare_sites(p).reshape(-1, 12)
    rng = np.random.default_rng(step)
    prev = rng.integers(0, n + 5, (h, w, 4)).astype(np.uint32)  # ids past n are stale
    prev[rng.random((h, w, 4)) < 0.3] = NONE
    got = ref.jfa_flood(d, h, w, prev, step, width)
    for j in range(h):
        for i in range(w):
            cand = []
            for b in (-1, 0, 1):
                for a in (-1, 0, 1):
                    ii, jj = i + a * step, j + b * step
                    if 0 <= ii < w and 0 <= jj < h:
                        cand.extend(prev[jj, ii])
            r = ranked(ref, d, n, cand, i + 0.5, j + 0.5)[:4]
            want = r + [NONE] * (width - len(r))
            assert list(got[j, i]) == want, (j, i)


@pytest.mark.parametrize("n", [1, 2, 4])
def test_round_with_few_sites_reaches_every_pixel(ref, n):
    h, w = 23, 37
    p = synth.sites(50 + n, n, h, w)
    d = ref.prepare_sites(p)
    cur = ref.jfa_seed(d, h, w)
    for s in ref.jfa_steps(h, w):
        cur = ref.jfa_flood(d, h, w, cur, s)
    exact = ref.brute_topk(d, h, w)
    assert np.array_equal(cur, exact[..., :4])


def test_round_finds_the_voronoi_owner(ref):
    """Ordinary Voronoi (isotropic, r = 0, one temperature), every site on a
    pixel of its own so that each is seeded: the JFA round's first entry is
    the nearest site at nearly every pixel."""
    h, w, n = 96, 80, 200
    p = synth.sites(61, n, h, w)
    cells = np.random.default_rng(61).choice(h * w, n, replace=False)  # one site per pixel: all seeded
    p[:, 0] = (cells % w) + 0.25 + 0.5 * p[:, 0] / w
    p[:, 1] = (cells // w) + 0.25 + 0.5 * p[:, 1] / h
    p[:, 2] = 0.0  # log tau
    p[:, 3] = 0.0  # r
    p[:, 7] = 0.0  # theta
    p[:, 8] = p[:, 9] = np.log(3.0)
    d = ref.prepare_sites(p)
    cur = ref.jfa_seed(d, h, w)
    for s in ref.jfa_steps(h, w):
        cur = ref.jfa_flood(d, h, w, cur, s)
    exact = ref.brute_topk(d, h, w)
    assert (cur[..., 0] == exact[..., 0]).mean() >= 0.999


def test_full_refresh_rebuilds_the_lists(ref):
    wl = synth.C1
    d = ref.prepare_sites(wl.make_sites())
    m = ref.full_refresh(d, wl.h, wl.w, 7)
    exact = ref.brute_topk(d, wl.h, wl.w)
    assert (m == exact).all(-1).mean() >= 0.99
    assert (m[..., 0] == exact[..., 0]).mean() >= 0.999
