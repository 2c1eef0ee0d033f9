"""Pins for the oracle's top-K propagation (paper Sec. 4.3 update
C~_t = C_{t-1} u P_t u G_t, C_t = topK; Figure 5 steps 1-5; Sec. 4.6 fixed-K
list; Sec. 6.5 exact-match protocol) and its injection generator.

The propagation is an approximation, so the oracle implements the algorithm
itself.  It is pinned by a brute-force restatement with Python sets on tiny
inputs, by properties the update must have (exact top-K is a fixed point,
scores never get worse, the map converges to the exact top-K), and the
generator by SplitMix64's reference outputs.
"""
import numpy as np
import pytest

import synth


def _tiny(seed, n=30, h=19, w=21):
    p = synth.sites(seed, n, h, w)
    return p, h, w


def _set_pass(ref, d, h, w, prev, stride, seed, pass_index, inject):
    """One pass written with Python sets, pixel by pixel."""
    n = d.shape[0]
    tiles_x = (w + 7) // 8
    out = np.empty((h, w, 8), np.uint32)
    for j in range(h):
        for i in range(w):
            ids = set()
            if prev is not None:
                for di, dj in ((0, 0), (stride, 0), (-stride, 0), (0, stride), (0, -stride)):
                    ii, jj = i + di, j + dj
                    if 0 <= ii < w and 0 <= jj < h:
                        ids.update(int(v) for v in prev[jj, ii])
            tile = (j // 8) * tiles_x + i // 8
            ids.update(ref.inject_id(seed, pass_index, tile, q, n) for q in range(inject))
            scored = []
            for s in ids:
                if s >= n or d[s, 0] < 0:
                    continue
                sc = ref.score(d, s, i + 0.5, j + 0.5)
                if not np.isnan(sc):
                    scored.append((-sc, s))
            scored.sort()
            lst = [s for _, s in scored[:8]]
            out[j, i] = lst + [ref.NONE] * (8 - len(lst))
    return out


@pytest.mark.parametrize("stride,inject", [(1, 64), (3, 5), (8, 0), (16, 64)])
def test_pass_matches_set_restatement(ref, stride, inject):
    p, h, w = _tiny(31)
    p[7, 0] = -1.0  # an inactive site is never listed
    d = ref.prepare_sites(p)
    prev = ref.propagate(d, h, w, None, 4, 99, 0, 6)  # a partial map to start from
    prev[3, 4, 2] = 1000  # out-of-range id in the previous map: skipped
    got = ref.propagate(d, h, w, prev, stride, 1234, 5, inject)
    want = _set_pass(ref, d, h, w, prev, stride, 1234, 5, inject)
    assert np.array_equal(got, want)
    assert not np.any(got == 7)


def test_pixel_subset_matches_full_pass(ref):
    p, h, w = _tiny(32)
    d = ref.prepare_sites(p)
    prev = ref.propagate(d, h, w, None, 4, 7, 0, 10)
    full = ref.propagate(d, h, w, prev, 2, 7, 1, 64)
    pix = np.array([0, 5, 77, h * w - 1, 200])
    sub = ref.propagate_pixels(d, h, w, prev, 2, 7, 1, 64, pix)
    assert np.array_equal(sub, full.reshape(-1, 8)[pix])


def test_exact_topk_is_a_fixed_point(ref):
    p, h, w = _tiny(33, n=80, h=30, w=26)
    d = ref.prepare_sites(p)
    exact = ref.brute_topk(d, h, w)
    for stride in (1, 2, 8):
        assert np.array_equal(ref.propagate(d, h, w, exact, stride, 5, stride, 64), exact)


def test_scores_never_get_worse(ref):
    """C_{t-1}(x) is part of C~_t(x), so each pixel's k-th best score is
    non-decreasing from pass to pass."""
    wl = synth.C1
    d = ref.prepare_sites(wl.make_sites())
    h, w = wl.h, wl.w
    cur = None
    prev_scores = np.full((h, w, 8), -np.inf)
    for t, s in enumerate(wl.strides[:10]):
        cur = ref.propagate(d, h, w, cur, s, wl.inject_seed, t, wl.inject)
        sc = np.full((h, w, 8), -np.inf)
        for j in range(0, h, 3):
            for i in range(0, w, 3):
                for k in range(8):
                    if cur[j, i, k] != ref.NONE:
                        sc[j, i, k] = ref.score(d, int(cur[j, i, k]), i + 0.5, j + 0.5)
        assert np.all(sc[::3, ::3] >= prev_scores[::3, ::3])
        prev_scores = sc


def test_c1_converges_to_exact_topk(ref):
    """The 64x64 / 256-site workload reaches the exact top-8 everywhere after
    its 20 warm-up passes (Sec. 6.5 measures the same exact-match fraction)."""
    wl = synth.C1
    d = ref.prepare_sites(wl.make_sites())
    got = ref.propagate_schedule(d, wl.h, wl.w, None, wl.strides, wl.inject_seed, 0, wl.inject)
    exact = ref.brute_topk(d, wl.h, wl.w)
    assert (got == exact).all(axis=-1).mean() >= 0.99


def test_empty_map_and_no_injection_stays_empty(ref):
    p, h, w = _tiny(34)
    d = ref.prepare_sites(p)
    assert np.all(ref.propagate(d, h, w, None, 1, 0, 0, 0) == ref.NONE)


def test_splitmix64_reference_outputs(ref):
    """Known outputs of the reference SplitMix64 generator (Vigna's
    splitmix64.c): the first output from state 0, and the first five from
    state 1234567.  Output t of the stream from state s is the counter value t."""
    assert ref.splitmix64(0, 0) == 0xE220A8397B1DCDAF
    want = [6457827717110365317, 3203168211198807973, 9817491932198370423,
            4593380528125082431, 16408922859458223821]
    assert [ref.splitmix64(1234567, t) for t in range(5)] == want


def test_inject_ids_counter_layout_and_range(ref):
    n = 50_000
    seed = 3002
    got = ref.inject_id(seed, 7, 1234, 5, n)
    z = ref.splitmix64(seed, (7 << 32) | (1234 << 6) | 5)
    assert got == ((z >> 32) * n) >> 32
    ids = np.array([ref.inject_id(seed, t, tile, j, n) for t in range(4) for tile in range(40) for j in range(64)])
    assert ids.min() >= 0 and ids.max() < n
    # roughly uniform: chi-square over 16 equal bins
    hist = np.bincount(ids * 16 // n, minlength=16)
    exp = ids.size / 16
    chi2 = ((hist - exp) ** 2 / exp).sum()
    assert chi2 < 45.0  # p ~ 1e-4 for 15 degrees of freedom


def test_brute_force_at_chosen_pixels(ref):
    """The sampled exact top-K equals the full one at those pixels (including
    the image's last pixel and repeats)."""
    h, w = 21, 34
    p = synth.sites(8, 90, h, w)
    p[::11, 0] = -1.0
    d = ref.prepare_sites(p)
    full = ref.brute_topk(d, h, w).reshape(-1, 8)
    pix = np.concatenate([np.random.default_rng(2).integers(0, h * w, 50), [0, h * w - 1, 7, 7]])
    assert np.array_equal(ref.brute_topk_pixels(d, h, w, pix), full[pix])
