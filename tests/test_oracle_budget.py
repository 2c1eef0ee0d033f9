"""Pins of the oracle's budget control (Sec. 4.5 "Adaptive Budget: Densify
and Prune"; Appendix B.5 "Densification scores", "Split kernel", "Pruning").

Selections are checked against rankings made here with numpy (for alpha 0
and 1 the densification score needs no power); the split geometry against
covariances built by hand from a known rotation and pair of spreads (the
children must sit on the major axis at offset * spread), and against a
target ramp for the Sobel fallback; the bookkeeping (slots, counts, Adam
moments, colours, prepared records) directly.
"""
import math

import numpy as np
import pytest

import synth

W, H = 48, 40


def base_state(seed=3, n=120, inactive=0.15):
    p = synth.sites(seed, n, H, W)
    rng = np.random.default_rng(seed)
    p[rng.random(n) < inactive, 0] = -1.0
    m = rng.normal(size=p.shape).astype(np.float32)
    v = rng.random(p.shape).astype(np.float32)
    t = rng.random((H, W, 3)).astype(np.float32)
    return p, m, v, t


def random_stats(seed, n):
    rng = np.random.default_rng(seed)
    st = np.zeros((n, 8), np.float32)
    st[:, 0] = rng.random(n) * 10
    st[:, 1] = rng.random(n) * 2
    st[:, 2] = rng.normal(size=n)
    st[:, 3:5] = rng.normal(size=(n, 2))
    st[:, 5] = st[:, 7] = rng.random(n) * 20 + 5
    st[:, 6] = rng.normal(size=n)
    return st


def test_prune_takes_the_lowest_removal_deltas(ref):
    p, m, v, t = base_state()
    d = ref.prepare_sites(p)
    st = random_stats(1, len(p))
    st[7, 2] = np.nan
    st[8, 2] = st[9, 2] = -5.0  # a tie: lower id first
    active = np.flatnonzero(p[:, 0] >= 0)
    key = np.where(np.isnan(st[active, 2]), np.inf, st[active, 2].astype(np.float64))
    for k in (0, 1, 13, len(active) + 5):
        P2, _, _, D2, done = ref.densify_prune(p, m, v, d, H, W, st, t, 0, k, 1.0, 0.0, 0.5, 0.85, 0.1)
        want = active[np.lexsort((active, key))][:k]
        assert done == (min(k, len(active)), 0)
        off = np.flatnonzero((p[:, 0] >= 0) & (P2[:, 0] < 0))
        assert sorted(off) == sorted(want)
        assert (P2[want, :2] == -1).all()
        assert np.array_equal(D2, ref.prepare_sites(P2))


@pytest.mark.parametrize("alpha", [0.0, 1.0])
def test_split_takes_the_best_scores_into_free_slots(ref, alpha):
    p, m, v, t = base_state(5)
    d = ref.prepare_sites(p)
    st = random_stats(2, len(p))
    st[3, 0] = 0.0  # no mass: never split
    n_prune, n_split, min_mass = 6, 9, 1.0
    P2, M2, V2, D2, done = ref.densify_prune(p, m, v, d, H, W, st, t, n_split, n_prune, alpha, min_mass,
                                             0.5, 0.85, 0.1)
    active = np.flatnonzero(p[:, 0] >= 0)
    key = st[active, 2].astype(np.float64)
    pruned = active[np.lexsort((active, key))][:n_prune]
    alive = np.setdiff1d(active, pruned)
    mass = st[alive, 0].astype(np.float64)
    ok = alive[(mass >= min_mass) & (mass > 0)]
    score = st[ok, 1].astype(np.float64) / (1.0 if alpha == 0 else st[ok, 0].astype(np.float64))
    parents = ok[np.lexsort((ok, -score))]
    free = np.flatnonzero(~(p[:, 0] >= 0) | np.isin(np.arange(len(p)), pruned))
    k = min(n_split, len(parents), len(free))
    assert done == (n_prune, k)
    assert (P2[:, 0] >= 0).sum() == len(active) - n_prune + k
    for par, slot in zip(parents[:k], free[:k]):
        # the two children are the parent moved both ways along one axis
        mid = (P2[par, :2].astype(np.float64) + P2[slot, :2]) / 2
        inside = (P2[[par, slot], 0] > 0).all() & (P2[[par, slot], 0] < W).all() & \
                 (P2[[par, slot], 1] > 0).all() & (P2[[par, slot], 1] < H).all()
        if inside:
            assert np.allclose(mid, p[par, :2], atol=1e-4)
        for c in (par, slot):
            assert P2[c, 2] == np.float32(p[par, 2] - np.float32(0.1))
            assert P2[c, 3] == np.float32(p[par, 3] * np.float32(0.85))
            assert np.array_equal(P2[c, 7:10], p[par, 7:10])
            ci = min(max(int(np.floor(P2[c, 0])), 0), W - 1)
            cj = min(max(int(np.floor(P2[c, 1])), 0), H - 1)
            assert np.array_equal(P2[c, 4:7], t[cj, ci])
            assert (M2[c] == 0).all() and (V2[c] == 0).all()
    untouched = np.setdiff1d(np.arange(len(p)), np.concatenate([parents[:k], free[:k]]))
    assert np.array_equal(M2[untouched], m[untouched]) and np.array_equal(V2[untouched], v[untouched])
    assert np.array_equal(D2, ref.prepare_sites(P2))


@pytest.mark.parametrize("phi,s1,s2,mean", [(0.5, 2.0, 1.0, (0.0, 0.0)), (2.3, 3.0, 0.5, (0.7, -1.2)),
                                            (-1.0, 1.5, 1.2, (2.0, 0.5))])
def test_split_axis_is_the_major_axis_of_the_covariance(ref, phi, s1, s2, mean):
    p, m, v, t = base_state(7, n=4, inactive=0.0)
    p[:, 0], p[:, 1] = [20.0, 30.0, 10.0, 40.0], [20.0, 10.0, 30.0, 5.0]
    p[3, 0] = -1.0  # the free slot
    d = ref.prepare_sites(p)
    st = np.zeros((4, 8), np.float32)
    mass = 2.5
    c, s = math.cos(phi), math.sin(phi)
    cov = np.array([[c, -s], [s, c]]) @ np.diag([s1 ** 2, s2 ** 2]) @ np.array([[c, s], [-s, c]])
    mx, my = mean
    st[:, 0] = 0.1
    st[0] = [mass, 1.0, 0.0, mass * mx, mass * my, mass * (cov[0, 0] + mx * mx), mass * (cov[0, 1] + mx * my),
             mass * (cov[1, 1] + my * my)]
    off = 0.5
    P2, _, _, _, done = ref.densify_prune(p, m, v, d, H, W, st, t, 1, 0, 0.0, 1.0, off, 1.0, 0.0)
    assert done == (0, 1)
    step = (P2[0, :2].astype(np.float64) - P2[3, :2]) / 2
    axis = np.array([c, s]) * (1 if s1 >= s2 else 0) + np.array([-s, c]) * (0 if s1 >= s2 else 1)
    assert abs(np.linalg.norm(step) - off * max(s1, s2)) < 1e-4
    assert abs(abs(step @ axis) - np.linalg.norm(step)) < 1e-4


def test_split_falls_back_to_the_target_gradient(ref):
    p, m, v, _ = base_state(9, n=3, inactive=0.0)
    p[:, 0], p[:, 1] = [24.0, 5.0, 5.0], [20.0, 5.0, 35.0]
    p[2, 0] = -1.0
    p[0, 8], p[0, 9] = math.log(2.0), math.log(0.5)  # larger scale 2
    d = ref.prepare_sites(p)
    g = np.array([0.6, -0.8])
    jj, ii = np.mgrid[0:H, 0:W]
    ramp = (0.01 * (g[0] * ii + g[1] * jj) + 0.5).astype(np.float32)
    t = np.repeat(ramp[..., None], 3, axis=-1)
    st = np.zeros((3, 8), np.float32)
    st[0, :3] = [3.0, 1.0, 0.0]  # mass, but no spread: the covariance is degenerate
    st[1, 0] = 0.1
    P2, _, _, _, done = ref.densify_prune(p, m, v, d, H, W, st, t, 1, 0, 0.0, 1.0, 0.5, 1.0, 0.0)
    assert done == (0, 1)
    step = (P2[0, :2].astype(np.float64) - P2[2, :2]) / 2
    assert np.allclose(step, 0.5 * 2.0 * g, atol=1e-4)


def test_split_stops_when_no_slot_is_free(ref):
    p, m, v, t = base_state(11, n=30, inactive=0.0)
    p[[4, 9], 0] = -1.0
    d = ref.prepare_sites(p)
    st = random_stats(4, 30)
    P2, _, _, _, done = ref.densify_prune(p, m, v, d, H, W, st, t, 10, 0, 1.0, 0.0, 0.5, 0.85, 0.1)
    assert done == (0, 2)
    assert (P2[:, 0] >= 0).all()
