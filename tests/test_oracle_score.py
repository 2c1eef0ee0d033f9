"""Pins for the oracle's logit and exact top-K (paper Sec. 3 "Connection to
SAD", Sec. 4.1 metric, Sec. 4.2 logit, Sec. 4.3 top-K under the same score).

The logit is l = -tau (||x - p||_G - r) with G = R diag(s1^-2, s2^-2) R^T.
Pins: points placed on the site's ellipse by float64 geometry; the special
cases that reduce to the ordinary Voronoi diagram (k nearest neighbours from
scipy's cKDTree) and to the Apollonius diagram; exact symmetries of the
formula; and the tie-break by site index.
"""
import math

import numpy as np
import pytest
from scipy.spatial import cKDTree

import synth


def _derived_one(ref, x, y, logtau, r, theta, s1, s2, col=(0.5, 0.5, 0.5)):
    p = np.zeros((1, 12), np.float32)
    p[0, :10] = [x, y, logtau, r, *col, theta, math.log(s1), math.log(s2)]
    return ref.prepare_sites(p), p


def test_ellipse_boundary(ref):
    """A point at p + rho * r * R(theta) (s1 cos phi, s2 sin phi) has
    ||x - p||_G = rho * r, so l = -tau * r * (rho - 1)."""
    rng = np.random.default_rng(11)
    for _ in range(300):
        x, y = rng.uniform(20, 40, 2)
        theta = rng.uniform(-3, 3)
        s1, s2 = np.exp(rng.uniform(np.log(0.5), np.log(16), 2))
        r = rng.uniform(0.5, 2.0)
        logtau = rng.uniform(np.log(0.5), np.log(20))
        d, p = _derived_one(ref, x, y, logtau, r, theta, s1, s2)
        # geometry in float64 from the float32 parameters the oracle sees
        xs, ys, th = float(p[0, 0]), float(p[0, 1]), float(p[0, 7])
        S1, S2 = math.exp(float(p[0, 8])), math.exp(float(p[0, 9]))
        tau = math.exp(float(p[0, 2]))
        rr = float(p[0, 3])
        for rho in (0.25, 1.0, 1.7):
            phi = rng.uniform(0, 2 * np.pi)
            u, v = S1 * rho * rr * math.cos(phi), S2 * rho * rr * math.sin(phi)
            qx = xs + math.cos(th) * u - math.sin(th) * v
            qy = ys + math.sin(th) * u + math.cos(th) * v
            qx32, qy32 = np.float32(qx), np.float32(qy)
            # exact logit at the float32 point, in float64
            dx, dy = float(qx32) - xs, float(qy32) - ys
            a = (dx * math.cos(th) + dy * math.sin(th)) / S1
            b = (-dx * math.sin(th) + dy * math.cos(th)) / S2
            want = -tau * (math.hypot(a, b) - rr)
            got = ref.score(d, 0, float(qx32), float(qy32))
            assert abs(want - (-tau * rr * (rho - 1))) < 1e-4 * tau * rr * max(rho, 1) + 1e-5 * tau * 40 / min(S1, S2)
            assert abs(got - want) <= 2e-6 * tau * (abs(a) + abs(b) + rr) * 4 + 1e-6, (got, want)


def test_isotropic_zero_radius_is_ordinary_voronoi(ref):
    """s1 = s2, r = 0, equal tau: the top-K lists are the K nearest sites by
    Euclidean distance (the ordinary Voronoi diagram of Sec. 3 and its
    K-th order refinement)."""
    h, w, n = 40, 56, 120
    rng = np.random.default_rng(3)
    p = np.zeros((n, 12), np.float32)
    p[:, 0] = rng.uniform(0, w, n)
    p[:, 1] = rng.uniform(0, h, n)
    p[:, 2] = 0.7
    p[:, 3] = 0.0
    p[:, 4:7] = rng.uniform(0, 1, (n, 3))
    p[:, 7] = rng.uniform(0, np.pi, n)  # rotation is irrelevant when isotropic
    p[:, 8] = p[:, 9] = np.log(3.0)
    d = ref.prepare_sites(p)
    topk = ref.brute_topk(d, h, w)
    tree = cKDTree(p[:, :2].astype(np.float64))
    yy, xx = np.mgrid[0:h, 0:w]
    pts = np.stack([xx.ravel() + 0.5, yy.ravel() + 0.5], 1)
    dist, idx = tree.query(pts, k=9)
    checked = 0
    for t in range(pts.shape[0]):
        # skip pixels where the 8th and 9th distances are too close to call
        if dist[t, 8] - dist[t, 7] < 1e-4 * dist[t, 8]:
            continue
        got = topk.reshape(-1, 8)[t]
        assert set(got.tolist()) == set(idx[t, :8].tolist())
        # the ordering is by distance (ties aside)
        order = np.argsort(dist[t, :8], kind="stable")
        gaps = np.diff(dist[t, :8])
        if np.all(gaps > 1e-4 * dist[t, 8]):
            assert got.tolist() == idx[t, :8][order].tolist()
        checked += 1
    assert checked > 0.95 * pts.shape[0]


def test_apollonius_isotropic_radius(ref):
    """Isotropic unit scales and equal tau: ranking by ||x - p|| - r
    (the additively weighted diagram of Sec. 3)."""
    h, w, n = 24, 30, 60
    rng = np.random.default_rng(5)
    p = np.zeros((n, 12), np.float32)
    p[:, 0] = rng.uniform(0, w, n)
    p[:, 1] = rng.uniform(0, h, n)
    p[:, 2] = 1.3
    p[:, 3] = rng.uniform(0, 6, n)
    p[:, 7] = rng.uniform(0, np.pi, n)
    d = ref.prepare_sites(p)
    topk = ref.brute_topk(d, h, w)
    for j in range(h):
        for i in range(w):
            sc = np.hypot(i + 0.5 - p[:, 0].astype(np.float64), j + 0.5 - p[:, 1].astype(np.float64)) - p[:, 3]
            order = np.argsort(sc, kind="stable")
            if sc[order[8]] - sc[order[7]] < 1e-4:
                continue
            assert set(topk[j, i].tolist()) == set(order[:8].tolist())


def test_exact_symmetries(ref):
    """Rotating by pi (cos, sin -> -cos, -sin) and rotating by pi/2 while
    swapping the two scales leave the float32 logit bit-identical."""
    p = synth.sites(21, 50, 32, 32)
    d = ref.prepare_sites(p)
    d_pi = d.copy()
    d_pi[:, 4:6] = -d[:, 4:6]
    d_sw = d.copy()
    d_sw[:, 4], d_sw[:, 5] = -d[:, 5], d[:, 4]
    d_sw[:, 6], d_sw[:, 7] = d[:, 7], d[:, 6]
    rng = np.random.default_rng(0)
    for _ in range(500):
        i = int(rng.integers(50))
        px, py = (float(v) for v in rng.uniform(0, 32, 2).astype(np.float32))
        s = ref.score(d, i, px, py)
        assert s == ref.score(d_pi, i, px, py)
        assert s == ref.score(d_sw, i, px, py)


def test_scale_absorbed_by_tau(ref):
    """Scaling both metric scales by lam, r by 1/lam and tau by lam leaves the
    logit unchanged (Sec. 4.1: a constant scale is absorbed into tau)."""
    p = synth.sites(22, 40, 32, 32)
    q = p.copy()
    lam = 2.0  # powers of two keep the float32 parameters exact
    q[:, 8:10] += np.float32(math.log(lam))
    q[:, 3] /= lam
    q[:, 2] += np.float32(math.log(lam))
    d, e = ref.prepare_sites(p), ref.prepare_sites(q)
    for i in range(40):
        for (px, py) in ((3.5, 7.5), (20.5, 11.5), (31.5, 0.5)):
            a, b = ref.score(d, i, px, py), ref.score(e, i, px, py)
            assert abs(a - b) <= 1e-5 * (abs(a) + d[i, 2] * d[i, 3]) + 1e-5


def test_tie_break_by_site_index(ref):
    """Identical sites have identical logits; the lower index ranks first."""
    p = synth.sites(23, 20, 16, 16)
    p[13] = p[4]
    p[17] = p[4]
    d = ref.prepare_sites(p)
    topk = ref.brute_topk(d, 16, 16)
    for lst in topk.reshape(-1, 8):
        lst = lst.tolist()
        for a, b in ((4, 13), (13, 17)):
            if b in lst:
                assert a in lst and lst.index(a) + 1 == lst.index(b)


def test_brute_topk_lists_are_sorted_distinct_and_padded(ref):
    p = synth.sites(24, 5, 12, 12)
    p[2, 0] = -1.0  # inactive: never listed
    d = ref.prepare_sites(p)
    topk = ref.brute_topk(d, 12, 12)
    for j in range(12):
        for i in range(12):
            lst = topk[j, i].tolist()
            assert lst[4:] == [ref.NONE] * 4 and 2 not in lst
            sc = [ref.score(d, k, i + 0.5, j + 0.5) for k in lst[:4]]
            assert sc == sorted(sc, reverse=True)
            assert len(set(lst[:4])) == 4


def test_tie_break_independent_of_candidate_order(ref):
    """Candidates arriving in descending id order (from a previous list) are
    still ranked lower id first when their logits tie."""
    p = synth.sites(25, 12, 8, 8)
    p[9] = p[2]
    p[5] = p[2]
    d = ref.prepare_sites(p)
    prev = np.full((8, 8, 8), ref.NONE, np.uint32)
    prev[..., :3] = [9, 5, 2]
    out = ref.propagate(d, 8, 8, prev, 1, 0, 0, 0)
    assert np.all(out[..., :3] == np.array([2, 5, 9], np.uint32))
