"""Pins of the oracle's per-site budget statistics (Sec. 4.5 "Adaptive
Budget: Densify and Prune"; Appendix B.5 "Densification scores", "Pruning").

Columns: mass sum w, energy sum w |c - I|^2, removal delta, and the weighted
moments sum w dx, sum w dy, sum w dx^2, sum w dx dy, sum w dy^2 of the pixel
offsets from the site.  Each is pinned by something other than its own
formula: the softmax weights form a partition of unity per pixel, the
energies add up to the rendered loss, a site's removal delta is the change of
the squared error when the site is switched off with the lists held fixed
(measured with the separately pinned render), the moments reassemble into the
plain pixel-coordinate sums, and a lone site has closed forms.
"""
import numpy as np
import pytest

import synth


def covered(ref, d, h, w, m):
    """Mask of the pixels whose list has a usable entry."""
    img = ref.render_fwd(d, h, w, m)
    lists = m.reshape(h, w, 8)
    n = d.reshape(-1, 12).shape[0]
    ok = np.zeros((h, w), bool)
    for k in range(8):
        ids = lists[..., k]
        valid = ids < n
        ok |= valid & (d.reshape(-1, 12)[np.minimum(ids, n - 1), 0] >= 0)
    return ok, img


@pytest.fixture(scope="module")
def case(ref):
    """64x64 / 256 sites with the exact top-8 lists, plus a second map that
    has empty lists, stale ids and an inactive site."""
    wl = synth.C1
    p = wl.make_sites()
    p[5, 0] = -1.0
    d = ref.prepare_sites(p)
    t = wl.make_target()
    m = ref.brute_topk(d, wl.h, wl.w)
    rng = np.random.default_rng(3)
    m2 = m.copy()
    m2[rng.random(m2.shape[:2]) < 0.05] = 0xFFFFFFFF
    m2[..., 7][rng.random(m2.shape[:2]) < 0.2] = 5  # the inactive site
    m2[..., 6][rng.random(m2.shape[:2]) < 0.1] = 999  # out of range
    return wl, d, t, [m, m2]


def test_mass_is_a_partition_of_unity(ref, case):
    wl, d, t, maps = case
    for m in maps:
        st, _ = ref.site_stats(d, wl.h, wl.w, m, t)
        ok, _ = covered(ref, d, wl.h, wl.w, m)
        assert abs(st[:, 0].sum() - ok.sum()) < 1e-9 * ok.sum()
        assert (st[:, 0] >= 0).all()


def test_energy_adds_up_to_the_loss(ref, case):
    wl, d, t, maps = case
    for m in maps:
        st, _ = ref.site_stats(d, wl.h, wl.w, m, t)
        ok, img = covered(ref, d, wl.h, wl.w, m)
        err = ((img - t) ** 2).sum(-1)
        assert abs(st[:, 1].sum() - err[ok].sum()) < 1e-9 * err.sum()
        _, _, loss, _ = ref.render_bwd(d, wl.h, wl.w, m, t)
        assert abs(err.sum() - loss * wl.h * wl.w) < 1e-9 * err.sum()


def test_removal_delta_is_the_error_change_without_the_site(ref, case):
    wl, d, t, maps = case
    for m in maps:
        st, _ = ref.site_stats(d, wl.h, wl.w, m, t)
        base = ((ref.render_fwd(d, wl.h, wl.w, m) - t) ** 2).sum()
        listed = np.unique(m[m < 256])
        for site in listed[:: max(1, len(listed) // 12)]:
            d2 = d.reshape(-1, 12).copy()
            d2[site, 0] = -1.0  # switched off: the render skips it, the others renormalise
            without = ((ref.render_fwd(d2, wl.h, wl.w, m) - t) ** 2).sum()
            assert abs(st[site, 2] - (without - base)) < 1e-9 * max(1.0, abs(without - base)), site


def test_moments_reassemble_into_pixel_sums(ref, case):
    wl, d, t, maps = case
    x = d.reshape(-1, 12)[:, 0].astype(np.float64)
    y = d.reshape(-1, 12)[:, 1].astype(np.float64)
    for m in maps:
        st, _ = ref.site_stats(d, wl.h, wl.w, m, t)
        ok, _ = covered(ref, d, wl.h, wl.w, m)
        jj, ii = np.nonzero(ok)
        px, py = ii + 0.5, jj + 0.5
        mass, sx, sy, sxx, sxy, syy = st[:, 0], st[:, 3], st[:, 4], st[:, 5], st[:, 6], st[:, 7]
        # sum over sites of w (p - x_i) shifted back by x_i gives sum over pixels of p
        checks = [
            ((sx + x * mass).sum(), px.sum()),
            ((sy + y * mass).sum(), py.sum()),
            ((sxx + 2 * x * sx + x * x * mass).sum(), (px * px).sum()),
            ((syy + 2 * y * sy + y * y * mass).sum(), (py * py).sum()),
            ((sxy + x * sy + y * sx + x * y * mass).sum(), (px * py).sum()),
        ]
        for got, want in checks:
            assert abs(got - want) < 1e-9 * abs(want), (got, want)


def test_lone_site_closed_forms(ref):
    h, w = 9, 13
    p = synth.sites(5, 1, h, w)
    d = ref.prepare_sites(p)
    t = np.random.default_rng(4).random((h, w, 3)).astype(np.float32)
    m = np.full((h, w, 8), 0xFFFFFFFF, np.uint32)
    m[..., 0] = 0
    st, mag = ref.site_stats(d, h, w, m, t)
    dd = d.reshape(-1, 12)[0].astype(np.float64)
    col = dd[8:11]
    ii, jj = np.meshgrid(np.arange(w) + 0.5, np.arange(h) + 0.5)
    dx, dy = ii - dd[0], jj - dd[1]
    tt = t.astype(np.float64)
    err = ((col - tt) ** 2).sum(-1)
    want = [h * w, err.sum(), ((tt ** 2).sum(-1) - err).sum(),  # removing the only site leaves black
            dx.sum(), dy.sum(), (dx * dx).sum(), (dx * dy).sum(), (dy * dy).sum()]
    np.testing.assert_allclose(st[0], want, rtol=1e-12, atol=1e-9)
    assert (mag[0] >= np.abs(st[0]) - 1e-9).all()
