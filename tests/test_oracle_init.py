"""Pins of the oracle's gradient-weighted initialisation (Sec. 4.4, the
density P_init mixing the normalised gradient magnitude with the uniform
density by lambda_init).

The gradient magnitude is checked against scipy.ndimage.sobel (float64,
borders repeated); single draws against a restatement with Python integers
(prefix sums, the 128-bit product, the search) on the oracle's own float32
magnitudes; the histogram of many draws against P_init computed in float64
from scipy's derivatives (chi-square); special cases: lambda = 1 and a flat
image give the uniform density, lambda = 0 never leaves the support of the
gradient; the records carry the sampled pixel's colour and the given values.
"""
import math

import numpy as np
import pytest
from scipy import ndimage, stats

import synth


def scipy_grad(t):
    t = t.astype(np.float64)
    acc = np.zeros(t.shape[:2])
    for c in range(3):
        gx = ndimage.sobel(t[..., c], axis=1, mode="nearest")
        gy = ndimage.sobel(t[..., c], axis=0, mode="nearest")
        acc += gx * gx + gy * gy
    return np.sqrt(acc)


def p_init(t, lam):
    g = scipy_grad(t)
    h, w = g.shape
    return (1 - lam) * g / g.sum() + lam / (h * w)


@pytest.mark.parametrize("h,w", [(23, 31), (1, 9), (8, 1), (1, 1)])
def test_gradient_magnitude_is_the_sobel_norm(ref, h, w):
    t = np.random.default_rng(h * 100 + w).random((h, w, 3)).astype(np.float32)
    g = ref.grad_mag(t, h, w)
    np.testing.assert_allclose(g, scipy_grad(t), rtol=2e-6, atol=1e-6)


def test_gradient_of_a_ramp(ref):
    """Interior pixels of I = a x + b y (each channel) have |grad| = 8 sqrt(3 (a^2 + b^2))."""
    h, w, a, b = 12, 15, 0.03, -0.02
    jj, ii = np.mgrid[0:h, 0:w]
    t = np.repeat((a * ii + b * jj + 0.5)[..., None], 3, axis=-1).astype(np.float32)
    g = ref.grad_mag(t, h, w)
    np.testing.assert_allclose(g[1:-1, 1:-1], 8 * math.sqrt(3 * (a * a + b * b)), rtol=1e-4)


def restated_draw(ref, g, lam, seed, s):
    h, w = g.shape
    units = [ref.grad_units(v) for v in g.ravel()]
    cum, tot = [], 0
    for u in units:
        tot += u
        cum.append(tot)
    z = [ref.splitmix64(seed, 4 * s + k) for k in range(4)]
    if float(np.float32(z[0] >> 40) * np.float32(2.0 ** -24)) < lam or tot == 0:
        x = ((z[1] >> 32) * h * w) >> 32
    else:
        t = (z[1] * tot) >> 64
        x = next(k for k, c in enumerate(cum) if c > t)
    return x % w, x // w, z


@pytest.mark.parametrize("lam", [0.0, 0.25, 1.0])
def test_single_draws_restated(ref, lam):
    h, w, n, seed = 9, 13, 300, 77
    t = synth.target_polygons(5, h, w, n_poly=3).astype(np.float32)
    g = ref.grad_mag(t, h, w)
    p, d = ref.init_sites(t, h, w, n, lam, seed, log_tau=0.5, r=0.25, log_scale=-0.3)
    for s in range(n):
        i, j, z = restated_draw(ref, g, lam, seed, s)
        fx = np.float32(i) + np.float32(z[2] >> 40) * np.float32(2.0 ** -24)
        fy = np.float32(j) + np.float32(z[3] >> 40) * np.float32(2.0 ** -24)
        assert (p[s, 0], p[s, 1]) == (fx, fy), s
        assert np.array_equal(p[s, 4:7], t[j, i]), s
    assert (p[:, 2] == np.float32(0.5)).all() and (p[:, 3] == np.float32(0.25)).all()
    assert (p[:, 7] == 0).all() and (p[:, 8:10] == np.float32(-0.3)).all() and (p[:, 10:] == 0).all()
    assert np.array_equal(d, ref.prepare_sites(p))


@pytest.mark.parametrize("lam", [0.0, 0.3, 1.0])
def test_histogram_follows_p_init(ref, lam):
    h, w, n = 12, 16, 120_000
    t = synth.target_polygons(8, h, w, n_poly=4).astype(np.float32)
    p, _ = ref.init_sites(t, h, w, n, lam, 1234 + int(lam * 10))
    cell = np.floor(p[:, 1]).astype(int) * w + np.floor(p[:, 0]).astype(int)
    count = np.bincount(cell, minlength=h * w)
    expect = p_init(t, lam).ravel() * n
    keep = expect > 0
    assert count[~keep].sum() == 0
    chi2 = (((count - expect) ** 2)[keep] / expect[keep]).sum()
    assert stats.chi2.sf(chi2, keep.sum() - 1) > 1e-4, chi2


def test_lambda_zero_stays_on_the_gradient(ref):
    h, w = 20, 20
    t = np.zeros((h, w, 3), np.float32)
    t[5:8, 9:12] = 1.0  # gradient only within one pixel of the square
    p, _ = ref.init_sites(t, h, w, 5000, 0.0, 9)
    g = scipy_grad(t)
    cells = np.floor(p[:, :2]).astype(int)
    assert (g[cells[:, 1], cells[:, 0]] > 0).all()


def test_flat_image_samples_uniformly(ref):
    h, w, n = 7, 11, 77_000
    t = np.full((h, w, 3), 0.4, np.float32)
    p, _ = ref.init_sites(t, h, w, n, 0.0, 3)
    cell = np.floor(p[:, 1]).astype(int) * w + np.floor(p[:, 0]).astype(int)
    count = np.bincount(cell, minlength=h * w)
    assert stats.chisquare(count).pvalue > 1e-4
    assert (p[:, 0] >= 0).all() and (p[:, 0] <= w).all() and (p[:, 1] >= 0).all() and (p[:, 1] <= h).all()


def test_grad_units():
    import oracle as ref

    assert ref.grad_units(0.0) == 0
    assert ref.grad_units(1.0) == 1 << 24
    assert ref.grad_units(2.0 ** -25) == 0
    assert ref.grad_units(1e9) == 1 << 32
    assert ref.grad_units(float("nan")) == 0


def test_draws_with_a_few_gradient_units(ref):
    """Gradients of a few units of 2^-24: the total is small, so the draw's
    t often equals a prefix sum, and pixels of zero weight sit between the
    others; a draw must never land on them (lambda = 0)."""
    h, w, n, seed = 10, 12, 2000, 5
    t = np.zeros((h, w, 3), np.float32)
    t[4, 6, 0] = 2.0 ** -22
    t[7, 2, 1] = 2.0 ** -23
    g = ref.grad_mag(t, h, w)
    units = np.array([ref.grad_units(v) for v in g.ravel()]).reshape(h, w)
    assert 0 < units.sum() < 200 and (units == 0).any()
    p, _ = ref.init_sites(t, h, w, n, 0.0, seed)
    cells = np.floor(p[:, :2]).astype(int)
    assert (units[cells[:, 1], cells[:, 0]] > 0).all()
    for s in range(0, n, 10):
        i, j, _ = restated_draw(ref, g, 0.0, seed, s)
        assert (cells[s, 0], cells[s, 1]) == (i, j), s
