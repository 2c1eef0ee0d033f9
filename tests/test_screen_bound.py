"""The propagation pass's screen of queued neighbour ids (may_rank_before in
sad_propagate.h), restated on the CPU: it drops a candidate only when its
approximate logit l' (fused multiply-adds, the hardware square root) plus the
bound M lies below the list's 8th logit, which is safe when the float32
logit l of the ranking (sad_device.h `logit`: one rounding per operation,
correctly rounded square root) satisfies l <= l' + M.  This checks
|l - l'| <= M on adversarial inputs (offsets that cancel, anisotropy far
beyond the workloads', tiny and huge offsets, subnormal q), with the fused
multiply-adds rounded exactly and the hardware root taken as any of the three
float32 values within one ulp of the correctly rounded root (the accuracy a
run over every float32 input measured on the MI355X)."""
from fractions import Fraction as Fr

import numpy as np

f32 = np.float32


def rn32(x: Fr) -> np.float32:
    """x rounded to the nearest float32 (ties to even), from the exact value."""
    f = f32(float(x))  # within one float32 step of the answer (double rounding)
    cands = [np.nextafter(f, f32(-np.inf)), f, np.nextafter(f, f32(np.inf))]
    best = None
    for c in cands:
        if not np.isfinite(c):
            continue
        d = abs(Fr(float(c)) - x)
        key = (d, int(c.view(np.uint32)) & 1)  # nearer first, then the even significand
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def fma(a, b, c) -> np.float32:
    return rn32(Fr(float(a)) * Fr(float(b)) + Fr(float(c)))


def exact_logit(g, px, py) -> np.float32:
    x, y, tau, r, c, s, i1, i2 = (f32(v) for v in g)
    dx = f32(px) - x
    dy = f32(py) - y
    a = (dx * c + dy * s) * i1
    b = (dy * c - dx * s) * i2
    q = a * a + b * b
    d = np.sqrt(q) - r
    return -(tau * d)


def screen(g, px, py):
    """l' and M of may_rank_before, for each hardware root within one ulp."""
    x, y, tau, r, c, s, i1, i2 = (f32(v) for v in g)
    dx = f32(px) - x
    dy = f32(py) - y
    a = fma(dx, c, dy * s) * i1
    b = fma(dy, c, -(dx * s)) * i2
    q = fma(a, a, b * b)
    root = f32(np.sqrt(q))
    out = []
    for sq in (np.nextafter(root, f32(-np.inf)), root, np.nextafter(root, f32(np.inf))):
        if sq < 0:
            continue
        l_ = tau * (r - sq)
        T = (abs(dx) + abs(dy)) * (i1 + i2)
        M = tau * fma(f32(2.0 ** -20), fma(f32(2.0), sq + abs(r), T), f32(2.0 ** -60))
        out.append((l_, M))
    return out


def site(rng, px, py, kind):
    th = rng.uniform(-4, 4)
    ls1, ls2 = rng.uniform(-4, 6, 2)
    if kind == "aniso":
        ls1, ls2 = -4.0, 7.0  # anisotropy e^11
    tau = np.exp(rng.uniform(-6, 6))
    r = rng.uniform(-4, 12)
    off = {"near": 10.0, "far": 3000.0, "tiny": 1e-3, "sub": 1e-21}.get(kind, 50.0)
    x = px + rng.uniform(-off, off)
    y = py + rng.uniform(-off, off)
    if kind == "zero":
        x, y = px, py
    return (x, y, tau, r, np.cos(th), np.sin(th), np.exp(-ls1), np.exp(-ls2))


def test_screen_bound_holds():
    rng = np.random.default_rng(7)
    worst = 0.0
    kinds = ["near", "far", "tiny", "sub", "aniso", "zero", "mid"]
    for t in range(4200):
        kind = kinds[t % len(kinds)]
        px = float(rng.integers(0, 8192)) + 0.5
        py = float(rng.integers(0, 8192)) + 0.5
        g = site(rng, px, py, kind)
        l = exact_logit(g, px, py)
        assert np.isfinite(l)
        for l_, M in screen(g, px, py):
            assert np.isfinite(l_) and np.isfinite(M) and M > 0
            err = abs(Fr(float(l)) - Fr(float(l_)))
            ratio = float(err / Fr(float(M)))
            worst = max(worst, ratio)
            assert ratio <= 1.0, (kind, g, px, py, l, l_, M)
    # the bound is several times the largest error seen, not a tight fit
    assert worst < 0.5, worst


def test_screen_bound_on_cancelling_offsets():
    """Offsets along the direction where dx cos + dy sin cancels (a near 0)
    and the other axis strongly scaled: the error of a is absolute, not
    relative to a."""
    rng = np.random.default_rng(11)
    for _ in range(600):
        th = rng.uniform(0, np.pi)
        c, s = np.cos(th), np.sin(th)
        px, py = float(rng.integers(0, 4096)) + 0.5, float(rng.integers(0, 4096)) + 0.5
        t = rng.uniform(1, 500)
        x, y = px + s * t, py - c * t  # (dx, dy) = -t (s, -c): a cancels
        g = (x, y, np.exp(rng.uniform(-3, 3)), rng.uniform(0, 3), c, s, np.exp(rng.uniform(-1, 8)),
             np.exp(rng.uniform(-8, 1)))
        l = exact_logit(g, px, py)
        for l_, M in screen(g, px, py):
            assert abs(Fr(float(l)) - Fr(float(l_))) <= Fr(float(M))
