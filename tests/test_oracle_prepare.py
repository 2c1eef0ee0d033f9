"""Pins for the oracle's site preparation (paper Sec. 4.1: tau = exp(log tau),
the metric's rotation and inverse scales).

The oracle promises the float32 nearest to the exact value of exp, cos and
sin.  mpmath (arbitrary precision, independent of the C library) decides what
that float is.
"""
import math

import mpmath
import numpy as np
import pytest

import synth

mpmath.mp.prec = 200


def nearest_f32(v: mpmath.mpf) -> np.float32:
    """Round-to-nearest-even of an exact real to float32, decided in mpmath."""
    f = np.float32(float(v))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    best = None
    for c in cands:
        if not np.isfinite(c):
            continue
        err = abs(mpmath.mpf(float(c)) - v)
        key = (err, int(np.array(c, dtype=np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def f32_values(seed, count, lo, hi):
    rng = np.random.default_rng(seed)
    return rng.uniform(lo, hi, count).astype(np.float32)


@pytest.mark.parametrize("fname,lo,hi", [("exp", -20.0, 20.0), ("exp", -103.0, 88.0),
                                         ("cos", -7.0, 7.0), ("sin", -7.0, 7.0),
                                         ("cos", -300.0, 300.0), ("sin", -300.0, 300.0)])
def test_correctly_rounded_against_mpmath(ref, fname, lo, hi):
    xs = f32_values(int(abs(lo) * 10) + len(fname), 1500, lo, hi)
    fn = {"exp": ref.exp_f32, "cos": ref.cos_f32, "sin": ref.sin_f32}[fname]
    mfn = {"exp": mpmath.exp, "cos": mpmath.cos, "sin": mpmath.sin}[fname]
    for x in xs:
        got = np.float32(fn(float(x)))
        want = nearest_f32(mfn(mpmath.mpf(float(x))))
        assert got == want or (got == 0 and want == 0), (fname, float(x), got, want)
    assert ref.ambiguous_count() == 0


def test_special_values(ref):
    assert ref.exp_f32(0.0) == 1.0
    assert ref.cos_f32(0.0) == 1.0 and ref.sin_f32(0.0) == 0.0
    assert math.isinf(ref.exp_f32(89.0))  # exp(89) > FLT_MAX
    assert ref.exp_f32(-104.0) == 0.0  # below half the smallest subnormal
    # a subnormal result, rounded correctly
    x = np.float32(-95.5)
    assert np.float32(ref.exp_f32(float(x))) == nearest_f32(mpmath.exp(mpmath.mpf(float(x))))
    # values the site recipes produce: log-scales of 0.5..16 px and tau of 0.5..20
    for s in (0.5, 1.0, 2.0, 8.0, 16.0):
        ls = np.float32(math.log(s))
        assert np.float32(ref.exp_f32(float(-ls))) == nearest_f32(mpmath.exp(-mpmath.mpf(float(ls))))


def test_prepared_record_layout(ref):
    p = synth.sites(7, 64, 32, 48)
    p[5, 0] = -1.0  # inactive site (Appendix B.2: x < 0)
    p[6, 7] = 3.0e6  # rotation beyond the supported range -> inactive
    d = ref.prepare_sites(p)
    for i in (0, 1, 17, 63):
        assert d[i, 0] == p[i, 0] and d[i, 1] == p[i, 1]
        assert d[i, 2] == ref.exp_f32(float(p[i, 2]))
        assert d[i, 3] == p[i, 3]
        assert d[i, 4] == ref.cos_f32(float(p[i, 7])) and d[i, 5] == ref.sin_f32(float(p[i, 7]))
        assert d[i, 6] == ref.exp_f32(float(-p[i, 8])) and d[i, 7] == ref.exp_f32(float(-p[i, 9]))
        assert np.array_equal(d[i, 8:11], p[i, 4:7]) and d[i, 11] == 0.0
    assert d[5, 0] < 0 and d[6, 0] < 0
    # tau and the inverse scales agree with float64 math to float32 precision
    assert np.allclose(d[:, 2], np.exp(p[:, 2].astype(np.float64)), rtol=1e-7)
    assert np.allclose(d[:, 6], np.exp(-p[:, 8].astype(np.float64)), rtol=1e-7)
