"""Pins of the oracle's packed evaluation records (Appendix B.2, "Packed
storage for evaluation") and of random access from them (Sec. 6.6).

float16 rounding is checked against numpy's float16 conversion; the bit
layout against codes recomputed in float64 with numpy; the per-image ranges
against numpy minima and maxima; the reparameterisation (determinant-1
metric with log tau' and r') by comparing logits of decoded records with the
logit of the original site written out in float64 from its angle and two
scales, on a small image where the codes are fine; angle codes modulo the
metric's period; queries against the float32-record query (already pinned)
within the quantisation's effect, and special cases (one colour everywhere,
a dominant temperature, stale ids, non-finite points).
"""
import math

import numpy as np
import pytest

import synth


def test_half_bits_match_numpy(ref):
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32)
    vals = bits.view(np.float32)
    special = np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, -65520.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26,
                        2.0 ** -14, 2.0 ** -14 * (1 - 2 ** -12), 1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11, np.inf, -np.inf,
                        0.1, -0.75, 1e-8, 6.1e-5], np.float32)
    small = (rng.random(5000) * 2.0 ** -13).astype(np.float32)
    for v in np.concatenate([vals[np.isfinite(vals)], special, small]):
        with np.errstate(over="ignore"):  # overflow to infinity is the expected result
            want = int(np.array(v, np.float32).astype(np.float16).view(np.uint16))
        assert ref.half_bits(v) == want, v
        assert ref.half_value(want) == float(np.array(want, np.uint16).view(np.float16)), want
    assert (ref.half_bits(np.float32("nan")) & 0x7C00) == 0x7C00 and (ref.half_bits(np.float32("nan")) & 0x3FF)


def sites_case(seed, n, h, w, inactive=0.1):
    p = synth.sites(seed, n, h, w)
    p[np.random.default_rng(seed).random(n) < inactive, 0] = -1.0
    return p


def transformed(ref, p):
    """(log tau', r', c_r, c_g, c_b) in float32 with the oracle's operation order."""
    hs = np.float32(0.5) * (p[:, 8] + p[:, 9])
    lt = p[:, 2] - hs
    rr = p[:, 3] * np.array([ref.exp_f32(float(v)) for v in hs], np.float32)
    return np.stack([lt, rr, p[:, 4], p[:, 5], p[:, 6]], axis=1)


def test_ranges_and_layout(ref):
    h, w, n = 48, 64, 400
    p = sites_case(3, n, h, w)
    d = ref.prepare_sites(p)
    pk, qp = ref.pack_sites(p, d, h, w)
    use = d[:, 0] >= 0
    v = transformed(ref, p)[use]
    assert np.array_equal(qp[0::2], v.min(0)) and np.array_equal(qp[1::2], v.max(0) - v.min(0))
    assert (pk[~use] == 0).all() and (pk[use, 0] >> 31 == 1).all()
    pu = p[use].astype(np.float64)
    vv = v.astype(np.float64)
    th = np.mod(pu[:, 7] + np.pi, 2 * np.pi) - np.pi
    fields = [
        (pk[use, 0] & 32767, pu[:, 0] / w * 32767),
        ((pk[use, 0] >> 15) & 32767, pu[:, 1] / h * 32767),
        (pk[use, 1] & 2047, (vv[:, 2] - qp[4]) / qp[5] * 2047),
        ((pk[use, 1] >> 11) & 2047, (vv[:, 3] - qp[6]) / qp[7] * 2047),
        (pk[use, 1] >> 22, (vv[:, 4] - qp[8]) / qp[9] * 1023),
        (pk[use, 2] & 65535, (vv[:, 0] - qp[0]) / qp[1] * 65535),
        (pk[use, 2] >> 16, (vv[:, 1] - qp[2]) / qp[3] * 65535),
        (pk[use, 3] & 65535, (th + np.pi) / (2 * np.pi) * 65535),
    ]
    for k, (got, want) in enumerate(fields):
        assert (np.abs(got.astype(np.float64) - want) <= 0.5 + 0.01).all(), k  # float32 rounding of t * maxq
    a = (pk[use, 3] >> 16).astype(np.uint16).view(np.float16).astype(np.float64)
    assert np.array_equal(a, (p[use, 9] - p[use, 8]).astype(np.float16).astype(np.float64))


def original_logit(p, px, py):
    """The logit of a site written out in float64 from its angle and two scales."""
    x, y, lt, r, th, l1, l2 = (float(p[k]) for k in (0, 1, 2, 3, 7, 8, 9))
    dx, dy = px - x, py - y
    u = math.cos(th) * dx + math.sin(th) * dy
    v = -math.sin(th) * dx + math.cos(th) * dy
    return -math.exp(lt) * (math.sqrt(u * u * math.exp(-2 * l1) + v * v * math.exp(-2 * l2)) - r)


def test_decoded_logit_is_the_original(ref):
    """On an 8x8 image (positions in steps of 1/4096 px) with log tau', r' in
    narrow ranges and log-anisotropies exact in float16, a decoded record's
    logit is the original site's up to the codes' resolution."""
    h = w = 8
    rng = np.random.default_rng(5)
    n = 60
    p = np.zeros((n, 12), np.float32)
    p[:, 0] = rng.uniform(0, w, n)
    p[:, 1] = rng.uniform(0, h, n)
    p[:, 8] = rng.choice([0.25, 0.5, 1.0, -0.5], n)
    p[:, 9] = rng.choice([0.25, 0.75, 1.5, 0.0], n)
    hs = 0.5 * (p[:, 8] + p[:, 9])
    p[:, 2] = (0.3 + hs + rng.uniform(0, 0.01, n)).astype(np.float32)  # log tau' in [0.3, 0.31]
    p[:, 3] = (rng.uniform(1.0, 1.01, n) * np.exp(-hs)).astype(np.float32)  # r' near [1, 1.01]
    p[:, 4:7] = rng.random((n, 3))
    p[:, 7] = rng.uniform(-6, 6, n)
    d = ref.prepare_sites(p)
    pk, qp = ref.pack_sites(p, d, h, w)
    worst = 0.0
    for i in range(n):
        v = ref.unpack_site(pk[i], qp, h, w)
        assert abs(v[8] - (p[i, 9] - p[i, 8])) == 0.0
        for px, py in rng.uniform(0, w, (20, 2)):
            a, b = ref.packed_logit(v, px, py), original_logit(p[i], px, py)
            worst = max(worst, abs(a - b))
    assert worst < 2e-3, worst


def test_angle_codes_respect_the_metric_period(ref):
    h = w = 16
    p = sites_case(9, 40, h, w, inactive=0.0)
    d = ref.prepare_sites(p)
    pk, qp = ref.pack_sites(p, d, h, w)
    base = [ref.unpack_site(pk[i], qp, h, w) for i in range(len(p))]
    for shift in (math.pi, 2 * math.pi, -3 * math.pi):
        p2 = p.copy()
        p2[:, 7] = (p[:, 7].astype(np.float64) + shift).astype(np.float32)
        pk2, qp2 = ref.pack_sites(p2, ref.prepare_sites(p2), h, w)
        for i in range(len(p)):
            v2 = ref.unpack_site(pk2[i], qp2, h, w)
            for px, py in ((3.3, 4.1), (12.0, 0.5), (8.5, 15.2)):
                b = ref.packed_logit(base[i], px, py)
                # a shift by pi moves the code by half a step: the logit moves by that angle
                assert abs(ref.packed_logit(v2, px, py) - b) < 2e-3 * max(1.0, abs(b))


@pytest.fixture(scope="module")
def c1_packed(ref):
    wl = synth.C1
    p = wl.make_sites()
    p[3, 0] = -1.0
    d = ref.prepare_sites(p)
    m = ref.brute_topk(d, wl.h, wl.w)
    pk, qp = ref.pack_sites(p, d, wl.h, wl.w)
    return wl, p, d, m, pk, qp


def test_query_packed_follows_the_float_records(ref, c1_packed):
    wl, p, d, m, pk, qp = c1_packed
    xy = synth.queries(11, 4000, wl.h, wl.w)
    a = ref.query_packed(pk, qp, wl.h, wl.w, m, xy)
    b = ref.query_points(d, wl.h, wl.w, m, xy)
    err = np.abs(a - b)
    assert err.max() < 0.05 and np.median(err) < 2e-3, (err.max(), np.median(err))


def test_query_packed_special_cases(ref, c1_packed):
    wl, p, d, m, pk, qp = c1_packed
    # one colour everywhere: every covered query returns the decoded colour
    p1 = p.copy()
    p1[:, 4:7] = [0.2, 0.5, 0.9]
    pk1, qp1 = ref.pack_sites(p1, ref.prepare_sites(p1), wl.h, wl.w)
    xy = synth.queries(12, 500, wl.h, wl.w)
    out = ref.query_packed(pk1, qp1, wl.h, wl.w, m, xy)
    np.testing.assert_allclose(out, np.tile(np.float32([0.2, 0.5, 0.9]), (500, 1)), atol=1e-7)
    # stale ids and unusable entries are skipped; a list of only those renders black
    m2 = m.copy()
    m2[0, 0] = [3, 999, 3, 0xFFFFFFFF, 3, 1000, 3, 3]
    got = ref.query_packed(pk, qp, wl.h, wl.w, m2, np.float32([[0.5, 0.5], [np.nan, 1.0], [-5.0, -5.0]]))
    assert (got[0] == 0).all() and np.isnan(got[1]).all() and (got[2] == 0).all()
    # a dominant temperature: the top entry's decoded colour
    p3 = p.copy()
    p3[:, 2] = 8.0
    d3 = ref.prepare_sites(p3)
    pk3, qp3 = ref.pack_sites(p3, d3, wl.h, wl.w)
    for j, i in ((20, 30), (5, 60), (63, 0)):
        vals = [ref.unpack_site(pk3[s], qp3, wl.h, wl.w) for s in m[j, i] if s < len(p) and d3[s, 0] >= 0]
        lg = [ref.packed_logit(v, i + 0.5, j + 0.5) for v in vals]
        out = ref.query_packed(pk3, qp3, wl.h, wl.w, m, np.float32([[i + 0.5, j + 0.5]]))[0]
        np.testing.assert_allclose(out, vals[int(np.argmax(lg))][4:7], atol=1e-6)
