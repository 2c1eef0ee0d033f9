"""Pins for the oracle's render, random-access query, hand-derived gradients
and Adam step (paper Sec. 4.2 softmax blend, Table 1 convexity / partition of
unity, Sec. 6.6 random access, Appendix B.4 gradients, Sec. 5 Adam).

The gradients are pinned against torch.autograd (float64, CPU) applied to the
forward written with torch operations, and against central finite
differences of the oracle's own forward; Adam against torch.optim.Adam.
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import expit

import synth


def _small(ref, seed=41, n=24, h=13, w=17):
    p = synth.sites(seed, n, h, w)
    d = ref.prepare_sites(p)
    topk = ref.brute_topk(d, h, w)
    return p, d, topk, h, w


def test_partition_of_unity_and_convexity(ref):
    p, d, topk, h, w = _small(ref)
    d1 = d.copy()
    d1[:, 8:11] = 1.0
    img1 = ref.render_fwd(d1, h, w, topk)
    assert np.allclose(img1, 1.0, atol=1e-14, rtol=0)  # weights sum to one
    img = ref.render_fwd(d, h, w, topk)
    for j in range(h):
        for i in range(w):
            cols = d[topk[j, i], 8:11].astype(np.float64)
            assert np.all(img[j, i] >= cols.min(0) - 1e-14) and np.all(img[j, i] <= cols.max(0) + 1e-14)


def test_two_site_logistic(ref):
    """With two entries the weight of the first is the logistic function of
    the logit difference."""
    p, d, topk, h, w = _small(ref)
    two = np.full_like(topk, ref.NONE)
    two[..., 0] = 3
    two[..., 1] = 11
    img = ref.render_fwd(d, h, w, two)
    for j in range(h):
        for i in range(w):
            l0 = ref.score(d, 3, i + 0.5, j + 0.5)
            l1 = ref.score(d, 11, i + 0.5, j + 0.5)
            w0 = expit(float(l0) - float(l1))
            want = w0 * d[3, 8:11].astype(np.float64) + (1 - w0) * d[11, 8:11].astype(np.float64)
            assert np.allclose(img[j, i], want, rtol=0, atol=1e-13)


def test_equal_logits_average_and_hard_limit(ref):
    p, d, topk, h, w = _small(ref)
    # eight copies of one site with different colours: equal logits, w = 1/8
    q = np.repeat(p[:1], 8, axis=0)
    q[:, 4:7] = np.random.default_rng(0).uniform(0, 1, (8, 3)).astype(np.float32)
    dq = ref.prepare_sites(q)
    lists = np.broadcast_to(np.arange(8, dtype=np.uint32), (h, w, 8)).copy()
    img = ref.render_fwd(dq, h, w, lists)
    assert np.allclose(img, q[:, 4:7].astype(np.float64).mean(0), atol=1e-14)
    # tau -> infinity: the blend becomes the top-1 colour (hard Voronoi ownership)
    p2 = p.copy()
    p2[:, 2] += 30.0
    d2 = ref.prepare_sites(p2)
    top = ref.brute_topk(d2, h, w)
    img2 = ref.render_fwd(d2, h, w, top)
    ok = 0
    for j in range(h):
        for i in range(w):
            l = [ref.score(d2, int(s), i + 0.5, j + 0.5) for s in top[j, i][:2]]
            if l[0] - l[1] > 50:
                assert np.array_equal(img2[j, i], d2[top[j, i][0], 8:11].astype(np.float64))
                ok += 1
    assert ok > 0.9 * h * w


def test_empty_list_and_invalid_entries(ref):
    p, d, topk, h, w = _small(ref)
    e = np.full_like(topk, ref.NONE)
    assert np.all(ref.render_fwd(d, h, w, e) == 0.0)
    t2 = topk.copy()
    t2[..., 5:] = ref.NONE
    t3 = t2.copy()
    t3[..., 5] = 999  # out-of-range id: skipped like the sentinel
    assert np.array_equal(ref.render_fwd(d, h, w, t2), ref.render_fwd(d, h, w, t3))


def test_query_at_pixel_centres_equals_render(ref):
    p, d, topk, h, w = _small(ref)
    yy, xx = np.mgrid[0:h, 0:w]
    xy = np.stack([xx.ravel() + 0.5, yy.ravel() + 0.5], 1).astype(np.float32)
    q = ref.query_points(d, h, w, topk, xy)
    assert np.array_equal(q, ref.render_fwd(d, h, w, topk).reshape(-1, 3))
    # points outside the image use the clamped pixel; non-finite points give NaN
    xy2 = np.array([[-3.0, 2.2], [w + 5.0, h + 1.0], [np.nan, 1.0], [1.0, np.inf]], np.float32)
    q2 = ref.query_points(d, h, w, topk, xy2)
    l0 = [int(s) for s in topk[2, 0] if s != ref.NONE]
    sc = np.array([ref.score(d, s, -3.0, np.float32(2.2)) for s in l0], np.float64)
    wts = np.exp(sc - sc.max())
    wts /= wts.sum()
    assert np.allclose(q2[0], (wts[:, None] * d[l0, 8:11]).sum(0), atol=1e-13)
    assert np.all(np.isnan(q2[2:]))


def _torch_loss(params64, lists, target, h, w):
    """The forward of Sec. 4.2 written with torch ops (float64) for autograd."""
    x, y, lt, r = params64[:, 0], params64[:, 1], params64[:, 2], params64[:, 3]
    col = params64[:, 4:7]
    th, l1, l2 = params64[:, 7], params64[:, 8], params64[:, 9]
    tau, cs, sn = torch.exp(lt), torch.cos(th), torch.sin(th)
    is1, is2 = torch.exp(-l1), torch.exp(-l2)
    yy, xx = torch.meshgrid(torch.arange(h, dtype=torch.float64), torch.arange(w, dtype=torch.float64),
                            indexing="ij")
    px, py = (xx + 0.5)[..., None], (yy + 0.5)[..., None]
    ids = torch.as_tensor(lists.astype(np.int64))
    dx, dy = px - x[ids], py - y[ids]
    a = (dx * cs[ids] + dy * sn[ids]) * is1[ids]
    b = (dy * cs[ids] - dx * sn[ids]) * is2[ids]
    logit = -tau[ids] * (torch.sqrt(a * a + b * b) - r[ids])
    wts = torch.softmax(logit, dim=-1)
    img = (wts[..., None] * col[ids]).sum(-2)
    return ((img - torch.as_tensor(target, dtype=torch.float64)) ** 2).sum() / (h * w)


def test_gradients_match_autograd(ref):
    p, d, topk, h, w = _small(ref, seed=43, n=30, h=14, w=18)
    target = synth.target_polygons(5, h, w)
    grad, gabs, loss, img = ref.render_bwd(d, h, w, topk, target)
    P = torch.tensor(p[:, :10].astype(np.float64), requires_grad=True)
    L = _torch_loss(P, topk, target, h, w)
    L.backward()
    auto = P.grad.numpy()
    assert abs(loss - L.item()) <= 1e-6 * L.item()
    # float32 logits in the oracle vs float64 in torch: agreement to ~1e-6 relative
    scale = np.abs(auto).max(0) + 1e-30
    err = np.abs(grad[:, :10] - auto) / scale
    assert err.max() < 2e-5, err.max(0)
    assert np.all(grad[:, 10:] == 0)
    assert np.all(gabs[:, :10] >= np.abs(grad[:, :10]) * (1 - 1e-12))  # the magnitude bounds the value


def test_gradients_match_finite_differences(ref):
    p, d, topk, h, w = _small(ref, seed=44, n=20, h=12, w=12)
    target = synth.target_polygons(6, h, w)
    grad, _, _, _ = ref.render_bwd(d, h, w, topk, target)

    def loss_of(pp):
        dd = ref.prepare_sites(pp)
        img = ref.render_fwd(dd, h, w, topk)
        return float(((img - target.astype(np.float64)) ** 2).sum() / (h * w))

    rng = np.random.default_rng(1)
    for _ in range(25):
        i, k = int(rng.integers(20)), int(rng.integers(10))
        step = {0: 1e-2, 1: 1e-2, 7: 1e-3}.get(k, 1e-3)
        pp, pm = p.copy(), p.copy()
        pp[i, k] += np.float32(step)
        pm[i, k] -= np.float32(step)
        actual = float(pp[i, k]) - float(pm[i, k])
        fd = (loss_of(pp) - loss_of(pm)) / actual
        assert abs(fd - grad[i, k]) <= 2e-2 * abs(grad[i, k]) + 1e-7, (i, k, fd, grad[i, k])


def test_gradient_invariants(ref):
    """Sum over sites of the colour gradients equals the sum over pixels of
    dL/dc (the weights of each list sum to one); the loss is the mean
    squared error of the rendered image."""
    p, d, topk, h, w = _small(ref, seed=45)
    target = synth.target_polygons(7, h, w)
    grad, _, loss, img = ref.render_bwd(d, h, w, topk, target)
    g = 2 * (img - target.astype(np.float64)) / (h * w)
    assert np.allclose(grad[:, 4:7].sum(0), g.reshape(-1, 3).sum(0), rtol=1e-12, atol=1e-15)
    assert abs(loss - ((img - target) ** 2).sum() / (h * w)) < 1e-12
    assert np.array_equal(img, ref.render_fwd(d, h, w, topk))


@pytest.mark.parametrize("b1,b2,rtol", [(0.875, 1 - 2.0 ** -9, 2e-7), (0.9, 0.999, 2e-5)])
def test_adam_against_torch(ref, b1, b2, rtol):
    """torch.optim.Adam with lr = 1 moves each parameter by the unit step
    m_hat / (sqrt(v_hat) + eps); the oracle must move it by that step times
    the rate of its group, then clamp the position into the image.  With
    betas exact in float32 the two agree to float32 rounding; with 0.9/0.999
    the float32 value of 1 - beta differs from torch's float64 one by ~1e-5
    relative, which bounds the unit step's difference."""
    n, h, w = 300, 40, 60
    p = synth.sites(46, n, h, w)
    p[3, 0] = -1.0  # inactive: left as it is
    lr = np.array([1e-2, 2e-3, 3e-3, 4e-3, 5e-3], np.float32)
    group_of = [0, 0, 1, 2, 3, 3, 3, 4, 4, 4]
    eps = 1e-8
    m = np.zeros_like(p)
    v = np.zeros_like(p)
    cur = p.copy()
    tp = torch.zeros((n, 10), dtype=torch.float32, requires_grad=True)
    opt = torch.optim.Adam([tp], lr=1.0, betas=(b1, b2), eps=eps)
    act = np.delete(np.arange(n), 3)
    for t in range(1, 4):
        g = synth.gradients(100 + t, n)
        bc1, bc2 = ref.bias_corrections(b1, b2, t)
        prev = cur.copy()
        cur, gz, m, v, der = ref.adam_step(cur, g, m, v, h, w, lr, b1, b2, eps, bc1, bc2)
        assert np.all(gz == 0)
        assert np.array_equal(der, ref.prepare_sites(cur))
        before = tp.detach().clone()
        tp.grad = torch.tensor(g[:, :10])
        opt.step()
        unit = (before - tp.detach()).numpy().astype(np.float64)
        want = prev[:, :10].astype(np.float64) - unit * lr[group_of].astype(np.float64)
        want[:, 0] = np.clip(want[:, 0], 0, w)
        want[:, 1] = np.clip(want[:, 1], 0, h)
        tol = 4e-7 * np.abs(prev[act, :10]) + rtol * lr[group_of] * np.abs(unit[act]) + 1e-12
        assert np.all(np.abs(cur[act, :10] - want[act]) <= tol)
        assert np.array_equal(cur[3], p[3])


def test_adam_clamps_positions(ref):
    p = synth.sites(47, 4, 10, 10)
    p[0, 0], p[1, 1] = 0.0, 10.0
    g = np.zeros_like(p)
    g[0, 0], g[1, 1] = 1.0, -1.0  # steps push x below 0 and y above H
    lr = np.full(5, 0.5, np.float32)
    bc1, bc2 = ref.bias_corrections(0.9, 0.999, 1)
    out, *_ = ref.adam_step(p, g, np.zeros_like(p), np.zeros_like(p), 10, 10, lr, 0.9, 0.999, 1e-8, bc1, bc2)
    assert out[0, 0] == 0.0 and out[1, 1] == 10.0
