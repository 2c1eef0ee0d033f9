"""Seeded synthetic inputs for the SAD hot path.

This module only draws numbers: site parameters, target images and query
points, with the shapes and value ranges of the workloads the SAD paper times
(Kodak-sized 768x512 images with 50k sites, 2048^2 images, random-access
decoding).  It holds none of the method's arithmetic, so both the CPU oracle
tests and the HIP path can take their inputs from here.

Site record layout (float32, 12 values per site, 48 bytes):
    0 x, 1 y          position in pixels, image plane [0, W) x [0, H)
    2 log_tau         log temperature
    3 r               additive radius, in the units of the anisotropic norm
    4..6 colour       RGB in [0, 1]
    7 theta           rotation of the metric (radians)
    8 log_s1, 9 log_s2  log scales (pixels) along the rotated axes
    10, 11            padding, always 0

All draws use numpy's PCG64 ``default_rng(seed)`` in float64 and are cast to
float32 at the end.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

PARAM_STRIDE = 12


@dataclass(frozen=True)
class SiteRecipe:
    ls_lo: float  # log-scale range lower end (log pixels)
    ls_hi: float
    r_lo: float = 0.0
    r_hi: float = 2.0
    logtau_lo: float = math.log(0.5)
    logtau_hi: float = math.log(20.0)
    fixed_logtau: float | None = None


SMALL_SCALES = SiteRecipe(ls_lo=math.log(1.0), ls_hi=math.log(8.0))
WIDE_SCALES = SiteRecipe(ls_lo=math.log(0.5), ls_hi=math.log(16.0))
WIDE_SCALES_TAU1 = SiteRecipe(ls_lo=math.log(0.5), ls_hi=math.log(16.0), fixed_logtau=0.0)


def sites(seed: int, n: int, h: int, w: int, recipe: SiteRecipe = SMALL_SCALES) -> np.ndarray:
    """Draw ``n`` site records ([n][12] float32)."""
    rng = np.random.default_rng(seed)
    p = np.zeros((n, PARAM_STRIDE), dtype=np.float64)
    p[:, 0] = rng.uniform(0.0, w, n)
    p[:, 1] = rng.uniform(0.0, h, n)
    if recipe.fixed_logtau is None:
        p[:, 2] = rng.uniform(recipe.logtau_lo, recipe.logtau_hi, n)
    else:
        rng.uniform(recipe.logtau_lo, recipe.logtau_hi, n)  # keep later draws aligned
        p[:, 2] = recipe.fixed_logtau
    p[:, 3] = rng.uniform(recipe.r_lo, recipe.r_hi, n)
    p[:, 4:7] = rng.uniform(0.0, 1.0, (n, 3))
    p[:, 7] = rng.uniform(0.0, math.pi, n)
    p[:, 8] = rng.uniform(recipe.ls_lo, recipe.ls_hi, n)
    p[:, 9] = rng.uniform(recipe.ls_lo, recipe.ls_hi, n)
    out = p.astype(np.float32)
    # uniform(0, w) can round up to w in float32; keep sites inside [0, W) x [0, H)
    out[:, 0] = np.minimum(out[:, 0], np.nextafter(np.float32(w), np.float32(0)))
    out[:, 1] = np.minimum(out[:, 1], np.nextafter(np.float32(h), np.float32(0)))
    return out


def sites_unique_cells(seed: int, n: int, h: int, w: int, recipe: SiteRecipe = WIDE_SCALES) -> np.ndarray:
    """Site records whose centres lie in n distinct pixels (drawn without
    replacement) at uniform offsets inside them, the other values as sites()
    draws them: the collision-free layout of the top-K convergence protocol."""
    p = sites(seed, n, h, w, recipe)
    rng = np.random.default_rng(seed + 1)
    cells = rng.choice(h * w, n, replace=False)
    off = rng.random((n, 2))
    p[:, 0] = ((cells % w) + off[:, 0]).astype(np.float32)
    p[:, 1] = ((cells // w) + off[:, 1]).astype(np.float32)
    return p


def target_polygons(seed: int, h: int, w: int, n_poly: int = 8) -> np.ndarray:
    """Linear colour ramp plus ``n_poly`` opaque convex polygons ([h][w][3] float32).

    The ramp is c0 + (c1 - c0) * clamp(0.5 + n.(x - centre) / W) along a random
    unit direction n.  Each polygon has 3-7 vertices at sorted random angles
    around a random centre, at radii U[4, 20] px; pixel centres inside every
    edge half-plane take the polygon's colour (hard edges), later polygons on top.
    """
    rng = np.random.default_rng(seed)
    yy, xx = np.mgrid[0:h, 0:w].astype(np.float64)
    px, py = xx + 0.5, yy + 0.5
    c0 = rng.uniform(0, 1, 3)
    c1 = rng.uniform(0, 1, 3)
    ang = rng.uniform(0, 2 * math.pi)
    nx, ny = math.cos(ang), math.sin(ang)
    t = 0.5 + (nx * (px - w / 2) + ny * (py - h / 2)) / w
    t = np.clip(t, 0.0, 1.0)[..., None]
    img = c0 + (c1 - c0) * t
    for _ in range(n_poly):
        cx, cy = rng.uniform(0, w), rng.uniform(0, h)
        nv = int(rng.integers(3, 8))
        angles = np.sort(rng.uniform(0, 2 * math.pi, nv))
        radii = rng.uniform(4.0, 20.0, nv)
        col = rng.uniform(0, 1, 3)
        vx = cx + radii * np.cos(angles)
        vy = cy + radii * np.sin(angles)
        inside = np.ones((h, w), dtype=bool)
        for k in range(nv):
            ax, ay = vx[k], vy[k]
            bx, by = vx[(k + 1) % nv], vy[(k + 1) % nv]
            # counter-clockwise vertex order: inside is the left side of each edge
            cross = (bx - ax) * (py - ay) - (by - ay) * (px - ax)
            inside &= cross >= 0
        img[inside] = col
    return img.astype(np.float32)


def target_noise_edges(seed: int, h: int, w: int, n_waves: int = 8, n_edges: int = 200) -> np.ndarray:
    """Smooth low-frequency noise plus ``n_edges`` hard edges ([h][w][3] float32).

    Per channel: 0.5 + sum_m a_m cos(2 pi k_m.(x/W, y/H) + phi_m) with integer
    k_m in {-4..4}^2 minus 0 and a_m ~ U[0, 0.06].  Each edge adds a colour
    offset ~ U[-0.3, 0.3]^3 to the pixels of a disc (radius U[16, 96] px) that
    lie on the positive side of a random line through the disc centre.
    The result is clamped to [0, 1].
    """
    rng = np.random.default_rng(seed)
    yy, xx = np.mgrid[0:h, 0:w].astype(np.float64)
    u, v = (xx + 0.5) / w, (yy + 0.5) / h
    img = np.full((h, w, 3), 0.5)
    for ch in range(3):
        for _ in range(n_waves):
            while True:
                k = rng.integers(-4, 5, 2)
                if k[0] != 0 or k[1] != 0:
                    break
            a = rng.uniform(0, 0.06)
            phi = rng.uniform(0, 2 * math.pi)
            img[..., ch] += a * np.cos(2 * math.pi * (k[0] * u + k[1] * v) + phi)
    px, py = xx + 0.5, yy + 0.5
    for _ in range(n_edges):
        cx, cy = rng.uniform(0, w), rng.uniform(0, h)
        rad = rng.uniform(16.0, 96.0)
        ang = rng.uniform(0, 2 * math.pi)
        delta = rng.uniform(-0.3, 0.3, 3)
        # only the disc's bounding box (with a pixel of margin) can be inside;
        # the test itself is evaluated exactly as over the whole image
        i0, i1 = max(0, int(math.floor(cx - rad)) - 1), min(w, int(math.ceil(cx + rad)) + 1)
        j0, j1 = max(0, int(math.floor(cy - rad)) - 1), min(h, int(math.ceil(cy + rad)) + 1)
        if i0 >= i1 or j0 >= j1:
            continue
        dxp, dyp = px[j0:j1, i0:i1] - cx, py[j0:j1, i0:i1] - cy
        mask = (dxp * dxp + dyp * dyp <= rad * rad) & (math.cos(ang) * dxp + math.sin(ang) * dyp > 0)
        img[j0:j1, i0:i1][mask] += delta
    return np.clip(img, 0.0, 1.0).astype(np.float32)


def queries(seed: int, m: int, h: int, w: int) -> np.ndarray:
    """``m`` uniformly random continuous points in [0, W) x [0, H) ([m][2] float32)."""
    rng = np.random.default_rng(seed)
    q = np.empty((m, 2), dtype=np.float64)
    q[:, 0] = rng.uniform(0.0, w, m)
    q[:, 1] = rng.uniform(0.0, h, m)
    out = q.astype(np.float32)
    out[:, 0] = np.minimum(out[:, 0], np.nextafter(np.float32(w), np.float32(0)))
    out[:, 1] = np.minimum(out[:, 1], np.nextafter(np.float32(h), np.float32(0)))
    return out


def gradients(seed: int, n: int, scale: float = 1e-3) -> np.ndarray:
    """Random per-site gradient records ([n][12] float32, padding 0) for optimizer tests."""
    rng = np.random.default_rng(seed)
    g = rng.normal(0.0, scale, (n, PARAM_STRIDE))
    g[:, 10:] = 0.0
    return g.astype(np.float32)


def jfa_strides(h: int, w: int, n_pass: int) -> list[int]:
    """Jump steps of the warm-up schedule: B/2, B/4, ..., 1, then 1.

    B is the smallest power of two >= max(H, W); the step at refresh t is
    max(1, B / 2^(min(t, log2 B - 1) + 1)).
    """
    b = 1
    while b < max(h, w):
        b *= 2
    lb = b.bit_length() - 1
    out = []
    for t in range(n_pass):
        out.append(max(1, b >> (min(t, max(lb - 1, 0)) + 1)))
    return out


@dataclass(frozen=True)
class Workload:
    name: str
    h: int
    w: int
    n: int
    recipe: SiteRecipe
    target: str  # "polygons" or "noise"
    strides: tuple[int, ...]  # propagation strides of one step
    inject: int = 64
    warm_passes: int = 16
    n_queries: int = 0

    @property
    def param_seed(self) -> int:
        return 1000 + int(self.name[1])

    @property
    def target_seed(self) -> int:
        return 2000 + int(self.name[1])

    @property
    def inject_seed(self) -> int:
        return 3000 + int(self.name[1])

    @property
    def query_seed(self) -> int:
        return 4000 + int(self.name[1])

    def make_sites(self) -> np.ndarray:
        return sites(self.param_seed, self.n, self.h, self.w, self.recipe)

    def make_target(self) -> np.ndarray:
        if self.target == "polygons":
            return target_polygons(self.target_seed, self.h, self.w)
        return target_noise_edges(self.target_seed, self.h, self.w)

    def make_queries(self, m: int | None = None) -> np.ndarray:
        return queries(self.query_seed, self.n_queries if m is None else m, self.h, self.w)


# C1: 64x64, 256 sites, 20 passes from an empty map on the warm-up schedule.
C1 = Workload("C1", 64, 64, 256, SMALL_SCALES, "polygons", tuple(jfa_strides(64, 64, 20)), warm_passes=0)
# C2: 768x512 (Kodak-sized), 50k sites; one step = strides 8,4,2,1 + forward + backward.
C2 = Workload("C2", 512, 768, 50_000, WIDE_SCALES, "noise", (8, 4, 2, 1))
# C3: the C2 shape trained with Adam, tau initialised at 1.
C3 = Workload("C3", 512, 768, 50_000, WIDE_SCALES_TAU1, "noise", (8, 4, 2, 1))
# C4: 2048x2048, 400k sites; one step = strides 16,8,4,2,1 + forward + backward.
C4 = Workload("C4", 2048, 2048, 400_000, WIDE_SCALES, "noise", (16, 8, 4, 2, 1))
# C5: random-access decode of a 768x512, 50k-site representation at 2^24 points.
C5 = Workload("C5", 512, 768, 50_000, SMALL_SCALES, "noise", (), n_queries=1 << 24)

WORKLOADS = {wl.name: wl for wl in (C1, C2, C3, C4, C5)}
