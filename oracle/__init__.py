"""CPU oracle for the SAD hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never calls it, and it never calls the product path.

The arithmetic lives in ``sadref.c`` (plain C, built with gcc, no FMA
contraction).  This module only compiles it and marshals numpy arrays; see the
C file for the definitions and the paper sections they follow.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from pathlib import Path

import numpy as np

HERE = Path(__file__).resolve().parent
SRC = HERE / "sadref.c"
BUILD_DIR = HERE / "_build"
LIB = BUILD_DIR / "libsadref.so"

K = 8
NONE = 0xFFFFFFFF
REC = 12

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-fno-finite-math-only", "-fopenmp", "-Wall", "-Wextra"]


def build(force: bool = True) -> Path:
    """Compile the oracle with gcc into ``oracle/_build/libsadref.so``."""
    if LIB.exists() and not force and LIB.stat().st_mtime >= SRC.stat().st_mtime:
        return LIB
    BUILD_DIR.mkdir(exist_ok=True)
    tmp = LIB.with_suffix(".so.tmp%d" % os.getpid())
    subprocess.run(["gcc", *CFLAGS, str(SRC), "-o", str(tmp), "-lm"], check=True)
    os.replace(tmp, LIB)
    return LIB


_lib = None


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        build(force=False)
        L = C.CDLL(str(LIB))
        f32p, u32p, f64p, i64p = (C.POINTER(C.c_float), C.POINTER(C.c_uint32),
                                  C.POINTER(C.c_double), C.POINTER(C.c_int64))
        i32, u32, u64, i64 = C.c_int32, C.c_uint32, C.c_uint64, C.c_int64
        i32p = C.POINTER(C.c_int32)
        L.sadref_prepare_sites.argtypes = [f32p, i32, f32p]
        L.sadref_brute_topk.argtypes = [f32p, i32, i32, i32, u32p]
        L.sadref_brute_topk_pixels.argtypes = [f32p, i32, i32, i32, i64p, i64, u32p]
        L.sadref_propagate.argtypes = [f32p, i32, i32, i32, u32p, u32p, i32, u64, u32, i32]
        L.sadref_propagate_pixels.argtypes = [f32p, i32, i32, i32, u32p, i32, u64, u32, i32, i64p, i64, u32p]
        L.sadref_render_fwd.argtypes = [f32p, i32, i32, i32, u32p, f64p]
        L.sadref_render_bwd.argtypes = [f32p, i32, i32, i32, u32p, f32p, f64p, f64p, f64p, f64p]
        L.sadref_site_stats.argtypes = [f32p, i32, i32, i32, u32p, f32p, f64p, f64p]
        L.sadref_jfa_seed.argtypes = [f32p, i32, i32, i32, u32p]
        L.sadref_jfa_flood.argtypes = [f32p, i32, i32, i32, u32p, u32p, i32, i32]
        f32 = C.c_float
        L.sadref_densify_prune.argtypes = [f32p, f32p, f32p, f32p, i32, i32, i32, f32p, f32p, i32, i32, f32, f32, f32,
                                           f32, f32, C.POINTER(C.c_int32)]
        L.sadref_half_bits.argtypes = [C.c_float]
        L.sadref_half_bits.restype = u32
        L.sadref_half_value.argtypes = [u32]
        L.sadref_half_value.restype = C.c_double
        L.sadref_pack_sites.argtypes = [f32p, f32p, i32, i32, i32, u32p, f32p]
        L.sadref_unpack_site.argtypes = [u32p, f32p, i32, i32, f64p]
        L.sadref_unpack_sites.argtypes = [u32p, f32p, i32, i32, i32, f64p, i32p]
        L.sadref_packed_logit.argtypes = [f64p, C.c_double, C.c_double]
        L.sadref_packed_logit.restype = C.c_double
        L.sadref_query_packed.argtypes = [u32p, f32p, i32, i32, i32, u32p, f32p, i64, f64p]
        L.sadref_grad_mag.argtypes = [f32p, i32, i32, f32p]
        L.sadref_grad_units.argtypes = [C.c_float]
        L.sadref_grad_units.restype = u64
        L.sadref_init_sites.argtypes = [f32p, i32, i32, i32, C.c_float, u64, C.c_float, C.c_float, C.c_float, f32p,
                                        f32p]
        L.sadref_query_points.argtypes = [f32p, i32, i32, i32, u32p, f32p, i64, f64p]
        L.sadref_adam_step.argtypes = [f32p, f32p, f32p, f32p, i32, i32, i32, f32p,
                                       C.c_float, C.c_float, C.c_float, C.c_float, C.c_float, f32p]
        L.sadref_score.argtypes = [f32p, i32, u32, C.c_float, C.c_float]
        L.sadref_score.restype = C.c_float
        for name in ("sadref_exp_f32", "sadref_cos_f32", "sadref_sin_f32"):
            getattr(L, name).argtypes = [C.c_float]
            getattr(L, name).restype = C.c_float
        L.sadref_splitmix64.argtypes = [u64, u64]
        L.sadref_splitmix64.restype = u64
        L.sadref_inject_id.argtypes = [u64, u32, u32, u32, i32]
        L.sadref_inject_id.restype = u32
        L.sadref_ambiguous_count.argtypes = []
        L.sadref_ambiguous_count.restype = C.c_long
        _lib = L
    return _lib


def _p(a: np.ndarray, ct):
    return a.ctypes.data_as(C.POINTER(ct))


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def _u32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.uint32)


def set_threads(n: int | None) -> None:
    """Thread count of the OpenMP loops (takes effect for the next parallel region)."""
    if n is not None:
        os.environ["OMP_NUM_THREADS"] = str(n)
        try:
            C.CDLL("libgomp.so.1").omp_set_num_threads(int(n))
        except OSError:
            pass


def ambiguous_count() -> int:
    """Number of prepared values whose float32 rounding the guard could not certify."""
    return int(lib().sadref_ambiguous_count())


def prepare_sites(params: np.ndarray) -> np.ndarray:
    params = _f32(params).reshape(-1, REC)
    out = np.empty_like(params)
    lib().sadref_prepare_sites(_p(params, C.c_float), params.shape[0], _p(out, C.c_float))
    return out


def exp_f32(x: float) -> float:
    return lib().sadref_exp_f32(x)


def cos_f32(x: float) -> float:
    return lib().sadref_cos_f32(x)


def sin_f32(x: float) -> float:
    return lib().sadref_sin_f32(x)


def score(derived: np.ndarray, site: int, px: float, py: float) -> float:
    derived = _f32(derived).reshape(-1, REC)
    return lib().sadref_score(_p(derived, C.c_float), derived.shape[0], site, px, py)


def brute_topk(derived: np.ndarray, h: int, w: int) -> np.ndarray:
    derived = _f32(derived).reshape(-1, REC)
    out = np.empty((h, w, K), dtype=np.uint32)
    lib().sadref_brute_topk(_p(derived, C.c_float), derived.shape[0], h, w, _p(out, C.c_uint32))
    return out


def brute_topk_pixels(derived: np.ndarray, h: int, w: int, pixels: np.ndarray) -> np.ndarray:
    """Exact top-K lists ([m][8]) at the given flat pixel indices."""
    derived = _f32(derived).reshape(-1, REC)
    pixels = np.ascontiguousarray(pixels, dtype=np.int64)
    out = np.empty((pixels.shape[0], K), np.uint32)
    lib().sadref_brute_topk_pixels(_p(derived, C.c_float), derived.shape[0], h, w, _p(pixels, C.c_int64),
                                   pixels.shape[0], _p(out, C.c_uint32))
    return out


def empty_map(h: int, w: int) -> np.ndarray:
    return np.full((h, w, K), NONE, dtype=np.uint32)


def splitmix64(seed: int, counter: int) -> int:
    return int(lib().sadref_splitmix64(seed, counter))


def inject_id(seed: int, pass_index: int, tile: int, j: int, n: int) -> int:
    return int(lib().sadref_inject_id(seed, pass_index, tile, j, n))


def propagate(derived: np.ndarray, h: int, w: int, prev: np.ndarray | None, stride: int,
              seed: int, pass_index: int, inject: int = 64) -> np.ndarray:
    derived = _f32(derived).reshape(-1, REC)
    out = np.empty((h, w, K), dtype=np.uint32)
    prev_p = None
    if prev is not None:
        prev = _u32(prev).reshape(h, w, K)
        prev_p = _p(prev, C.c_uint32)
    lib().sadref_propagate(_p(derived, C.c_float), derived.shape[0], h, w, prev_p, _p(out, C.c_uint32),
                           stride, seed, pass_index, inject)
    return out


def propagate_pixels(derived: np.ndarray, h: int, w: int, prev: np.ndarray | None, stride: int,
                     seed: int, pass_index: int, inject: int, pixels: np.ndarray) -> np.ndarray:
    derived = _f32(derived).reshape(-1, REC)
    pixels = np.ascontiguousarray(pixels, dtype=np.int64)
    out = np.empty((pixels.shape[0], K), dtype=np.uint32)
    prev_p = None
    if prev is not None:
        prev = _u32(prev).reshape(h, w, K)
        prev_p = _p(prev, C.c_uint32)
    lib().sadref_propagate_pixels(_p(derived, C.c_float), derived.shape[0], h, w, prev_p, stride, seed,
                                  pass_index, inject, _p(pixels, C.c_int64), pixels.shape[0],
                                  _p(out, C.c_uint32))
    return out


def propagate_schedule(derived: np.ndarray, h: int, w: int, prev: np.ndarray | None, strides,
                       seed: int, first_pass: int = 0, inject: int = 64) -> np.ndarray:
    """Successive passes, one per stride, with pass indices first_pass, first_pass+1, ..."""
    cur = prev
    for t, s in enumerate(strides):
        cur = propagate(derived, h, w, cur, int(s), seed, first_pass + t, inject)
    if cur is None:
        cur = empty_map(h, w)
    return cur


def densify_prune(params: np.ndarray, m: np.ndarray, v: np.ndarray, derived: np.ndarray, h: int, w: int,
                  stats: np.ndarray, target: np.ndarray, n_split: int, n_prune: int, alpha: float, min_mass: float,
                  offset: float, r_scale: float, logtau_shift: float):
    """Budget control (see sadref_densify_prune) on copies of the site
    arrays: returns (params, m, v, derived, (pruned, split))."""
    params = _f32(params).reshape(-1, REC).copy()
    n = params.shape[0]
    m = _f32(m).reshape(n, REC).copy()
    v = _f32(v).reshape(n, REC).copy()
    derived = _f32(derived).reshape(n, REC).copy()
    stats = _f32(stats).reshape(n, 8)
    target = _f32(target).reshape(h, w, 3)
    done = (C.c_int32 * 2)()
    lib().sadref_densify_prune(_p(params, C.c_float), _p(m, C.c_float), _p(v, C.c_float), _p(derived, C.c_float),
                               n, h, w, _p(stats, C.c_float), _p(target, C.c_float), n_split, n_prune, alpha,
                               min_mass, offset, r_scale, logtau_shift, done)
    return params, m, v, derived, (int(done[0]), int(done[1]))


JFA_K = 4


def half_bits(f: float) -> int:
    """float16 bits of a float32, rounded to nearest even (own conversion)."""
    return int(lib().sadref_half_bits(float(f)))


def half_value(bits: int) -> float:
    return float(lib().sadref_half_value(int(bits)))


def pack_sites(params: np.ndarray, derived: np.ndarray, h: int, w: int):
    """Packed evaluation records (see sadref_pack_sites): ([n][4] uint32, qp float32[10])."""
    p = _f32(params).reshape(-1, REC)
    d = _f32(derived).reshape(-1, REC)
    n = p.shape[0]
    out = np.zeros((n, 4), np.uint32)
    qp = np.zeros(10, np.float32)
    lib().sadref_pack_sites(_p(p, C.c_float), _p(d, C.c_float), n, h, w, _p(out, C.c_uint32), _p(qp, C.c_float))
    return out, qp


def unpack_site(record: np.ndarray, qp: np.ndarray, h: int, w: int):
    """(x, y, tau', r', c_r, c_g, c_b, theta, a) of one packed record in float64, or None if not usable."""
    rec = _u32(record).reshape(4)
    q = _f32(qp)
    v = np.zeros(9, np.float64)
    ok = lib().sadref_unpack_site(_p(rec, C.c_uint32), _p(q, C.c_float), h, w, _p(v, C.c_double))
    return v if ok else None


def unpack_sites(packed: np.ndarray, qp: np.ndarray, h: int, w: int):
    """All records decoded ([n][9] float64 as unpack_site; zeros where not usable) and the usable mask."""
    pk = _u32(packed).reshape(-1, 4)
    q = _f32(qp)
    n = pk.shape[0]
    out = np.zeros((n, 9), np.float64)
    ok = np.zeros(n, np.int32)
    lib().sadref_unpack_sites(_p(pk, C.c_uint32), _p(q, C.c_float), n, h, w, _p(out, C.c_double),
                              _p(ok, C.c_int32))
    return out, ok.astype(bool)


def packed_logit(values: np.ndarray, px: float, py: float) -> float:
    v = np.ascontiguousarray(values, dtype=np.float64)
    return float(lib().sadref_packed_logit(_p(v, C.c_double), float(px), float(py)))


def query_packed(packed: np.ndarray, qp: np.ndarray, h: int, w: int, topk: np.ndarray, xy: np.ndarray) -> np.ndarray:
    pk = _u32(packed).reshape(-1, 4)
    q = _f32(qp)
    m = _u32(topk)
    pts = _f32(xy).reshape(-1, 2)
    out = np.zeros((pts.shape[0], 3), np.float64)
    lib().sadref_query_packed(_p(pk, C.c_uint32), _p(q, C.c_float), pk.shape[0], h, w, _p(m, C.c_uint32),
                              _p(pts, C.c_float), pts.shape[0], _p(out, C.c_double))
    return out


def grad_mag(target: np.ndarray, h: int, w: int) -> np.ndarray:
    """float32 |grad I| per pixel ([h][w]; see sadref_grad_mag)."""
    t = _f32(target).reshape(h, w, 3)
    g = np.empty((h, w), np.float32)
    lib().sadref_grad_mag(_p(t, C.c_float), h, w, _p(g, C.c_float))
    return g


def grad_units(g: float) -> int:
    """The integer weight (units of 2^-24) the sampler gives a float32 gradient magnitude."""
    return int(lib().sadref_grad_units(float(g)))


def init_sites(target: np.ndarray, h: int, w: int, n: int, lam: float, seed: int, log_tau: float = 0.0,
               r: float = 0.0, log_scale: float = 0.0):
    """Gradient-weighted initialisation (see sadref_init_sites): returns (params, derived)."""
    t = _f32(target).reshape(h, w, 3)
    p = np.zeros((n, REC), np.float32)
    d = np.zeros((n, REC), np.float32)
    lib().sadref_init_sites(_p(t, C.c_float), h, w, n, lam, seed, log_tau, r, log_scale, _p(p, C.c_float),
                            _p(d, C.c_float))
    return p, d


def jfa_steps(h: int, w: int) -> list[int]:
    """Jump steps of a JFA round: B/2, B/4, ..., 1 with B = 2^ceil(log2 max(h, w))."""
    b = 1
    while b < max(h, w):
        b *= 2
    out = []
    s = b // 2
    while s >= 1:
        out.append(s)
        s //= 2
    return out


def jfa_seed(derived: np.ndarray, h: int, w: int) -> np.ndarray:
    """Seed pass of the JFA prepass (see sadref_jfa_seed): [h][w][4] u32."""
    derived = _f32(derived).reshape(-1, REC)
    out = np.empty((h, w, JFA_K), dtype=np.uint32)
    lib().sadref_jfa_seed(_p(derived, C.c_float), derived.shape[0], h, w, _p(out, C.c_uint32))
    return out


def jfa_flood(derived: np.ndarray, h: int, w: int, prev: np.ndarray, step: int, out_width: int = JFA_K) -> np.ndarray:
    """One flood pass (see sadref_jfa_flood): [h][w][out_width] u32."""
    derived = _f32(derived).reshape(-1, REC)
    prev = _u32(prev).reshape(h, w, JFA_K)
    out = np.empty((h, w, out_width), dtype=np.uint32)
    lib().sadref_jfa_flood(_p(derived, C.c_float), derived.shape[0], h, w, _p(prev, C.c_uint32),
                           _p(out, C.c_uint32), step, out_width)
    return out


def full_refresh(derived: np.ndarray, h: int, w: int, seed: int, n_pass: int = 16, inject: int = 64) -> np.ndarray:
    """The render protocol's list rebuild (Sec. 6.6): one JFA round (seed and
    flood passes, the last one writing a top-K map), then n_pass propagation
    passes on the warm-up schedule with pass indices 0, 1, ..."""
    steps = jfa_steps(h, w)
    cur = jfa_seed(derived, h, w)
    for t, s in enumerate(steps):
        cur = jfa_flood(derived, h, w, cur, s, K if t == len(steps) - 1 else JFA_K)
    if not steps:  # a 1x1 image: the seed alone, widened
        cur = np.concatenate([cur, np.full((h, w, K - JFA_K), 0xFFFFFFFF, np.uint32)], axis=-1)
    strides = []
    b = 1
    while b < max(h, w):
        b *= 2
    lb = b.bit_length() - 1
    for t in range(n_pass):
        strides.append(max(1, b >> (min(t, max(lb - 1, 0)) + 1)))
    return propagate_schedule(derived, h, w, cur, strides, seed, 0, inject)


def render_fwd(derived: np.ndarray, h: int, w: int, topk: np.ndarray) -> np.ndarray:
    derived = _f32(derived).reshape(-1, REC)
    topk = _u32(topk).reshape(h, w, K)
    out = np.empty((h, w, 3), dtype=np.float64)
    lib().sadref_render_fwd(_p(derived, C.c_float), derived.shape[0], h, w, _p(topk, C.c_uint32),
                            _p(out, C.c_double))
    return out


def render_bwd(derived: np.ndarray, h: int, w: int, topk: np.ndarray, target: np.ndarray):
    """Returns (grad [n][12] f64, grad_mag [n][12] f64, loss, image [h][w][3] f64).

    grad_mag is the running error magnitude of each gradient sum (see
    sadref_render_bwd): it bounds how far a lower-precision evaluation of the
    same sums can drift, cancellation included."""
    derived = _f32(derived).reshape(-1, REC)
    n = derived.shape[0]
    topk = _u32(topk).reshape(h, w, K)
    target = _f32(target).reshape(h, w, 3)
    grad = np.zeros((n, REC), dtype=np.float64)
    gabs = np.zeros((n, REC), dtype=np.float64)
    loss = np.zeros(1, dtype=np.float64)
    img = np.empty((h, w, 3), dtype=np.float64)
    lib().sadref_render_bwd(_p(derived, C.c_float), n, h, w, _p(topk, C.c_uint32), _p(target, C.c_float),
                            _p(grad, C.c_double), _p(gabs, C.c_double), _p(loss, C.c_double),
                            _p(img, C.c_double))
    return grad, gabs, float(loss[0]), img


def site_stats(derived: np.ndarray, h: int, w: int, topk: np.ndarray, target: np.ndarray):
    """Per-site budget statistics (Sec. 4.5, Appendix B.5): returns (stats
    [n][8] f64, stats_mag [n][8] f64) with columns mass, energy, removal
    delta, sum w dx, sum w dy, sum w dx^2, sum w dx dy, sum w dy^2 (see
    sadref_site_stats); stats_mag holds the sums of the terms' magnitudes."""
    derived = _f32(derived).reshape(-1, REC)
    n = derived.shape[0]
    topk = _u32(topk).reshape(h, w, K)
    target = _f32(target).reshape(h, w, 3)
    stats = np.zeros((n, 8), dtype=np.float64)
    mag = np.zeros((n, 8), dtype=np.float64)
    lib().sadref_site_stats(_p(derived, C.c_float), n, h, w, _p(topk, C.c_uint32), _p(target, C.c_float),
                            _p(stats, C.c_double), _p(mag, C.c_double))
    return stats, mag


def query_points(derived: np.ndarray, h: int, w: int, topk: np.ndarray, xy: np.ndarray) -> np.ndarray:
    derived = _f32(derived).reshape(-1, REC)
    topk = _u32(topk).reshape(h, w, K)
    xy = _f32(xy).reshape(-1, 2)
    out = np.empty((xy.shape[0], 3), dtype=np.float64)
    lib().sadref_query_points(_p(derived, C.c_float), derived.shape[0], h, w, _p(topk, C.c_uint32),
                              _p(xy, C.c_float), xy.shape[0], _p(out, C.c_double))
    return out


def adam_step(params, grad, m, v, h: int, w: int, lr, beta1: float, beta2: float, eps: float,
              bc1: float, bc2: float):
    """In-place Adam on copies; returns (params, grad, m, v, derived)."""
    params = _f32(params).reshape(-1, REC).copy()
    grad = _f32(grad).reshape(-1, REC).copy()
    m = _f32(m).reshape(-1, REC).copy()
    v = _f32(v).reshape(-1, REC).copy()
    lr = _f32(lr).reshape(5)
    derived = np.empty_like(params)
    lib().sadref_adam_step(_p(params, C.c_float), _p(grad, C.c_float), _p(m, C.c_float), _p(v, C.c_float),
                           params.shape[0], h, w, _p(lr, C.c_float), beta1, beta2, eps, bc1, bc2,
                           _p(derived, C.c_float))
    return params, grad, m, v, derived


def bias_corrections(beta1: float, beta2: float, t: int) -> tuple[float, float]:
    """Adam's 1 - beta^t in float32, computed on the host as the step contract requires."""
    return float(np.float32(1.0 - float(beta1) ** t)), float(np.float32(1.0 - float(beta2) ** t))
