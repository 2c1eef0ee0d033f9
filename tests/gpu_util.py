"""Helpers for the GPU parity tests: moving seeded inputs to the device and
results back, and the tolerances the comparisons use.

Tolerances (floating-point outputs; integer outputs are compared bit for bit):
- colours: |gpu - oracle| <= 1e-5 absolute.  The GPU blends in float32
  from the same float32 logits the oracle uses; the oracle blends in float64.
- gradients, per site and parameter: |gpu - oracle| <= 1e-4 max(|oracle|,
  1e-3 M) with M the largest |oracle| value of that parameter over all sites
  (the parameter's column), and per column ||gpu - oracle||_2 <= 1e-4
  ||oracle||_2.  A NaN on one side only is an error.  When the GPU sums a
  site's terms in fixed point, each of the `count` terms (count = the number
  of pixels listing the site) is rounded to a multiple of 2^-E first, which
  adds count * 2^-E to the element bound.
- loss: relative 1e-5.
- budget statistics, per site and column: 1e-4 |oracle| + 1e-5 S, S the
  oracle's sum of the terms' magnitudes (for the removal delta, of the two
  squared errors it subtracts), plus count * 2^-E_q, the resolution of the
  GPU's fixed-point sums of that column (2^E_q chosen per column from the
  range of its terms).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

COLOUR_ATOL = 1e-5
GRAD_RTOL = 1e-4
GRAD_STOL = 1e-5


def dev() -> torch.device:
    if not torch.cuda.is_available():
        raise RuntimeError("GPU test run without a visible GPU")
    return torch.device("cuda", 0)


def to_gpu(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32)).to(dev())
    return torch.from_numpy(a).to(dev())


def map_to_np(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def fixed_point_resolution(h: int, w: int) -> float:
    e = 45
    while (1 << (e - 45)) < h * w:
        e += 1
    return 2.0 ** -e


GRAD_FLOOR = 1e-3
GRAD_NORM_RTOL = 1e-4
GRAD_COLUMNS = ("x", "y", "log_tau", "r", "red", "green", "blue", "theta", "log_s1", "log_s2")


def grad_ratios(gpu: np.ndarray, ref: np.ndarray, slack: np.ndarray | None = None):
    """Per site and gradient column, |gpu - oracle| / element bound; per
    column, ||gpu - oracle||_2 / (1e-4 ||oracle||_2 + ||slack||_2).  Either
    check passes at a ratio <= 1.  A NaN on one side only gives inf."""
    gpu = gpu[:, :10].astype(np.float64)
    ref = ref[:, :10].astype(np.float64)
    both_nan = np.isnan(gpu) & np.isnan(ref)
    err = np.abs(gpu - ref)
    err[both_nan] = 0.0
    err[np.isnan(err)] = np.inf
    fin = np.where(np.isfinite(ref), np.abs(ref), 0.0)
    colmax = fin.max(axis=0) if len(fin) else np.zeros(10)
    bound = GRAD_RTOL * np.maximum(np.abs(ref), GRAD_FLOOR * colmax[None, :])
    sl = np.zeros_like(bound) if slack is None else np.broadcast_to(slack, bound.shape)
    bound = bound + sl
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(err == 0.0, 0.0, err / bound)
    ratio[np.isnan(ratio)] = np.inf
    d = np.where(both_nan, 0.0, gpu - ref)
    r0 = np.where(both_nan, 0.0, ref)
    dn = np.sqrt((d ** 2).sum(axis=0))
    nb = GRAD_NORM_RTOL * np.sqrt((r0 ** 2).sum(axis=0)) + np.sqrt((sl ** 2).sum(axis=0))
    with np.errstate(divide="ignore", invalid="ignore"):
        norm = np.where(dn == 0.0, 0.0, dn / nb)
    norm[np.isnan(norm)] = np.inf
    return ratio, norm


def grad_summary(gpu: np.ndarray, ref: np.ndarray, slack: np.ndarray | None = None) -> str:
    ratio, norm = grad_ratios(gpu, ref, slack)
    mx = ratio.max(axis=0) if len(ratio) else np.zeros(10)
    return " ".join(f"{c} {m:.3g}/{nv:.3g}" for c, m, nv in zip(GRAD_COLUMNS, mx, norm))


def assert_grad_close(gpu: np.ndarray, ref: np.ndarray, what: str = "grad", topk: np.ndarray | None = None,
                      hw: tuple | None = None, resolution: float | None = None) -> None:
    """The element bound and the column norm bound above; with topk and a
    fixed-point resolution 2^-E both bounds gain count * 2^-E per site."""
    slack = None
    if topk is not None and resolution is not None:
        ids = topk.reshape(-1)
        ids = ids[ids < ref.shape[0]].astype(np.int64)
        count = np.bincount(ids, minlength=ref.shape[0]).astype(np.float64)
        slack = (count * resolution)[:, None]
    ratio, norm = grad_ratios(gpu, ref, slack)
    say(f"[gpu] {what}: per column, max |err|/bound of the elements / of the norm: {grad_summary(gpu, ref, slack)}")
    bad = ratio > 1.0
    if bad.any():
        i, k = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} entries out of tolerance; first site {i} {GRAD_COLUMNS[k]}: "
                             f"gpu {gpu[i, k]!r} oracle {ref[i, k]!r}")
    if (norm > 1.0).any():
        k = int(np.argmax(norm))
        raise AssertionError(f"{what}: column {GRAD_COLUMNS[k]}: norm error {norm[k]:.3g} of its bound")


def stats_resolution(h: int, w: int) -> np.ndarray:
    """Per-column resolution of the GPU's fixed-point statistics sums: 2^-E_q
    with E_q = 52, 50, 49 for mass, energy and removal delta and 52 - lg,
    52 - 2 lg for the first and second moments, 2^lg >= max(h, w)."""
    lg = 0
    while (1 << lg) < max(h, w):
        lg += 1
    e = np.array([52, 50, 49, 52 - lg, 52 - lg, 52 - 2 * lg, 52 - 2 * lg, 52 - 2 * lg], dtype=np.float64)
    return 2.0 ** -e


def assert_stats_close(gpu: np.ndarray, ref: np.ndarray, mag: np.ndarray, topk: np.ndarray, hw: tuple,
                       what: str = "stats", calls: int = 1) -> None:
    """ref and mag cover all `calls` accumulated calls over the map topk."""
    gpu = gpu.astype(np.float64)
    ids = topk.reshape(-1)
    ids = ids[ids < ref.shape[0]].astype(np.int64)
    count = calls * np.bincount(ids, minlength=ref.shape[0]).astype(np.float64)
    tol = GRAD_RTOL * np.abs(ref) + GRAD_STOL * mag + count[:, None] * stats_resolution(*hw)[None, :]
    err = np.abs(gpu - ref)
    bad = ~(err <= tol)
    if bad.any():
        i, k = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} entries out of tolerance; first site {i} column {k}: "
                             f"gpu {gpu[i, k]!r} oracle {ref[i, k]!r} magnitude {mag[i, k]!r}")


def assert_colour_close(gpu: np.ndarray, ref: np.ndarray, what: str = "colour") -> None:
    err = np.abs(gpu.astype(np.float64) - ref)
    nan_ok = np.isnan(gpu) & np.isnan(ref)
    err[nan_ok] = 0
    if not (err <= COLOUR_ATOL).all():
        idx = np.unravel_index(np.nanargmax(err), err.shape)
        raise AssertionError(f"{what}: max |diff| {np.nanmax(err):.3g} at {idx}")
