"""Helpers for the GPU parity tests: moving seeded inputs to the device and
results back, and the tolerances the comparisons use.

Tolerances (floating-point outputs; integer outputs are compared bit for bit):
- colours: |gpu - oracle| <= 1e-5 absolute.  The GPU blends in float32
  from the same float32 logits the oracle uses; the oracle blends in float64.
- gradients, per site and parameter: |gpu - oracle| <= 1e-4 |oracle|
  + 1e-5 S, with S the oracle's running error magnitude of that sum (every
  term evaluated with the absolute values of its inputs and intermediate
  sums).  A float32 evaluation of a term with m roundings is off by at most
  about m 2^-24 of its magnitude (m ~ 30 here), and a float32 sum in any
  order adds at most (count - 1) 2^-24 of the summed magnitudes, typically
  sqrt(count) 2^-24; 1e-5 = 168 x 2^-24 covers both for the sizes tested.
  The GPU sums each site's contributions in 64-bit fixed point with
  resolution 2^-E, 2^E = 2^45 * (the power of two >= h*w), rounding each
  contribution toward zero; that adds at most count * 2^-E, count = the number of
  pixels listing the site.
- loss: relative 1e-5.
- budget statistics, per site and column: the gradients' bar (1e-4 |oracle|
  + 1e-5 S, S the oracle's sum of the terms' magnitudes; for the removal
  delta, of the two squared errors it subtracts) plus count * 2^-E_q, the
  resolution of the GPU's fixed-point sums of that column (2^E_q chosen per
  column from the range of its terms).
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


def assert_grad_close(gpu: np.ndarray, ref: np.ndarray, ref_abs: np.ndarray, what: str = "grad",
                      topk: np.ndarray | None = None, hw: tuple | None = None) -> None:
    gpu = gpu[:, :10].astype(np.float64)
    ref = ref[:, :10]
    tol = GRAD_RTOL * np.abs(ref) + GRAD_STOL * ref_abs[:, :10]
    if topk is not None:
        ids = topk.reshape(-1)
        ids = ids[ids < ref.shape[0]].astype(np.int64)
        count = np.bincount(ids, minlength=ref.shape[0]).astype(np.float64)
        tol = tol + (count * fixed_point_resolution(*hw))[:, None]
    err = np.abs(gpu - ref)
    bad = err > tol
    if bad.any():
        i, k = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} entries out of tolerance; first site {i} param {k}: "
                             f"gpu {gpu[i, k]!r} oracle {ref[i, k]!r} |term| sum {ref_abs[i, k]!r}")


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
