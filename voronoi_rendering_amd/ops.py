"""Thin torch-facing wrappers of the SAD C ABI (include/sad.h).

PyTorch only provides device memory and the current stream: every wrapper
checks shapes, dtypes and devices, passes raw pointers to libsad.so, and the
work runs in the HIP kernels.  Top-K maps are torch.int32 tensors holding the
uint32 site ids bit for bit (empty slot 0xffffffff reads as -1); the passes
also take torch.int16 maps holding uint16 ids (empty slot 0xffff, read as -1)
when there are at most 65,535 sites.
"""
from __future__ import annotations

import ctypes as C
from typing import Sequence

import torch

from . import _native

K = 8
REC = 12
NSTAT = 8  # budget statistics per site
EMPTY_I32 = -1


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape: tuple | None = None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU (the SAD kernels have no CPU path)")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def prepare_sites(params: torch.Tensor, derived: torch.Tensor | None = None) -> torch.Tensor:
    n = params.shape[0]
    _need(params, "params", torch.float32, (n, REC))
    if derived is None:
        derived = torch.empty_like(params)
    _need(derived, "derived", torch.float32, (n, REC))
    _native.check("sad_prepare_sites", _native.lib().sad_prepare_sites(_ptr(params), n, _ptr(derived),
                                                                        _stream(params)))
    return derived


def empty_map(h: int, w: int, device="cuda") -> torch.Tensor:
    return torch.full((h, w, K), EMPTY_I32, dtype=torch.int32, device=device)


def _map_bits(t: torch.Tensor, name: str, h: int, w: int) -> int:
    """Id width of a top-K map tensor: int32 holds 32-bit ids, int16 16-bit ids."""
    if isinstance(t, torch.Tensor) and t.dtype == torch.int16:
        _need(t, name, torch.int16, (h, w, K))
        return 16
    _need(t, name, torch.int32, (h, w, K))
    return 32


def _pass_maps(h: int, w: int, n: int, prev, prev_scores, prev_thr, prev_probe, out, out_scores, out_thr,
               out_probe) -> _native.PassMaps:
    """Checked tensors of a propagation pass as a sad_pass_maps."""
    pbits = _map_bits(prev, "prev", h, w) if prev is not None else 32
    obits = _map_bits(out, "out", h, w)
    for t, name in ((prev_scores, "prev_scores"), (out_scores, "out_scores")):
        if t is not None:
            _need(t, name, torch.float32, (h, w, K))
    for t, name in ((prev_thr, "prev_thr"), (out_thr, "out_thr")):
        if t is not None:
            _need(t, name, torch.float32, (h, w))
    for t, name in ((prev_probe, "prev_probe"), (out_probe, "out_probe")):
        if t is not None:
            _need(t, name, torch.float32, (n, 4))
    return _native.PassMaps(_ptr(prev), _ptr(prev_scores), _ptr(prev_thr), _ptr(prev_probe), _ptr(out),
                            _ptr(out_scores), _ptr(out_thr), _ptr(out_probe), pbits, obits)


def propagate_topk(derived: torch.Tensor, h: int, w: int, prev: torch.Tensor | None, out: torch.Tensor | None = None,
                   *, stride: int, seed: int, pass_index: int, inject: int = 64,
                   prev_scores: torch.Tensor | None = None, out_scores: torch.Tensor | None = None,
                   prev_thr: torch.Tensor | None = None, out_thr: torch.Tensor | None = None,
                   prev_probe: torch.Tensor | None = None, out_probe: torch.Tensor | None = None) -> torch.Tensor:
    """One propagation pass.  ``prev_scores`` (optional) must hold the logits of
    ``prev``'s entries under ``derived`` as a previous pass wrote them to its
    ``out_scores``; pass it only while the sites are unchanged.  ``prev`` and
    ``out`` may be int16 maps (16-bit ids); ``prev_thr`` / ``out_thr``
    ([h][w] float32) hand on only each list's 8th logit instead, and
    ``prev_probe`` / ``out_probe`` ([n][4] float32) the sites' probe records
    (sad_propagate_pass)."""
    n = derived.shape[0]
    _need(derived, "derived", torch.float32, (n, REC))
    if out is None:
        out = torch.empty((h, w, K), dtype=torch.int32, device=derived.device)
    maps = _pass_maps(h, w, n, prev, prev_scores, prev_thr, prev_probe, out, out_scores, out_thr, out_probe)
    tail = (int(stride), int(seed) & 0xFFFFFFFFFFFFFFFF, int(pass_index) & 0xFFFFFFFF, int(inject), _stream(derived))
    if (maps.prev_bits, maps.next_bits) == (32, 32) and not (maps.thr_prev or maps.thr_next or maps.probe_prev
                                                             or maps.probe_next):
        st = _native.lib().sad_propagate_topk(_ptr(derived), n, h, w, _ptr(prev), _ptr(prev_scores), _ptr(out),
                                              _ptr(out_scores), *tail)
        _native.check("sad_propagate_topk", st)
    else:
        st = _native.lib().sad_propagate_pass(_ptr(derived), n, h, w, C.byref(maps), *tail)
        _native.check("sad_propagate_pass", st)
    return out


def render_fwd(derived: torch.Tensor, h: int, w: int, topk: torch.Tensor, image: torch.Tensor | None = None
               ) -> torch.Tensor:
    n = derived.shape[0]
    _need(derived, "derived", torch.float32, (n, REC))
    _need(topk, "topk", torch.int32, (h, w, K))
    if image is None:
        image = torch.empty((h, w, 3), dtype=torch.float32, device=derived.device)
    _need(image, "image", torch.float32, (h, w, 3))
    _native.check("sad_render_fwd", _native.lib().sad_render_fwd(_ptr(derived), n, h, w, _ptr(topk), _ptr(image),
                                                                  _stream(derived)))
    return image


_workspaces: dict = {}


def stats_workspace(h: int, w: int, device) -> torch.Tensor:
    """A per-device scratch buffer for site_stats, grown on demand and reused.
    Calls that share it must be ordered (one stream, or explicit waits)."""
    need = int(_native.lib().sad_site_stats_workspace_bytes(h, w))
    dev = torch.device(device)
    ws = _workspaces.get(dev)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        _workspaces[dev] = ws
    return ws


def render_bwd(derived: torch.Tensor, h: int, w: int, topk: torch.Tensor, target: torch.Tensor, grad: torch.Tensor,
               loss: torch.Tensor | None = None, image: torch.Tensor | None = None) -> None:
    """Accumulate the loss gradient into ``grad`` ([n][12]); optionally add the
    loss into ``loss`` (one float32) and write the rendered image."""
    n = derived.shape[0]
    _need(derived, "derived", torch.float32, (n, REC))
    _need(topk, "topk", torch.int32, (h, w, K))
    _need(target, "target", torch.float32, (h, w, 3))
    _need(grad, "grad", torch.float32, (n, REC))
    if loss is not None:
        _need(loss, "loss", torch.float32, (1,))
    if image is not None:
        _need(image, "image", torch.float32, (h, w, 3))
    st = _native.lib().sad_render_bwd(_ptr(derived), n, h, w, _ptr(topk), _ptr(target), _ptr(grad), _ptr(loss),
                                      _ptr(image), _stream(derived))
    _native.check("sad_render_bwd", st)


def site_stats(derived: torch.Tensor, h: int, w: int, topk: torch.Tensor, target: torch.Tensor,
               stats: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Accumulate the per-site budget statistics ([n][8]: mass, energy,
    removal delta, sum w dx, sum w dy, sum w dx^2, sum w dx dy, sum w dy^2)
    into ``stats`` (zeros when not given) and return it."""
    n = derived.shape[0]
    _need(derived, "derived", torch.float32, (n, REC))
    _need(topk, "topk", torch.int32, (h, w, K))
    _need(target, "target", torch.float32, (h, w, 3))
    if stats is None:
        stats = torch.zeros((n, NSTAT), dtype=torch.float32, device=derived.device)
    _need(stats, "stats", torch.float32, (n, NSTAT))
    if workspace is None:
        workspace = stats_workspace(h, w, derived.device)
    st = _native.lib().sad_site_stats(_ptr(derived), n, h, w, _ptr(topk), _ptr(target), _ptr(stats),
                                      _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _stream(derived))
    _native.check("sad_site_stats", st)
    return stats


def site_stats_noalloc(derived: torch.Tensor, h: int, w: int, topk: torch.Tensor, target: torch.Tensor,
                       stats: torch.Tensor) -> torch.Tensor:
    """site_stats with the library's own device scratch (no workspace, no
    allocation); ``stats`` must be given.  Calls on one GPU must not overlap."""
    n = derived.shape[0]
    _need(derived, "derived", torch.float32, (n, REC))
    _need(topk, "topk", torch.int32, (h, w, K))
    _need(target, "target", torch.float32, (h, w, 3))
    _need(stats, "stats", torch.float32, (n, NSTAT))
    st = _native.lib().sad_site_stats_noalloc(_ptr(derived), n, h, w, _ptr(topk), _ptr(target), _ptr(stats),
                                              _stream(derived))
    _native.check("sad_site_stats_noalloc", st)
    return stats


def budget_workspace(n: int, device) -> torch.Tensor:
    """Scratch memory for sad_densify_prune with n sites."""
    nb = int(_native.lib().sad_budget_workspace_bytes(int(n)))
    return torch.empty(max(nb, 1), dtype=torch.uint8, device=device)


def densify_prune(params: torch.Tensor, m: torch.Tensor, v: torch.Tensor, derived: torch.Tensor, h: int, w: int,
                  stats: torch.Tensor, target: torch.Tensor, *, n_split: int, n_prune: int, alpha: float = 1.0,
                  min_mass: float = 1.0, offset: float = 0.5, r_scale: float = 0.85, logtau_shift: float = 0.1,
                  workspace: torch.Tensor | None = None, done: torch.Tensor | None = None) -> torch.Tensor:
    """Prune and split sites in place (see sad_densify_prune); returns the
    numbers pruned and split as a device int32[2] (``done`` when given)."""
    n = params.shape[0]
    for t, name in ((params, "params"), (m, "m"), (v, "v"), (derived, "derived")):
        _need(t, name, torch.float32, (n, REC))
    _need(stats, "stats", torch.float32, (n, NSTAT))
    _need(target, "target", torch.float32, (h, w, 3))
    if workspace is None:
        workspace = budget_workspace(n, params.device)
    if done is None:
        done = torch.zeros(2, dtype=torch.int32, device=params.device)
    _need(done, "done", torch.int32, (2,))
    st = _native.lib().sad_densify_prune(_ptr(params), _ptr(m), _ptr(v), _ptr(derived), n, h, w, _ptr(stats),
                                         _ptr(target), int(n_split), int(n_prune), float(alpha), float(min_mass),
                                         float(offset), float(r_scale), float(logtau_shift), _ptr(done),
                                         _ptr(workspace), workspace.numel(), _stream(params))
    _native.check("sad_densify_prune", st)
    return done


def init_workspace(h: int, w: int, device) -> torch.Tensor:
    """Scratch memory for sad_init_sites on an h x w target."""
    nb = int(_native.lib().sad_init_workspace_bytes(int(h), int(w)))
    return torch.empty(max(nb, 1), dtype=torch.uint8, device=device)


def init_sites(target: torch.Tensor, n: int, *, lam: float, seed: int, log_tau: float = 0.0, r: float = 0.0,
               log_scale: float = 0.0, params: torch.Tensor | None = None, derived: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """Gradient-weighted initialisation of n sites from the [h][w][3] target
    (see sad_init_sites); returns (params, derived)."""
    if target.dim() != 3 or target.shape[2] != 3:
        raise ValueError(f"target must have shape (h, w, 3), got {tuple(target.shape)}")
    h, w = int(target.shape[0]), int(target.shape[1])
    _need(target, "target", torch.float32, (h, w, 3))
    dev = target.device
    if params is None:
        params = torch.empty((n, REC), dtype=torch.float32, device=dev)
    if derived is None:
        derived = torch.empty((n, REC), dtype=torch.float32, device=dev)
    _need(params, "params", torch.float32, (n, REC))
    _need(derived, "derived", torch.float32, (n, REC))
    if workspace is None:
        workspace = init_workspace(h, w, dev)
    st = _native.lib().sad_init_sites(_ptr(target), h, w, int(n), float(lam), int(seed) & (2 ** 64 - 1),
                                      float(log_tau), float(r), float(log_scale), _ptr(params), _ptr(derived),
                                      _ptr(workspace), workspace.numel(), _stream(target))
    _native.check("sad_init_sites", st)
    return params, derived


NQP = 10  # per-image parameters of the packed records


def pack_sites(params: torch.Tensor, derived: torch.Tensor, h: int, w: int, packed: torch.Tensor | None = None,
               qparams: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """Packed 16-byte evaluation records ([n][4] int32 holding uint32 words)
    and their per-image parameters (float32[10]); see sad_pack_sites."""
    n = params.shape[0]
    _need(params, "params", torch.float32, (n, REC))
    _need(derived, "derived", torch.float32, (n, REC))
    if packed is None:
        packed = torch.empty((n, 4), dtype=torch.int32, device=params.device)
    if qparams is None:
        qparams = torch.empty(NQP, dtype=torch.float32, device=params.device)
    _need(packed, "packed", torch.int32, (n, 4))
    _need(qparams, "qparams", torch.float32, (NQP,))
    st = _native.lib().sad_pack_sites(_ptr(params), _ptr(derived), n, h, w, _ptr(packed), _ptr(qparams),
                                      _stream(params))
    _native.check("sad_pack_sites", st)
    return packed, qparams


def query_packed(packed: torch.Tensor, qparams: torch.Tensor, h: int, w: int, topk: torch.Tensor, xy: torch.Tensor,
                 rgb: torch.Tensor | None = None) -> torch.Tensor:
    """Colours at points [m][2] from packed records (see sad_query_packed)."""
    n = packed.shape[0]
    _need(packed, "packed", torch.int32, (n, 4))
    _need(qparams, "qparams", torch.float32, (NQP,))
    _need(topk, "topk", torch.int32, (h, w, K))
    m = xy.shape[0]
    _need(xy, "xy", torch.float32, (m, 2))
    if rgb is None:
        rgb = torch.empty((m, 3), dtype=torch.float32, device=xy.device)
    _need(rgb, "rgb", torch.float32, (m, 3))
    st = _native.lib().sad_query_packed(_ptr(packed), _ptr(qparams), n, h, w, _ptr(topk), _ptr(xy), m, _ptr(rgb),
                                        _stream(xy))
    _native.check("sad_query_packed", st)
    return rgb


JFA_K = 4  # ids per pixel in the JFA prepass


def jfa_steps(h: int, w: int) -> list[int]:
    """Jump steps of a JFA round: B/2, B/4, ..., 1, B the smallest power of two >= max(h, w)."""
    b = 1
    while b < max(h, w):
        b *= 2
    steps, s = [], b // 2
    while s >= 1:
        steps.append(s)
        s //= 2
    return steps


def jfa_seed(derived: torch.Tensor, h: int, w: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """Seed pass of the JFA prepass into ``out`` ([h][w][4] int32)."""
    n = derived.shape[0]
    _need(derived, "derived", torch.float32, (n, REC))
    if out is None:
        out = torch.empty((h, w, JFA_K), dtype=torch.int32, device=derived.device)
    _need(out, "out", torch.int32, (h, w, JFA_K))
    _native.check("sad_jfa_seed", _native.lib().sad_jfa_seed(_ptr(derived), n, h, w, _ptr(out), _stream(derived)))
    return out


def jfa_flood(derived: torch.Tensor, h: int, w: int, prev: torch.Tensor, step: int, out_width: int = JFA_K,
              out: torch.Tensor | None = None) -> torch.Tensor:
    """One flood pass of the JFA prepass; ``out`` is [h][w][4], or with
    out_width 8 a top-K map [h][w][8]."""
    n = derived.shape[0]
    _need(derived, "derived", torch.float32, (n, REC))
    _need(prev, "prev", torch.int32, (h, w, JFA_K))
    if out is None:
        out = torch.empty((h, w, out_width), dtype=torch.int32, device=derived.device)
    _need(out, "out", torch.int32, (h, w, out_width))
    _native.check("sad_jfa_flood", _native.lib().sad_jfa_flood(_ptr(derived), n, h, w, _ptr(prev), _ptr(out),
                                                                int(step), int(out_width), _stream(derived)))
    return out


def widen_map(topk16: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """The lists of an int16 (16-bit-id) map as an int32 map (sad_widen_map)."""
    h, w = int(topk16.shape[0]), int(topk16.shape[1])
    _need(topk16, "topk16", torch.int16, (h, w, K))
    if out is None:
        out = torch.empty((h, w, K), dtype=torch.int32, device=topk16.device)
    _need(out, "out", torch.int32, (h, w, K))
    st = _native.lib().sad_widen_map(_ptr(topk16), h, w, _ptr(out), _stream(topk16))
    _native.check("sad_widen_map", st)
    return out


def step_fused(derived: torch.Tensor, h: int, w: int, prev: torch.Tensor | None, out: torch.Tensor,
               target: torch.Tensor, grad: torch.Tensor, *, stride: int, seed: int, pass_index: int,
               inject: int = 64, prev_scores: torch.Tensor | None = None, out_scores: torch.Tensor | None = None,
               loss: torch.Tensor | None = None, image: torch.Tensor | None = None,
               prev_thr: torch.Tensor | None = None, prev_probe: torch.Tensor | None = None) -> torch.Tensor:
    """propagate_topk(...) into ``out`` followed by render_bwd over ``out``, in
    one call (both launches checked before either is enqueued).  ``prev`` may
    be an int16 map (16-bit ids) and come with ``prev_thr`` (each list's 8th
    logit) instead of ``prev_scores``, and the pass may read the sites' probe
    records ``prev_probe``; ``out`` has 32-bit ids, or 16-bit ones (an int16
    map, n <= 65535) for the next step's first pass."""
    n = derived.shape[0]
    _need(derived, "derived", torch.float32, (n, REC))
    maps = _pass_maps(h, w, n, prev, prev_scores, prev_thr, prev_probe, out, out_scores, None, None)
    _need(target, "target", torch.float32, (h, w, 3))
    _need(grad, "grad", torch.float32, (n, REC))
    if loss is not None:
        _need(loss, "loss", torch.float32, (1,))
    if image is not None:
        _need(image, "image", torch.float32, (h, w, 3))
    tail = (int(stride), int(seed) & 0xFFFFFFFFFFFFFFFF, int(pass_index) & 0xFFFFFFFF, int(inject), _ptr(target),
            _ptr(grad), _ptr(loss), _ptr(image), _stream(derived))
    if maps.prev_bits == 32 and maps.next_bits == 32 and not (maps.thr_prev or maps.probe_prev):
        st = _native.lib().sad_step_fused(_ptr(derived), n, h, w, _ptr(prev), _ptr(prev_scores), _ptr(out),
                                          _ptr(out_scores), *tail)
        _native.check("sad_step_fused", st)
    else:
        st = _native.lib().sad_step_fused_pass(_ptr(derived), n, h, w, C.byref(maps), *tail)
        _native.check("sad_step_fused_pass", st)
    return out


def adam_step(params: torch.Tensor, grad: torch.Tensor, m: torch.Tensor, v: torch.Tensor, h: int, w: int,
              lr: Sequence[float], beta1: float, beta2: float, eps: float, bias_corr1: float, bias_corr2: float,
              derived: torch.Tensor | None = None, probe: torch.Tensor | None = None) -> None:
    """One Adam step; ``derived`` (optional) receives the new prepared
    records and ``probe`` (optional, [n][4] float32, needs ``derived``) the
    sites' probe records from them (sad_adam_step_probe)."""
    n = params.shape[0]
    for t, name in ((params, "params"), (grad, "grad"), (m, "m"), (v, "v")):
        _need(t, name, torch.float32, (n, REC))
    if derived is not None:
        _need(derived, "derived", torch.float32, (n, REC))
    if probe is not None:
        _need(probe, "probe", torch.float32, (n, 4))
    lr_arr = (C.c_float * 5)(*[float(x) for x in lr])
    st = _native.lib().sad_adam_step_probe(_ptr(params), _ptr(grad), _ptr(m), _ptr(v), n, h, w, lr_arr, beta1, beta2,
                                           eps, bias_corr1, bias_corr2, _ptr(derived), _ptr(probe), _stream(params))
    _native.check("sad_adam_step_probe", st)


def query_points(derived: torch.Tensor, h: int, w: int, topk: torch.Tensor, xy: torch.Tensor,
                 rgb: torch.Tensor | None = None) -> torch.Tensor:
    n = derived.shape[0]
    m = xy.shape[0]
    _need(derived, "derived", torch.float32, (n, REC))
    _need(topk, "topk", torch.int32, (h, w, K))
    _need(xy, "xy", torch.float32, (m, 2))
    if rgb is None:
        rgb = torch.empty((m, 3), dtype=torch.float32, device=derived.device)
    _need(rgb, "rgb", torch.float32, (m, 3))
    st = _native.lib().sad_query_points(_ptr(derived), n, h, w, _ptr(topk), _ptr(xy), m, _ptr(rgb),
                                        _stream(derived))
    _native.check("sad_query_points", st)
    return rgb


def jfa_strides(h: int, w: int, n_pass: int) -> list[int]:
    """Jump steps of the warm-up schedule (Sec. 4.3): B/2, B/4, ..., 1, then 1,
    with B the smallest power of two >= max(h, w)."""
    b = 1
    while b < max(h, w):
        b *= 2
    lb = b.bit_length() - 1
    return [max(1, b >> (min(t, max(lb - 1, 0)) + 1)) for t in range(n_pass)]
