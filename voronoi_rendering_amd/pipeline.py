"""A GPU-resident SAD fitting loop built from the C-ABI calls.

One training iteration (Sec. 5: no CPU work inside the loop besides launches)
is: propagation passes over the top-K map, the forward + backward render that
accumulates the site gradients and the loss, and the Adam step that also
rewrites the prepared site records.  The map lives in two ping-pong buffers
because a pass only reads the previous map.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Sequence

import torch

from . import ops


@dataclass
class AdamConfig:
    lr: tuple = (1e-3, 1e-3, 1e-3, 1e-3, 1e-3)  # (x, y), log tau, r, colour, (theta, log s1, log s2)
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8


def bias_corrections(beta1: float, beta2: float, t: int) -> tuple[float, float]:
    """1 - beta^t for Adam step t, computed on the host in float64 and handed
    to the kernel as float32."""
    import numpy as np

    return float(np.float32(1.0 - float(beta1) ** t)), float(np.float32(1.0 - float(beta2) ** t))


@dataclass
class BudgetSchedule:
    """When and how much budget control a fit runs (Sec. 4.5; the pages leave
    the numbers open): at iterations start, start + every, ... up to stop, split
    n_split and prune n_prune sites with the budget step's constants, then
    rebuild the lists from the sites (a JFA round and refresh_passes
    propagation passes), since the new sites are in no list yet."""
    every: int = 100
    start: int = 100
    stop: int = 800
    n_split: int = 0
    n_prune: int = 0
    alpha: float = 1.0
    min_mass: float = 1.0
    offset: float = 0.5
    r_scale: float = 0.85
    logtau_shift: float = 0.1
    refresh_passes: int = 4

    def due(self, it: int) -> bool:
        return self.start <= it <= self.stop and (it - self.start) % self.every == 0


@dataclass
class SadField:
    params: torch.Tensor  # [n][12] float32 on the GPU
    h: int
    w: int
    seed: int
    inject: int = 64
    adam: AdamConfig = field(default_factory=AdamConfig)

    def __post_init__(self):
        dev = self.params.device
        n = self.params.shape[0]
        self.derived = ops.prepare_sites(self.params)
        self.grad = torch.zeros((n, ops.REC), dtype=torch.float32, device=dev)
        self.m = torch.zeros_like(self.grad)
        self.v = torch.zeros_like(self.grad)
        self.maps = [ops.empty_map(self.h, self.w, dev), ops.empty_map(self.h, self.w, dev)]
        # logits of each map's entries, valid while the sites do not change
        self.scores = [torch.empty((self.h, self.w, ops.K), dtype=torch.float32, device=dev) for _ in range(2)]
        self.scores_valid = False
        # 16-bit-id maps and 8th-logit maps through which a step's passes hand
        # on their lists (made on first use; only when every id fits in 16 bits)
        self.inter = None  # the maps a step's passes hand on (int16 ids when n <= 65535)
        self.thr = None
        self.probe = None  # [n][4] probe records of the sites (a step's first pass or the Adam step writes them)
        self.probe_valid = False  # whether they are those of the current prepared sites
        # a training step's last pass hands its lists to the next step at width 16
        # (when every id fits): then map16 holds the current lists and
        # maps[cur] is refreshed from it only when a 32-bit map is asked for
        self.map16 = None
        self.cur16 = False
        self.cur = 0
        self.pass_index = 0
        self.adam_t = 0
        self.loss = torch.zeros(1, dtype=torch.float32, device=dev)
        self._jfa = None  # ping-pong 4-lists of the JFA prepass, made on first use

    @classmethod
    def from_target(cls, target: torch.Tensor, n: int, *, lam: float, seed: int, log_tau: float = 0.0,
                    r: float = 0.0, log_scale: float = 0.0, **kw) -> "SadField":
        """A field of n sites drawn from the gradient-weighted density of the
        [h][w][3] target (Sec. 4.4; see ops.init_sites); ``seed`` also seeds
        the probes."""
        params, _ = ops.init_sites(target, n, lam=lam, seed=seed, log_tau=log_tau, r=r, log_scale=log_scale)
        return cls(params, int(target.shape[0]), int(target.shape[1]), seed, **kw)

    @property
    def topk(self) -> torch.Tensor:
        """The current lists as a 32-bit-id map."""
        return self._map32()

    def _map32(self) -> torch.Tensor:
        """maps[cur], first widened from map16 when a step's last pass left
        the current lists there."""
        if self.cur16:
            ops.widen_map(self.map16, self.maps[self.cur])
            self.cur16 = False
        return self.maps[self.cur]

    def propagate(self, strides: Sequence[int]) -> None:
        if strides:
            self._map32()  # the passes below read and write the 32-bit maps
        for s in strides:
            ops.propagate_topk(self.derived, self.h, self.w, self.maps[self.cur], self.maps[1 - self.cur],
                               stride=int(s), seed=self.seed, pass_index=self.pass_index, inject=self.inject,
                               prev_scores=self.scores[self.cur] if self.scores_valid else None,
                               out_scores=self.scores[1 - self.cur])
            self.cur = 1 - self.cur
            self.pass_index += 1
            self.scores_valid = True

    def sites_changed(self, probe_records_current: bool = False) -> None:
        """The prepared sites were rewritten: the cached logits are stale, and
        so are the probe records unless they were rewritten with the sites
        (``probe_records_current``, as the Adam step does)."""
        self.scores_valid = False
        self.probe_valid = self.probe_valid and probe_records_current

    def warm(self, n_pass: int) -> None:
        """Fill the map from scratch with the warm-up jump schedule."""
        self.propagate(ops.jfa_strides(self.h, self.w, n_pass))

    def densify_prune(self, target: torch.Tensor, **budget) -> torch.Tensor:
        """Budget control over the current map: the per-site statistics, then
        prune and split (keyword arguments as ops.densify_prune).  Returns the
        numbers pruned and split (device int32[2])."""
        stats = ops.site_stats(self.derived, self.h, self.w, self.topk, target)
        done = ops.densify_prune(self.params, self.m, self.v, self.derived, self.h, self.w, stats, target, **budget)
        self.sites_changed()
        return done

    def refresh(self, n_pass: int = 16) -> None:
        """Rebuild the map from the sites alone (the render protocol of Sec. 6.6):
        one JFA round (seed, then flood passes B/2, ..., 1, the last one writing
        the top-K map), then n_pass propagation passes on the warm-up schedule."""
        steps = ops.jfa_steps(self.h, self.w)
        self.cur16 = False  # the lists are rebuilt into maps[cur]
        if not steps:  # a 1x1 image: the seed alone
            self.maps[self.cur].fill_(-1)
            self.maps[self.cur][..., :ops.JFA_K] = ops.jfa_seed(self.derived, self.h, self.w)
        else:
            if self._jfa is None:
                self._jfa = [torch.empty((self.h, self.w, ops.JFA_K), dtype=torch.int32, device=self.params.device)
                             for _ in range(2)]
            a, b = self._jfa
            ops.jfa_seed(self.derived, self.h, self.w, a)
            for t, s in enumerate(steps):
                if t == len(steps) - 1:
                    ops.jfa_flood(self.derived, self.h, self.w, a, s, ops.K, self.maps[self.cur])
                else:
                    ops.jfa_flood(self.derived, self.h, self.w, a, s, ops.JFA_K, b)
                    a, b = b, a
        self.scores_valid = False
        self.propagate(ops.jfa_strides(self.h, self.w, n_pass))

    def forward_backward(self, target: torch.Tensor, image: torch.Tensor | None = None) -> None:
        ops.render_bwd(self.derived, self.h, self.w, self.topk, target, self.grad, self.loss, image)

    def step(self, strides: Sequence[int], target: torch.Tensor, fused: bool = True,
             before_last: Callable[[], None] | None = None) -> None:
        """Propagation passes + forward + backward (gradients accumulate).  With
        ``fused`` the last pass and the backward run as one call, and
        ``before_last`` (if given) is called between the enqueueing of the other
        passes and of that call (a place for timing events)."""
        if not fused or len(strides) == 0:
            self.propagate(strides)
            self.forward_backward(target)
            return
        n = self.params.shape[0]
        probe = None
        out = self.maps[1 - self.cur]
        if len(strides) < 2:
            prev, prev_thr = self._map32(), None
            prev_scores = self.scores[self.cur] if self.scores_valid else None
        else:
            # the passes before the last hand their lists on with only each
            # list's 8th logit, and with 16-bit ids when every id fits (20
            # instead of 64 bytes per pixel each way; 36 with 32-bit ids); the
            # passes cull their probes from the sites' probe records, which the
            # first pass writes unless the Adam step already has
            dev = self.params.device
            dt = torch.int16 if n <= 0xFFFF else torch.int32
            if self.inter is None or self.inter[0].dtype != dt:
                self.inter = [torch.empty((self.h, self.w, ops.K), dtype=dt, device=dev) for _ in range(2)]
            if self.thr is None:
                self.thr = [torch.empty((self.h, self.w), dtype=torch.float32, device=dev) for _ in range(2)]
            if self.probe is None or self.probe.shape[0] != n:
                self.probe = torch.empty((n, 4), dtype=torch.float32, device=dev)
                self.probe_valid = False
            probe = self.probe
            if self.cur16:  # the previous step's lists (their logits are recomputed)
                prev, prev_thr, prev_scores = self.map16, None, None
            else:
                prev, prev_thr = self.maps[self.cur], None
                prev_scores = self.scores[self.cur] if self.scores_valid else None
            for k, s in enumerate(strides[:-1]):
                out, out_thr = self.inter[k % 2], self.thr[k % 2]
                write = not self.probe_valid
                ops.propagate_topk(self.derived, self.h, self.w, prev, out, stride=int(s), seed=self.seed,
                                   pass_index=self.pass_index, inject=self.inject, prev_scores=prev_scores,
                                   prev_thr=prev_thr, out_thr=out_thr, prev_probe=None if write else probe,
                                   out_probe=probe if write else None)
                self.probe_valid = True
                prev, prev_scores, prev_thr = out, None, out_thr
                self.pass_index += 1
            if dt == torch.int16:
                # the last pass writes 16-bit lists for the next step's first pass
                # (the first pass has read map16 by then)
                if self.map16 is None:
                    self.map16 = torch.empty((self.h, self.w, ops.K), dtype=torch.int16, device=dev)
                out = self.map16
            else:
                out = self.maps[1 - self.cur]
        if before_last is not None:
            before_last()
        # The last pass's logits are not kept: a training iteration rewrites the
        # sites next, so the following pass recomputes them anyway.
        ops.step_fused(self.derived, self.h, self.w, prev, out, target, self.grad,
                       stride=int(strides[-1]), seed=self.seed, pass_index=self.pass_index, inject=self.inject,
                       prev_scores=prev_scores, out_scores=None, loss=self.loss, prev_thr=prev_thr,
                       prev_probe=probe)
        if out is self.map16:
            self.cur16 = True
        else:
            self.cur = 1 - self.cur
            self.cur16 = False
        self.pass_index += 1
        self.scores_valid = False

    def adam_step(self) -> None:
        self.adam_t += 1
        bc1, bc2 = bias_corrections(self.adam.beta1, self.adam.beta2, self.adam_t)
        # the probe records (once a step has made them) are rewritten with the
        # prepared sites, so the next step's first pass culls from them
        probe = self.probe if self.probe is not None and self.probe.shape[0] == self.params.shape[0] else None
        ops.adam_step(self.params, self.grad, self.m, self.v, self.h, self.w, self.adam.lr, self.adam.beta1,
                      self.adam.beta2, self.adam.eps, bc1, bc2, self.derived, probe)
        self.probe_valid = probe is not None
        self.sites_changed(probe_records_current=True)

    def train_iter(self, strides: Sequence[int], target: torch.Tensor, fused: bool = True) -> None:
        self.step(strides, target, fused)
        self.adam_step()

    def fit(self, target: torch.Tensor, iters: int, strides: Sequence[int],
            budget: BudgetSchedule | None = None) -> None:
        """iters training iterations (propagation passes, forward, backward,
        Adam), with budget control on the given schedule."""
        for it in range(1, iters + 1):
            self.train_iter(strides, target)
            if budget is not None and budget.due(it):
                self.budget_step(target, budget)

    def budget_step(self, target: torch.Tensor, budget: BudgetSchedule) -> torch.Tensor:
        """One scheduled budget step: statistics, prune and split, then the
        lists rebuilt from the sites.  Returns the numbers pruned and split."""
        done = self.densify_prune(target, n_split=budget.n_split, n_prune=budget.n_prune, alpha=budget.alpha,
                                  min_mass=budget.min_mass, offset=budget.offset, r_scale=budget.r_scale,
                                  logtau_shift=budget.logtau_shift)
        self.refresh(budget.refresh_passes)
        return done

    def active_sites(self) -> int:
        return int((self.params[:, 0] >= 0).sum())

    def render(self) -> torch.Tensor:
        return ops.render_fwd(self.derived, self.h, self.w, self.topk)
