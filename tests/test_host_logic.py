"""Host-side logic of the binding and the fitting loop, on the CPU: the jump
schedules, Adam's bias corrections, the budget schedule, and the refusal of
tensors that are not on the GPU (there is no CPU path)."""
import math

import numpy as np
import pytest
import torch

import synth
from voronoi_rendering_amd import ops
from voronoi_rendering_amd.pipeline import BudgetSchedule, bias_corrections


@pytest.mark.parametrize("h,w", [(1, 1), (1, 2), (3, 5), (64, 64), (512, 768), (2048, 2048), (45, 131), (1000, 3)])
def test_jfa_steps_halve_from_half_the_power_of_two(ref, h, w):
    b = 1 << math.ceil(math.log2(max(h, w)))
    want = [b >> k for k in range(1, int(math.log2(b)) + 1)]
    assert ops.jfa_steps(h, w) == want == ref.jfa_steps(h, w)


@pytest.mark.parametrize("h,w,n", [(64, 64, 20), (512, 768, 16), (2048, 2048, 21), (1, 1, 3), (5, 3, 6)])
def test_warm_up_schedule(h, w, n):
    """s_t = max(1, B / 2^(min(t, log2 B - 1) + 1)): halving from B/2, then 1."""
    b = 1 << math.ceil(math.log2(max(h, w)))
    lb = int(math.log2(b))
    want = [max(1, b // 2 ** (min(t, max(lb - 1, 0)) + 1)) for t in range(n)]
    assert ops.jfa_strides(h, w, n) == want == synth.jfa_strides(h, w, n)


@pytest.mark.parametrize("t", [1, 2, 10, 1000])
def test_bias_corrections_match_the_oracle(ref, t):
    assert bias_corrections(0.9, 0.999, t) == ref.bias_corrections(0.9, 0.999, t)
    assert bias_corrections(0.9, 0.999, t)[0] == np.float32(1 - 0.9 ** t)


def test_budget_schedule():
    b = BudgetSchedule(every=100, start=100, stop=800)
    due = [it for it in range(1, 1001) if b.due(it)]
    assert due == list(range(100, 801, 100))
    assert [it for it in range(1, 30) if BudgetSchedule(every=5, start=3, stop=20).due(it)] == [3, 8, 13, 18]


def test_cpu_tensors_are_refused():
    p = torch.zeros((4, 12), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU"):
        ops.prepare_sites(p)
    with pytest.raises(ValueError, match="GPU"):
        ops.render_fwd(p, 2, 2, torch.zeros((2, 2, 8), dtype=torch.int32))


class _Recorder:
    """Stands in for the binding's calls (no GPU here): records which maps and
    probe records each call reads and writes."""

    def __init__(self):
        self.calls = []

    def prepare_sites(self, params, derived=None):
        return torch.zeros_like(params)

    def empty_map(self, h, w, device="cpu"):
        return torch.full((h, w, ops.K), -1, dtype=torch.int32)

    def propagate_topk(self, derived, h, w, prev, out, **kw):
        self.calls.append(("pass", prev, out, kw.get("prev_probe"), kw.get("out_probe")))
        return out

    def step_fused(self, derived, h, w, prev, out, target, grad, **kw):
        self.calls.append(("fused", prev, out, kw.get("prev_probe"), None))
        return out

    def adam_step(self, params, grad, m, v, h, w, lr, b1, b2, eps, bc1, bc2, derived=None, probe=None):
        self.calls.append(("adam", None, None, None, probe))

    def widen_map(self, topk16, out=None):
        self.calls.append(("widen", topk16, out, None, None))
        return out


@pytest.mark.parametrize("n", [1000, 70000])
def test_field_hand_off_bookkeeping(monkeypatch, n):
    """The fitting loop's hand-off between steps: the last pass writes a
    16-bit map (n <= 65535) that the next step's first pass reads, the field
    widens it only when a 32-bit map is asked for; the first pass writes the
    probe records unless the Adam step has rewritten them with the sites, and
    a change of the sites by other means makes the next step write them again."""
    from voronoi_rendering_amd import pipeline

    rec = _Recorder()
    for name in ("prepare_sites", "empty_map", "propagate_topk", "step_fused", "adam_step", "widen_map"):
        monkeypatch.setattr(pipeline.ops, name, getattr(rec, name))
    f = pipeline.SadField(torch.zeros((n, ops.REC)), 16, 24, 5)
    tgt = torch.zeros((16, 24, 3))
    small = n <= 0xFFFF
    strides = [8, 4, 2, 1]

    f.step(strides, tgt)
    (k0, p0, o0, pp0, op0), *mid, (kf, pf, of, ppf, _) = rec.calls
    assert k0 == "pass" and p0 is f.maps[0] and pp0 is None and op0 is f.probe  # records written
    assert all(c[0] == "pass" and c[3] is f.probe and c[4] is None for c in mid)  # and read
    assert kf == "fused" and ppf is f.probe and pf is mid[-1][2]
    assert f.cur16 == small and (of is f.map16 if small else of is f.maps[1] and f.cur == 1)

    f.adam_step()
    assert rec.calls[-1][0] == "adam" and rec.calls[-1][4] is f.probe and f.probe_valid
    rec.calls.clear()
    f.step(strides, tgt)
    first = rec.calls[0]
    assert first[3] is f.probe and first[4] is None  # culled from the Adam step's records
    assert first[1] is (f.map16 if small else f.maps[1])
    assert not any(c[0] == "widen" for c in rec.calls)

    rec.calls.clear()
    m = f.topk
    assert [c[0] for c in rec.calls] == (["widen"] if small else [])
    assert m is f.maps[f.cur] and not f.cur16
    if small:
        assert rec.calls[0][1] is f.map16 and rec.calls[0][2] is m

    f.sites_changed()  # e.g. a budget step: the probe records are stale
    assert not f.probe_valid
    rec.calls.clear()
    f.step(strides, tgt)
    assert rec.calls[0][1] is m and rec.calls[0][3] is None and rec.calls[0][4] is f.probe
