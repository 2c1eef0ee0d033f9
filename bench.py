"""Throughput of the SAD hot path on one MI355X.

Workload (default): 768x512 RGB float32 target, 50,000 sites, K = 8.  One
step = 4 top-K propagation passes (strides 8, 4, 2, 1, 64 injected sites per
8x8 tile) + forward render + backward with the loss.  The timed map is a
settled one: built by the full refresh (a JFA round and 16 passes) and then
500 untimed steps, so that the lists are the exact top-8 almost everywhere,
as in a fit after its first iterations.  The timed steps run the last pass
and the backward as one call (sad_step_fused).  Metric: Mpixel-iters/s =
H*W per step / step time.  All inputs are synthetic (synth.C2) and already
resident in GPU memory when the timed region starts.

The first pass of each step recomputes the logits of the pixels' previous
lists (as after an Adam update, which also rewrites the sites' probe
records, so that every pass culls its probes from them); the following
passes reuse the logits the previous pass wrote.  Every pass hands its lists on
with 16-bit ids (every id of the 50,000 fits): the last pass writes the 16-bit
map the next step's first pass reads.

Prints ONE JSON line.  Per-kernel durations come from HIP events in up to 50
further steps made of the same launches, on the stream the kernels run on
(torch's current stream): one event pair around a step's first passes, one
around its last pass + backward kernel.  The per-stride figures time single
passes on 32-bit maps, and the standalone backward, one event pair each.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def algorithmic_bytes(h: int, w: int, n: int, n_pass: int) -> dict:
    """Bytes the method must move (not counting re-reads served by caches).
    propagate:  read + write one 32-byte list per pixel per pass.
    render_bwd: read list (32 B) + target (12 B) per pixel, read the 48-byte
                prepared record and read-modify-write the 40-byte gradient
                record (80 B) per site.
    step_last:  the last pass and the backward in one kernel: read + write
                the list (64 B) + the target (12 B) per pixel, 128 B per site.
    step:       the whole step with the last list handed from the pass to the
                backward: 64 B per pixel per pass + the target + 128 B per site."""
    p = h * w
    prop = 64 * p
    bwd = p * (32 + 12) + n * (48 + 80)
    last = p * (64 + 12) + n * 128
    step = n_pass * 64 * p + 12 * p + n * 128
    return {"propagate": prop, "render_bwd": bwd, "step_last": last, "step": step}


KERNEL_OF = {"propagate": "k_propagate", "render_bwd": "k_backward", "step_last": "k_step_last"}


def counter_record(kind: str):
    """The kernel's entry of the committed rocprofv3 counter summary, or None
    when the kernel's sources changed since the counters were taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "hbm_counters_768x512.json")
    try:
        data = json.load(open(path))
        rec = data["kernels"][KERNEL_OF[kind]]
        h = hashlib.sha256()
        for f in rec["sources"]:
            h.update(open(os.path.join(ROOT, f), "rb").read())
        return rec if h.hexdigest() == rec["source_sha256"] else None
    except (OSError, KeyError, ValueError):
        return None


def measured_traffic(kind: str):
    """HBM bytes per launch of the kernel (scaled FETCH_SIZE + WRITE_SIZE), or None."""
    rec = counter_record(kind)
    return int(rec["bytes"]) if rec else None


# Vector ALU issue peak: the published fp32 vector peak (157.3 TFLOP/s, an FMA
# counted as two flops) in lane-operations: 256 CUs x 4 SIMDs x 32 lanes per
# clock at 2.4 GHz, i.e. a wave64 fp32 instruction every 2 cycles per SIMD.  A
# kernel of nothing but independent v_fma_f32 reaches about 51 T of it on the
# MI355X (its clock under that load reads about 2.1 GHz).
VALU_PEAK_T = 157.3 / 2


def valu_roofline(kind: str, seconds: float):
    """Vector-ALU lane-operations per second of the kernel (instructions per
    wavefront and wavefronts per launch from the counter summary, duration
    measured live) against the issue peak, or None without valid counters.
    Every VALU instruction counts as 64 lane-operations (float64 and
    transcendental instructions take longer to issue, so for a kernel with
    many of them the fraction understates how busy the ALU is)."""
    rec = counter_record(kind)
    if not rec or "valu_insts_per_wave" not in rec:
        return None
    ops = rec["valu_insts_per_wave"] * rec["waves_per_dispatch"] * 64
    ach = ops / seconds / 1e12
    return {"bound": "alu", "achieved": round(ach, 2), "peak": round(VALU_PEAK_T, 2), "unit": "T lane-op/s",
            "frac": round(ach / VALU_PEAK_T, 4), "valu_insts_per_wave": round(rec["valu_insts_per_wave"], 1),
            "valu_busy_pct_counter": round(rec["valu_busy_pct"], 1), "kernel": kind}


def cpu_baseline(wl, budget_s: float) -> dict:
    """The oracle as it stands, timed on the host cores on whole C2 steps
    (4 passes + backward over the full image) until ~budget_s seconds."""
    import numpy as np

    import oracle as ref
    import synth

    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    ref.set_threads(threads)
    p = wl.make_sites()
    tgt = wl.make_target()
    d = ref.prepare_sites(p)
    warm = synth.jfa_strides(wl.h, wl.w, wl.warm_passes)
    cur = ref.propagate_schedule(d, wl.h, wl.w, None, warm, wl.inject_seed, 0, wl.inject)
    pi = len(warm)
    steps = 0
    t0 = time.perf_counter()
    while True:
        cur = ref.propagate_schedule(d, wl.h, wl.w, cur, wl.strides, wl.inject_seed, pi, wl.inject)
        pi += len(wl.strides)
        ref.render_bwd(d, wl.h, wl.w, cur, tgt)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    value = wl.h * wl.w * steps / el / 1e6
    return {"value": round(value, 4), "unit": "Mpixel-iters/s", "cores": threads, "kind": "oracle",
            "sample": f"{steps} full {wl.w}x{wl.h} steps (4 passes + forward/backward), {el:.1f} s, "
                      f"{threads} OpenMP threads"}


def cpu_other(include_2048: bool) -> dict:
    """The oracle on the other workloads: the 64x64 run (20 passes from an
    empty map + backward), 2^20 of the 2^24 random queries on the 768x512
    query map (rate extrapolated linearly), one 768x512 step on one thread,
    and with include_2048 one 2048x2048 step after the oracle's own 16-pass
    warm-up (about a minute)."""
    import oracle as ref
    import synth

    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    ref.set_threads(threads)
    out = {"cores": threads, "kind": "oracle"}
    wl = synth.C1
    d = ref.prepare_sites(wl.make_sites())
    tgt = wl.make_target()
    t0 = time.perf_counter()
    m = ref.propagate_schedule(d, wl.h, wl.w, None, wl.strides, wl.inject_seed, 0, wl.inject)
    ref.render_bwd(d, wl.h, wl.w, m, tgt)
    out["run_64x64_ms"] = round((time.perf_counter() - t0) * 1e3, 2)
    wl = synth.C5
    d = ref.prepare_sites(wl.make_sites())
    m = ref.propagate_schedule(d, wl.h, wl.w, None, synth.jfa_strides(wl.h, wl.w, wl.warm_passes), wl.inject_seed,
                               0, wl.inject)
    xy = wl.make_queries(1 << 20)
    t0 = time.perf_counter()
    ref.query_points(d, wl.h, wl.w, m, xy)
    out["query_Mqueries_per_s"] = round((1 << 20) / (time.perf_counter() - t0) / 1e6, 3)
    out["query_sample"] = "2^20 of the 2^24 points, rate extrapolated linearly"
    # one whole 768x512 step on a single thread, beside the all-core figure
    wl = synth.C2
    d = ref.prepare_sites(wl.make_sites())
    tgt = wl.make_target()
    m = ref.propagate_schedule(d, wl.h, wl.w, None, synth.jfa_strides(wl.h, wl.w, wl.warm_passes), wl.inject_seed,
                               0, wl.inject)
    ref.set_threads(1)
    t0 = time.perf_counter()
    m = ref.propagate_schedule(d, wl.h, wl.w, m, wl.strides, wl.inject_seed, wl.warm_passes, wl.inject)
    ref.render_bwd(d, wl.h, wl.w, m, tgt)
    out["step_768x512_one_thread_Mpixel_iters_per_s"] = round(wl.h * wl.w / (time.perf_counter() - t0) / 1e6, 4)
    ref.set_threads(threads)
    if include_2048:
        wl = synth.C4
        d = ref.prepare_sites(wl.make_sites())
        tgt = wl.make_target()
        m = ref.propagate_schedule(d, wl.h, wl.w, None, synth.jfa_strides(wl.h, wl.w, wl.warm_passes),
                                   wl.inject_seed, 0, wl.inject)
        t0 = time.perf_counter()
        m = ref.propagate_schedule(d, wl.h, wl.w, m, wl.strides, wl.inject_seed, wl.warm_passes, wl.inject)
        ref.render_bwd(d, wl.h, wl.w, m, tgt)
        out["step_2048x2048_Mpixel_iters_per_s"] = round(wl.h * wl.w / (time.perf_counter() - t0) / 1e6, 4)
    return out


INIT = {"lam": 0.3, "log_tau": 0.0, "r": 0.0, "log_scale": 0.7}  # encode from the gradient-weighted density


def encode_run(torch, synth, SadField, wl, tgt, iters: int, init: dict | None = None, n0: int | None = None,
               budget=None) -> dict:
    """The training workload end to end: wall clock from the initial
    parameters in device memory (or, with ``init``, from the target alone:
    the gradient-weighted draw of the sites is inside the clock), site
    preparation, the first map (16 passes from empty, or a full refresh for
    drawn sites), then ``iters`` iterations of propagate +
    forward + backward + Adam, to the last kernel's end; then an untimed
    second run of the same iterations that renders the fit at a few
    iterations for its PSNR against the target.  ``n0`` sites are drawn
    (default: the workload's count) and ``budget`` is the fit's
    budget-control schedule."""
    strides = list(wl.strides)

    def build_map(f):
        # from drawn sites the pages' full refresh; from given sites 16 passes from an empty map
        if init is not None:
            f.refresh(wl.warm_passes)
        else:
            f.warm(wl.warm_passes)

    def start():
        if init is not None:
            return SadField.from_target(tgt, n0 or wl.n, seed=wl.inject_seed, inject=wl.inject, **init)
        return SadField(p0.clone(), wl.h, wl.w, wl.inject_seed, inject=wl.inject)

    p0 = torch.from_numpy(wl.make_sites()).to("cuda") if init is None else None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    f = start()
    build_map(f)
    f.fit(tgt, iters, strides, budget)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    del f
    f = start()
    build_map(f)
    psnr = {}
    marks = {1, 10, 100, iters}
    for it in range(1, iters + 1):
        f.train_iter(strides, tgt)
        if budget is not None and budget.due(it):  # the same schedule, one iteration at a time
            f.budget_step(tgt, budget)
        if it in marks:  # the updated sites over the iteration's map
            mse = float(((f.render() - tgt) ** 2).mean())
            psnr[str(it)] = round(10.0 * math.log10(1.0 / mse), 3)
    first = "a full refresh (JFA round, 16 passes)" if init is not None else "16 passes from an empty map"
    out = {"s": round(wall, 4), "ms_per_iteration": round(wall / iters * 1e3, 4), "psnr_db_at_iteration": psnr,
           "note": f"setup, {first} and all iterations inside the wall clock"}
    if init is not None:
        out["init"] = dict(init, sites=n0 or wl.n,
                           note="sites drawn from the target's gradient-weighted density inside the clock")
    if budget is not None:
        out["budget"] = {"every": budget.every, "start": budget.start, "stop": budget.stop, "n_split": budget.n_split,
                         "n_prune": budget.n_prune, "refresh_passes": budget.refresh_passes,
                         "final_sites": f.active_sites()}
    return out


# The pages' per-call times of the same protocol on an NVIDIA RTX 5090 at 1.0
# bits per pixel (Table 8: full refresh = one JFA round + 16 propagation
# passes + render; Table 9: the stages), in ms.  Context only: other
# hardware, and site counts set by the pages' bit budget rather than these.
PAGES_REFRESH_MS = {512: {"total": 1.100, "render": 0.015, "passes16": 0.728, "pass1": 0.053},
                    1024: {"total": 4.614, "render": 0.034, "passes16": 2.568, "pass1": 0.168},
                    2048: {"total": 26.539, "render": 0.132, "passes16": 16.009, "pass1": 1.006}}


def refresh_timings(torch, synth, ops, SadField) -> dict:
    """The render protocol from the sites alone at 512^2, 1024^2 and 2048^2
    (site density of the 2048^2 workload: 25k, 100k, 400k sites): one JFA
    round, 16 propagation passes, the render, and for comparison one pass;
    HIP events on the launch stream, 10 warm-up + 30 timed calls, medians."""
    import numpy as np

    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream(dev)
    out = {}
    for side, n in ((512, 25_000), (1024, 100_000), (2048, 400_000)):
        p = torch.from_numpy(synth.sites(7000 + side, n, side, side, synth.WIDE_SCALES)).to(dev)
        f = SadField(p, side, side, 5000 + side)
        img = torch.empty((side, side, 3), dtype=torch.float32, device=dev)
        steps = ops.jfa_steps(side, side)
        strides16 = ops.jfa_strides(side, side, 16)
        rec = []
        for it in range(40):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
            ev[0].record(stream)
            f.refresh(0)  # the JFA round alone
            ev[1].record(stream)
            f.propagate(strides16)
            ev[2].record(stream)
            ops.render_fwd(f.derived, side, side, f.topk, img)
            ev[3].record(stream)
            f.sites_changed()
            f.propagate([1])
            ev[4].record(stream)
            if it >= 10:
                rec.append(ev)
        torch.cuda.synchronize()
        t = {k: [] for k in ("jfa_round", "passes16", "render", "pass1")}
        for ev in rec:
            for k, (a, b) in zip(t, ((0, 1), (1, 2), (2, 3), (3, 4))):
                t[k].append(ev[a].elapsed_time(ev[b]))
        med = {k: float(np.median(v)) for k, v in t.items()}
        out[f"{side}x{side}_{n // 1000}k"] = {
            "total_ms": round(med["jfa_round"] + med["passes16"] + med["render"], 4),
            "jfa_round_ms": round(med["jfa_round"], 4), "jfa_passes": len(steps) + 1,
            "passes16_ms": round(med["passes16"], 4), "render_ms": round(med["render"], 4),
            "pass1_ms": round(med["pass1"], 4), "pages_rtx5090_ms": PAGES_REFRESH_MS[side]}
        del f, p, img
    return out


def budget_timings(torch, synth, ops, SadField) -> dict:
    """The budget step on the 768x512 / 50k-site training workload after the
    warm-up passes: the statistics of the map, then prune and split 500 sites
    each; every timed call starts from the same copy of the sites (the copy is
    outside the events).  HIP events on the launch stream, 5 warm-up + 20
    timed calls, median."""
    import numpy as np

    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream(dev)
    wl = synth.C3
    f = SadField(torch.from_numpy(wl.make_sites()).to(dev), wl.h, wl.w, wl.inject_seed, inject=wl.inject)
    tgt = torch.from_numpy(wl.make_target()).to(dev)
    f.warm(wl.warm_passes)
    stats = ops.site_stats(f.derived, wl.h, wl.w, f.topk, tgt)
    ws = ops.budget_workspace(wl.n, dev)
    done = torch.zeros(2, dtype=torch.int32, device=dev)
    state = (f.params, f.m, f.v, f.derived)
    saved = [x.clone() for x in state]
    rec = []
    for it in range(25):
        for x, y in zip(state, saved):
            x.copy_(y)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        ops.densify_prune(*state, wl.h, wl.w, stats, tgt, n_split=500, n_prune=500, workspace=ws, done=done)
        ev[1].record(stream)
        if it >= 5:
            rec.append(ev)
    torch.cuda.synchronize()
    t = float(np.median([a.elapsed_time(b) for a, b in rec]))
    pruned, split = (int(x) for x in done.cpu())
    return {"us": round(t * 1e3, 2), "pruned": pruned, "split": split, "sites": wl.n,
            "note": "2 stable radix sorts over 50k keys, a stable select and 4 small kernels; launch- and latency-bound"}


def secondary(torch, synth, ops, SadField) -> dict:
    """The other workloads, timed briefly with inputs resident on the GPU (not
    the headline): the 2048x2048 / 400k-site step, a training iteration
    (step + Adam, the 768x512 training workload), the Adam step alone, the
    budget statistics pass and the budget step, the 1,000-iteration encode (from the
    synthetic sites and from a gradient-weighted draw), the draw alone, and 2^24
    random-access queries on a 768x512 / 50k-site map, from the float32 records
    and from the packed ones."""
    dev = torch.device("cuda", 0)

    def per_call(fn, reps):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3 / reps

    out = {}
    wl = synth.C1
    p1 = torch.from_numpy(wl.make_sites()).to(dev)
    tgt1 = torch.from_numpy(wl.make_target()).to(dev)

    def run1():
        f1 = SadField(p1, wl.h, wl.w, wl.inject_seed, inject=wl.inject)
        f1.step(list(wl.strides), tgt1, fused=True)

    t = per_call(run1, 20)
    out["run_64x64_20_passes"] = {"ms": round(t * 1e3, 4), "note": "launch-bound: 20 passes + backward, setup included"}
    wl = synth.C4
    f = SadField(torch.from_numpy(wl.make_sites()).to(dev), wl.h, wl.w, wl.inject_seed, inject=wl.inject)
    tgt = torch.from_numpy(wl.make_target()).to(dev)
    f.warm(wl.warm_passes)

    def step4():
        f.sites_changed(probe_records_current=True)  # as after an Adam update
        f.step(list(wl.strides), tgt, fused=True)

    t = per_call(step4, 10)
    out["step_2048x2048_400k"] = {"Mpixel_iters_per_s": round(wl.h * wl.w / t / 1e6, 1), "ms_per_step": round(t * 1e3, 4),
                                  "passes_per_step": len(wl.strides)}
    del f, tgt
    wl = synth.C3
    f = SadField(torch.from_numpy(wl.make_sites()).to(dev), wl.h, wl.w, wl.inject_seed, inject=wl.inject)
    tgt = torch.from_numpy(wl.make_target()).to(dev)
    f.warm(wl.warm_passes)
    t = per_call(lambda: f.train_iter(list(wl.strides), tgt), 50)
    out["training_iteration_768x512_50k"] = {"ms_per_iteration": round(t * 1e3, 4),
                                             "Mpixel_iters_per_s": round(wl.h * wl.w / t / 1e6, 1)}
    t = per_call(f.adam_step, 50)
    adam_bytes = 9 * 48 * wl.n  # params, grad, m, v read; params, m, v, grad, derived written
    out["adam_step_50k"] = {"us": round(t * 1e6, 2), "GB_per_s": round(adam_bytes / t / 1e9, 1),
                            "algorithmic_bytes": adam_bytes}
    stats = torch.zeros((wl.n, ops.NSTAT), dtype=torch.float32, device=dev)
    ws = ops.stats_workspace(wl.h, wl.w, dev)
    t = per_call(lambda: ops.site_stats(f.derived, wl.h, wl.w, f.topk, tgt, stats, ws), 20)
    stat_bytes = wl.h * wl.w * (32 + 12) + wl.n * (48 + 2 * 32)  # lists, target; records, stats read + written
    out["site_stats_768x512_50k"] = {"us": round(t * 1e6, 2), "GB_per_s": round(stat_bytes / t / 1e9, 1),
                                     "algorithmic_bytes": stat_bytes}
    del f, stats, ws
    out["densify_prune_768x512_50k"] = budget_timings(torch, synth, ops, SadField)
    out["encode_768x512_50k_1000_iterations"] = encode_run(torch, synth, SadField, wl, tgt, 1000)
    out["encode_768x512_50k_1000_iterations_gradient_init"] = encode_run(torch, synth, SadField, wl, tgt, 1000, INIT)
    from voronoi_rendering_amd.pipeline import BudgetSchedule

    prune = BudgetSchedule(every=100, start=100, stop=800, n_prune=6250)  # 100k drawn, 50k left after iteration 800
    out["encode_768x512_100k_to_50k_1000_iterations_budget"] = encode_run(torch, synth, SadField, wl, tgt, 1000, INIT,
                                                                          100_000, prune)
    ws = ops.init_workspace(wl.h, wl.w, dev)
    prm = torch.empty((wl.n, ops.REC), dtype=torch.float32, device=dev)
    drv = torch.empty_like(prm)
    t = per_call(lambda: ops.init_sites(tgt, wl.n, seed=7, params=prm, derived=drv, workspace=ws, **INIT), 20)
    out["init_sites_768x512_50k"] = {"us": round(t * 1e6, 2)}
    del ws, prm, drv
    del tgt
    wl = synth.C5
    f = SadField(torch.from_numpy(wl.make_sites()).to(dev), wl.h, wl.w, wl.inject_seed, inject=wl.inject)
    f.warm(wl.warm_passes)
    xy = torch.from_numpy(wl.make_queries()).to(dev)
    rgb = torch.empty((xy.shape[0], 3), dtype=torch.float32, device=dev)
    t = per_call(lambda: ops.query_points(f.derived, wl.h, wl.w, f.topk, xy, rgb), 5)
    m = xy.shape[0]
    out["query_2e24_points"] = {"Mqueries_per_s": round(m / t / 1e6, 1), "ms": round(t * 1e3, 3),
                                "GB_per_s_algorithmic": round(52 * m / t / 1e9, 1)}
    pk, qp = ops.pack_sites(f.params, f.derived, wl.h, wl.w)
    tp = per_call(lambda: ops.pack_sites(f.params, f.derived, wl.h, wl.w, pk, qp), 20)
    t = per_call(lambda: ops.query_packed(pk, qp, wl.h, wl.w, f.topk, xy, rgb), 5)
    out["query_packed_2e24_points"] = {"Mqueries_per_s": round(m / t / 1e6, 1), "ms": round(t * 1e3, 3),
                                       "GB_per_s_algorithmic": round(52 * m / t / 1e9, 1),
                                       "pack_50k_us": round(tp * 1e6, 2),
                                       "note": "16-byte packed records (Appendix B.2) instead of 48-byte ones"}
    del pk, qp
    del f, xy, rgb
    out["full_refresh"] = refresh_timings(torch, synth, ops, SadField)
    return out


SETTLE_STEPS = 500  # untimed steps after the refresh, before the warm-up steps


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-secondary", action="store_true", help="skip the other workloads' timings")
    ap.add_argument("--cpu-all", action="store_true",
                    help="also time the oracle on one 2048x2048 step (adds about a minute)")
    ap.add_argument("--refresh-only", action="store_true",
                    help="only time the full refresh (JFA round + 16 passes + render) at 512^2, 1024^2, 2048^2")
    ap.add_argument("--budget-only", action="store_true",
                    help="only time the budget step (statistics given; prune and split 500 of 50k sites)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy 5 times (reference for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the SAD hot path here has no multi-GPU mode "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if args.calibrate_copy:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4, "launches": 5}))
        return 0

    import synth
    from voronoi_rendering_amd import ops
    from voronoi_rendering_amd.pipeline import SadField

    if args.refresh_only:
        print(json.dumps({"full_refresh": refresh_timings(torch, synth, ops, SadField)}), flush=True)
        return 0
    if args.budget_only:
        print(json.dumps({"densify_prune_768x512_50k": budget_timings(torch, synth, ops, SadField)}), flush=True)
        return 0
    wl = synth.C2
    dev = torch.device("cuda", 0)
    params = torch.from_numpy(wl.make_sites()).to(dev)
    target = torch.from_numpy(wl.make_target()).to(dev)
    f = SadField(params, wl.h, wl.w, wl.inject_seed, inject=wl.inject)
    strides = list(wl.strides)
    # The map a long fit works on: the pages' full refresh (a JFA round and 16
    # passes), then steps until the lists have settled (on these static sites
    # they reach the exact top-8 everywhere; a step on settled lists is a few
    # per cent slower than on fresh ones, whose neighbours are mostly listed).
    f.refresh(16)
    for _ in range(SETTLE_STEPS):
        f.sites_changed()
        f.step(strides, target, fused=True)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev = []  # (kind, start event, end event, launches between them)

    def step(record: bool):
        # In training the Adam update rewrites the sites between steps, so the
        # first pass of every step recomputes the previous lists' logits; it
        # rewrites the sites' probe records with them.
        f.sites_changed(probe_records_current=True)
        if not record:
            f.step(strides, target, fused=True)
            return
        # the same launches as the timed steps: one event pair around the
        # step's first passes (their average is the per-pass duration; an
        # event pair per launch would add its own gaps) and one around the
        # last pass and the backward (one kernel)
        a, b, c = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        a.record(stream)
        f.step(strides, target, fused=True, before_last=lambda: b.record(stream))
        c.record(stream)
        ev.append(("propagate", a, b, len(strides) - 1))
        ev.append(("step_last", b, c, 1))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    # Timed region: K plain steps give the throughput; then up to 50 steps with
    # HIP events give the per-kernel durations (events add gaps of their own,
    # so they stay out of the headline).
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(False)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ev_steps = min(args.steps, 50)
    for _ in range(ev_steps):
        step(True)
    torch.cuda.synchronize()

    # per-pass durations by stride: one event pair per pass (each pair adds a
    # small gap of its own), over a few more steps
    by_stride = {s: [] for s in strides}
    evs = []
    for _ in range(min(args.steps, 20)):
        f.sites_changed()
        for s_ in strides:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            f.propagate([s_])
            b.record(stream)
            evs.append((s_, a, b))
        # the backward alone (its own kernel, as sad_render_bwd runs it)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        f.forward_backward(target)
        b.record(stream)
        evs.append(("bwd", a, b))
    torch.cuda.synchronize()
    bwd_alone = []
    for s_, a, b in evs:
        if s_ == "bwd":
            bwd_alone.append(a.elapsed_time(b) * 1e3)
        else:
            by_stride[s_].append(a.elapsed_time(b) * 1e3)
    # a plain device copy of 256 MiB: the bandwidth this machine's HBM reaches
    src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(10):
        dst.copy_(src)
    b.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * src.numel() * 4 * 10 / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst

    per = {}
    for kind, a, b, launches in ev:
        per.setdefault(kind, []).append((a.elapsed_time(b) * 1e-3 / launches, launches))
    avg = {k: float(np.mean([d for d, _ in v])) for k, v in per.items()}
    ms_per_step = elapsed / args.steps * 1e3
    pix = wl.h * wl.w
    value = pix / (elapsed / args.steps) / 1e6
    ab = algorithmic_bytes(wl.h, wl.w, wl.n, len(strides))
    total = {k: avg[k] * sum(n for _, n in per[k]) / ev_steps for k in avg}
    dom = max(total, key=total.get)
    achieved = ab[dom] / avg[dom] / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(dom), "kernel": dom,
                "kernel_us": round(avg[dom] * 1e6, 3),
                "bytes_per_launch": ab[dom],
                "copy_GBps_measured": round(copy_gbs, 1),
                "frac_of_measured_copy": round(achieved / copy_gbs, 4)}
    out = {
        "metric": "Mpixel-iters/s (propagate+fwd+bwd), 768x512 @ 50k sites; % HBM roofline",
        "value": round(value, 2),
        "unit": "Mpixel-iters/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "C2: 768x512 RGB f32, 50,000 sites, K=8, strides 8,4,2,1, 64 injected per 8x8 "
                               "tile, forward+backward with loss",
                   "map": f"full refresh (JFA round + 16 passes), then {SETTLE_STEPS} settling steps",
                   "pixels": pix, "sites": wl.n, "passes_per_step": len(strides), "parallelism": "single GPU"},
        "step_frac_of_hbm_roofline": round(ab["step"] / (elapsed / args.steps) / 1e9 / HBM_PEAK_GBS, 4),
        "kernel_us": {k: round(v * 1e6, 3) for k, v in avg.items()},
        "pass_us_by_stride": {str(k): round(float(np.median(v)), 3) for k, v in by_stride.items()},
        "render_bwd_alone_us": round(float(np.median(bwd_alone)), 3),
        "kernel_timing": f"HIP events on the launch stream over {ev_steps} further steps of the timed launches: one "
                         "pair around the step's first passes (per-pass average), one around the last pass + backward "
                         "kernel; per-stride passes (32-bit maps) and the backward alone (sad_render_bwd) from one pair "
                         "per launch",
        "roofline": roofline,
        "valu_roofline": valu_roofline(dom, avg[dom]),
    }
    if not args.no_secondary:
        out["secondary"] = secondary(torch, synth, ops, SadField)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
        out["cpu_other"] = cpu_other(args.cpu_all)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
