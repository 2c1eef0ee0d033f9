"""Host-side checks of bench.py: the one-GPU contract and the bookkeeping
that needs no GPU (algorithmic bytes, counter summaries, the roofline peaks)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_of_the_step():
    ab = bench.algorithmic_bytes(512, 768, 50_000, 4)
    pix = 512 * 768
    assert ab["propagate"] == 64 * pix
    # four passes of lists, the target, and per site the record read and the gradient read and written
    assert ab["step"] == pix * (64 * 4 + 12) + 50_000 * (48 + 80)
    # the last pass and the backward in one kernel: lists read and written, the target, 128 B per site
    assert ab["step_last"] == pix * (64 + 12) + 50_000 * 128


def test_counter_summary_matches_the_sources():
    """The committed counters were taken on the current kernel sources (else the
    bench reports traffic as null) and carry the instruction counts."""
    rec = bench.counter_record("propagate")
    if rec is None:  # the bench then reports traffic as null, which is what it should do
        pytest.skip("the committed counters predate the propagation kernel's current sources")
    assert rec["waves_per_dispatch"] == 6144 and rec["valu_insts_per_wave"] > 0
    assert bench.measured_traffic("propagate") == int(rec["bytes"])
    v = bench.valu_roofline("propagate", 25e-6)
    # the fp32 vector peak, 157.3 TFLOP/s, in lane-operations (an FMA is two flops)
    assert v["bound"] == "alu" and abs(v["peak"] - 78.65) < 0.01 and 0 < v["frac"] < 1
    for kind in ("step_last", "render_bwd"):
        r = bench.counter_record(kind)
        assert r is not None and r["waves_per_dispatch"] == 6144 and r["bytes"] > 0


def test_profiles_are_short_text():
    for f in os.listdir(os.path.join(ROOT, "profiles")):
        path = os.path.join(ROOT, "profiles", f)
        assert f.endswith((".md", ".txt", ".json")), f
        assert os.path.getsize(path) < 64 * 1024, f
        if f.endswith(".json"):
            json.load(open(path))
