"""Build libsad.so, the HIP library behind the SAD C ABI, for gfx950.

Compiles every ``csrc/*.hip`` with hipcc into ``voronoi_rendering_amd/libsad.so``.
Floating point: no contraction into fused multiply-adds (the logit and Adam
are specified one rounding per operation), correctly rounded float32 division
and square root, subnormals kept, and packed float32 instructions disabled.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
LIB = PKG / "libsad.so"
ARCH = os.environ.get("SAD_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-munsafe-fp-atomics",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the SAD HIP library cannot be built")


def sources() -> list[Path]:
    return sorted(CSRC.glob("*.hip"))


def build(verbose: bool = False, jobs: int = 8) -> Path:
    """Compile all sources (always) and link libsad.so in place."""
    objdir = PKG / "_build"
    objdir.mkdir(exist_ok=True)
    cc = hipcc()
    procs = []
    objs = []
    for src in sources():
        obj = objdir / (src.stem + ".o")
        objs.append(obj)
        cmd = [cc, *HIPCC_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", "-c", str(src), "-o", str(obj)]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        if len(procs) >= jobs:
            _wait(procs.pop(0))
    for pr in procs:
        _wait(pr)
    tmp = LIB.with_suffix(".so.tmp%d" % os.getpid())
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def _wait(item) -> None:
    src, proc = item
    out, _ = proc.communicate()
    # hipcc's host pass does not know the device-only target feature: not an error
    lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln and "not a recognized feature" not in ln]
    if proc.returncode != 0:
        sys.stderr.write("\n".join(lines) + "\n")
        raise RuntimeError(f"hipcc failed on {src.name}")
    if lines and any(ln.strip() for ln in lines):
        sys.stderr.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
