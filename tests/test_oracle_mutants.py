"""The oracle's pins must catch plausible mistakes.

Each case copies the oracle into a temporary directory, plants one mistake in
the C source (a transposed rotation, a swapped scale, a wrong sign or factor
in a gradient, a wrong stencil, a missing bias correction, ...), rebuilds it
there and runs the oracle's pin tests against the copy, which must fail.
Runs on the CPU only; the repository's oracle is never modified.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = [
    ("rotation transposed", "float a = (dx * d[4] + dy * d[5]) * d[6];", "float a = (dx * d[4] - dy * d[5]) * d[6];"),
    ("scales swapped", "float a = (dx * d[4] + dy * d[5]) * d[6];", "float a = (dx * d[4] + dy * d[5]) * d[7];"),
    ("radius sign", "float dist = sqrtf(q) - d[3];", "float dist = sqrtf(q) + d[3];"),
    ("y gradient sign", "t[1] = kappa * -2.0 * (a * is1 * sn + b * is2 * cs);",
     "t[1] = kappa * -2.0 * (a * is1 * sn - b * is2 * cs);"),
    ("theta gradient factor", "t[7] = kappa * 2.0 * ar * br * (is1 * is1 - is2 * is2);",
     "t[7] = kappa * 2.0 * ar * br * (is1 - is2);"),
    ("log tau gradient", "t[2] = delta * (double)e.l[k];", "t[2] = delta;"),
    ("diagonal neighbour", "{0, 0}, {stride, 0}, {-stride, 0}, {0, stride}, {0, -stride}",
     "{0, 0}, {stride, stride}, {-stride, 0}, {0, stride}, {0, -stride}"),
    ("tile index transposed", "uint32_t tile = (uint32_t)((j / TILE) * tiles_x + (i / TILE));",
     "uint32_t tile = (uint32_t)((i / TILE) * tiles_x + (j / TILE));"),
    ("tie-break reversed", "if (a->id < b->id) return -1;\n    if (a->id > b->id) return 1;",
     "if (a->id > b->id) return -1;\n    if (a->id < b->id) return 1;"),
    ("softmax sign", "e->w[k] = exp((double)e->l[k] - m);", "e->w[k] = exp(m - (double)e->l[k]);"),
    ("adam without bias correction", "float vhat = vv[k] / bc2;", "float vhat = vv[k];"),
    ("no position clamp", "p[1] = fminf(fmaxf(p[1], 0.0f), (float)h);", "(void)h;"),
    ("energy unweighted", "double t[8] = {wk, wk * err,", "double t[8] = {wk, err,"),
    ("removal blend not renormalised", "if (z > 0.0) cp[ch] /= z;", "(void)z;"),
    ("moment about the wrong axis", "double wk = e.w[k];\n                double dx = (double)px - (double)d[0], dy = (double)py - (double)d[1];",
     "double wk = e.w[k];\n                double dx = (double)px - (double)d[0], dy = (double)py - (double)d[0];"),
    ("cross moment missing the weight", "wk * dx * dy, wk * dy * dy};", "dx * dy, wk * dy * dy};"),
    ("flood without the diagonal neighbours", "for (int a = -1; a <= 1; ++a) {",
     "for (int a = -1; a <= 1; ++a) {\n                    if (a != 0 && b != 0) continue;"),
    ("seed keeps the worst-ranked site", "if (cur == NONE || s > best[p] ||", "if (cur == NONE || s < best[p] ||"),
    ("flood step only along x", "jj = (int64_t)j + (int64_t)b * step;", "jj = (int64_t)j + (int64_t)b;"),
    ("prune the highest removal deltas", "r[nr].key = isnan(dl) ? INFINITY : (double)dl;",
     "r[nr].key = isnan(dl) ? INFINITY : -(double)dl;"),
    ("split along the minor axis", "float lam = (a + c) * 0.5f + sqrtf(half * half + b * b);",
     "float lam = (a + c) * 0.5f - sqrtf(half * half + b * b);"),
    ("children keep the parent's colour", "o[4] = t[0];", "o[4] = base[4];"),
    ("children keep their Adam moments", "m[(size_t)oi * REC + q] = 0.0f;", "(void)oi;"),
    ("Sobel centre weight 1", "float gx = (tpx(target, h, w, i + 1, j - 1, c) + 2.0f * tpx(target, h, w, i + 1, j, c) +",
     "float gx = (tpx(target, h, w, i + 1, j - 1, c) + 1.0f * tpx(target, h, w, i + 1, j, c) +"),
    ("mixture weights swapped", "if (u0 < lambda || total == 0) {", "if (u0 >= lambda || total == 0) {"),
    ("inverse CDF off by one", "if (cum[mid] > t) hi = mid; else lo = mid + 1;",
     "if (cum[mid] >= t) hi = mid; else lo = mid + 1;"),
    ("init colour channels reversed", "for (int c = 0; c < 3; ++c) p[4 + c] = target[x * 3 + c];",
     "for (int c = 0; c < 3; ++c) p[4 + c] = target[x * 3 + (2 - c)];"),
    ("packed anisotropy sign", "o[3] = qt | (sadref_half_bits(p[9] - p[8]) << 16);",
     "o[3] = qt | (sadref_half_bits(p[8] - p[9]) << 16);"),
    ("packed r without the scale", "v[1] = p[3] * sadref_exp_f32(hs);", "v[1] = p[3];"),
    ("packed colour fields shifted", "o[1] = q[2] | (q[3] << 11) | (q[4] << 22);",
     "o[1] = q[2] | (q[3] << 10) | (q[4] << 21);"),
    ("packed angle decoded over half the circle",
     "out[7] = (double)(o[3] & 65535u) / 65535.0 * (2.0 * SADREF_PI) - SADREF_PI;",
     "out[7] = (double)(o[3] & 65535u) / 65535.0 * SADREF_PI - SADREF_PI;"),
    ("packed half rounding truncates", "double r = nearbyint(a / ulp) * ulp;", "double r = floor(a / ulp) * ulp;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle",
                    ignore=shutil.ignore_patterns("_build", "__pycache__"))
    shutil.copytree(os.path.join(ROOT, "synth"), tmp_path / "synth",
                    ignore=shutil.ignore_patterns("__pycache__"))
    os.mkdir(tmp_path / "tests")
    for f in os.listdir(os.path.join(ROOT, "tests")):
        if f.startswith("test_oracle_") and f != "test_oracle_mutants.py" or f == "conftest.py":
            shutil.copy(os.path.join(ROOT, "tests", f), tmp_path / "tests" / f)
    shutil.copy(os.path.join(ROOT, "pytest.ini"), tmp_path / "pytest.ini")
    src = tmp_path / "oracle" / "sadref.c"
    text = src.read_text()
    assert text.count(old) == 1, name
    src.write_text(text.replace(old, new))
    env = dict(os.environ, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "tests"], cwd=tmp_path,
                       capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 1, f"mutant '{name}' survived:\n{r.stdout[-2000:]}"
