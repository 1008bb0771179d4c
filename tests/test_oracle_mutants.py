"""Planted mistakes in the oracle are caught by its pins.

Each case copies the oracle's C sources, plants one plausible mistake in the copy,
builds it with the oracle's own flags and runs the pins that should catch it in a
child process that loads the mutant (GM_ORACLE_LIB); the child must fail.  The
tracked oracle is never modified.  Mistakes planted:

* the camera-frame covariance formed as W^T Sigma W instead of W Sigma W^T;
* the camera centre taken as -W t instead of -W^T t (the colour's view direction);
* Blinn-Phong's half vector in place of Phong's reflected light vector;
* the light position used as a camera-space point, not carried by W L + t;
* the back layer of the two-layer composite going on after its pixel's front layer
  has stopped.
"""
import os
import shutil
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "wtsw": ([
        ("A[r * 3 + c] = (W[r * 3 + 0] * S[0 * 3 + c] + W[r * 3 + 1] * S[1 * 3 + c]) + W[r * 3 + 2] * S[2 * 3 + c];",
         "A[r * 3 + c] = (W[0 * 3 + r] * S[0 * 3 + c] + W[1 * 3 + r] * S[1 * 3 + c]) + W[2 * 3 + r] * S[2 * 3 + c];"),
        ("float v = (A[r * 3 + 0] * W[c * 3 + 0] + A[r * 3 + 1] * W[c * 3 + 1]) + A[r * 3 + 2] * W[c * 3 + 2];",
         "float v = (A[r * 3 + 0] * W[0 * 3 + c] + A[r * 3 + 1] * W[1 * 3 + c]) + A[r * 3 + 2] * W[2 * 3 + c];"),
    ], "projection"),
    "minus_w_t": ([
        ("Cw[j] = -((double)W[0 * 3 + j] * tt[0] + (double)W[1 * 3 + j] * tt[1] + (double)W[2 * 3 + j] * tt[2]);",
         "Cw[j] = -((double)W[j * 3 + 0] * tt[0] + (double)W[j * 3 + 1] * tt[1] + (double)W[j * 3 + 2] * tt[2]);"),
    ], "sh_colour_direction"),
    "blinn": ([
        ("double rde = rv[0] * e[0] + rv[1] * e[1] + rv[2] * e[2];",
         "double hh[3] = {l[0] + e[0], l[1] + e[1], l[2] + e[2]};"
         " double hn = sqrt(hh[0] * hh[0] + hh[1] * hh[1] + hh[2] * hh[2]);"
         " double rde = (n[0] * hh[0] + n[1] * hh[1] + n[2] * hh[2]) / hn; (void)rv;"),
    ], "phong_off_axis"),
    "light_in_camera_space": ([
        ("L[r] = R[r * 3 + 0] * (double)m->light->pos[0] + R[r * 3 + 1] * (double)m->light->pos[1] +\n"
         "                   R[r * 3 + 2] * (double)m->light->pos[2] + cam->t[r];",
         "L[r] = (double)m->light->pos[r];"),
    ], "phong_off_axis"),
    "back_layer_outlives_front": ([
        ("if (layer == 0) aliveB = 0; /* the pixel stops with its front layer */",
         "(void)0;"),
    ], "front_layer", "test_oracle_aa.py"),
}


def _build_mutant(tmp, edits):
    src_dir = os.path.join(ROOT, "oracle")
    for f in os.listdir(src_dir):
        if f.endswith(".c"):
            shutil.copy(os.path.join(src_dir, f), tmp)
    path = os.path.join(tmp, "gm_oracle.c")
    text = open(path).read()
    for old, new in edits:
        assert text.count(old) == 1, "the mutation's target is no longer in gm_oracle.c: " + old[:60]
        text = text.replace(old, new)
    open(path, "w").write(text)
    so = os.path.join(tmp, "libmutant.so")
    srcs = [os.path.join(tmp, os.path.basename(s)) for s in oracle._SRCS]
    subprocess.check_call(["gcc", *oracle.GCC_FLAGS, *srcs, "-o", so, "-lm"])
    return so


def _run_pins(selector, lib=None, test_file="test_oracle_camera_pins.py"):
    env = dict(os.environ)
    env.pop("GM_ORACLE_LIB", None)
    if lib:
        env["GM_ORACLE_LIB"] = lib
    env["OMP_NUM_THREADS"] = env.get("OMP_NUM_THREADS", "4")
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", test_file), "-q", "-x",
           "-k", selector, "-p", "no:cacheprovider", "-m", "not gpu"]
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_fails_a_pin(name, tmp_path, oracle_lib):
    edits, selector, *test_file = MUTANTS[name]
    so = _build_mutant(str(tmp_path), edits)
    res = _run_pins(selector, so, *test_file)
    assert res.returncode == 1, (name, res.returncode, res.stdout[-2000:], res.stderr[-2000:])
    assert "failed" in res.stdout


def test_pins_pass_on_the_oracle(oracle_lib):
    for sel, *test_file in sorted({tuple(m[1:]) for m in MUTANTS.values()}):
        res = _run_pins(sel, None, *test_file)
        assert res.returncode == 0, (sel, res.stdout[-2000:])
