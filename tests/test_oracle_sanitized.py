"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

The oracle's C sources are built once more with -fsanitize=address,undefined (host
code only; gcc, the oracle's own flags otherwise) and a selection of the oracle pins
runs in a child process that loads that build (GM_ORACLE_LIB) with the ASan
runtime preloaded.  Any invalid access, leak-free heap misuse or undefined
behaviour the sanitizers report fails the test.  Command, for running by hand:

    gcc -O1 -g -fsanitize=address,undefined -fno-omit-frame-pointer -fopenmp \
        -ffp-contract=off -fno-fast-math -std=c11 -shared -fPIC oracle/*.c -o /tmp/liboracle_asan.so -lm
    LD_PRELOAD=$(gcc -print-file-name=libasan.so) ASAN_OPTIONS=detect_leaks=0 \
        GM_ORACLE_LIB=/tmp/liboracle_asan.so python -m pytest tests/test_oracle_pins.py -m "not gpu"
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# pins covering every C entry point of the oracle on small inputs
SELECTION = [
    "tests/test_oracle_pins.py",
    "tests/test_oracle_project_bwd.py",
    "tests/test_oracle_mesh_bwd.py",
    "tests/test_oracle_aa.py",
]


def _asan_runtime():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return path if path and os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.slow
def test_oracle_pins_clean_under_asan_ubsan(tmp_path):
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    so = str(tmp_path / "liboracle_asan.so")
    flags = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined",
             "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-shared", "-fPIC"]
    subprocess.check_call(["gcc", *flags, *oracle._SRCS, "-o", so, "-lm"])
    env = dict(os.environ)
    env.update(GM_ORACLE_LIB=so, LD_PRELOAD=rt, OMP_NUM_THREADS="4",
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    cmd = [sys.executable, "-m", "pytest", *[os.path.join(ROOT, p) for p in SELECTION], "-q", "-x",
           "-m", "not gpu and not slow", "-p", "no:cacheprovider"]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=1500)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in res.stdout
