"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

``oracle/kda_oracle.c`` is compiled with ``-fsanitize=address,undefined`` and
the forward, decode, comparison and backward pins run against it in a
subprocess with the ASan runtime preloaded into Python: every out-of-bounds
access, use after free or undefined operation in the oracle ends that run with
a report.  A copy with a planted one-element heap overflow shows that such a
report does end the run.
"""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kda_oracle.c")
SAN_FLAGS = ["-std=c99", "-O1", "-g", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-fopenmp", "-fPIC", "-shared"]


def _asan_runtime():
    try:
        path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                              text=True, check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _build(src_text, tmp_path):
    c = tmp_path / "oracle_san.c"
    c.write_text(src_text)
    lib = tmp_path / "liboracle_san.so"
    subprocess.run(["gcc", *SAN_FLAGS, str(c), "-o", str(lib), "-lm"], check=True)
    return str(lib)


def _env(lib, runtime):
    preload = runtime + (":" + os.environ["LD_PRELOAD"] if os.environ.get("LD_PRELOAD") else "")
    return dict(os.environ, KDA_ORACLE_LIB=lib, LD_PRELOAD=preload,
                ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=23",
                UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=24")


@pytest.fixture(scope="module")
def runtime():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("gcc has no AddressSanitizer runtime here")
    return rt


def test_oracle_pins_are_clean_under_sanitizers(runtime, tmp_path):
    lib = _build(open(SRC).read(), tmp_path)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_backward.py")],
                       env=_env(lib, runtime), cwd=ROOT, capture_output=True, text=True,
                       timeout=600)
    report = r.stdout[-3000:] + r.stderr[-3000:]
    assert "AddressSanitizer" not in report and "runtime error" not in report, report
    assert r.returncode == 0, report


def test_sanitizer_reports_a_planted_overflow(runtime, tmp_path):
    src = open(SRC).read()
    old = "            for (int64_t e = 0; e < dk * dv; ++e)\n                S[e] = S0 ? S0[e] : 0.0;"
    assert src.count(old) >= 1
    # one element past the end of the malloc'd state, in the forward only
    lib = _build(src.replace(old, old.replace("e < dk * dv", "e <= dk * dv"), 1), tmp_path)
    code = ("import numpy as np, oracle\n"
            "r = np.random.default_rng(0)\n"
            "a = [r.standard_normal((5, 1, 4)).astype(np.float32) for _ in range(6)]\n"
            "a[4] = r.uniform(0, 1, (5, 1)).astype(np.float32)\n"
            "oracle.forward(*a)\n")
    r = subprocess.run([sys.executable, "-c", code], env=_env(lib, runtime), cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]
