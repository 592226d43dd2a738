"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/asan_oracle_driver.c calls every entry point of oracle/lto.c on small
ragged shapes with buffers allocated at their exact sizes; built here with
gcc and the sanitizers, any read or write outside a tensor, use after free,
leak or undefined arithmetic fails the run.  Host code only: no GPU code is
built with a sanitizer.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_clean_under_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = tmp_path / "oracle_driver"
    cmd = [gcc, "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-fopenmp",
           os.path.join(ROOT, "tests", "asan_oracle_driver.c"),
           os.path.join(ROOT, "oracle", "lto.c"), "-lm", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=240)
    if r.returncode != 0 and "sanitize" in r.stderr:
        pytest.skip("sanitizer runtime not available: " + r.stderr[-300:])
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="2")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=240, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr
    assert "all checks passed" in r.stdout
