"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host
code only, g++): tests/oracle_sanitize.cpp drives every exported oracle
function on small inputs with ragged vocabularies, -inf / NaN logits, empty
rows, truncation and invalid policies; any sanitizer report fails the run."""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_oracle_under_asan_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = str(tmp_path / "oracle_sanitize")
    build = subprocess.run(
        [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
         "-fsanitize=address,undefined,float-cast-overflow", "-fno-sanitize-recover=all",
         os.path.join(HERE, "oracle_sanitize.cpp"), os.path.join(ROOT, "oracle", "dspark_oracle.cpp"),
         "-o", exe], capture_output=True, text=True, timeout=600)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert run.returncode == 0, (run.stdout[-2000:], run.stderr[-6000:])
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr, run.stderr[-6000:]
    assert "oracle sanitizer run done (0" in run.stdout
