"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Builds two small drivers with gcc/g++ and runs them: tests/sanitize/plan_check.cpp
over the forward's host planning code (gated_linear_attention_amd/csrc/plan_host.h:
segment lengths, workspace layout, overlap checks) on a grid of batch shapes, and
tests/sanitize/oracle_check.c over the fp64 C oracle (forward, backward, decode).
Any sanitizer report or failed invariant fails the test. Host code only: no GPU
code is built here.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


def _run(cmd_build, exe, tmp_path):
    r = subprocess.run(cmd_build, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    # the environment is passed as it is; ASan is told not to insist on being
    # the first library loaded
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out[-4000:]
    return out


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_plan_host_code_sanitized(tmp_path):
    exe = str(tmp_path / "plan_check")
    out = _run(["g++", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"),
                "-I", os.path.join(ROOT, "gated_linear_attention_amd", "csrc"),
                os.path.join(ROOT, "tests", "sanitize", "plan_check.cpp"), "-o", exe], exe, tmp_path)
    assert "plan_check: ok" in out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_c_sanitized(tmp_path):
    exe = str(tmp_path / "oracle_check")
    out = _run(["gcc", "-std=c11", *SAN, "-fopenmp",
                os.path.join(ROOT, "oracle", "gla_oracle.c"),
                os.path.join(ROOT, "tests", "sanitize", "oracle_check.c"), "-o", exe, "-lm"],
               exe, tmp_path)
    assert "oracle_check: ok" in out
