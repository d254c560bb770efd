"""The host-side code under the address and undefined-behaviour sanitizers
(gcc/g++ -fsanitize=address,undefined, no recovery): the CPU oracle
(tests/sanitize/oracle_check.c runs every entry point on small layers) and the
library's planning code -- configuration checks, workspace carving, launch
plans -- which is plain C++ in csrc/plan.h (tests/sanitize/plan_check.cpp
sweeps the configurations of the tests and the benchmark and a seeded set of
random ones).  No GPU is involved."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]


def _run(exe):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_check")
    subprocess.run(["gcc", "-std=c99", "-ffp-contract=off", *SAN,
                    os.path.join(HERE, "oracle_check.c"), "-o", exe, "-lm"], check=True)
    assert "0 failures" in _run(exe)


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_planning_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "plan_check")
    subprocess.run(["g++", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "sparse_moe_decode_router_amd", "csrc"),
                    os.path.join(HERE, "plan_check.cpp"), "-o", exe], check=True)
    assert "0 failures" in _run(exe)
