"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer: a small
C++ driver (oracle_sanitize_driver.cpp) calls every oracle entry point on ragged
shapes, block sizes from per-token scales to 256-key steps, causal masks,
variable lengths and Q smoothing, with the oracle compiled in.  Any out-of-bounds
access, leak or undefined operation in the oracle's raw-pointer indexing aborts
the run.  Host code only (g++); no GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "orc_sanitized")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           os.path.join(ROOT, "tests", "oracle_sanitize_driver.cpp"),
           os.path.join(ROOT, "oracle", "rotattn_oracle.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0 and "sanitized oracle run: ok" in r.stdout, r.stdout + r.stderr[-4000:]
