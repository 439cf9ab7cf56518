"""The fp64 oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds oracle/spec_oracle.cpp with a small driver (tests/helpers/
oracle_sanitize_main.cpp) that calls every C entry point of the oracle on
seeded inputs and edge cases (V = 1, -inf logits, out-of-range tokens,
ragged lengths including zero, tree parents, invalid per-request settings,
rows without mass), and checks that the run is clean: no sanitizer report,
every documented return code and output range respected.  CPU only.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_oracle_clean_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "oracle_sanitize"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fopenmp", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           os.path.join(ROOT, "oracle", "spec_oracle.cpp"),
           os.path.join(ROOT, "tests", "helpers", "oracle_sanitize_main.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="2")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    assert "oracle sanitizer run: ok" in r.stdout
