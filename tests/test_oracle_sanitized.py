"""The oracle's C++ under AddressSanitizer and UndefinedBehaviorSanitizer:
oracle/sanitize_check.cpp calls every oracle entry point (all key kinds,
value widths, bit ranges and digit widths 1..16, sizes 0..4097, edge
patterns) with buffers of exactly the documented size and cross-checks the
counting-sort LSD against the one-bit split sort.  Built as a standalone
executable with g++, so no sanitizer runtime has to be preloaded."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")


@pytest.fixture(scope="module")
def sanitized_exe(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("san") / "sanitize_check")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-ffp-contract=off", "-I", ORACLE, os.path.join(ORACLE, "oracle.cpp"),
           os.path.join(ORACLE, "sanitize_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "sanitize" in r.stderr and "cannot find" in r.stderr:
        pytest.skip("sanitizer runtime not installed")
    assert r.returncode == 0, r.stderr
    return exe


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_oracle_clean_under_sanitizers(sanitized_exe, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sanitized_exe, str(seed)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "sanitize_check ok" in r.stdout
