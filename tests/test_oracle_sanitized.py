"""The float64 oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/oracle_sanitize_driver.c calls every oracle entry point on small
seeded inputs (both gate kinds, snapshots, shared q/k heads, rollback with
invalid indices, the chunked form with a ragged tail, empty problems); it is
built here with gcc -fsanitize=address,undefined together with
oracle/gdn_oracle.c, and must exit 0 with no sanitizer report.  CPU only.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not available")
    exe = tmp_path / "oracle_asan"
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "oracle", "gdn_oracle.c"), os.path.join(ROOT, "tests", "oracle_sanitize_driver.c"),
           "-lm", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr
