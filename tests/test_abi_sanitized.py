"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library's sources are compiled with the sanitizers on the host pass
only (the device code is built as usual and never launched here), and the
argument validation of every entry point (tests/abi_sanitize_calls.py) runs
in a process that preloads the sanitizer runtime.  Every call must return its
documented status with no sanitizer report.  CPU only.
"""

import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_attention_recurrence_net_amd", "csrc")


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_abi_validation_under_sanitizers(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    rt = _asan_runtime()
    if not os.path.exists(hipcc) or rt is None:
        pytest.skip("hipcc or the clang sanitizer runtime is not available")
    so = tmp_path / "libgdn_sanitized.so"
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, *srcs, "-o", str(so)]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=600)
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "abi_sanitize_calls.py"), str(so)],
                       capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "checks ok" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr
