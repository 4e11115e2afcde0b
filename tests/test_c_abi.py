"""The library from plain C.

tests/c_abi_driver.c calls libgdn.so through include/gdn.h alone: it is built
with gcc against the HIP runtime (no hipcc, no C++, no Python), allocates
device memory and a stream itself, and checks a shared-q/k-head verification
with K = 4 slots and a final state, the rollback (bit for bit), the chunked
KDA prefill with float32 inputs and the rollback fused in, and an error
return against the float64 oracle (2e-4 for the token kernel, 1e-2 for the
chunked path).  On the CPU: the program is built and every library it needs
resolves.  On the GPU: it runs and passes.
"""

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "c_abi_driver")


def test_c_driver_builds_and_links():
    from linear_attention_recurrence_net_amd import _binding, build
    if not os.path.exists(_binding.library_path()):
        build.build()
    import oracle
    oracle.build()
    import __graft_entry__
    __graft_entry__.build_c_driver()
    out = subprocess.run(["ldd", DRIVER], capture_output=True, text=True, check=True).stdout
    assert "not found" not in out, out
    for lib in ("libgdn.so", "libgdn_oracle.so", "libamdhip64.so"):
        assert lib in out, (lib, out)


@pytest.mark.gpu
def test_c_driver_runs_on_the_gpu():
    assert os.path.exists(DRIVER), "tests/c_abi_driver is built by __graft_entry__.build()"
    print("running", DRIVER, flush=True)
    r = subprocess.run([DRIVER], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
