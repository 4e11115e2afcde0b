"""GPU check of gdn_prefill_chunked_ex_noalloc, the chunked prefill that uses
the library's fixed scratch array instead of a caller workspace.

It is called through the C ABI (ctypes, no Python wrapper) and compared with
gdn_prefill_chunked_ex on the same inputs, bit for bit, on consecutive calls
whose second input is smaller than the first (the array keeps the first
call's contents).  The two entry points run the same kernels, so the bar is
exact equality, stricter than the 1e-2 prefill bar; the first call is also
checked against the float64 oracle at that bar.  A problem larger than the
array is refused before any launch, with its outputs untouched.
"""

import ctypes

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
from helpers import ensure_built, oracle_args, rel_err, upload

pytestmark = pytest.mark.gpu

GDN_F32, GDN_BF16 = 0, 1
ERR_SCRATCH = 6
SCRATCH_BYTES = 256 * 1024 * 1024


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()
    assert torch.cuda.is_available()


def _gdn():
    import linear_attention_recurrence_net_amd as gdn
    return gdn


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _noalloc(case, d, state, final, o, head_map=0):
    lib = _gdn().library()
    dt = GDN_BF16 if case.qkv_dtype == "bf16" else GDN_F32
    gate = 1 if case.gate == "kda" else 0
    K = state.shape[2] if state.dim() == 5 else 1
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.gdn_prefill_chunked_ex_noalloc(
        case.B, case.T, case.H, case.H_qk, head_map, case.d_k, case.d_v, 64, dt, gate, K,
        _p(d["q"]), _p(d["k"]), _p(d["v"]), _p(d["g"]), _p(d["beta"]), _p(state), _p(final), _p(o),
        stream)


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int32).numpy()


# consecutive calls: the second one smaller than the first
CASES = [
    dict(B=1, T=8192, H=16, d_k=128, gate="gda", qkv_dtype="bf16", K=1, zero_state=True),  # the prefill workload
    dict(B=2, T=200, H=4, d_k=64, gate="kda", qkv_dtype="bf16", K=1),
    dict(B=3, T=150, H=4, d_k=128, gate="gda", qkv_dtype="f32", K=5),
    dict(B=1, T=70, H=2, d_k=128, gate="kda", qkv_dtype="f32", K=1),
]


def test_noalloc_matches_workspace_entry_point_on_consecutive_calls():
    gdn = _gdn()
    for i, kw in enumerate(CASES):
        kw = dict(kw)
        K = kw.pop("K")
        c = gi.make_case(kw.pop("B"), kw.pop("T"), kw.pop("H"), kw.pop("d_k"), K=K, seed=800 + i, **kw)
        print(f"call {i}: B={c.B} T={c.T} H={c.H} d={c.d_k} {c.gate} {c.qkv_dtype} K={K}", flush=True)
        d = upload(c)
        st_ref = d["state"].clone() if K > 1 else d["state"][:, :, 0].contiguous()
        st_na = st_ref.clone()
        fin_ref = torch.empty((c.B, c.H, c.d_k, c.d_v), device="cuda") if K > 1 else None
        fin_na = torch.full_like(fin_ref, float("nan")) if K > 1 else None
        o_ref = gdn.gdn_prefill_chunked_ex(d["q"], d["k"], d["v"], d["g"], d["beta"], st_ref,
                                           final_state=fin_ref)
        o_na = torch.full((c.B, c.T, c.H, c.d_v), float("nan"), device="cuda")
        assert _noalloc(c, d, st_na, fin_na, o_na) == 0
        torch.cuda.synchronize()
        assert np.array_equal(_bits(o_na), _bits(o_ref)), i
        assert np.array_equal(_bits(st_na), _bits(st_ref)), i
        if K > 1:
            assert np.array_equal(_bits(fin_na), _bits(fin_ref)), i
        if i == 0:
            ro, rst, _ = oracle.forward(*oracle_args(c), c.f64("state"))
            assert rel_err(o_na, ro, "o") <= 1e-2
            assert rel_err(st_na, rst[:, :, 0], "state") <= 1e-2


def test_noalloc_refuses_problems_beyond_the_scratch_array():
    gdn = _gdn()
    lib = gdn.library()
    per_chunk = lib.gdn_prefill_workspace_size_ex(1, 64, 1, 128, 128, 64, GDN_BF16, 0)
    T = 64 * (SCRATCH_BYTES // per_chunk) + 1  # one chunk more than the array holds, one head
    assert lib.gdn_prefill_workspace_size_ex(1, T, 1, 128, 128, 64, GDN_BF16, 0) > SCRATCH_BYTES
    c = gi.make_case(1, 4, 1, 128, seed=5)  # small inputs; the refusal comes before any launch
    q = torch.zeros((1, T, 1, 128), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros((1, T, 1), device="cuda")
    st = torch.full((1, 1, 128, 128), 7.0, device="cuda")
    o = torch.full((1, T, 1, 128), float("nan"), device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    r = lib.gdn_prefill_chunked_ex_noalloc(1, T, 1, 1, 0, 128, 128, 64, GDN_BF16, 0, 1, _p(q), _p(q), _p(q),
                                           _p(g), _p(g), _p(st), None, _p(o), stream)
    torch.cuda.synchronize()
    assert r == ERR_SCRATCH
    assert b"scratch" in lib.gdn_status_str(r)
    assert torch.isnan(o).all() and (st == 7.0).all()
    del c
