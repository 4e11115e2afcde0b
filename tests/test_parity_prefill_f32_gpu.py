"""GPU parity of the general chunked prefill entry point with float32 q/k/v.

The float32 inputs are rounded to bf16 (nearest even) for the MFMA
products, so the bar is the prefill's (1e-2 against the float64 oracle on
the float32 inputs).  When the float32 inputs hold bf16 values exactly, the
rounding is exact and the result must equal the bf16 path bit for bit; this
is checked for both gate kinds.
"""

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
from helpers import bits, dev, ensure_built, oracle_args, rel_err, upload

pytestmark = pytest.mark.gpu

TOL = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()
    assert torch.cuda.is_available()


def _gdn():
    import linear_attention_recurrence_net_amd as gdn
    return gdn


def _run_ex(u, head_map="grouped", state=None, final=None):
    st = (u["state"][:, :, 0].contiguous() if state is None else state)
    o = _gdn().gdn_prefill_chunked_ex(u["q"], u["k"], u["v"], u["g"], u["beta"], st,
                                      head_map=head_map, final_state=final)
    torch.cuda.synchronize()
    return o, st


@pytest.mark.parametrize("B,T,H,Hq,d,gate,head_map", [
    (1, 200, 4, 4, 128, "gda", "grouped"),
    (2, 97, 3, 3, 64, "gda", "grouped"),
    (1, 150, 8, 2, 128, "gda", "tiled"),
    (2, 130, 2, 2, 128, "kda", "grouped"),
    (1, 65, 4, 2, 64, "kda", "grouped"),
])
def test_prefill_f32_inputs(B, T, H, Hq, d, gate, head_map):
    c = gi.make_case(B, T, H, d, gate=gate, qkv_dtype="f32", seed=900 + T + H, H_qk=Hq)
    u = upload(c)
    assert u["q"].dtype == torch.float32
    o, s = _run_ex(u, head_map)
    ro, rst, _ = oracle.forward(*oracle_args(c), c.f64("state"), kda=gate == "kda", head_map=head_map)
    eo, es = rel_err(o, ro), rel_err(s, rst[:, :, 0])
    print(f"f32 {gate} B={B} T={T} H={H} H_qk={Hq} d={d}: o {eo:.3e} state {es:.3e}", flush=True)
    assert eo <= TOL and es <= TOL


def test_prefill_f32_workload_full_size():
    c = gi.workload_case(4, qkv_dtype="f32")
    u = upload(c)
    o, s = _run_ex(u)
    ro, rst, _ = oracle.forward(*oracle_args(c), c.f64("state"))
    eo, es = rel_err(o, ro), rel_err(s, rst[:, :, 0])
    print(f"f32 prefill workload: o {eo:.3e} state {es:.3e}", flush=True)
    assert eo <= TOL and es <= TOL


@pytest.mark.parametrize("gate", ["gda", "kda"])
def test_prefill_f32_bf16_exact_inputs_equal_bf16_path(gate):
    c = gi.make_case(2, 150, 4, 128, gate=gate, qkv_dtype="bf16", seed=33, H_qk=2)
    ub = upload(c)  # bf16 tensors
    uf = dict(ub)
    for n in ("q", "k", "v"):
        uf[n] = dev(getattr(c, n))  # the same values as float32
    ob, sb = _run_ex(ub)
    of, sf = _run_ex(dict(uf, state=upload(c)["state"]))
    assert np.array_equal(bits(ob), bits(of))
    assert np.array_equal(bits(sb), bits(sf))


def test_prefill_f32_snapshots():
    B, T, H, d, K = 2, 40, 4, 128, 5
    c = gi.make_case(B, T, H, d, K=K, qkv_dtype="f32", seed=71)
    c.state[:, :, 1:] = np.float32(np.nan)
    u = upload(c)
    fin = torch.empty((B, H, d, d), device="cuda")
    o, st = _run_ex(u, state=u["state"], final=fin)
    ro, rst, rfin = oracle.forward(*oracle_args(c), c.f64("state"), want_final=True)
    assert rel_err(o, ro) <= TOL and rel_err(fin, rfin) <= TOL
    for t in range(1, K):
        assert rel_err(st[:, :, t], rst[:, :, t]) <= TOL
    assert np.array_equal(bits(st[:, :, 0]), c.state[:, :, 0].view(np.int32))


def test_prefill_ex_kda_snapshots_float32():
    """KDA with K snapshot slots and float32 inputs through the general entry
    point (more shapes in the snapshot tests)."""
    B, T, H, d, K = 2, 20, 2, 64, 6
    c = gi.make_case(B, T, H, d, K=K, gate="kda", qkv_dtype="f32", seed=4)
    c.state[:, :, 1:] = np.float32(np.nan)
    u = upload(c)
    fin = torch.empty((B, H, d, d), device="cuda")
    o, st = _run_ex(u, state=u["state"], final=fin)
    ro, rst, rfin = oracle.forward(*oracle_args(c), c.f64("state"), kda=True, want_final=True)
    assert rel_err(o, ro) <= TOL and rel_err(fin, rfin) <= TOL
    for t in range(1, K):
        assert rel_err(st[:, :, t], rst[:, :, t]) <= TOL
    assert np.array_equal(bits(st[:, :, 0]), c.state[:, :, 0].view(np.int32))
