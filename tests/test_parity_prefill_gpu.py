"""GPU parity of the chunked prefill (bf16 MFMA, chunk 64) against the float64
oracle's sequential recurrence.

Bar: max|gpu - ref| / max|ref| <= 1e-2 per output tensor (o and the final
state).  Covered: the full prefill workload (B=1, T=8192, H=16, d=128, zero
initial state) compared on every output; ragged lengths around the chunk
size (1, 63, 64, 65, 150, 200); d = 64; several sequences; a non-zero
initial state; the exact special case beta = 0 with gate 1 (the state must
come back bit-identical); agreement with the token-by-token GPU kernel.
"""

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
from helpers import bits, ensure_built, oracle_args, rel_err, upload

pytestmark = pytest.mark.gpu

TOL = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()
    assert torch.cuda.is_available()


def _gdn():
    import linear_attention_recurrence_net_amd as gdn
    return gdn


def _prefill(case):
    d = upload(case)
    s = d["state"][:, :, 0].contiguous()
    o = _gdn().gdn_prefill_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], s)
    torch.cuda.synchronize()
    return o, s, d


def _check(case, o, s, tol=TOL):
    ro, rst, _ = oracle.forward(*oracle_args(case), case.f64("state"))
    eo, es = rel_err(o, ro, "o"), rel_err(s, rst[:, :, 0], "state")
    print(f"B={case.B} T={case.T} H={case.H} d={case.d_k} o {eo:.3e} state {es:.3e}", flush=True)
    assert eo <= tol and es <= tol, (eo, es)
    return eo, es


def test_prefill_workload_full_size():
    c = gi.workload_case(4)
    o, s, _ = _prefill(c)
    _check(c, o, s)


@pytest.mark.parametrize("T", [1, 63, 64, 65, 150, 200])
def test_prefill_ragged_lengths(T):
    c = gi.make_case(1, T, 2, 128, qkv_dtype="bf16", seed=200 + T, zero_state=True)
    o, s, _ = _prefill(c)
    _check(c, o, s)


@pytest.mark.parametrize("B,T,H,d", [(2, 130, 3, 64), (3, 97, 2, 128), (1, 300, 4, 64)])
def test_prefill_batches_and_d64_nonzero_state(B, T, H, d):
    c = gi.make_case(B, T, H, d, qkv_dtype="bf16", seed=300 + T)
    o, s, _ = _prefill(c)
    _check(c, o, s)


def test_prefill_beta0_gate1_state_bitwise():
    c = gi.make_case(1, 130, 2, 128, qkv_dtype="bf16", seed=7)
    c.beta[:] = 0.0
    c.g[:] = 0.0
    o, s, _ = _prefill(c)
    assert np.array_equal(bits(s), c.state[:, :, 0].view(np.int32))
    _check(c, o, s)


def test_prefill_matches_token_kernel():
    c = gi.make_case(2, 257, 4, 128, qkv_dtype="bf16", seed=9, zero_state=True)
    o, s, d = _prefill(c)
    s2 = upload(c)["state"][:, :, 0].contiguous()
    o2 = _gdn().gdn_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], s2)
    torch.cuda.synchronize()
    assert rel_err(o, o2.double().cpu().numpy()) <= TOL
    assert rel_err(s, s2.double().cpu().numpy()) <= TOL


def test_prefill_rejects_kda_and_fp32():
    c = gi.make_case(1, 8, 1, 64, qkv_dtype="f32", gate="kda", seed=1)
    d = upload(c)
    s = d["state"][:, :, 0].contiguous()
    with pytest.raises(Exception):
        _gdn().gdn_prefill_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], s)


def test_prefill_graph_replay_matches_eager():
    """The bench times HIP-graph replays of the prefill: every replay must
    equal the eager result bit for bit, with eager work between replays.
    Covers the uniform, variable-length (its offset table is rebuilt by a
    kernel on every call) and KDA prefills."""
    gdn = _gdn()
    c = gi.make_case(1, 200, 4, 128, qkv_dtype="bf16", seed=41)
    ck = gi.make_case(1, 150, 2, 64, gate="kda", qkv_dtype="bf16", seed=42)
    vc = gi.make_varlen_case([70, 0, 130], 4, 64, seed=43)
    u, uk = upload(c), upload(ck)
    bf = torch.bfloat16
    t = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dt)
    vq, vk, vv, vg, vb = t(vc.q, bf), t(vc.k, bf), t(vc.v, bf), t(vc.g), t(vc.beta)
    vcu = t(vc.cu_seqlens, torch.int32)
    s0, sk0, sv0 = (u["state"][:, :, 0].contiguous(), uk["state"][:, :, 0].contiguous(), t(vc.state))
    ws = torch.empty(gdn.gdn_prefill_workspace_size(1, 200, 4, 128, 128), dtype=torch.uint8, device="cuda")
    wsk = torch.empty(gdn.gdn_prefill_kda_workspace_size(1, 150, 2, 64, 64), dtype=torch.uint8, device="cuda")
    wsv = torch.empty(gdn.gdn_prefill_varlen_workspace_size(3, vc.total, 4, 64, 64), dtype=torch.uint8,
                      device="cuda")
    s, sk, sv = torch.empty_like(s0), torch.empty_like(sk0), torch.empty_like(sv0)
    o = torch.empty((1, 200, 4, 128), device="cuda")
    ok = torch.empty((1, 150, 2, 64), device="cuda")
    ov = torch.zeros((vc.total, 4, 64), device="cuda")

    def run():
        torch.mul(s0, 1.0, out=s)  # reset the states with kernels (x * 1 is exact)
        torch.mul(sk0, 1.0, out=sk)
        torch.mul(sv0, 1.0, out=sv)
        gdn.gdn_prefill_chunked(u["q"], u["k"], u["v"], u["g"], u["beta"], s, o=o, workspace=ws)
        gdn.gdn_prefill_chunked_kda(uk["q"], uk["k"], uk["v"], uk["g"], uk["beta"], sk, o=ok, workspace=wsk)
        gdn.gdn_prefill_chunked_varlen(vcu, vq, vk, vv, vg, vb, sv, o=ov, workspace=wsv)

    run()
    torch.cuda.synchronize()
    ref = [bits(x) for x in (o, s, ok, sk, ov[:70], ov[70:], sv)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for _ in range(3):
        for x in (o, s, ok, sk, sv, ov, ws, wsk, wsv):
            x.fill_(0 if x.dtype == torch.uint8 else float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [bits(x) for x in (o, s, ok, sk, ov[:70], ov[70:], sv)]
        for a, b in zip(ref, got):
            assert np.array_equal(a, b)
