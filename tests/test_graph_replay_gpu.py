"""Calls captured into a HIP graph and replayed give the bits of the same
calls issued one by one.

Each entry point is captured once (torch.cuda.CUDAGraph, whose capture
stream the binding launches on), then replayed several times with eager
work and a synchronisation between the replays; every replay is compared
bit for bit with the eager result of the same call on the same inputs.
Calls that update the state in place are compared step by step against a
run of eager calls from the same start state.  The kernels are
deterministic (fixed summation orders), so equality is exact.
"""

import numpy as np
import pytest
import torch

import gdn_inputs as gi
from helpers import bits, ensure_built, upload

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()
    assert torch.cuda.is_available()


def _gdn():
    import linear_attention_recurrence_net_amd as gdn
    return gdn


def _capture(fn):
    """Warm up fn eagerly on a side stream (as torch asks before a
    capture), then capture one call of it."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _in_place_replays(call, state, o, s0):
    """call() updates `state` in place and writes `o`.  Eager reference:
    REPLAYS calls from s0, recording state and o after each.  Then the
    captured call is replayed REPLAYS times from s0."""
    ref = []
    state.copy_(s0)
    for _ in range(REPLAYS):
        call()
        torch.cuda.synchronize()
        ref.append((bits(state), bits(o)))
    g = _capture(call)  # the warm-up inside runs the call once more
    state.copy_(s0)
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(state), ref[i][0]), f"state after replay {i}"
        assert np.array_equal(bits(o), ref[i][1]), f"o after replay {i}"
        # eager work between replays on the same stream
        torch.cuda.synchronize()
        _ = (state.sum() + o.sum()).item()


@pytest.mark.parametrize("gate,d", [("gda", 128), ("kda", 64)])
def test_decode_in_place_graph_replays(gate, d):
    c = gi.make_case(4, 1, 4, d, gate=gate, qkv_dtype="bf16", seed=71)
    u = upload(c)
    state = u["state"][:, :, 0].contiguous()
    s0 = state.clone()
    o = torch.empty((c.B, c.T, c.H, c.d_v), device="cuda")
    gdn = _gdn()
    _in_place_replays(lambda: gdn.gdn_forward(u["q"], u["k"], u["v"], u["g"], u["beta"], state, o=o),
                      state, o, s0)


@pytest.mark.parametrize("gate,d", [("gda", 128), ("kda", 64)])
def test_verify_snapshots_graph_replays(gate, d):
    c = gi.make_case(4, 4, 4, d, K=4, gate=gate, qkv_dtype="bf16", seed=72)
    u = upload(c)
    state = u["state"]
    o = torch.empty((c.B, c.T, c.H, c.d_v), device="cuda")
    fin = torch.empty((c.B, c.H, c.d_k, c.d_v), device="cuda")
    gdn = _gdn()
    call = lambda: gdn.gdn_forward_snapshots(u["q"], u["k"], u["v"], u["g"], u["beta"], state, fin, o=o)
    call()
    torch.cuda.synchronize()
    ref = (bits(state), bits(o), bits(fin))  # slot 0 is read only: every call gives these
    g = _capture(call)
    for i in range(REPLAYS):
        state[:, :, 1:].fill_(float("nan"))
        fin.fill_(float("nan"))
        o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(state), ref[0]), f"snapshots after replay {i}"
        assert np.array_equal(bits(o), ref[1]), f"o after replay {i}"
        assert np.array_equal(bits(fin), ref[2]), f"final state after replay {i}"


def test_rollback_graph_replays():
    c = gi.make_case(8, 4, 4, 128, K=4, gate="gda", qkv_dtype="bf16", seed=73)
    u = upload(c)
    state = u["state"]
    gdn = _gdn()
    gdn.gdn_forward_snapshots(u["q"], u["k"], u["v"], u["g"], u["beta"], state)
    torch.cuda.synchronize()
    snap = state.clone()
    accepted = torch.tensor([0, 1, 2, 3, 3, 2, 1, 0], dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    call = lambda: gdn.gdn_rollback_select(accepted, state, err)
    expect = snap.clone()
    for b, a in enumerate(accepted.tolist()):
        expect[b, :, 0] = snap[b, :, a]
    g = _capture(call)
    for i in range(REPLAYS):
        state.copy_(snap)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(state), bits(expect)), f"state after replay {i}"
        assert int(err.item()) == 0


@pytest.mark.parametrize("entry", ["workspace", "noalloc"])
@pytest.mark.parametrize("gate", ["gda", "kda"])
def test_prefill_in_place_graph_replays(entry, gate):
    # several chunks and a ragged tail
    c = gi.make_case(2, 200, 4, 128, gate=gate, qkv_dtype="bf16", seed=74)
    u = upload(c)
    state = u["state"][:, :, 0].contiguous()
    s0 = state.clone()
    o = torch.empty((c.B, c.T, c.H, c.d_v), device="cuda")
    gdn = _gdn()
    if entry == "workspace":
        code = gdn.GDN_GATE_KEY if gate == "kda" else gdn.GDN_GATE_HEAD
        ws = torch.empty(gdn.gdn_prefill_workspace_size_ex(c.B, c.T, c.H, 128, 128, 64, gdn.GDN_BF16, code),
                         dtype=torch.uint8, device="cuda")
        call = lambda: gdn.gdn_prefill_chunked_ex(u["q"], u["k"], u["v"], u["g"], u["beta"], state, o=o,
                                                  workspace=ws)
    else:
        call = lambda: gdn.gdn_prefill_chunked_ex_noalloc(u["q"], u["k"], u["v"], u["g"], u["beta"], state, o)
    _in_place_replays(call, state, o, s0)


@pytest.mark.parametrize("gate", ["gda", "kda"])
def test_prefill_varlen_graph_replays(gate):
    # packed sequences: the device table of sequence starts is built inside the
    # captured work, from offsets that stay on the device
    lengths = [0, 70, 1, 130, 64, 0, 9]
    vc = gi.make_varlen_case(lengths, 4, 64, seed=75, gate=gate)
    bf = torch.bfloat16
    q, k, v = (torch.from_numpy(x).to(bf).cuda() for x in (vc.q, vc.k, vc.v))
    g, beta = torch.from_numpy(vc.g).cuda(), torch.from_numpy(vc.beta).cuda()
    cu = torch.from_numpy(vc.cu_seqlens).cuda()
    state = torch.from_numpy(vc.state).cuda()
    s0 = state.clone()
    o = torch.zeros((vc.total, vc.H, vc.d), device="cuda")
    gdn = _gdn()
    code = gdn.GDN_GATE_KEY if gate == "kda" else gdn.GDN_GATE_HEAD
    ws = torch.empty(gdn.gdn_prefill_varlen_workspace_size_ex(len(lengths), vc.total, vc.H, vc.d, vc.d, 64,
                                                               gdn.GDN_BF16, code),
                     dtype=torch.uint8, device="cuda")
    call = lambda: gdn.gdn_prefill_chunked_varlen_ex(cu, q, k, v, g, beta, state, o=o, workspace=ws)
    _in_place_replays(call, state, o, s0)


@pytest.mark.parametrize("gate", ["gda", "kda"])
def test_prefill_snapshots_graph_replays(gate):
    # the chunked path with K = 5 slots and a final state (slots 1..4 after
    # tokens 1..4, the final state after all 90)
    c = gi.make_case(2, 90, 2, 128, K=5, gate=gate, qkv_dtype="bf16", seed=76)
    u = upload(c)
    state = u["state"]
    s0 = state.clone()
    fin = torch.zeros((c.B, c.H, c.d_k, c.d_v), device="cuda")
    o = torch.empty((c.B, c.T, c.H, c.d_v), device="cuda")
    gdn = _gdn()
    code = gdn.GDN_GATE_KEY if gate == "kda" else gdn.GDN_GATE_HEAD
    ws = torch.empty(gdn.gdn_prefill_workspace_size_ex(c.B, c.T, c.H, 128, 128, 64, gdn.GDN_BF16, code),
                     dtype=torch.uint8, device="cuda")
    call = lambda: gdn.gdn_prefill_chunked_ex(u["q"], u["k"], u["v"], u["g"], u["beta"], state, final_state=fin,
                                              o=o, workspace=ws)
    call()
    torch.cuda.synchronize()
    ref = (bits(state), bits(o), bits(fin))
    g = _capture(call)
    for i in range(REPLAYS):
        state.copy_(s0)
        fin.fill_(float("nan"))
        o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(state), ref[0]), f"snapshots after replay {i}"
        assert np.array_equal(bits(o), ref[1]), f"o after replay {i}"
        assert np.array_equal(bits(fin), ref[2]), f"final state after replay {i}"


@pytest.mark.parametrize("gate,d", [("gda", 128), ("kda", 64)])
def test_rollback_fused_into_verify_graph_replays(gate, d):
    c = gi.make_case(6, 4, 4, d, K=4, gate=gate, qkv_dtype="bf16", seed=77)
    u = upload(c)
    state = u["state"]
    state[:, :, 1:] = torch.randn_like(state[:, :, 1:])
    s0 = state.clone()
    o = torch.empty((c.B, c.T, c.H, c.d_v), device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    acc = torch.tensor([0, 1, 2, 3, 3, 1], dtype=torch.int32, device="cuda")
    gdn = _gdn()
    call = lambda: gdn.gdn_forward_snapshots_after_rollback(acc, u["q"], u["k"], u["v"], u["g"], u["beta"], state,
                                                            o=o, err_flag=err)
    _in_place_replays(call, state, o, s0)
    assert int(err.item()) == 0
