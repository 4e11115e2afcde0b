"""GPU parity of the chunked prefill that emits K state snapshots.

The slot semantics are those of gdn_forward_snapshots: slot 0 is the input
(not written for K > 1), slot t holds the state after t tokens for
1 <= t <= min(T, K-1), slots past T are untouched, and the final state goes
to final_state (K > 1) or back to slot 0 (K = 1).  Each written tensor is
compared with the float64 oracle's per-token loop at the prefill bar (1e-2);
o and the final state must also equal, bit for bit, the plain chunked
prefill on the same inputs (the snapshots do not change the chain).  Both
gate kinds are covered (KDA with bf16 and float32 inputs), and a rollback
after each is a byte copy of the accepted slot.
"""

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
from helpers import bits, dev, ensure_built, oracle_args, rel_err, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()
    assert torch.cuda.is_available()


def _gdn():
    import linear_attention_recurrence_net_amd as gdn
    return gdn


CASES = [
    # B, T, H, H_qk, d, K, head map
    (2, 16, 4, 4, 128, 4, "grouped"),    # a 16-token draft, 3 snapshots
    (1, 2, 4, 2, 64, 5, "tiled"),        # T < K-1: slots 3, 4 untouched
    (2, 150, 2, 2, 128, 67, "grouped"),  # snapshots 65, 66 fall in the second chunk
    (1, 64, 3, 1, 64, 65, "grouped"),    # one full chunk, a snapshot after every token
    (3, 37, 2, 2, 128, 2, "grouped"),
]


@pytest.mark.parametrize("B,T,H,Hq,d,K,head_map", CASES)
def test_prefill_snapshots(B, T, H, Hq, d, K, head_map):
    c = gi.make_case(B, T, H, d, K=K, qkv_dtype="bf16", seed=800 + T + K, H_qk=Hq)
    c.state[:, :, 1:] = np.float32(np.nan)  # slots the call may not read
    u = upload(c)
    fin = torch.full((B, H, d, d), float("nan"), device="cuda")
    o = _gdn().gdn_prefill_chunked_snapshots(u["q"], u["k"], u["v"], u["g"], u["beta"], u["state"],
                                             head_map=head_map, final_state=fin)
    torch.cuda.synchronize()
    ro, rst, rfin = oracle.forward(*oracle_args(c), c.f64("state"), want_final=True,
                                   head_map=head_map)
    st = u["state"]
    eo, ef = rel_err(o, ro), rel_err(fin, rfin)
    print(f"B={B} T={T} H={H} H_qk={Hq} d={d} K={K}: o {eo:.2e} final {ef:.2e}", flush=True)
    assert eo <= 1e-2 and ef <= 1e-2
    # slot 0 is the input, unchanged
    assert np.array_equal(bits(st[:, :, 0]), c.state[:, :, 0].view(np.int32))
    n = min(T, K - 1)
    worst = 0.0
    for t in range(1, n + 1):
        e = rel_err(st[:, :, t], rst[:, :, t])
        worst = max(worst, e)
        assert e <= 1e-2, (t, e)
    print(f"  {n} snapshots, worst {worst:.2e}", flush=True)
    # slots past T were not written
    if n + 1 < K:
        assert torch.isnan(st[:, :, n + 1:]).all()

    # o and the final state equal the plain chunked prefill's bit for bit
    u2 = upload(c)
    s2 = u2["state"][:, :, 0].contiguous()
    o2 = _gdn().gdn_prefill_chunked_qk_broadcast(u2["q"], u2["k"], u2["v"], u2["g"], u2["beta"], s2,
                                                 head_map=head_map)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o), bits(o2))
    assert np.array_equal(bits(fin), bits(s2))


def test_prefill_snapshots_k1_is_in_place_prefill():
    c = gi.make_case(2, 97, 4, 128, qkv_dtype="bf16", seed=77)
    u, u2 = upload(c), upload(c)
    o = _gdn().gdn_prefill_chunked_snapshots(u["q"], u["k"], u["v"], u["g"], u["beta"], u["state"])
    s2 = u2["state"][:, :, 0].contiguous()
    o2 = _gdn().gdn_prefill_chunked(u2["q"], u2["k"], u2["v"], u2["g"], u2["beta"], s2)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o), bits(o2))
    assert np.array_equal(bits(u["state"][:, :, 0]), bits(s2))


def test_prefill_snapshots_then_rollback():
    """Verify a draft with the chunked path, then roll back: slot 0 must hold
    the state after the accepted number of tokens (within the prefill bar of
    the oracle), and be a byte copy of that snapshot."""
    B, T, H, d, K = 4, 12, 2, 128, 5
    c = gi.make_case(B, T, H, d, K=K, qkv_dtype="bf16", seed=91, with_accepted=True)
    u = upload(c)
    _gdn().gdn_prefill_chunked_snapshots(u["q"], u["k"], u["v"], u["g"], u["beta"], u["state"])
    torch.cuda.synchronize()
    before = u["state"].clone()
    acc = dev(c.accepted)
    _gdn().gdn_rollback_select(acc, u["state"])
    torch.cuda.synchronize()
    _, rst, _ = oracle.forward(*oracle_args(c), c.f64("state"))
    for b in range(B):
        a = int(c.accepted[b])
        assert np.array_equal(bits(u["state"][b, :, 0]), bits(before[b, :, a]))
        ref = rst[b, :, a] if a > 0 else c.f64("state")[b, :, 0]
        assert rel_err(u["state"][b, :, 0], ref) <= 1e-2


def test_prefill_snapshots_empty_copies_slot0():
    c = gi.make_case(2, 1, 3, 64, K=3, qkv_dtype="bf16", seed=5)
    u = upload(c)
    fin = torch.full((2, 3, 64, 64), float("nan"), device="cuda")
    e = torch.empty((2, 0, 3, 64), dtype=torch.bfloat16, device="cuda")
    ge = torch.empty((2, 0, 3), dtype=torch.float32, device="cuda")
    _gdn().gdn_prefill_chunked_snapshots(e, e, e, ge, ge, u["state"], final_state=fin)
    torch.cuda.synchronize()
    assert np.array_equal(bits(fin), bits(u["state"][:, :, 0]))


# KDA (one log-gate per key row) through gdn_prefill_chunked_ex
KDA_CASES = [
    # B, T, H, H_qk, d, K, dtype
    (2, 16, 4, 4, 128, 4, "bf16"),   # a 16-token draft, 3 snapshots
    (1, 2, 4, 2, 64, 5, "bf16"),     # T < K-1: slots 3, 4 untouched
    (2, 150, 2, 2, 128, 67, "bf16"), # snapshots 65, 66 fall in the second chunk
    (1, 64, 3, 1, 64, 65, "bf16"),   # one full chunk, a snapshot after every token
    (2, 37, 2, 2, 128, 9, "f32"),    # float32 inputs (rounded to bf16 on this path)
    (3, 23, 2, 2, 128, 6, "bf16"),   # a partial last batch of the snapshot loop
]


@pytest.mark.parametrize("B,T,H,Hq,d,K,dt", KDA_CASES)
def test_prefill_snapshots_kda(B, T, H, Hq, d, K, dt):
    c = gi.make_case(B, T, H, d, K=K, gate="kda", qkv_dtype=dt, seed=850 + T + K, H_qk=Hq)
    c.state[:, :, 1:] = np.float32(np.nan)  # slots the call may not read
    u = upload(c)
    fin = torch.full((B, H, d, d), float("nan"), device="cuda")
    o = _gdn().gdn_prefill_chunked_ex(u["q"], u["k"], u["v"], u["g"], u["beta"], u["state"],
                                      final_state=fin)
    torch.cuda.synchronize()
    ro, rst, rfin = oracle.forward(*oracle_args(c), c.f64("state"), kda=True, want_final=True)
    st = u["state"]
    eo, ef = rel_err(o, ro, "o"), rel_err(fin, rfin, "final")
    print(f"KDA B={B} T={T} H={H} H_qk={Hq} d={d} K={K} {dt}: o {eo:.2e} final {ef:.2e}", flush=True)
    assert eo <= 1e-2 and ef <= 1e-2
    assert np.array_equal(bits(st[:, :, 0]), c.state[:, :, 0].view(np.int32))
    n = min(T, K - 1)
    worst = 0.0
    for t in range(1, n + 1):
        e = rel_err(st[:, :, t], rst[:, :, t], f"slot{t}")
        worst = max(worst, e)
        assert e <= 1e-2, (t, e)
    print(f"  {n} snapshots, worst {worst:.2e}", flush=True)
    if n + 1 < K:
        assert torch.isnan(st[:, :, n + 1:]).all()
    # o and the final state equal the plain KDA chunked prefill's bit for bit
    u2 = upload(c)
    s2 = u2["state"][:, :, 0].contiguous()
    o2 = _gdn().gdn_prefill_chunked_ex(u2["q"], u2["k"], u2["v"], u2["g"], u2["beta"], s2)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o), bits(o2))
    assert np.array_equal(bits(fin), bits(s2))


def test_prefill_snapshots_kda_then_rollback():
    """KDA draft verified with the chunked path, then rolled back: slot 0 is a
    byte copy of the accepted snapshot and within the prefill bar of the
    oracle's state after that many tokens."""
    B, T, H, d, K = 4, 12, 2, 64, 5
    c = gi.make_case(B, T, H, d, K=K, gate="kda", qkv_dtype="bf16", seed=93, with_accepted=True)
    u = upload(c)
    _gdn().gdn_prefill_chunked_ex(u["q"], u["k"], u["v"], u["g"], u["beta"], u["state"])
    torch.cuda.synchronize()
    before = u["state"].clone()
    _gdn().gdn_rollback_select(dev(c.accepted), u["state"])
    torch.cuda.synchronize()
    _, rst, _ = oracle.forward(*oracle_args(c), c.f64("state"), kda=True)
    for b in range(B):
        a = int(c.accepted[b])
        assert np.array_equal(bits(u["state"][b, :, 0]), bits(before[b, :, a]))
        ref = rst[b, :, a] if a > 0 else c.f64("state")[b, :, 0]
        assert rel_err(u["state"][b, :, 0], ref) <= 1e-2
