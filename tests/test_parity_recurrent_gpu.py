"""GPU parity of the decode / verify / rollback path against the float64 oracle.

Bars: max|gpu - ref| / max|ref| <= 2e-4 per output tensor (o, every written
state slot, final state) for the fp32 recurrent path; bit-exact for slot
selection, rollback copies and the special cases whose result is exact in
IEEE arithmetic (beta = 0 with gate 1, K = 1 against the single-slot call).

The workloads are run at their full sizes (decode B=64 H=16 d=128; verify
B=32 H=16 d=128 T=4 K=4; KDA verify B=32 H=32 d=64 T=4 K=4) in the launch
configuration the benchmark times, and compared on every output.
"""

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
from helpers import bits, ensure_built, oracle_args, rel_err, upload

pytestmark = pytest.mark.gpu

TOL = 2e-4


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()
    import linear_attention_recurrence_net_amd as gdn
    gdn.library()
    assert torch.cuda.is_available()


def _gdn():
    import linear_attention_recurrence_net_amd as gdn
    return gdn


def _run_snapshots(case, want_final=True):
    d = upload(case)
    fin = torch.empty((case.B, case.H, case.d_k, case.d_v), device="cuda") if want_final else None
    o = _gdn().gdn_forward_snapshots(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], fin)
    torch.cuda.synchronize()
    return o, d["state"], fin


def _check_against_oracle(case, o, st, fin):
    ro, rst, rfin = oracle.forward(*oracle_args(case), case.f64("state"), kda=case.gate == "kda",
                                   want_final=fin is not None)
    errs = {"o": rel_err(o, ro, "o")}
    n_written = min(case.T, case.K - 1) if case.K > 1 else 0
    if case.K == 1:
        errs["state"] = rel_err(st[:, :, 0], rst[:, :, 0], "state")
    for s in range(1, n_written + 1):
        errs[f"slot{s}"] = rel_err(st[:, :, s], rst[:, :, s], f"slot{s}")
    if fin is not None:
        errs["final"] = rel_err(fin, rfin, "final")
    print(case.B, case.T, case.H, case.d_k, case.gate, case.qkv_dtype, errs, flush=True)
    for name, e in errs.items():
        assert e <= TOL, (name, e)
    # slots not written must be bit-identical to their input
    if case.K > 1:
        assert np.array_equal(bits(st[:, :, 0]), case.state[:, :, 0].view(np.int32))
        for s in range(n_written + 1, case.K):
            assert np.array_equal(bits(st[:, :, s]), case.state[:, :, s].view(np.int32))
    return rst


def test_config0_tiny_fp32():
    c = gi.workload_case(0)
    o, st, fin = _run_snapshots(c)
    _check_against_oracle(c, o, st, fin)


def test_config1_decode_full_size():
    c = gi.workload_case(1)
    d = upload(c)
    state = d["state"][:, :, 0].contiguous()  # [B,H,d,d], K = 1
    o = _gdn().gdn_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], state)
    torch.cuda.synchronize()
    ro, rst, _ = oracle.forward(*oracle_args(c), c.f64("state"))
    eo, es = rel_err(o, ro, "o"), rel_err(state, rst[:, :, 0], "state")
    print("decode", eo, es, flush=True)
    assert eo <= TOL and es <= TOL


@pytest.mark.parametrize("cfg", [2, 3])
@pytest.mark.parametrize("with_final", [True, False])
def test_verify_and_rollback_full_size(cfg, with_final):
    """The verify workloads at full size, with a final state and without one
    (the launch the benchmark times: then no state after the last token is
    stored anywhere, and slot 0 must keep the input bit for bit)."""
    c = gi.workload_case(cfg)
    d = upload(c)
    fin = torch.empty((c.B, c.H, c.d_k, c.d_v), device="cuda") if with_final else None
    o = _gdn().gdn_forward_snapshots(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], fin)
    torch.cuda.synchronize()
    st = d["state"]
    rst = _check_against_oracle(c, o, st, fin)
    assert np.array_equal(bits(st[:, :, 0]), c.state[:, :, 0].view(np.int32))

    before = bits(st)
    acc = torch.from_numpy(c.accepted).to("cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    _gdn().gdn_rollback_select(acc, st, err)
    torch.cuda.synchronize()
    after = bits(st)
    assert int(err.item()) == 0
    ref_rolled, n_bad = oracle.rollback(c.accepted, rst)
    assert n_bad == 0
    for b in range(c.B):
        a = int(c.accepted[b])
        # slot 0 <- the GPU's own slot a, bit for bit; other slots unchanged
        assert np.array_equal(after[b, :, 0], before[b, :, a]), b
        assert np.array_equal(after[b, :, 1:], before[b, :, 1:]), b
    # the selected state agrees with the oracle's selection
    assert rel_err(st[:, :, 0], ref_rolled[:, :, 0]) <= TOL


@pytest.mark.parametrize("B,T,H,d,gate,dt,K", [
    (3, 37, 4, 128, "gda", "bf16", 1),
    (2, 19, 3, 128, "kda", "bf16", 1),
    (2, 23, 3, 64, "gda", "f32", 1),
    (5, 9, 2, 64, "kda", "f32", 1),
    (4, 7, 2, 128, "gda", "f32", 6),
    (3, 2, 2, 128, "kda", "bf16", 5),   # T < K-1: slots 3, 4 untouched
    (2, 8, 2, 64, "gda", "bf16", 3),    # T > K-1
    (1, 1, 1, 64, "kda", "bf16", 2),
])
def test_shapes_and_modes(B, T, H, d, gate, dt, K):
    c = gi.make_case(B, T, H, d, K=K, gate=gate, qkv_dtype=dt, seed=100 + B * T + d)
    if K > 1:  # poison the slots the call may not write
        c.state[:, :, 1:] = np.float32(np.nan)
    o, st, fin = _run_snapshots(c)
    _check_against_oracle(c, o, st, fin)


def test_k1_snapshots_equal_single_slot_bitwise():
    c = gi.make_case(4, 5, 3, 128, K=1, gate="gda", seed=31)
    d1, d2 = upload(c), upload(c)
    s1 = d1["state"][:, :, 0].contiguous()
    o1 = _gdn().gdn_forward(d1["q"], d1["k"], d1["v"], d1["g"], d1["beta"], s1)
    o2 = _gdn().gdn_forward_snapshots(d2["q"], d2["k"], d2["v"], d2["g"], d2["beta"], d2["state"])
    torch.cuda.synchronize()
    assert np.array_equal(bits(o1), bits(o2))
    assert np.array_equal(bits(s1), bits(d2["state"][:, :, 0]))


@pytest.mark.parametrize("gate", ["gda", "kda"])
def test_beta0_gate1_state_unchanged_bitwise(gate):
    c = gi.make_case(3, 6, 2, 128, K=1, gate=gate, seed=41)
    c.beta[:] = 0.0
    c.g[:] = 0.0
    d = upload(c)
    s = d["state"][:, :, 0].contiguous()
    o = _gdn().gdn_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], s)
    torch.cuda.synchronize()
    assert np.array_equal(bits(s), c.state[:, :, 0].view(np.int32))
    ro, _, _ = oracle.forward(*oracle_args(c), c.f64("state"), kda=gate == "kda")
    assert rel_err(o, ro) <= TOL


def test_zero_tokens_copies_final_state_only():
    c = gi.make_case(2, 0, 2, 64, K=3, seed=5)
    c.state[:, :, 1:] = 3.5
    d = upload(c)
    fin = torch.full((2, 2, 64, 64), -1.0, device="cuda")
    o = _gdn().gdn_forward_snapshots(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], fin)
    torch.cuda.synchronize()
    assert o.numel() == 0
    assert np.array_equal(bits(fin), c.state[:, :, 0].view(np.int32))
    assert np.array_equal(bits(d["state"]), c.state.view(np.int32))


def test_repeat_runs_bitwise_deterministic():
    c = gi.workload_case(2)
    outs = []
    for _ in range(2):
        o, st, fin = _run_snapshots(c)
        outs.append((bits(o), bits(st), bits(fin)))
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("d", [64, 128])  # 128: few 64 KiB tiles, each copied by four workgroups
def test_rollback_edge_cases_and_error_flag(d):
    rng = np.random.default_rng(8)
    B, H, K = 6, 3, 4
    st_np = rng.standard_normal((B, H, K, d, d)).astype(np.float32)
    st = torch.from_numpy(st_np.copy()).to("cuda")
    acc_np = np.array([0, 3, -1, 4, 1, 2], dtype=np.int32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    _gdn().gdn_rollback_select(torch.from_numpy(acc_np).to("cuda"), st, err)
    torch.cuda.synchronize()
    out = st.cpu().numpy()
    assert int(err.item()) == 1
    ref, n_bad = oracle.rollback(acc_np, st_np.astype(np.float64))
    assert n_bad == 2
    assert np.array_equal(out.view(np.int32), ref.astype(np.float32).view(np.int32))


@pytest.mark.parametrize("d_k,d_v", [(48, 48), (128, 128), (32, 96)])
def test_rollback_any_tile(d_k, d_v):
    rng = np.random.default_rng(d_k + d_v)
    B, H, K = 5, 2, 3
    st_np = rng.standard_normal((B, H, K, d_k, d_v)).astype(np.float32)
    st = torch.from_numpy(st_np.copy()).to("cuda")
    acc_np = rng.integers(0, K, B).astype(np.int32)
    _gdn().gdn_rollback_select(torch.from_numpy(acc_np).to("cuda"), st)
    torch.cuda.synchronize()
    ref, _ = oracle.rollback(acc_np, st_np.astype(np.float64))
    assert np.array_equal(st.cpu().numpy().view(np.int32), ref.astype(np.float32).view(np.int32))


def test_graph_replay_matches_eager():
    """The bench times HIP-graph replays of these launches: every replay must
    equal the eager result bit for bit, with eager work between replays."""
    c = gi.make_case(8, 4, 4, 128, K=4, gate="gda", seed=77, with_accepted=True)
    d = upload(c)
    acc = torch.from_numpy(c.accepted).to("cuda")
    base = d["state"].clone()
    gdn = _gdn()

    work = base.clone()
    o = torch.empty((c.B, c.T, c.H, c.d_v), device="cuda")
    gdn.gdn_forward_snapshots(d["q"], d["k"], d["v"], d["g"], d["beta"], work, None, o)
    gdn.gdn_rollback_select(acc, work)
    torch.cuda.synchronize()
    ref_o, ref_s = bits(o), bits(work)

    work2 = torch.empty_like(base)
    o2 = torch.empty_like(o)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        torch.mul(base, 1.0, out=work2)  # reset the state with a kernel (x * 1 is exact)
        gdn.gdn_forward_snapshots(d["q"], d["k"], d["v"], d["g"], d["beta"], work2, None, o2)
        gdn.gdn_rollback_select(acc, work2)
    for _ in range(3):
        work2.fill_(float("nan"))
        o2.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(o2), ref_o)
        assert np.array_equal(bits(work2), ref_s)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("gate", ["gda", "kda"])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_single_token_kernel_all_variants(d, gate, dt):
    """The single-token decode instantiation for every head size, gate mode
    and input dtype."""
    c = gi.make_case(6, 1, 5, d, K=1, gate=gate, qkv_dtype=dt, seed=500 + d)
    d_ = upload(c)
    s = d_["state"][:, :, 0].contiguous()
    o = _gdn().gdn_forward(d_["q"], d_["k"], d_["v"], d_["g"], d_["beta"], s)
    torch.cuda.synchronize()
    ro, rst, _ = oracle.forward(*oracle_args(c), c.f64("state"), kda=gate == "kda")
    assert rel_err(o, ro) <= TOL and rel_err(s, rst[:, :, 0]) <= TOL


def test_large_decode_grid_sampled_heads():
    """B=512 sequences x 16 heads (512 MiB of state, 8x the decode workload);
    the oracle checks a seeded sample of (sequence, head) pairs one by one."""
    B, H, d = 512, 16, 128
    c = gi.make_case(B, 1, H, d, K=1, gate="gda", qkv_dtype="bf16", seed=808)
    d_ = upload(c)
    s = d_["state"][:, :, 0].contiguous()
    o = _gdn().gdn_forward(d_["q"], d_["k"], d_["v"], d_["g"], d_["beta"], s)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    picks = [(int(b), int(h)) for b, h in zip(rng.integers(0, B, 24), rng.integers(0, H, 24))]
    picks += [(0, 0), (B - 1, H - 1)]
    for b, h in picks:
        one = lambda x: np.ascontiguousarray(x[b:b + 1, :, h:h + 1], dtype=np.float64)
        ro, rst, _ = oracle.forward(one(c.q), one(c.k), one(c.v), one(c.g), one(c.beta),
                                    np.asarray(c.state[b:b + 1, h:h + 1], dtype=np.float64))
        assert rel_err(o[b:b + 1, :, h:h + 1], ro) <= TOL, (b, h)
        assert rel_err(s[b:b + 1, h:h + 1], rst[:, :, 0]) <= TOL, (b, h)


@pytest.mark.parametrize("gate", ["gda", "kda"])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_decode_beyond_one_resident_round(gate, dt):
    """A single-token 128 x 128 grid with more heads than one resident round
    of two-wavefront workgroups holds (four per compute unit) runs four
    wavefronts per head; both sides of that threshold match the oracle."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    H, d = 16, 128
    for heads in (4 * cus, 4 * cus + H):
        B = heads // H
        c = gi.make_case(B, 1, H, d, K=1, gate=gate, qkv_dtype=dt, seed=900 + B)
        d_ = upload(c)
        s = d_["state"][:, :, 0].contiguous()
        o = _gdn().gdn_forward(d_["q"], d_["k"], d_["v"], d_["g"], d_["beta"], s)
        torch.cuda.synchronize()
        ro, rst, _ = oracle.forward(*oracle_args(c), c.f64("state"), kda=gate == "kda")
        eo, es = rel_err(o, ro), rel_err(s, rst[:, :, 0])
        print(B * H, gate, dt, eo, es, flush=True)
        assert eo <= TOL and es <= TOL, (B * H, eo, es)
