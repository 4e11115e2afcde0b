"""The rollback fused into the chunked prefill.

gdn_prefill_chunked_ex_after_rollback(accepted, ...) must give the bits of
gdn_rollback_select(accepted) followed by gdn_prefill_chunked_ex on the same
state: every slot, o, the final state and the error flag.  The state starts
with every slot holding a different random state (a previous draft's
snapshots); the accepted lengths cover 0, the last slot, slots that the call
overwrites with its own snapshots, and an invalid index.  The result is also
checked against the float64 oracle's rollback followed by its token loop at
the prefill bar (max|gpu - ref| / max|ref| <= 1e-2).  Covered: GDA and KDA,
bf16 and float32 inputs, both head maps with shared q/k heads, unequal head
sizes, token counts inside one chunk and across chunk edges, snapshots inside
one chunk and across two, with and without a final state, and the degenerate
T = 0 and K = 1 calls (which the entry point makes as the two calls).
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


CASES = [
    # B, T, H, H_qk, d_k, d_v, K, gate, dtype, head map, final state
    (4, 100, 4, 2, 128, 128, 5, "gda", "bf16", "grouped", True),
    (3, 130, 2, 1, 128, 64, 70, "gda", "f32", "tiled", False),
    (4, 64, 4, 4, 64, 128, 17, "kda", "bf16", "grouped", True),
    (3, 200, 6, 3, 128, 128, 70, "kda", "f32", "tiled", True),
    (5, 17, 2, 2, 64, 64, 4, "gda", "bf16", "grouped", False),
    (4, 65, 4, 1, 128, 128, 2, "kda", "bf16", "grouped", True),
]


def _accepted(B, K, seed):
    rng = np.random.default_rng(seed)
    acc = rng.integers(0, K, size=B).astype(np.int32)
    acc[0] = K - 1
    acc[1] = 1 if K > 1 else 0
    acc[-1] = K if B > 3 else -1  # invalid: flagged, the sequence starts from slot 0
    return acc


def _run_pair(gdn, u, state0, acc, hm, final, T):
    B, H, _, dk, dv = state0.shape

    def run(fused):
        st = state0.clone()
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        fin = torch.full((B, H, dk, dv), float("nan"), device="cuda") if final else None
        o = torch.full((B, T, H, dv), float("nan"), device="cuda")
        if fused:
            gdn.gdn_prefill_chunked_ex_after_rollback(acc, u["q"], u["k"], u["v"], u["g"], u["beta"], st,
                                                      head_map=hm, final_state=fin, o=o, err_flag=err)
        else:
            gdn.gdn_rollback_select(acc, st, err)
            gdn.gdn_prefill_chunked_ex(u["q"], u["k"], u["v"], u["g"], u["beta"], st, head_map=hm,
                                       final_state=fin, o=o)
        torch.cuda.synchronize()
        return st, o, fin, err

    return run(True), run(False)


@pytest.mark.parametrize("B,T,H,Hq,dk,dv,K,gate,dt,hm,final", CASES)
def test_prefill_fused_rollback_equals_two_calls_and_oracle(B, T, H, Hq, dk, dv, K, gate, dt, hm, final):
    gdn = _gdn()
    c = gi.make_case(B, T, H, dk, dv, K=K, gate=gate, qkv_dtype=dt, seed=710 + K + T, H_qk=Hq)
    # the previous draft: every slot a different state
    rng = np.random.default_rng(720 + K)
    c.state[:] = (rng.standard_normal(c.state.shape) * 0.1).astype(np.float32)
    u = upload(c)
    state0 = u["state"]
    acc_np = _accepted(B, K, seed=730 + B)
    acc = torch.from_numpy(acc_np).cuda()

    (st_f, o_f, fin_f, err_f), (st_t, o_t, fin_t, err_t) = _run_pair(gdn, u, state0, acc, hm, final, T)
    assert np.array_equal(bits(st_f), bits(st_t)), "state slots"
    assert np.array_equal(bits(o_f), bits(o_t)), "o"
    if final:
        assert np.array_equal(bits(fin_f), bits(fin_t)), "final state"
    assert int(err_f.item()) == int(err_t.item()) == 1

    # the oracle: rollback of the previous draft's state, then the token loop
    rolled, n_bad = oracle.rollback(acc_np, c.f64("state"))
    assert n_bad == 1
    ro, rst, rfin = oracle.forward(*oracle_args(c), rolled, kda=gate == "kda", want_final=True, head_map=hm)
    errs = {"o": rel_err(o_f, ro, "o")}
    n_snap = min(T, K - 1)
    for s in range(n_snap + 1):
        errs[f"slot{s}"] = rel_err(st_f[:, :, s], rst[:, :, s], f"slot{s}")
    # slots past the call's snapshots keep the previous draft's bits
    assert np.array_equal(bits(st_f)[:, :, n_snap + 1:], bits(state0)[:, :, n_snap + 1:])
    if final:
        errs["final"] = rel_err(fin_f, rfin, "final")
    worst = max(errs, key=errs.get)
    print(f"worst {worst} {errs[worst]:.2e}", flush=True)
    for name, e in errs.items():
        assert e <= TOL, (name, e)


@pytest.mark.parametrize("T,K", [(0, 4), (70, 1)])
def test_prefill_fused_rollback_degenerate_cases(T, K):
    # T = 0: the rollback alone (with a final-state copy); K = 1: only the flag
    gdn = _gdn()
    B, H, d = 4, 2, 64
    c = gi.make_case(B, max(T, 1), H, d, K=K, gate="gda", qkv_dtype="bf16", seed=740 + T)
    u = upload(c)
    u = {n: (x[:, :T] if n in ("q", "k", "v", "g", "beta") else x) for n, x in u.items()}
    base = u["state"].clone()
    base[:, :, 1:] = torch.randn_like(base[:, :, 1:])
    acc = torch.tensor([0, K - 1, min(1, K - 1), K], dtype=torch.int32, device="cuda")
    a, b = _run_pair(gdn, u, base, acc, "grouped", K > 1, T)
    assert np.array_equal(bits(a[0]), bits(b[0]))
    assert np.array_equal(bits(a[1]), bits(b[1]))
    if K > 1:
        assert np.array_equal(bits(a[2]), bits(b[2]))
    assert int(a[3].item()) == int(b[3].item()) == 1


def test_prefill_fused_rollback_graph_replays():
    """The fused call captured in a HIP graph, replayed three times from the
    same previous-draft state with different accepted lengths, each replay
    bit-identical to the eager two calls."""
    gdn = _gdn()
    B, T, H, d, K = 4, 100, 4, 128, 5
    c = gi.make_case(B, T, H, d, K=K, gate="gda", qkv_dtype="bf16", seed=750)
    rng = np.random.default_rng(751)
    c.state[:] = (rng.standard_normal(c.state.shape) * 0.1).astype(np.float32)
    u = upload(c)
    state0 = u["state"].clone()
    st = state0.clone()
    acc = torch.zeros(B, dtype=torch.int32, device="cuda")
    o = torch.empty((B, T, H, d), device="cuda")
    ws = torch.empty(gdn.gdn_prefill_workspace_size_ex(B, T, H, d, d), dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        gdn.gdn_prefill_chunked_ex_after_rollback(acc, u["q"], u["k"], u["v"], u["g"], u["beta"], st, o=o,
                                                  workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gdn.gdn_prefill_chunked_ex_after_rollback(acc, u["q"], u["k"], u["v"], u["g"], u["beta"], st, o=o,
                                                  workspace=ws)
    for rep, lens in enumerate(([0, 1, 2, 3], [4, 4, 1, 0], [2, 3, 4, 1])):
        st.copy_(state0)
        acc.copy_(torch.tensor(lens, dtype=torch.int32))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref_st = state0.clone()
        gdn.gdn_rollback_select(acc, ref_st)
        ref_o = gdn.gdn_prefill_chunked_ex(u["q"], u["k"], u["v"], u["g"], u["beta"], ref_st)
        torch.cuda.synchronize()
        assert np.array_equal(bits(st), bits(ref_st)), rep
        assert np.array_equal(bits(o), bits(ref_o)), rep
