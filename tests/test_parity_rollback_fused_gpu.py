"""The rollback fused into the next verification.

gdn_forward_snapshots_after_rollback(accepted, ...) must give the bits of
gdn_rollback_select(accepted) followed by gdn_forward_qk_broadcast on the
same state: every slot, o, the final state and the error flag.  The state
starts from a previous draft (slots 1..K-1 written by a verification), the
accepted lengths cover 0, every valid slot and an invalid index.  The result
is also checked against the float64 oracle's rollback followed by its token
loop at the fp32 bar (2e-4).  Covered: the 128 x 128 four-token draft form,
the streaming form (more tokens than the draft form takes), 64 x 64 KDA,
unequal head sizes with shared q/k heads, a final state, K = 1 and T = 0
(which the entry point runs as the two calls).
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
    assert torch.cuda.is_available()


def _gdn():
    import linear_attention_recurrence_net_amd as gdn
    return gdn


CASES = [
    # B, T, H, H_qk, d_k, d_v, K, gate, dtype, head map, final state
    (8, 4, 4, 4, 128, 128, 4, "gda", "bf16", "grouped", False),
    (6, 7, 2, 1, 128, 128, 5, "gda", "f32", "grouped", True),
    (8, 4, 4, 2, 64, 64, 4, "kda", "bf16", "tiled", False),
    (5, 3, 6, 3, 64, 128, 6, "kda", "f32", "grouped", True),
    (4, 1, 2, 2, 128, 64, 3, "gda", "bf16", "tiled", True),
]


def _accepted(B, K, seed):
    rng = np.random.default_rng(seed)
    acc = rng.integers(0, K, size=B).astype(np.int32)
    acc[0] = 0
    acc[1] = K - 1
    acc[-1] = K if B > 2 else -1  # invalid: flagged, the sequence starts from slot 0
    return acc


@pytest.mark.parametrize("B,T,H,Hq,dk,dv,K,gate,dt,hm,final", CASES)
def test_fused_rollback_equals_two_calls_and_oracle(B, T, H, Hq, dk, dv, K, gate, dt, hm, final):
    gdn = _gdn()
    # a previous draft fills slots 1..K-1
    prev = gi.make_case(B, K - 1, H, dk, dv, K=K, gate=gate, qkv_dtype=dt, seed=640 + K, H_qk=Hq)
    up = upload(prev)
    state0 = up["state"]
    gdn.gdn_forward_qk_broadcast(up["q"], up["k"], up["v"], up["g"], up["beta"], state0, head_map=hm)
    # the next draft's inputs
    c = gi.make_case(B, T, H, dk, dv, K=K, gate=gate, qkv_dtype=dt, seed=650 + T, H_qk=Hq)
    u = upload(c)
    acc_np = _accepted(B, K, seed=660 + B)
    acc = torch.from_numpy(acc_np).cuda()

    def run(fused):
        st = state0.clone()
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        fin = torch.full((B, H, dk, dv), float("nan"), device="cuda") if final else None
        if fused:
            o = gdn.gdn_forward_snapshots_after_rollback(acc, u["q"], u["k"], u["v"], u["g"], u["beta"], st,
                                                         head_map=hm, final_state=fin, err_flag=err)
        else:
            gdn.gdn_rollback_select(acc, st, err)
            o = gdn.gdn_forward_qk_broadcast(u["q"], u["k"], u["v"], u["g"], u["beta"], st, head_map=hm,
                                             final_state=fin)
        torch.cuda.synchronize()
        return st, o, fin, err

    st_f, o_f, fin_f, err_f = run(True)
    st_t, o_t, fin_t, err_t = run(False)
    assert np.array_equal(bits(st_f), bits(st_t)), "state slots"
    assert np.array_equal(bits(o_f), bits(o_t)), "o"
    if final:
        assert np.array_equal(bits(fin_f), bits(fin_t)), "final state"
    assert int(err_f.item()) == int(err_t.item()) == 1

    # the oracle: rollback of the previous draft's state, then the token loop
    prev_state = state0.double().cpu().numpy()
    rolled, n_bad = oracle.rollback(acc_np, prev_state)
    assert n_bad == 1
    ro, rst, rfin = oracle.forward(*oracle_args(c), rolled, kda=gate == "kda", want_final=True, head_map=hm)
    errs = {"o": rel_err(o_f, ro, "o")}
    n_snap = min(T, K - 1)
    for s in range(n_snap + 1):
        errs[f"slot{s}"] = rel_err(st_f[:, :, s], rst[:, :, s], f"slot{s}")
    if final:
        errs["final"] = rel_err(fin_f, rfin, "final")
    print({k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for name, e in errs.items():
        assert e <= TOL, (name, e)


@pytest.mark.parametrize("T,K", [(0, 4), (3, 1)])
def test_fused_rollback_degenerate_cases(T, K):
    # T = 0: the rollback alone (with a final-state copy); K = 1: only the flag
    gdn = _gdn()
    B, H, d = 4, 2, 64
    c = gi.make_case(B, max(T, 1), H, d, K=K, gate="gda", qkv_dtype="bf16", seed=670 + T)
    u = upload(c)
    q, k, v, g, beta = (x[:, :T] for x in (u["q"], u["k"], u["v"], u["g"], u["beta"]))
    base = u["state"].clone()
    base[:, :, 1:] = torch.randn_like(base[:, :, 1:])
    acc = torch.tensor([0, K - 1, min(1, K - 1), K], dtype=torch.int32, device="cuda")

    def run(fused):
        st = base.clone()
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        fin = torch.full((B, H, d, d), float("nan"), device="cuda") if K > 1 else None
        o = torch.zeros((B, T, H, d), device="cuda")
        if fused:
            gdn.gdn_forward_snapshots_after_rollback(acc, q, k, v, g, beta, st, final_state=fin, o=o, err_flag=err)
        else:
            gdn.gdn_rollback_select(acc, st, err)
            gdn.gdn_forward_qk_broadcast(q, k, v, g, beta, st, final_state=fin, o=o)
        torch.cuda.synchronize()
        return st, o, fin, err

    a, b = run(True), run(False)
    assert np.array_equal(bits(a[0]), bits(b[0]))
    assert np.array_equal(bits(a[1]), bits(b[1]))
    if K > 1:
        assert np.array_equal(bits(a[2]), bits(b[2]))
    assert int(a[3].item()) == int(b[3].item()) == 1
