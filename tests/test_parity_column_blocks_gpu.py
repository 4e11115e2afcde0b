"""Column-block launches of the token kernel against the float64 oracle.

A token-kernel grid that would fill less than one resident round (two
wavefronts per SIMD) is split into 4 or 2 column blocks per head; the
columns of the state are independent, so each block sums and updates its own
columns over every key row.  The sizes here are chosen from the device's
compute-unit count so that each launch form takes each block count: single
token (decode), a 128 x 128 draft of at most four tokens (half-round rule),
the streamed form (more tokens, or smaller tiles), and the rollback fused
into the verification, for head sizes 64 and 128 in every pairing, GDA and
KDA gates, bf16 and float32 inputs.  Bars: 2e-4 per output tensor (o, every
written slot, final state), and the rolled-back slot 0 bit for bit.
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


def _round_waves():
    # wavefronts of one resident round: two per SIMD, four SIMDs per compute unit
    return 8 * torch.cuda.get_device_properties(0).multi_processor_count


def _wph(T, dk, dv, kda):
    if T == 1:
        return 2
    return 4 if (dk == 128 and dv == 128) else 2


def _heads_for(ncb, T, dk, dv, kda):
    """Heads (B * H) for which the launcher picks `ncb` column blocks."""
    draft = T <= 4 and dk == 128 and dv == 128 and T > 1
    rnd = _round_waves() // (2 if draft else 1)
    w = _wph(T, dk, dv, kda)
    if ncb == 4:
        return max(1, rnd // (4 * w))           # 4 * waves <= round
    if ncb == 2:
        return rnd // (2 * w)                   # 2 * waves <= round < 4 * waves
    return rnd // w + 8                         # beyond: whole rows


CASES = []
for T, K in ((1, 1), (3, 4), (9, 5)):
    for dk, dv in ((128, 128), (64, 64), (64, 128), (128, 64)):
        for ncb in (4, 2, 1):
            if ncb == 4 and dv < 128:
                continue
            CASES.append((T, K, dk, dv, ncb))


@pytest.mark.parametrize("T,K,dk,dv,ncb", CASES)
def test_column_blocks_match_oracle(T, K, dk, dv, ncb):
    import linear_attention_recurrence_net_amd as gdn
    kda = dk == 64  # KDA at d_k = 64, GDA at 128
    heads = _heads_for(ncb, T, dk, dv, kda)
    H = 4
    B = max(1, heads // H)
    if ncb == 1 and B * H * _wph(T, dk, dv, kda) <= _round_waves():
        B += 1
    dt = "f32" if (dk + dv + T) % 3 == 0 else "bf16"
    c = gi.make_case(B, T, H, dk, dv, K=K, gate="kda" if kda else "gda", qkv_dtype=dt, seed=1500 + B + T + dk + dv)
    if K > 1:
        rng = np.random.default_rng(1501)
        c.state[:, :, 1:] = (rng.standard_normal(c.state[:, :, 1:].shape) * 0.1).astype(np.float32)
    u = upload(c)
    st = u["state"] if K > 1 else u["state"][:, :, 0].contiguous()
    fin = torch.full((B, H, dk, dv), float("nan"), device="cuda") if K > 1 else None
    o = gdn.gdn_forward_snapshots(u["q"], u["k"], u["v"], u["g"], u["beta"], st, fin) if K > 1 else \
        gdn.gdn_forward(u["q"], u["k"], u["v"], u["g"], u["beta"], st)
    torch.cuda.synchronize()
    ro, rst, rfin = oracle.forward(*oracle_args(c), c.f64("state"), kda=kda, want_final=True)
    errs = {"o": rel_err(o, ro, "o")}
    if K == 1:
        errs["state"] = rel_err(st, rst[:, :, 0], "state")
    else:
        for s in range(1, min(T, K - 1) + 1):
            errs[f"slot{s}"] = rel_err(st[:, :, s], rst[:, :, s], f"slot{s}")
        errs["final"] = rel_err(fin, rfin, "final")
    print(f"B={B} H={H} heads={B * H} ncb={ncb}", {k: f"{v:.1e}" for k, v in errs.items()}, flush=True)
    for name, e in errs.items():
        assert e <= TOL, (name, e)

    if K > 1:
        # the same launch with the previous draft's rollback fused in
        acc_np = np.random.default_rng(1502).integers(0, K, size=B).astype(np.int32)
        acc = torch.from_numpy(acc_np).cuda()
        u2 = upload(gi.make_case(B, T, H, dk, dv, K=K, gate="kda" if kda else "gda", qkv_dtype=dt, seed=1600 + B))
        prev = st.clone()  # the slots of the draft just verified
        st2 = st.clone()
        o2 = gdn.gdn_forward_snapshots_after_rollback(acc, u2["q"], u2["k"], u2["v"], u2["g"], u2["beta"], st2)
        torch.cuda.synchronize()
        ref_st = prev.clone()
        gdn.gdn_rollback_select(acc, ref_st)
        ref_o = gdn.gdn_forward_qk_broadcast(u2["q"], u2["k"], u2["v"], u2["g"], u2["beta"], ref_st)
        torch.cuda.synchronize()
        assert np.array_equal(bits(st2), bits(ref_st))
        assert np.array_equal(bits(o2), bits(ref_o))
        # slot 0 holds slot accepted[b] of the previous draft, bit for bit
        p, s2 = bits(prev), bits(st2)
        for b in range(B):
            assert np.array_equal(s2[b, :, 0], p[b, :, acc_np[b]])
