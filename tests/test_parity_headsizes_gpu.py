"""GPU parity with unequal key and value head sizes (d_k != d_v).

The pages name head sizes 64 and 128; the kernels take any pairing of the
two.  The state is d_k x d_v: q, k and KDA's gates run along the key axis,
v and o along the value axis.  Each case is compared with the float64
oracle at the path's bar (2e-4 for the token kernel).
"""

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
from helpers import bits, ensure_built, oracle_args, rel_err, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()
    assert torch.cuda.is_available()


def _gdn():
    import linear_attention_recurrence_net_amd as gdn
    return gdn


TOKEN_CASES = [
    # B, T, H, H_qk, d_k, d_v, K, gate, dtype
    (8, 1, 4, 4, 64, 128, 1, "gda", "bf16"),   # decode
    (8, 1, 4, 4, 128, 64, 1, "gda", "bf16"),
    (4, 4, 4, 2, 64, 128, 4, "gda", "bf16"),   # verify with snapshots, shared q/k heads
    (4, 4, 4, 4, 128, 64, 4, "kda", "bf16"),
    (2, 9, 3, 3, 128, 64, 1, "kda", "f32"),
    (2, 7, 2, 1, 64, 128, 3, "gda", "f32"),
]


@pytest.mark.parametrize("B,T,H,Hq,dk,dv,K,gate,dt", TOKEN_CASES)
def test_token_kernel_unequal_head_sizes(B, T, H, Hq, dk, dv, K, gate, dt):
    c = gi.make_case(B, T, H, dk, dv, K=K, gate=gate, qkv_dtype=dt, seed=1000 + dk + T, H_qk=Hq)
    if K > 1:
        c.state[:, :, 1:] = np.float32(np.nan)
    u = upload(c)
    st = u["state"] if K > 1 else u["state"][:, :, 0].contiguous()
    fin = torch.full((B, H, dk, dv), float("nan"), device="cuda") if K > 1 else None
    o = _gdn().gdn_forward_qk_broadcast(u["q"], u["k"], u["v"], u["g"], u["beta"], st, final_state=fin)
    torch.cuda.synchronize()
    assert o.shape == (B, T, H, dv)
    ro, rst, rfin = oracle.forward(*oracle_args(c), c.f64("state"), kda=gate == "kda",
                                   want_final=True)
    errs = {"o": rel_err(o, ro)}
    if K == 1:
        errs["state"] = rel_err(st, rst[:, :, 0])
    else:
        errs["final"] = rel_err(fin, rfin)
        for t in range(1, min(T, K - 1) + 1):
            errs[f"slot{t}"] = rel_err(st[:, :, t], rst[:, :, t])
        assert np.array_equal(bits(st[:, :, 0]), c.state[:, :, 0].view(np.int32))
    print(f"token d_k={dk} d_v={dv} K={K} {gate} {dt}: " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()),
          flush=True)
    for name, e in errs.items():
        assert e <= 2e-4, (name, e)


def test_rollback_unequal_head_sizes():
    c = gi.make_case(6, 4, 3, 128, 64, K=4, qkv_dtype="bf16", seed=5, with_accepted=True)
    u = upload(c)
    _gdn().gdn_forward_snapshots(u["q"], u["k"], u["v"], u["g"], u["beta"], u["state"])
    torch.cuda.synchronize()
    before = u["state"].clone()
    acc = torch.from_numpy(c.accepted).to("cuda")
    _gdn().gdn_rollback_select(acc, u["state"])
    torch.cuda.synchronize()
    for b in range(c.B):
        a = int(c.accepted[b])
        assert np.array_equal(bits(u["state"][b, :, 0]), bits(before[b, :, a]))


PREFILL_CASES = [
    # B, T, H, H_qk, d_k, d_v, gate, dtype
    (1, 200, 4, 4, 64, 128, "gda", "bf16"),
    (2, 130, 4, 2, 128, 64, "gda", "bf16"),
    (1, 150, 2, 2, 64, 128, "kda", "bf16"),
    (1, 97, 4, 4, 128, 64, "kda", "bf16"),
    (1, 100, 2, 2, 64, 128, "gda", "f32"),
    (1, 70, 2, 2, 128, 64, "kda", "f32"),
]


@pytest.mark.parametrize("B,T,H,Hq,dk,dv,gate,dt", PREFILL_CASES)
def test_prefill_unequal_head_sizes(B, T, H, Hq, dk, dv, gate, dt):
    c = gi.make_case(B, T, H, dk, dv, gate=gate, qkv_dtype=dt, seed=1100 + T + dk, H_qk=Hq)
    u = upload(c)
    s = u["state"][:, :, 0].contiguous()
    o = _gdn().gdn_prefill_chunked_ex(u["q"], u["k"], u["v"], u["g"], u["beta"], s)
    torch.cuda.synchronize()
    assert o.shape == (B, T, H, dv)
    ro, rst, _ = oracle.forward(*oracle_args(c), c.f64("state"), kda=gate == "kda")
    eo, es = rel_err(o, ro), rel_err(s, rst[:, :, 0])
    print(f"prefill d_k={dk} d_v={dv} {gate} {dt}: o {eo:.2e} state {es:.2e}", flush=True)
    assert eo <= 1e-2 and es <= 1e-2


def test_prefill_snapshots_unequal_head_sizes():
    B, T, H, dk, dv, K = 2, 20, 2, 128, 64, 5
    c = gi.make_case(B, T, H, dk, dv, K=K, qkv_dtype="bf16", seed=77)
    c.state[:, :, 1:] = np.float32(np.nan)
    u = upload(c)
    fin = torch.empty((B, H, dk, dv), device="cuda")
    _gdn().gdn_prefill_chunked_snapshots(u["q"], u["k"], u["v"], u["g"], u["beta"], u["state"],
                                         final_state=fin)
    torch.cuda.synchronize()
    _, rst, rfin = oracle.forward(*oracle_args(c), c.f64("state"), want_final=True)
    assert rel_err(fin, rfin) <= 1e-2
    for t in range(1, K):
        assert rel_err(u["state"][:, :, t], rst[:, :, t]) <= 1e-2


def test_prefill_varlen_unequal_head_sizes():
    lengths, H, dk, dv = [70, 0, 130], 2, 64, 128
    total = sum(lengths)
    c = gi.make_case(1, total, H, dk, dv, qkv_dtype="bf16", seed=88)
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    rng = np.random.default_rng(3)
    s0 = np.ascontiguousarray(rng.normal(0.0, 0.1, size=(len(lengths), H, dk, dv)), dtype=np.float32)
    bf = torch.bfloat16
    t = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dt)
    st = t(s0)
    o = torch.zeros((total, H, dv), device="cuda")
    _gdn().gdn_prefill_chunked_varlen(t(cu, torch.int32), t(c.q[0], bf), t(c.k[0], bf), t(c.v[0], bf),
                                      t(c.g[0]), t(c.beta[0]), st, o=o)
    torch.cuda.synchronize()
    for i, n in enumerate(lengths):
        a, b = int(cu[i]), int(cu[i + 1])
        if n == 0:
            assert np.array_equal(bits(st[i]), s0[i].view(np.int32))
            continue
        sl = lambda x: x[:, a:b].astype(np.float64)
        ro, rst, _ = oracle.forward(sl(c.q), sl(c.k), sl(c.v), sl(c.g), sl(c.beta),
                                    s0[i][None, :, None].astype(np.float64))
        assert rel_err(o[a:b], ro[0]) <= 1e-2 and rel_err(st[i], rst[0, :, 0]) <= 1e-2
