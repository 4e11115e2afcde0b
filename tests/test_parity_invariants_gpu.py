"""GPU checks of the recurrence's invariants and of strong decays.

* Invariant 2 on the token kernel: with gate 1 (g = 0), beta = 1 and a
  unit-norm float32 key, the delta rule writes v exactly into the key's
  direction, so S_t^T k_t = v_t after every token.  Checked on every snapshot
  slot, max|S^T k - v| / max|v| <= 2e-4 (the float32 path's bar).
* Invariant 1 on the token kernel: beta = 0 with gate 1 leaves the state
  bit-identical.
* Strong GDA decays (g = -30 per token, and single tokens at e^-300 among
  mild ones) on the token kernel (2e-4 against the float64 oracle) and on
  the chunked prefill (1e-2).
"""

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
from helpers import bits, ensure_built, oracle_args, rel_err, upload

pytestmark = pytest.mark.gpu

TOL_F32 = 2e-4
TOL_PREFILL = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()
    assert torch.cuda.is_available()


def _gdn():
    import linear_attention_recurrence_net_amd as gdn
    return gdn


@pytest.mark.parametrize("d_k,d_v", [(128, 128), (64, 64), (64, 128)])
def test_invariant2_delta_rule_writes_v(d_k, d_v):
    T = 6
    c = gi.make_case(3, T, 4, d_k, d_v, K=T + 1, gate="gda", qkv_dtype="f32", seed=900 + d_k + d_v)
    c.g[:] = 0.0
    c.beta[:] = 1.0
    # unit-norm keys in float32 (the generator normalises in float64 and rounds)
    kn = c.k.astype(np.float64)
    kn /= np.linalg.norm(kn, axis=-1, keepdims=True)
    c.k[:] = kn.astype(np.float32)
    d = upload(c)
    o = _gdn().gdn_forward_snapshots(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"])
    torch.cuda.synchronize()
    st = d["state"].double().cpu().numpy()  # slot t = S_t
    k = c.k.astype(np.float64)
    v = c.v.astype(np.float64)
    worst = 0.0
    for t in range(T):
        sk = np.einsum("bhij,bhi->bhj", st[:, :, t + 1], k[:, t])
        e = rel_err(sk, v[:, t], f"S{t + 1}^T k{t + 1} - v")
        worst = max(worst, e)
        assert e <= TOL_F32, (t, e)
    print(f"invariant 2 d_k={d_k} d_v={d_v}: worst {worst:.2e}", flush=True)
    assert torch.isfinite(o).all()


@pytest.mark.parametrize("gate", ["gda", "kda"])
def test_invariant1_beta0_gate1_token_kernel_bitwise(gate):
    c = gi.make_case(2, 5, 3, 128, gate=gate, qkv_dtype="bf16", seed=37)
    c.beta[:] = 0.0
    c.g[:] = 0.0
    d = upload(c)
    s = d["state"][:, :, 0].contiguous()
    _gdn().gdn_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], s)
    torch.cuda.synchronize()
    assert np.array_equal(bits(s), c.state[:, :, 0].view(np.int32))


def _gda_strong(c, regime):
    if regime == "const-30":
        c.g[:] = -30.0
    elif regime == "spikes":
        rng = np.random.default_rng(3)
        c.g[:] = np.where(rng.random(c.g.shape) < 0.1, -300.0, -0.05).astype(np.float32)
    else:
        raise ValueError(regime)


@pytest.mark.parametrize("regime", ["const-30", "spikes"])
@pytest.mark.parametrize("T,K", [(1, 1), (4, 4), (9, 1)])
def test_token_kernel_strong_gda_gates(regime, T, K):
    c = gi.make_case(8, T, 4, 128, K=K, gate="gda", qkv_dtype="bf16", seed=41 + T)
    _gda_strong(c, regime)
    d = upload(c)
    fin = torch.empty((c.B, c.H, c.d_k, c.d_v), device="cuda") if K > 1 else None
    o = _gdn().gdn_forward_snapshots(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], fin)
    torch.cuda.synchronize()
    ro, rst, rfin = oracle.forward(*oracle_args(c), c.f64("state"), want_final=fin is not None)
    errs = {"o": rel_err(o, ro, "o")}
    if K == 1:
        errs["state"] = rel_err(d["state"][:, :, 0], rst[:, :, 0], "state")
    else:
        for s in range(1, min(T, K - 1) + 1):
            errs[f"slot{s}"] = rel_err(d["state"][:, :, s], rst[:, :, s], f"slot{s}")
        errs["final"] = rel_err(fin, rfin, "final")
    print(regime, T, K, errs, flush=True)
    for name, e in errs.items():
        assert e <= TOL_F32, (name, e)


@pytest.mark.parametrize("regime", ["const-30", "spikes"])
@pytest.mark.parametrize("T,d", [(200, 128), (130, 64)])
def test_prefill_strong_gda_gates(regime, T, d):
    c = gi.make_case(2, T, 3, d, gate="gda", qkv_dtype="bf16", seed=51 + T)
    _gda_strong(c, regime)
    dd = upload(c)
    s = dd["state"][:, :, 0].contiguous()
    o = _gdn().gdn_prefill_chunked(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], s)
    torch.cuda.synchronize()
    ro, rst, _ = oracle.forward(*oracle_args(c), c.f64("state"))
    eo, es = rel_err(o, ro, "o"), rel_err(s, rst[:, :, 0], "state")
    print(f"prefill GDA {regime} T={T} d={d}: o {eo:.2e} state {es:.2e}", flush=True)
    assert eo <= TOL_PREFILL and es <= TOL_PREFILL, (eo, es)
