"""GPU parity of the KDA chunked prefill (one log-gate per key row) against
the float64 oracle's token loop.

Bar: max|gpu - ref| / max|ref| <= 1e-2 per output tensor (o and the final
state), as for the GDA prefill.  Covered: the prefill workload's shape with
KDA gates (B=1, T=8192, H=16, d=128), ragged lengths around the chunk size,
d = 64, several sequences, non-zero initial states, q/k heads shared by the
value heads (both orders), strong gates (three times the workload's, constant
and scaled log-gates down to -40 per token, sparse e^-300 decays, fast and
slow key rows mixed; also at the workload's shape and with float32 inputs),
the exact special case beta = 0 with gate 1 (state bit-identical), and
agreement with the token-by-token GPU kernel.
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


def _prefill(case, head_map="grouped"):
    d = upload(case)
    s = d["state"][:, :, 0].contiguous()
    o = _gdn().gdn_prefill_chunked_kda(d["q"], d["k"], d["v"], d["g"], d["beta"], s, head_map=head_map)
    torch.cuda.synchronize()
    return o, s, d


def _check(case, o, s, head_map="grouped"):
    ro, rst, _ = oracle.forward(*oracle_args(case), case.f64("state"), kda=True, head_map=head_map)
    eo, es = rel_err(o, ro, "o"), rel_err(s, rst[:, :, 0], "state")
    print(f"KDA B={case.B} T={case.T} H={case.H} H_qk={case.H_qk} d={case.d_k} o {eo:.3e} state {es:.3e}",
          flush=True)
    assert eo <= TOL and es <= TOL, (eo, es)


def test_prefill_kda_workload_shape_full_size():
    c = gi.workload_case(4, gate="kda")
    o, s, _ = _prefill(c)
    _check(c, o, s)


@pytest.mark.parametrize("T", [1, 63, 64, 65, 150])
def test_prefill_kda_ragged_lengths(T):
    c = gi.make_case(1, T, 2, 128, gate="kda", qkv_dtype="bf16", seed=400 + T, zero_state=True)
    o, s, _ = _prefill(c)
    _check(c, o, s)


@pytest.mark.parametrize("B,T,H,Hq,d,head_map", [
    (2, 130, 3, 3, 64, "grouped"),
    (3, 97, 2, 2, 128, "grouped"),
    (1, 300, 4, 4, 64, "grouped"),
    (2, 200, 8, 2, 128, "grouped"),
    (1, 150, 6, 3, 64, "tiled"),
])
def test_prefill_kda_batches_heads_nonzero_state(B, T, H, Hq, d, head_map):
    c = gi.make_case(B, T, H, d, gate="kda", qkv_dtype="bf16", seed=500 + T + H, H_qk=Hq)
    o, s, _ = _prefill(c, head_map)
    _check(c, o, s, head_map)


def _strong_gates(c, regime, rng):
    """Replace the case's log-gates by one of the strong-decay regimes."""
    g = c.g.astype(np.float64)
    if regime == "3x":  # three times the workload's gates
        g = 3.0 * g
    elif regime.startswith("const"):  # the same log-gate on every key row and token
        g = np.full_like(g, float(regime[5:]))
    elif regime.startswith("scaled"):  # the workload's gates scaled to a mean per token
        g = g * (float(regime[6:]) / g.mean())
    elif regime == "spikes":  # mostly mild decays, one in ten at e^-300
        g = np.where(rng.random(g.shape) < 0.1, -300.0, -0.05)
    elif regime == "mixed":  # half the key rows fast-forgetting, half slow
        g = np.where(np.arange(g.shape[-1]) % 2 == 0, -40.0 * g / g.mean(), 0.05 * g)
    c.g[:] = g.astype(np.float32)


@pytest.mark.parametrize("regime", ["3x", "const-12", "const-15", "const-40", "scaled-12",
                                    "scaled-40", "spikes", "mixed"])
@pytest.mark.parametrize("d", [64, 128])
def test_prefill_kda_strong_gates(regime, d):
    """Decays far beyond the workload's, down to e^-40 per token and single
    tokens at e^-300: every log-gate g <= 0 is in the chunked path's range.
    Chunks with a key row decaying by more than e^-40 across 16 tokens take
    the exact path for their diagonal blocks."""
    c = gi.make_case(2, 200, 2, d, gate="kda", qkv_dtype="bf16", seed=61 + d)
    _strong_gates(c, regime, np.random.default_rng(7))
    assert (c.g <= 0).all()
    o, s, _ = _prefill(c)
    _check(c, o, s)


def test_prefill_kda_strong_gates_workload_shape():
    """The prefill workload's shape (B=1, T=8192, H=16, d=128) with log-gates
    scaled to a mean of -12 per token on every key row."""
    c = gi.workload_case(4, gate="kda")
    _strong_gates(c, "scaled-12", None)
    o, s, _ = _prefill(c)
    _check(c, o, s)


def test_prefill_kda_strong_gates_float32_inputs():
    import linear_attention_recurrence_net_amd as gdn
    c = gi.make_case(2, 150, 3, 128, gate="kda", qkv_dtype="f32", seed=71)
    _strong_gates(c, "const-15", None)
    d = upload(c)
    s = d["state"][:, :, 0].contiguous()
    o = gdn.gdn_prefill_chunked_ex(d["q"], d["k"], d["v"], d["g"], d["beta"], s)
    torch.cuda.synchronize()
    _check(c, o, s)


def test_prefill_kda_beta0_gate1_state_bitwise():
    c = gi.make_case(1, 130, 2, 128, gate="kda", qkv_dtype="bf16", seed=17)
    c.beta[:] = 0.0
    c.g[:] = 0.0
    o, s, _ = _prefill(c)
    assert np.array_equal(bits(s), c.state[:, :, 0].view(np.int32))
    _check(c, o, s)


def test_prefill_kda_matches_token_kernel():
    c = gi.make_case(2, 257, 4, 64, gate="kda", qkv_dtype="bf16", seed=19)
    o, s, d = _prefill(c)
    s2 = upload(c)["state"][:, :, 0].contiguous()
    o2 = _gdn().gdn_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], s2)
    torch.cuda.synchronize()
    assert rel_err(o, o2.double().cpu().numpy()) <= TOL
    assert rel_err(s, s2.double().cpu().numpy()) <= TOL


def test_prefill_kda_rejects_head_gates():
    c = gi.make_case(1, 8, 2, 64, qkv_dtype="bf16", seed=3)  # GDA gates [B,T,H]
    d = upload(c)
    s = d["state"][:, :, 0].contiguous()
    with pytest.raises(Exception):
        _gdn().gdn_prefill_chunked_kda(d["q"], d["k"], d["v"], d["g"], d["beta"], s)
