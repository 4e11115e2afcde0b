"""GPU parity of the KDA chunked prefill (one log-gate per key row) against
the float64 oracle's token loop.

Bar: max|gpu - ref| / max|ref| <= 1e-2 per output tensor (o and the final
state), as for the GDA prefill.  Covered: the prefill workload's shape with
KDA gates (B=1, T=8192, H=16, d=128), ragged lengths around the chunk size,
d = 64, several sequences, non-zero initial states, q/k heads shared by the
value heads (both orders), gates three times the workload's strength, the
exact special case beta = 0 with gate 1 (state bit-identical), and agreement
with the token-by-token GPU kernel.
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
    eo, es = rel_err(o, ro), rel_err(s, rst[:, :, 0])
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


def test_prefill_kda_strong_gates():
    """Gates three times the workload's: decays across a chunk of e^-150 and
    beyond.  The chunked path's stated range (8 consecutive log-gates of a
    key row summing to more than -80) still holds for these inputs."""
    c = gi.make_case(2, 200, 2, 128, gate="kda", qkv_dtype="bf16", seed=61)
    c.g[:] = 3.0 * c.g
    win = np.lib.stride_tricks.sliding_window_view(c.g.astype(np.float64), 8, axis=1).sum(-1)
    assert win.min() > -80.0
    o, s, _ = _prefill(c)
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
