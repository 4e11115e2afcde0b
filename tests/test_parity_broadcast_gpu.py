"""GPU parity of the q/k head broadcast (value heads sharing q/k heads).

For each case the broadcast entry point is compared
  * with the float64 oracle, to the path's bar (2e-4 for the recurrent
    kernel, 1e-2 for the bf16-MFMA prefill), and
  * bit for bit with the plain entry point run on q and k repeated to H
    heads in the same order (grouped: numpy repeat; tiled: numpy tile) --
    the kernels read the same values, so the results must be identical.
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


def _repeat(a: np.ndarray, R: int, head_map: str) -> np.ndarray:
    return np.repeat(a, R, axis=2) if head_map == "grouped" else np.tile(a, (1, 1, R, 1))


def _repeated_upload(c, head_map):
    R = c.H // c.H_qk
    qdt = torch.bfloat16 if c.qkv_dtype == "bf16" else torch.float32
    return dev(_repeat(c.q, R, head_map), qdt), dev(_repeat(c.k, R, head_map), qdt)


RECURRENT_CASES = [
    # B, T, H, H_qk, d, K, gate, dtype
    (8, 1, 16, 4, 128, 1, "gda", "bf16"),   # decode shape with 4 value heads per q/k head
    (4, 4, 8, 2, 128, 4, "gda", "bf16"),    # verify with snapshots
    (4, 4, 16, 8, 64, 4, "kda", "bf16"),
    (2, 9, 6, 3, 64, 1, "gda", "f32"),
    (2, 5, 4, 1, 128, 3, "kda", "f32"),     # one q/k head for every value head
]


@pytest.mark.parametrize("head_map", ["grouped", "tiled"])
@pytest.mark.parametrize("B,T,H,Hq,d,K,gate,dt", RECURRENT_CASES)
def test_forward_qk_broadcast(B, T, H, Hq, d, K, gate, dt, head_map):
    c = gi.make_case(B, T, H, d, K=K, gate=gate, qkv_dtype=dt, seed=500 + H + Hq + T, H_qk=Hq)
    u = upload(c)
    st = u["state"] if K > 1 else u["state"][:, :, 0].contiguous()
    fin = torch.empty((B, H, d, d), dtype=torch.float32, device="cuda") if K > 1 else None
    o = _gdn().gdn_forward_qk_broadcast(u["q"], u["k"], u["v"], u["g"], u["beta"], st,
                                        head_map=head_map, final_state=fin)
    torch.cuda.synchronize()
    ro, rst, rfin = oracle.forward(*oracle_args(c), c.f64("state"), kda=gate == "kda",
                                   want_final=True, head_map=head_map)
    print(f"{head_map} B={B} T={T} H={H} H_qk={Hq} d={d} K={K} {gate} {dt}: o {rel_err(o, ro):.2e}",
          flush=True)
    assert rel_err(o, ro) <= 2e-4
    if K > 1:
        assert rel_err(st, rst) <= 2e-4
        assert rel_err(fin, rfin) <= 2e-4
    else:
        assert rel_err(st, rst[:, :, 0]) <= 2e-4

    # bit for bit against the plain kernel on materialised repeats
    q2, k2 = _repeated_upload(c, head_map)
    u2 = upload(c)
    st2 = u2["state"] if K > 1 else u2["state"][:, :, 0].contiguous()
    if K > 1:
        fin2 = torch.empty_like(fin)
        o2 = _gdn().gdn_forward_snapshots(q2, k2, u2["v"], u2["g"], u2["beta"], st2, final_state=fin2)
    else:
        o2 = _gdn().gdn_forward(q2, k2, u2["v"], u2["g"], u2["beta"], st2)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o), bits(o2))
    assert np.array_equal(bits(st), bits(st2))
    if K > 1:
        assert np.array_equal(bits(fin), bits(fin2))


@pytest.mark.parametrize("head_map", ["grouped", "tiled"])
@pytest.mark.parametrize("B,T,H,Hq,d", [(1, 200, 8, 2, 128), (2, 97, 6, 3, 64), (1, 130, 4, 1, 128)])
def test_prefill_qk_broadcast(B, T, H, Hq, d, head_map):
    c = gi.make_case(B, T, H, d, qkv_dtype="bf16", seed=600 + T + Hq, H_qk=Hq)
    u = upload(c)
    s = u["state"][:, :, 0].contiguous()
    o = _gdn().gdn_prefill_chunked_qk_broadcast(u["q"], u["k"], u["v"], u["g"], u["beta"], s,
                                                head_map=head_map)
    torch.cuda.synchronize()
    ro, rst, _ = oracle.forward(*oracle_args(c), c.f64("state"), head_map=head_map)
    eo, es = rel_err(o, ro), rel_err(s, rst[:, :, 0])
    print(f"prefill {head_map} B={B} T={T} H={H} H_qk={Hq} d={d}: o {eo:.2e} state {es:.2e}", flush=True)
    assert eo <= 1e-2 and es <= 1e-2

    q2, k2 = _repeated_upload(c, head_map)
    u2 = upload(c)
    s2 = u2["state"][:, :, 0].contiguous()
    o2 = _gdn().gdn_prefill_chunked(q2, k2, u2["v"], u2["g"], u2["beta"], s2)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o), bits(o2))
    assert np.array_equal(bits(s), bits(s2))


def test_qk_broadcast_rejects_bad_head_counts():
    c = gi.make_case(1, 2, 4, 64, qkv_dtype="bf16", seed=3, H_qk=2)
    u = upload(c)
    st = u["state"][:, :, 0].contiguous()
    q3 = torch.cat([u["q"], u["q"][:, :, :1]], dim=2).contiguous()  # 3 q/k heads for 4 value heads
    with pytest.raises(ValueError):
        _gdn().gdn_forward_qk_broadcast(q3, q3, u["v"], u["g"], u["beta"], st)
    with pytest.raises(ValueError):
        _gdn().gdn_forward_qk_broadcast(u["q"], u["k"], u["v"], u["g"], u["beta"], st,
                                        head_map="diagonal")
