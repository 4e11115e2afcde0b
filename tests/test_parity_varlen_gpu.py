"""GPU parity of the variable-length chunked prefill (packed sequences).

Each sequence of a packed batch is compared with the float64 oracle run on
that sequence alone (bar 1e-2, as for the prefill), and bit for bit with
gdn_prefill_chunked_qk_broadcast on that sequence alone; empty sequences must
leave their state bit-identical.  Malformed offsets are clamped on the device
(running maximum of offsets clamped to [0, total]); the result must equal
the run with the sanitised offsets.
"""

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
from helpers import bits, dev, ensure_built, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()
    assert torch.cuda.is_available()


def _gdn():
    import linear_attention_recurrence_net_amd as gdn
    return gdn


def _upload(vc: gi.VarlenCase):
    bf = torch.bfloat16
    return dict(q=dev(vc.q, bf), k=dev(vc.k, bf), v=dev(vc.v, bf), g=dev(vc.g), beta=dev(vc.beta),
                state=dev(vc.state), cu=dev(vc.cu_seqlens))


def _run(vc, u, head_map, cu=None):
    st = u["state"].clone()
    o = torch.full((vc.total, vc.H, vc.d), float("nan"), device="cuda")
    _gdn().gdn_prefill_chunked_varlen(u["cu"] if cu is None else cu, u["q"], u["k"], u["v"], u["g"],
                                      u["beta"], st, head_map=head_map, o=o)
    torch.cuda.synchronize()
    return o, st


CASES = [
    # lengths, H, H_qk, d, head map
    ([0, 1, 63, 64, 65, 200, 7, 0], 4, 2, 128, "grouped"),
    ([130, 0, 64, 97], 6, 3, 64, "tiled"),
    ([300], 4, 4, 128, "grouped"),
]


@pytest.mark.parametrize("lengths,H,Hq,d,head_map", CASES)
def test_prefill_varlen(lengths, H, Hq, d, head_map):
    vc = gi.make_varlen_case(lengths, H, d, H_qk=Hq, seed=700 + sum(lengths))
    u = _upload(vc)
    o, st = _run(vc, u, head_map)
    for i, n in enumerate(lengths):
        a, b = int(vc.cu_seqlens[i]), int(vc.cu_seqlens[i + 1])
        if n == 0:
            assert np.array_equal(bits(st[i]), vc.state[i].view(np.int32))
            continue
        c = vc.sequence(i)
        ro, rst, _ = oracle.forward(*[c.f64(x) for x in ("q", "k", "v", "g", "beta")], c.f64("state"),
                                    head_map=head_map)
        eo, es = rel_err(o[a:b], ro[0]), rel_err(st[i], rst[0, :, 0])
        print(f"seq {i} len {n}: o {eo:.2e} state {es:.2e}", flush=True)
        assert eo <= 1e-2 and es <= 1e-2
        # bit for bit with the sequence alone
        s1 = dev(vc.state[i][None])
        o1 = _gdn().gdn_prefill_chunked_qk_broadcast(u["q"][a:b][None].contiguous(),
                                                     u["k"][a:b][None].contiguous(),
                                                     u["v"][a:b][None].contiguous(),
                                                     u["g"][a:b][None].contiguous(),
                                                     u["beta"][a:b][None].contiguous(), s1,
                                                     head_map=head_map)
        torch.cuda.synchronize()
        assert np.array_equal(bits(o[a:b]), bits(o1[0]))
        assert np.array_equal(bits(st[i]), bits(s1[0]))


def test_prefill_varlen_clamps_malformed_offsets():
    vc = gi.make_varlen_case([150, 130], 4, 64, seed=9)  # total 280
    u = _upload(vc)
    N = 4
    state = dev(np.concatenate([vc.state, vc.state], axis=0))  # 4 initial states
    bad = torch.tensor([0, 150, 90, 400, 250], dtype=torch.int32, device="cuda")
    good = torch.tensor([0, 150, 150, 280, 280], dtype=torch.int32, device="cuda")  # sanitised
    outs = []
    for cu in (bad, good):
        st = state.clone()
        o = torch.full((vc.total, vc.H, vc.d), float("nan"), device="cuda")
        _gdn().gdn_prefill_chunked_varlen(cu, u["q"], u["k"], u["v"], u["g"], u["beta"], st, o=o)
        torch.cuda.synchronize()
        outs.append((o, st))
    assert N == bad.numel() - 1
    assert np.array_equal(bits(outs[0][0]), bits(outs[1][0]))
    assert np.array_equal(bits(outs[0][1]), bits(outs[1][1]))
    # the emptied sequences 1 and 3 kept their initial states
    assert np.array_equal(bits(outs[0][1][1]), bits(state[1]))
    assert np.array_equal(bits(outs[0][1][3]), bits(state[3]))


# the general entry point: KDA gates and float32 inputs on packed sequences
EX_CASES = [
    # lengths, H, H_qk, d, head map, gate, q/k/v type
    ([0, 1, 63, 64, 65, 200, 7, 0], 4, 2, 128, "grouped", "kda", "bf16"),
    ([130, 0, 64, 97], 6, 3, 64, "tiled", "kda", "f32"),
    ([150, 33, 0, 64], 4, 4, 128, "grouped", "gda", "f32"),
]


def _upload_ex(vc: gi.VarlenCase):
    t = torch.bfloat16 if vc.qkv_dtype == "bf16" else torch.float32
    return dict(q=dev(vc.q, t), k=dev(vc.k, t), v=dev(vc.v, t), g=dev(vc.g), beta=dev(vc.beta),
                state=dev(vc.state), cu=dev(vc.cu_seqlens))


@pytest.mark.parametrize("lengths,H,Hq,d,head_map,gate,dt", EX_CASES)
def test_prefill_varlen_ex(lengths, H, Hq, d, head_map, gate, dt):
    vc = gi.make_varlen_case(lengths, H, d, H_qk=Hq, seed=800 + sum(lengths), gate=gate, qkv_dtype=dt)
    u = _upload_ex(vc)
    st = u["state"].clone()
    o = torch.full((vc.total, vc.H, vc.d), float("nan"), device="cuda")
    gdn = _gdn()
    gdn.gdn_prefill_chunked_varlen_ex(u["cu"], u["q"], u["k"], u["v"], u["g"], u["beta"], st,
                                      head_map=head_map, o=o)
    torch.cuda.synchronize()
    for i, n in enumerate(lengths):
        a, b = int(vc.cu_seqlens[i]), int(vc.cu_seqlens[i + 1])
        if n == 0:
            assert np.array_equal(bits(st[i]), vc.state[i].view(np.int32))
            continue
        c = vc.sequence(i)
        ro, rst, _ = oracle.forward(*[c.f64(x) for x in ("q", "k", "v", "g", "beta")], c.f64("state"),
                                    head_map=head_map, kda=gate == "kda")
        eo = rel_err(o[a:b], ro[0], f"seq{i} o")
        es = rel_err(st[i], rst[0, :, 0], f"seq{i} state")
        print(f"{gate} {dt} seq {i} len {n}: o {eo:.2e} state {es:.2e}", flush=True)
        assert eo <= 1e-2 and es <= 1e-2
        # bit for bit with the general entry point on the sequence alone
        s1 = dev(vc.state[i][None])
        o1 = gdn.gdn_prefill_chunked_ex(u["q"][a:b][None].contiguous(), u["k"][a:b][None].contiguous(),
                                        u["v"][a:b][None].contiguous(), u["g"][a:b][None].contiguous(),
                                        u["beta"][a:b][None].contiguous(), s1, head_map=head_map)
        torch.cuda.synchronize()
        assert np.array_equal(bits(o[a:b]), bits(o1[0]))
        assert np.array_equal(bits(st[i]), bits(s1[0]))


def test_prefill_varlen_ex_equals_varlen_for_bf16_gda():
    vc = gi.make_varlen_case([0, 1, 63, 64, 65, 200, 7, 0], 4, 128, H_qk=2, seed=901)
    u = _upload(vc)
    o0, s0 = _run(vc, u, "grouped")
    st = u["state"].clone()
    o = torch.full((vc.total, vc.H, vc.d), float("nan"), device="cuda")
    _gdn().gdn_prefill_chunked_varlen_ex(u["cu"], u["q"], u["k"], u["v"], u["g"], u["beta"], st, o=o)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o), bits(o0))
    assert np.array_equal(bits(st), bits(s0))


def test_prefill_varlen_many_sequences():
    # 40 sequences of a seeded log-uniform length mix (some below one chunk,
    # some several chunks) plus two empty ones, through the general entry point
    lengths = gi.varlen_lengths(2600, 40, seed=31)
    lengths = lengths[:7] + [0] + lengths[7:29] + [0] + lengths[29:]
    vc = gi.make_varlen_case(lengths, 4, 64, H_qk=2, seed=33)
    u = _upload(vc)
    st = u["state"].clone()
    o = torch.full((vc.total, vc.H, vc.d), float("nan"), device="cuda")
    _gdn().gdn_prefill_chunked_varlen_ex(u["cu"], u["q"], u["k"], u["v"], u["g"], u["beta"], st, o=o)
    torch.cuda.synchronize()
    worst = 0.0
    for i, n in enumerate(lengths):
        a, b = int(vc.cu_seqlens[i]), int(vc.cu_seqlens[i + 1])
        if n == 0:
            assert np.array_equal(bits(st[i]), vc.state[i].view(np.int32))
            continue
        c = vc.sequence(i)
        ro, rst, _ = oracle.forward(*[c.f64(x) for x in ("q", "k", "v", "g", "beta")], c.f64("state"))
        e = max(rel_err(o[a:b], ro[0], f"seq{i} o"), rel_err(st[i], rst[0, :, 0], f"seq{i} state"))
        worst = max(worst, e)
        assert e <= 1e-2, (i, n, e)
    print(f"{len(lengths)} sequences ({min(lengths)}..{max(lengths)} tokens): worst {worst:.2e}", flush=True)


def test_prefill_varlen_beyond_one_table_block():
    # 300 sequences: the device table of sanitised starts and chunk offsets is
    # built 64 offsets at a time, carrying the running maximum and the chunk
    # count from block to block; many sequences are shorter than a chunk and
    # some are empty, at positions on both sides of the block edges
    lengths = gi.varlen_lengths(9000, 290, seed=51)
    for pos in (0, 63, 64, 65, 127, 128, 200, 250, 280, 299):
        lengths.insert(pos, 0)
    assert len(lengths) == 300
    vc = gi.make_varlen_case(lengths, 2, 64, seed=53)
    u = _upload(vc)
    o, st = _run(vc, u, "grouped")
    worst = 0.0
    for i, n in enumerate(lengths):
        a, b = int(vc.cu_seqlens[i]), int(vc.cu_seqlens[i + 1])
        if n == 0:
            assert np.array_equal(bits(st[i]), vc.state[i].view(np.int32)), i
            continue
        c = vc.sequence(i)
        ro, rst, _ = oracle.forward(*[c.f64(x) for x in ("q", "k", "v", "g", "beta")], c.f64("state"))
        e = max(rel_err(o[a:b], ro[0], f"seq{i} o"), rel_err(st[i], rst[0, :, 0], f"seq{i} state"))
        worst = max(worst, e)
        assert e <= 1e-2, (i, n, e)
    assert not torch.isnan(o).any()  # every row belongs to a sequence and is written
    print(f"{len(lengths)} sequences ({min(lengths)}..{max(lengths)} tokens): worst {worst:.2e}", flush=True)
