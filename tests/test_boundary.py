"""C-ABI boundary checks that need no GPU.

* libgdn.so loads and exports every function include/gdn.h declares;
* argument validation happens on the host before any HIP call: NULL
  pointers, bad sizes, unsupported head sizes / dtypes / gates / chunk
  sizes, misalignment and a short prefill workspace return their status
  codes without launching (so these calls are safe without a GPU);
* the allocation-free prefill validates exactly as the general prefill and
  refuses, before any HIP call, a problem larger than its scratch array;
* the status strings exist for every code;
* the Python binding refuses CPU tensors (there is no CPU path).
"""

import ctypes
import os
import re

import pytest
import torch

import linear_attention_recurrence_net_amd as gdn
from linear_attention_recurrence_net_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUP, ERR_WS, ERR_HIP, ERR_SCRATCH, ERR_ALIAS = range(8)


def _declared_functions():
    txt = open(os.path.join(ROOT, "include", "gdn.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_binding.library_path()):
        from linear_attention_recurrence_net_amd import build
        build.build()
    return gdn.library()


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert set(declared) == set(_binding.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for s in range(8):
        assert lib.gdn_status_str(s)
    assert b"unknown" in lib.gdn_status_str(99)


P = ctypes.c_void_p(256)  # a fake, 16-byte aligned "device" pointer: never dereferenced
N = None
# distinct fake pointers, 1 TiB apart and 256-byte aligned (never dereferenced),
# for calls that must get past the check that written arrays overlap no other
D = [ctypes.c_void_p((i + 1) << 40) for i in range(24)]


def fwd(lib, B=1, T=1, H=1, dk=64, dv=64, dt=1, gate=0, q=P, k=P, v=P, g=P, beta=P, st=P, o=P):
    return lib.gdn_forward(B, T, H, dk, dv, dt, gate, q, k, v, g, beta, st, o, None)


def snap(lib, K=4, fin=N, **kw):
    a = dict(B=1, T=1, H=1, dk=64, dv=64, dt=1, gate=0, q=P, k=P, v=P, g=P, beta=P, st=P, o=P)
    a.update(kw)
    return lib.gdn_forward_snapshots(a["B"], a["T"], a["H"], a["dk"], a["dv"], a["dt"], a["gate"],
                                     K, a["q"], a["k"], a["v"], a["g"], a["beta"], a["st"], fin,
                                     a["o"], None)


def test_forward_validation(lib):
    assert fwd(lib, q=N) == ERR_NULL
    assert fwd(lib, st=N) == ERR_NULL
    assert fwd(lib, o=N) == ERR_NULL
    assert fwd(lib, B=-1) == ERR_SHAPE
    assert fwd(lib, T=-3) == ERR_SHAPE
    assert fwd(lib, dk=32, dv=32) == ERR_UNSUP  # head size 32 is not supported
    assert fwd(lib, dk=64, dv=96) == ERR_UNSUP   # head sizes are 64 or 128 (d_k and d_v may differ)
    assert fwd(lib, dk=96, dv=96) == ERR_UNSUP
    assert fwd(lib, dt=7) == ERR_UNSUP
    assert fwd(lib, gate=2) == ERR_UNSUP
    assert fwd(lib, q=ctypes.c_void_p(258)) == ERR_UNSUP  # misaligned
    # empty problems are valid and launch nothing
    assert fwd(lib, B=0) == OK
    assert fwd(lib, H=0) == OK
    assert fwd(lib, T=0) == OK


def test_snapshot_validation(lib):
    assert snap(lib, K=0) == ERR_SHAPE
    assert snap(lib, K=-2) == ERR_SHAPE
    assert snap(lib, K=4, fin=ctypes.c_void_p(264)) == ERR_UNSUP
    assert snap(lib, K=4, B=0) == OK


def test_forward_after_rollback_validation(lib):
    def far(B=1, T=1, H=1, Hq=1, hm=0, dk=64, dv=64, dt=1, gate=0, K=4, acc=P, q=P, k=P, v=P, g=P, beta=P,
            st=P, fin=N, o=P, err=N):
        return lib.gdn_forward_snapshots_after_rollback(B, T, H, Hq, hm, dk, dv, dt, gate, K, acc, q, k, v, g,
                                                        beta, st, fin, o, err, None)
    assert far(acc=N) == ERR_NULL
    assert far(st=N) == ERR_NULL
    assert far(q=N) == ERR_NULL
    assert far(K=0) == ERR_SHAPE
    assert far(H=4, Hq=3) == ERR_SHAPE
    assert far(hm=2) == ERR_UNSUP
    assert far(dk=96) == ERR_UNSUP
    assert far(gate=2) == ERR_UNSUP
    assert far(o=ctypes.c_void_p(264)) == ERR_UNSUP
    assert far(B=0, acc=N) == OK
    assert far(H=0) == OK


def test_rollback_validation(lib):
    rb = lib.gdn_rollback_select
    assert rb(1, 1, 4, 64, 64, N, P, N, None) == ERR_NULL
    assert rb(1, 1, 4, 64, 64, P, N, N, None) == ERR_NULL
    assert rb(1, 1, 0, 64, 64, P, P, N, None) == ERR_SHAPE
    assert rb(-1, 1, 4, 64, 64, P, P, N, None) == ERR_SHAPE
    assert rb(1, 1, 4, 3, 3, P, P, N, None) == ERR_UNSUP  # tile not a multiple of 4
    assert rb(0, 1, 4, 64, 64, P, P, N, None) == OK


def test_prefill_validation(lib):
    ws = lib.gdn_prefill_workspace_size
    need = ws(1, 8192, 16, 128, 128, 64)
    assert need > 0
    assert ws(1, 8192, 16, 128, 128, 32) == 0
    assert ws(1, 8192, 16, 32, 32, 64) == 0
    pf = lib.gdn_prefill_chunked
    big = need
    assert pf(1, 100, 2, 128, 128, 64, N, P, P, P, P, P, P, P, big, None) == ERR_NULL
    assert pf(1, 100, 2, 128, 128, 0, P, P, P, P, P, P, P, P, big, None) == ERR_SHAPE
    assert pf(1, 100, 2, 128, 128, 32, P, P, P, P, P, P, P, P, big, None) == ERR_UNSUP
    assert pf(1, 100, 2, 96, 96, 64, P, P, P, P, P, P, P, P, big, None) == ERR_UNSUP
    small = ws(1, 100, 2, 128, 128, 64)
    assert pf(1, 100, 2, 128, 128, 64, D[0], D[1], D[2], D[3], D[4], D[5], D[6], N, small, None) == ERR_WS
    assert pf(1, 100, 2, 128, 128, 64, D[0], D[1], D[2], D[3], D[4], D[5], D[6], D[7], small - 1, None) == ERR_WS
    assert pf(1, 100, 2, 128, 128, 64, D[0], D[1], D[2], D[3], D[4], D[5], D[6], ctypes.c_void_p(272), small, None) == ERR_WS
    assert pf(1, 0, 2, 128, 128, 64, D[0], D[1], D[2], D[3], D[4], D[5], D[6], N, 0, None) == OK
    # one sequence's [T,H,d] fp32 rows must stay below 2^31 bytes
    huge_T = (1 << 31) // (16 * 128 * 4)
    assert pf(1, huge_T, 16, 128, 128, 64, P, P, P, P, P, P, P, P, 1 << 40, None) == ERR_UNSUP
    assert pf(1, huge_T - 1, 16, 128, 128, 64, D[0], D[1], D[2], D[3], D[4], D[5], D[6], N, 0, None) == ERR_WS


def test_workspace_grows_with_tokens(lib):
    ws = lib.gdn_prefill_workspace_size
    assert ws(1, 64, 16, 128, 128, 64) <= ws(1, 65, 16, 128, 128, 64) <= ws(1, 8192, 16, 128, 128, 64)
    assert ws(2, 8192, 16, 128, 128, 64) >= ws(1, 8192, 16, 128, 128, 64)


def test_binding_rejects_cpu_tensors(lib):
    q = torch.zeros(1, 1, 1, 64, dtype=torch.bfloat16)
    g = torch.zeros(1, 1, 1)
    with pytest.raises(ValueError, match="GPU"):
        gdn.gdn_forward(q, q, q, g, g, torch.zeros(1, 1, 64, 64))


def test_qk_broadcast_validation(lib):
    fb = lib.gdn_forward_qk_broadcast
    # B, T, H, H_qk, head_map, dk, dv, dtype, gate, K, q, k, v, g, beta, state, final, o, stream
    assert fb(1, 1, 4, 3, 0, 64, 64, 1, 0, 1, P, P, P, P, P, P, N, P, None) == ERR_SHAPE  # 3 does not divide 4
    assert fb(1, 1, 4, 0, 0, 64, 64, 1, 0, 1, P, P, P, P, P, P, N, P, None) == ERR_SHAPE
    assert fb(1, 1, 4, 2, 2, 64, 64, 1, 0, 1, P, P, P, P, P, P, N, P, None) == ERR_UNSUP  # bad head map
    assert fb(1, 1, 4, 2, 1, 64, 64, 1, 0, 1, N, P, P, P, P, P, N, P, None) == ERR_NULL
    assert fb(1, 1, 4, 2, 1, 96, 96, 1, 0, 1, P, P, P, P, P, P, N, P, None) == ERR_UNSUP
    assert fb(0, 1, 4, 2, 1, 64, 64, 1, 0, 1, P, P, P, P, P, P, N, P, None) == OK
    pb = lib.gdn_prefill_chunked_qk_broadcast
    big = lib.gdn_prefill_workspace_size(1, 100, 4, 128, 128, 64)
    # B, T, H, H_qk, head_map, dk, dv, chunk, q, k, v, g, beta, state, o, ws, ws_bytes, stream
    assert pb(1, 100, 4, 3, 0, 128, 128, 64, P, P, P, P, P, P, P, P, big, None) == ERR_SHAPE
    assert pb(1, 100, 4, 2, 5, 128, 128, 64, P, P, P, P, P, P, P, P, big, None) == ERR_UNSUP
    assert pb(1, 100, 4, 2, 0, 128, 128, 64, D[0], D[1], D[2], D[3], D[4], D[5], D[6], N, big, None) == ERR_WS
    assert pb(1, 0, 4, 2, 0, 128, 128, 64, D[0], D[1], D[2], D[3], D[4], D[5], D[6], N, 0, None) == OK


def test_prefill_varlen_validation(lib):
    wsz = lib.gdn_prefill_varlen_workspace_size
    need = wsz(3, 300, 4, 128, 128, 64)
    assert need >= wsz(1, 300, 4, 128, 128, 64) > 0  # more sequences, more partial chunks
    assert wsz(3, 300, 4, 128, 128, 32) == 0
    pv = lib.gdn_prefill_chunked_varlen
    # N, total, H, H_qk, map, dk, dv, chunk, cu, q, k, v, g, beta, state, o, ws, ws_bytes, stream
    assert pv(3, 300, 4, 2, 0, 128, 128, 64, N, P, P, P, P, P, P, P, P, need, None) == ERR_NULL
    assert pv(-1, 300, 4, 2, 0, 128, 128, 64, P, P, P, P, P, P, P, P, P, need, None) == ERR_SHAPE
    assert pv(3, 300, 4, 3, 0, 128, 128, 64, P, P, P, P, P, P, P, P, P, need, None) == ERR_SHAPE
    assert pv(3, 300, 4, 2, 0, 128, 128, 32, P, P, P, P, P, P, P, P, P, need, None) == ERR_UNSUP
    assert pv(3, 300, 4, 2, 0, 128, 128, 64, D[0], D[1], D[2], D[3], D[4], D[5], D[6], D[7], D[8], need - 1, None) == ERR_WS
    assert pv(0, 300, 4, 2, 0, 128, 128, 64, N, D[0], D[1], D[2], D[3], D[4], D[5], D[6], N, 0, None) == OK
    assert pv(3, 0, 4, 2, 0, 128, 128, 64, P, N, N, N, N, N, P, N, N, 0, None) == OK


def test_prefill_varlen_ex_validation(lib):
    wsz = lib.gdn_prefill_varlen_workspace_size_ex
    base = wsz(3, 300, 4, 128, 128, 64, 1, 0)
    assert base == lib.gdn_prefill_varlen_workspace_size(3, 300, 4, 128, 128, 64) > 0
    kda, f32 = wsz(3, 300, 4, 128, 128, 64, 1, 1), wsz(3, 300, 4, 128, 128, 64, 0, 0)
    assert kda > base and f32 > base  # decayed images; bf16 images of the float32 rows
    assert wsz(3, 300, 4, 128, 128, 64, 2, 0) == 0 and wsz(3, 300, 4, 128, 128, 64, 1, 2) == 0
    pv = lib.gdn_prefill_chunked_varlen_ex
    # N, total, H, H_qk, map, dk, dv, chunk, dtype, gate, cu, q, k, v, g, beta, state, o, ws, ws_bytes, stream
    assert pv(3, 300, 4, 2, 0, 128, 128, 64, 1, 1, N, P, P, P, P, P, P, P, P, kda, None) == ERR_NULL
    assert pv(3, 300, 4, 2, 0, 128, 128, 64, 1, 1, P, P, P, P, N, P, P, P, P, kda, None) == ERR_NULL
    assert pv(-1, 300, 4, 2, 0, 128, 128, 64, 1, 1, P, P, P, P, P, P, P, P, P, kda, None) == ERR_SHAPE
    assert pv(3, 300, 4, 2, 0, 128, 128, 64, 2, 1, P, P, P, P, P, P, P, P, P, kda, None) == ERR_UNSUP
    assert pv(3, 300, 4, 2, 0, 128, 128, 64, 1, 2, P, P, P, P, P, P, P, P, P, kda, None) == ERR_UNSUP
    g8 = ctypes.c_void_p(264)  # 8-byte aligned: fine for GDA gates, not for KDA's 16-byte pieces
    assert pv(3, 300, 4, 2, 0, 128, 128, 64, 1, 1, P, P, P, P, g8, P, P, P, P, kda, None) == ERR_UNSUP
    assert pv(3, 300, 4, 2, 0, 128, 128, 64, 1, 1, D[0], D[1], D[2], D[3], D[4], D[5], D[6], D[7], D[8], kda - 1, None) == ERR_WS
    assert pv(3, 300, 4, 2, 0, 128, 128, 64, 0, 0, D[0], D[1], D[2], D[3], D[4], D[5], D[6], D[7], D[8], f32 - 1, None) == ERR_WS
    assert pv(0, 300, 4, 2, 0, 128, 128, 64, 1, 1, N, D[0], D[1], D[2], D[3], D[4], D[5], D[6], N, 0, None) == OK


def test_prefill_snapshots_validation(lib):
    need = lib.gdn_prefill_workspace_size(2, 100, 4, 128, 128, 64)
    ps = lib.gdn_prefill_chunked_snapshots
    # B, T, H, H_qk, map, dk, dv, chunk, K, q, k, v, g, beta, state, final, o, ws, ws_bytes, stream
    assert ps(2, 100, 4, 4, 0, 128, 128, 64, 0, P, P, P, P, P, P, P, P, P, need, None) == ERR_SHAPE
    assert ps(2, 100, 4, 3, 0, 128, 128, 64, 4, P, P, P, P, P, P, P, P, P, need, None) == ERR_SHAPE
    assert ps(2, 100, 4, 4, 0, 128, 128, 64, 4, P, P, P, P, P, N, P, P, P, need, None) == ERR_NULL
    assert ps(2, 100, 4, 4, 0, 128, 96, 64, 4, P, P, P, P, P, P, P, P, P, need, None) == ERR_UNSUP
    assert ps(2, 100, 4, 4, 2, 128, 128, 64, 4, P, P, P, P, P, P, P, P, P, need, None) == ERR_UNSUP
    assert ps(2, 100, 4, 4, 0, 128, 128, 64, 4, D[0], D[1], D[2], D[3], D[4], D[5], D[6], D[7], D[8], need - 1, None) == ERR_WS
    # empty problems launch nothing; T = 0 without final_state (or with K = 1) is a no-op
    assert ps(0, 100, 4, 4, 0, 128, 128, 64, 4, N, N, N, N, N, N, N, N, N, 0, None) == OK
    assert ps(2, 0, 4, 4, 0, 128, 128, 64, 4, N, N, N, N, N, P, N, N, N, 0, None) == OK
    assert ps(2, 0, 4, 4, 0, 128, 128, 64, 1, N, N, N, N, N, P, P, N, N, 0, None) == OK


def test_prefill_kda_validation(lib):
    wsz = lib.gdn_prefill_kda_workspace_size
    need = wsz(1, 100, 4, 128, 128, 64)
    assert need > lib.gdn_prefill_workspace_size(1, 100, 4, 128, 128, 64) > 0  # three more images
    assert wsz(1, 100, 4, 128, 128, 32) == 0
    pk = lib.gdn_prefill_chunked_kda
    # B, T, H, H_qk, map, dk, dv, chunk, q, k, v, g, beta, state, o, ws, ws_bytes, stream
    assert pk(1, 100, 4, 4, 0, 128, 128, 64, P, P, P, N, P, P, P, P, need, None) == ERR_NULL
    assert pk(1, 100, 4, 3, 0, 128, 128, 64, P, P, P, P, P, P, P, P, need, None) == ERR_SHAPE
    assert pk(1, 100, 4, 4, 0, 128, 128, 16, P, P, P, P, P, P, P, P, need, None) == ERR_UNSUP
    assert pk(1, 100, 4, 4, 0, 128, 128, 64, P, P, P, ctypes.c_void_p(260), P, P, P, P, need,
              None) == ERR_UNSUP
    assert pk(1, 100, 4, 4, 0, 128, 128, 64, D[0], D[1], D[2], D[3], D[4], D[5], D[6], D[7], need - 1, None) == ERR_WS
    assert pk(1, 0, 4, 4, 0, 128, 128, 64, N, N, N, N, N, D[0], N, N, 0, None) == OK


def test_prefill_ex_validation(lib):
    wsz = lib.gdn_prefill_workspace_size_ex
    gda_bf, gda_f, kda_bf, kda_f = (wsz(1, 100, 4, 128, 128, 64, dt, gt) for dt, gt in
                                    ((1, 0), (0, 0), (1, 1), (0, 1)))
    assert 0 < gda_bf < gda_f and gda_bf < kda_bf < kda_f  # images for f32 inputs and for KDA
    assert gda_bf == lib.gdn_prefill_workspace_size(1, 100, 4, 128, 128, 64)
    assert wsz(1, 100, 4, 128, 128, 64, 2, 0) == 0 and wsz(1, 100, 4, 128, 128, 64, 1, 2) == 0
    pe = lib.gdn_prefill_chunked_ex
    # B, T, H, H_qk, map, dk, dv, chunk, dtype, gate, K, q, k, v, g, beta, state, final, o, ws, ws_bytes, stream
    assert pe(1, 100, 4, 4, 0, 128, 128, 64, 0, 0, 0, P, P, P, P, P, P, N, P, P, gda_f, None) == ERR_SHAPE
    assert pe(1, 100, 4, 4, 0, 128, 128, 64, 5, 0, 1, P, P, P, P, P, P, N, P, P, gda_f, None) == ERR_UNSUP
    # KDA with K > 1 snapshot slots is accepted up to the workspace check
    assert pe(1, 100, 4, 4, 0, 128, 128, 64, 1, 1, 2, D[0], D[1], D[2], D[3], D[4], D[5], N, D[6], D[7], kda_bf - 1, None) == ERR_WS
    assert pe(1, 100, 4, 4, 0, 128, 128, 64, 0, 0, 1, D[0], D[1], D[2], D[3], D[4], D[5], N, D[6], D[7], gda_f - 1, None) == ERR_WS
    assert pe(1, 100, 4, 4, 0, 128, 128, 64, 0, 1, 1, D[0], D[1], D[2], D[3], D[4], D[5], N, D[6], D[7], kda_f - 1, None) == ERR_WS
    assert pe(1, 0, 4, 4, 0, 128, 128, 64, 0, 0, 1, N, N, N, N, N, D[0], N, N, N, 0, None) == OK



def test_prefill_ex_after_rollback_validation(lib):
    # accepted first, then every check of gdn_prefill_chunked_ex; none launches
    need = lib.gdn_prefill_workspace_size_ex(2, 100, 4, 128, 128, 64, 1, 0)
    wsa = ctypes.c_void_p(4096)

    def par(B=2, T=100, H=4, Hq=4, hm=0, dk=128, dv=128, chunk=64, dt=1, gate=0, K=4, acc=D[0], q=D[1], k=D[2],
            v=D[3], g=D[4], beta=D[5], st=D[6], fin=N, o=D[7], ws=wsa, wsb=need, err=N):
        return lib.gdn_prefill_chunked_ex_after_rollback(B, T, H, Hq, hm, dk, dv, chunk, dt, gate, K, acc, q, k, v,
                                                         g, beta, st, fin, o, ws, wsb, err, None)
    assert par(acc=N) == ERR_NULL
    assert par(st=N) == ERR_NULL
    assert par(beta=N) == ERR_NULL
    assert par(K=0) == ERR_SHAPE
    assert par(H=4, Hq=3) == ERR_SHAPE
    assert par(chunk=32) == ERR_UNSUP
    assert par(dk=96) == ERR_UNSUP
    assert par(dt=5) == ERR_UNSUP
    assert par(o=ctypes.c_void_p(264)) == ERR_UNSUP
    assert par(wsb=need - 1) == ERR_WS
    assert par(o=D[1]) == ERR_ALIAS      # o is q
    assert par(err=D[6]) == ERR_ALIAS    # the error flag inside the state
    assert par(acc=D[7]) == ERR_ALIAS    # the accepted lengths inside o
    assert par(ws=ctypes.c_void_p(4096 + 16)) == ERR_WS
    assert par(ws=N) == ERR_WS
    assert par(B=0, acc=N) == OK
    assert par(H=0) == OK



def test_overlapping_arrays_are_refused(lib):
    """An array the call writes may share no byte with another of its arrays:
    GDN_ERR_ALIAS, before any launch.  Inputs may share memory."""
    at = lambda p, off: ctypes.c_void_p(p.value + off)
    # decode, bf16, B=T=H=1, d=64: q, k, v are 128 bytes each
    fw = lambda q, k, v, g, b, st, o: lib.gdn_forward(1, 1, 1, 64, 64, 1, 0, q, k, v, g, b, st, o, None)
    assert fw(D[0], D[1], D[2], D[3], D[4], D[5], D[0]) == ERR_ALIAS             # o is q
    assert fw(D[0], D[1], D[2], D[3], D[4], at(D[2], 112), D[6]) == ERR_ALIAS    # state begins in v
    assert fw(D[0], D[1], D[2], D[3], D[4], D[5], at(D[5], 16368)) == ERR_ALIAS  # o ends the state
    # snapshots: the final state inside slot 3 of the state (K = 4 slots of 16 KiB)
    assert lib.gdn_forward_snapshots(1, 1, 1, 64, 64, 1, 0, 4, D[0], D[1], D[2], D[3], D[4], D[5],
                                     at(D[5], 3 * 16384), D[6], None) == ERR_ALIAS
    # rollback: the error flag in the last slot
    assert lib.gdn_rollback_select(2, 2, 4, 64, 64, D[0], D[1], at(D[1], 2 * 2 * 4 * 16384 - 4), None) == ERR_ALIAS
    # prefill: q (100 tokens x 2 heads x 128 bf16 = 51200 bytes) followed at once by o is fine
    # (the next check, a missing workspace, fails), one 16-byte piece earlier it is not
    pe = lambda o, ws, wsb: lib.gdn_prefill_chunked_ex(1, 100, 2, 2, 0, 128, 128, 64, 1, 0, 1, D[0], D[1], D[2],
                                                      D[3], D[4], D[5], N, o, ws, wsb, None)
    need = lib.gdn_prefill_workspace_size_ex(1, 100, 2, 128, 128, 64, 1, 0)
    assert pe(at(D[0], 51200), N, 0) == ERR_WS
    assert pe(at(D[0], 51200 - 16), N, 0) == ERR_ALIAS
    assert pe(D[6], at(D[6], 256), need) == ERR_ALIAS  # the workspace inside o
    assert pe(D[6], at(D[5], -(need - 256)), need) == ERR_ALIAS  # the workspace runs into the state
    # variable-length prefill: o over the sequence offsets
    assert lib.gdn_prefill_chunked_varlen(2, 100, 2, 2, 0, 128, 128, 64, D[0], D[1], D[2], D[3], D[4], D[5],
                                          D[6], at(D[0], 0), D[7], 1 << 30, None) == ERR_ALIAS


SCRATCH_BYTES = 256 * 1024 * 1024  # GDN_PREFILL_SCRATCH_BYTES in include/gdn.h


def test_prefill_ex_noalloc_validation(lib):
    hdr = open(os.path.join(ROOT, "include", "gdn.h")).read()
    assert "#define GDN_PREFILL_SCRATCH_BYTES (256u * 1024u * 1024u)" in hdr
    pn = lib.gdn_prefill_chunked_ex_noalloc
    # B, T, H, H_qk, map, dk, dv, chunk, dtype, gate, K, q, k, v, g, beta, state, final, o, stream
    assert pn(1, 100, 4, 4, 0, 128, 128, 64, 0, 0, 0, P, P, P, P, P, P, N, P, None) == ERR_SHAPE
    assert pn(1, 100, 4, 3, 0, 128, 128, 64, 1, 0, 1, P, P, P, P, P, P, N, P, None) == ERR_SHAPE
    assert pn(1, 100, 4, 4, 0, 128, 128, 64, 5, 0, 1, P, P, P, P, P, P, N, P, None) == ERR_UNSUP
    assert pn(1, 100, 4, 4, 0, 128, 128, 32, 1, 0, 1, P, P, P, P, P, P, N, P, None) == ERR_UNSUP
    assert pn(1, 100, 4, 4, 0, 128, 128, 64, 1, 1, 2, P, P, P, P, N, P, N, P, None) == ERR_NULL
    assert pn(1, 100, 4, 4, 0, 128, 128, 64, 1, 0, 1, N, P, P, P, P, P, N, P, None) == ERR_NULL
    assert pn(1, 0, 4, 4, 0, 128, 128, 64, 1, 0, 1, N, N, N, N, N, P, N, N, None) == OK
    assert pn(0, 100, 4, 4, 0, 128, 128, 64, 1, 0, 1, N, N, N, N, N, N, N, N, None) == OK
    # the largest workspace the scratch array holds, and one chunk more
    wsz = lib.gdn_prefill_workspace_size_ex
    for dt, gate in ((1, 0), (0, 0), (1, 1), (0, 1)):
        assert wsz(1, 8192, 16, 128, 128, 64, dt, gate) <= SCRATCH_BYTES  # the prefill workload fits
        per_chunk = wsz(1, 64, 1, 128, 128, 64, dt, gate)
        n = SCRATCH_BYTES // per_chunk  # chunks of one head that fit
        assert wsz(1, 64 * n, 1, 128, 128, 64, dt, gate) <= SCRATCH_BYTES
        assert wsz(1, 64 * n + 1, 1, 128, 128, 64, dt, gate) > SCRATCH_BYTES
        assert pn(1, 64 * n + 1, 1, 1, 0, 128, 128, 64, dt, gate, 1,
                  D[10], D[11], D[12], D[13], D[14], D[15], N, D[16], None) == ERR_SCRATCH


def test_bench_runs_on_one_gpu_only():
    """bench.py measures one GPU: any other --gpus value exits with status 2
    and says so, before it touches a GPU."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_bench_traffic_tied_to_kernel_sources(monkeypatch):
    """bench.py reports the counter-measured decode traffic only for the
    kernel sources it was measured on; for those it is the calibrated
    FETCH_SIZE + WRITE_SIZE, close to the algorithmic bytes of the launch."""
    import hashlib
    import importlib
    import sys
    sys.path.insert(0, ROOT)
    bench = importlib.import_module("bench")
    t = dict(bench.DECODE_TRAFFIC)
    h = hashlib.sha256()
    for rel in t["sources"]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    monkeypatch.setitem(bench.DECODE_TRAFFIC, "sha256", "0" * 64)
    assert bench.decode_traffic_bytes() is None
    monkeypatch.setitem(bench.DECODE_TRAFFIC, "sha256", h.hexdigest())
    got = bench.decode_traffic_bytes()
    copy = 64 * 1024 * 1024
    want = t["fetch_kib"] / t["copy_fetch_kib"] * copy + t["write_kib"] / t["copy_write_kib"] * copy
    assert got == pytest.approx(want, rel=1e-12)
    algorithmic = bench.recurrent_bytes(64, 1, 16, 128, 1, False, True)
    assert 0.9 < got / algorithmic < 1.3


def test_bench_decode_traffic_matches_kernel_sources():
    """bench.py reports the decode kernel's counter-measured HBM traffic only
    while the kernel sources are those the counters were taken on; the
    committed figures must describe the committed sources."""
    import sys
    sys.path.insert(0, ROOT)
    import bench
    nbytes = bench.decode_traffic_bytes()
    assert nbytes is not None, "decode traffic counters describe other kernel sources: collect them again"
    assert 1.0 <= nbytes / 135536640 < 1.05  # within 5% above the algorithmic bytes
