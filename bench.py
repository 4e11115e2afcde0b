#!/usr/bin/env python3
"""Benchmark of the GDN recurrence library on one MI355X.

Headline workload: batched decode, GDA, B=64 sequences, H=16 heads,
d_k=d_v=128, one token per sequence, bf16 q/k/v, fp32 gates and state
(state [64,16,128,128] fp32 = 64 MiB, read and written in place).

A step is one call of gdn_forward over the whole batch.  The timed region
holds exactly --steps steps between two device synchronisations: the steps
are captured once into a HIP graph (removing Python launch overhead) and one
replay is timed with HIP events on the stream the kernels run on.  Inputs
are resident in HBM before it starts.  To measure HBM rather than the 256 MB
Infinity Cache, the steps rotate over enough independent input/state sets to
span >= 1 GiB.

Printed: ONE JSON line with the throughput (tokens/s), the roofline of the
dominant kernel (algorithmic bytes per launch / mean launch time, against
8 TB/s), the other workloads of the path (speculative verify + rollback, KDA
verify + rollback, chunked prefill), and the float64 CPU oracle timed on a
bounded sample on the host cores as a baseline.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
ROTATE_BYTES = 1 << 30  # >= 1 GiB of rotating buffers defeats the 256 MB MALL

METRIC = "GDN tokens/s and achieved HBM GB/s (% peak), decode B=64 H=16 d=128"

# HBM traffic of one decode launch, from two rocprofv3 --pmc runs of
# `bench.py --only decode --copy-calibration` (FETCH_SIZE, then WRITE_SIZE, KiB
# per dispatch; summary in profiles/recurrent_decode_B64_H16_d128_traffic.md).
# Each counter is scaled by what it reads for a 64 MiB device-to-device copy
# (64 MiB read + 64 MiB written).  The figures describe the kernel built from
# the sources hashed below and are reported only while those are unchanged.
DECODE_TRAFFIC = {
    "sources": ["linear_attention_recurrence_net_amd/csrc/gdn_recurrent.hip",
                "linear_attention_recurrence_net_amd/csrc/device_common.hpp",
                "linear_attention_recurrence_net_amd/csrc/gdn_internal.hpp"],
    "sha256": "e061ddf4b1fe0583377e4f0182f5280529d2e4ead4e3c4ceacf4b710e90ad225",
    "fetch_kib": 33259.0,       # median over 162 decode dispatches
    "write_kib": 66085.3125,
    "copy_fetch_kib": 32779.5,  # median over 98 copies of 64 MiB
    "copy_write_kib": 65536.0,
}


def decode_traffic_bytes():
    """Calibrated HBM bytes per decode launch, or None if not measured for
    the current kernel sources."""
    import hashlib
    t = DECODE_TRAFFIC
    if t["sha256"] is None:
        return None
    h = hashlib.sha256()
    for rel in t["sources"]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != t["sha256"]:
        return None
    copy_bytes = 64 * 1024 * 1024
    fetch = t["fetch_kib"] * 1024 * copy_bytes / (t["copy_fetch_kib"] * 1024)
    write = t["write_kib"] * 1024 * copy_bytes / (t["copy_write_kib"] * 1024)
    return fetch + write


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------
# algorithmic work (minimum bytes the method must move)
# ----------------------------------------------------------------------------
def token_bytes(d: int, kda: bool, bf16: bool) -> int:
    """Per token and head: q, k, v in, o out (fp32), gate(s) and beta."""
    e = 2 if bf16 else 4
    gate = 4 * d if kda else 4
    return 3 * d * e + gate + 4 + 4 * d


def recurrent_bytes(B, T, H, d, K, kda, bf16, final=False) -> int:
    tile = 4 * d * d
    n_snap = min(T, K - 1) if K > 1 else 0
    state = tile + (tile if K == 1 else n_snap * tile) + (tile if final else 0)
    return B * H * (state + T * token_bytes(d, kda, bf16))


def broadcast_bytes(B, T, H, Hq, d, bf16=True) -> int:
    """Decode with H value heads sharing Hq q/k heads: the state in and out
    and v, o, g, beta per value head; q and k once per q/k head."""
    e = 2 if bf16 else 4
    tile = 4 * d * d
    return B * H * (2 * tile + T * (d * e + 4 * d + 8)) + B * Hq * T * 2 * d * e


def recurrent_flops(B, T, H, d) -> int:
    # per token-head: two d x d reductions and one rank-1 update (3 d^2 FMA)
    return B * T * H * 7 * d * d


def prefill_bytes(B, T, H, d) -> int:
    return B * T * H * (3 * 2 * d + 8 + 4 * d) + 2 * B * H * 4 * d * d


def prefill_kda_bytes(B, T, H, d) -> int:
    """As prefill_bytes, with one fp32 log-gate per key row instead of one per head."""
    return B * T * H * (3 * 2 * d + 4 * d + 4 + 4 * d) + 2 * B * H * 4 * d * d


def prefill_flops(B, T, H, d, C=64) -> int:
    """Dense-tile MFMA work of the chunk form per head-token: 2 (5 C d + 3 d^2)."""
    return B * T * H * 2 * (5 * C * d + 3 * d * d)


# ----------------------------------------------------------------------------
# GPU timing helpers
# ----------------------------------------------------------------------------
def run_timed(torch, calls, steps, warmup):
    """Time exactly `steps` launches (rotating over `calls`).

    Each call takes the HIP stream handle to launch on.  Warmup: `warmup`
    eager launches, then the `steps` launches are captured once into a HIP
    graph and the graph is replayed once untimed.  The timed region is one
    replay of that graph between two HIP events recorded on the stream the
    kernels run on, bracketed by device synchronisations.  Returns
    (region_ms, eager_ms_per_step) where the second figure times the same
    launches issued one by one from Python (launch overhead included).
    """
    cur = torch.cuda.current_stream()
    sp = ctypes.c_void_p(cur.cuda_stream)
    for i in range(warmup):
        calls[i % len(calls)](sp)
    torch.cuda.synchronize()
    # eager reference timing (host launch overhead included)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_eager = min(steps, 50)
    e0.record(cur)
    for i in range(n_eager):
        calls[i % len(calls)](sp)
    e1.record(cur)
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / n_eager

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for i in range(steps):
            calls[i % len(calls)](gs)
    graph.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(cur)
    graph.replay()
    end.record(cur)
    torch.cuda.synchronize()
    region_ms = start.elapsed_time(end)
    del graph
    return region_ms, eager_ms


def launch_spread(torch, calls, n=100):
    """Per-launch GPU time of `n` eager launches (rotating over `calls`),
    each bracketed by its own pair of HIP events on the launch stream.
    Returns (p10, median, p90) in microseconds."""
    cur = torch.cuda.current_stream()
    sp = ctypes.c_void_p(cur.cuda_stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i, (a, b) in enumerate(ev):
        a.record(cur)
        calls[i % len(calls)](sp)
        b.record(cur)
    torch.cuda.synchronize()
    us = np.sort(np.array([a.elapsed_time(b) * 1e3 for a, b in ev]))
    return float(np.percentile(us, 10)), float(np.median(us)), float(np.percentile(us, 90))


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------
def upload_case(torch, case):
    qdt = torch.bfloat16 if case.qkv_dtype == "bf16" else torch.float32
    dev = lambda a, dt=None: (torch.from_numpy(np.ascontiguousarray(a)).to(dt) if dt else
                              torch.from_numpy(np.ascontiguousarray(a))).to("cuda")
    return dict(q=dev(case.q, qdt), k=dev(case.k, qdt), v=dev(case.v, qdt), g=dev(case.g),
                beta=dev(case.beta), state=dev(case.state))


def raw_forward_call(lib, case, d, state, o, K=None, final=None):
    """Pre-marshalled ctypes call of gdn_forward / gdn_forward_snapshots (no
    per-call Python checks inside the timed loop)."""
    dt = 1 if case.qkv_dtype == "bf16" else 0
    gate = 1 if case.gate == "kda" else 0
    p = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
    args_common = (p(d["q"]), p(d["k"]), p(d["v"]), p(d["g"]), p(d["beta"]))
    if K is None:
        args = (case.B, case.T, case.H, case.d_k, case.d_v, dt, gate, *args_common, p(state),
                p(o))
        fn = lib.gdn_forward
    else:
        args = (case.B, case.T, case.H, case.d_k, case.d_v, dt, gate, K, *args_common, p(state),
                p(final), p(o))
        fn = lib.gdn_forward_snapshots

    def call(stream):
        st = fn(*args, stream)
        if st != 0:
            raise RuntimeError(f"libgdn status {st}")
    return call


def _rotating_sets(torch, d, case, with_state_slot0=False):
    """Independent copies of all inputs and the state, >= 1 GiB in total."""
    state = d["state"][:, :, 0].contiguous() if with_state_slot0 else d["state"]
    n_sets = max(2, -(-ROTATE_BYTES // (state.numel() * 4)))
    sets = []
    for _ in range(n_sets):
        ds = {k: v.clone() for k, v in d.items() if k != "state"}
        ds["state"] = state.clone()
        ds["o"] = torch.empty((case.B, case.T, case.H, case.d_v), device="cuda")
        sets.append(ds)
    return sets


def _timing(region_ms, eager_ms, steps):
    per = region_ms / steps
    return dict(ms_per_step=per, us_per_launch=per * 1e3, eager_us_per_launch=eager_ms * 1e3)


def bench_copy_context(torch, steps, warmup):
    """A plain device-to-device copy of 64 MiB (torch's copy_), timed like the
    decode: graph-replayed launches over 8 rotating source/destination pairs
    (1 GiB), so each copy reads and writes HBM.  Context for the decode's
    fraction of peak: what a copy of the decode's state size reaches here."""
    n = 16 * 1024 * 1024
    pairs = [(torch.randn(n, device="cuda"), torch.empty(n, device="cuda")) for _ in range(8)]
    calls = [lambda sp, s=s, d=d: d.copy_(s) for s, d in pairs]
    t = _timing(*run_timed(torch, calls, steps, warmup), steps)
    nbytes = 2 * n * 4
    gbs = nbytes / (t["us_per_launch"] * 1e-6) / 1e9
    del pairs, calls
    torch.cuda.empty_cache()
    return {"what": "device-to-device copy of 64 MiB (torch copy_), 8 rotating pairs, graph-replayed",
            "bytes_per_copy": nbytes, "us_per_copy": t["us_per_launch"], "achieved_gbs": gbs,
            "frac_of_hbm_peak": gbs / HBM_PEAK_GBS}


def bench_decode(torch, lib, steps, warmup):
    import gdn_inputs as gi
    case = gi.workload_case(1)
    d = upload_case(torch, case)
    sets = _rotating_sets(torch, d, case, with_state_slot0=True)
    calls = [raw_forward_call(lib, case, s, s["state"], s["o"]) for s in sets]
    region_ms, eager_ms = run_timed(torch, calls, steps, warmup)
    spread = launch_spread(torch, calls)
    nbytes = recurrent_bytes(case.B, case.T, case.H, case.d_k, 1, False, True)
    t = _timing(region_ms, eager_ms, steps)
    res = dict(case=case, n_sets=len(sets), region_ms=region_ms, spread_us=spread,
               tokens_per_s=case.B * case.T * steps / (region_ms * 1e-3),
               bytes=nbytes, achieved_gbs=nbytes / (t["us_per_launch"] * 1e-6) / 1e9, **t)
    del sets, calls
    torch.cuda.empty_cache()
    return res


BROADCAST_WORKLOAD = dict(name="decode GDA B=64 H=32 value heads sharing H_qk=16 q/k heads "
                               "(grouped) d=128 T=1", B=64, T=1, H=32, H_qk=16, d_k=128)


def bench_decode_broadcast(torch, lib, steps, warmup):
    """Decode where two value heads share each q/k head (gdn_forward_qk_broadcast)."""
    import gdn_inputs as gi
    w = BROADCAST_WORKLOAD
    case = gi.make_case(w["B"], w["T"], w["H"], w["d_k"], qkv_dtype="bf16", seed=11, H_qk=w["H_qk"])
    d = upload_case(torch, case)
    sets = _rotating_sets(torch, d, case, with_state_slot0=True)
    p = lambda t: ctypes.c_void_p(t.data_ptr())

    def mk(s):
        args = (case.B, case.T, case.H, case.H_qk, 0, case.d_k, case.d_v, 1, 0, 1, p(s["q"]),
                p(s["k"]), p(s["v"]), p(s["g"]), p(s["beta"]), p(s["state"]), None, p(s["o"]))

        def call(stream):
            st = lib.gdn_forward_qk_broadcast(*args, stream)
            if st != 0:
                raise RuntimeError(f"libgdn status {st}")
        return call
    calls = [mk(s) for s in sets]
    t = _timing(*run_timed(torch, calls, steps, warmup), steps)
    nbytes = broadcast_bytes(case.B, case.T, case.H, case.H_qk, case.d_k)
    gbs = nbytes / (t["us_per_launch"] * 1e-6) / 1e9
    del sets, calls
    torch.cuda.empty_cache()
    return dict(workload=w["name"], bytes=nbytes, achieved_gbs=gbs, frac_of_hbm_peak=gbs / HBM_PEAK_GBS,
                tokens_per_s=case.B * case.T / (t["us_per_launch"] * 1e-6), **t)


SMALL_BATCHES = (1, 8)


def bench_small_batch(torch, lib, steps, warmup):
    """Decode (one token) and the four-token verify (K = 4) of GDA H=16 d=128
    at small batches, whose grids fill less than one resident round and are
    launched in column blocks."""
    import gdn_inputs as gi
    out = {}
    for kind, T, K in (("decode", 1, 1), ("verify", 4, 4)):
        for B in SMALL_BATCHES:
            case = gi.make_case(B, T, 16, 128, K=K, gate="gda", qkv_dtype="bf16", seed=17 + B)
            d = upload_case(torch, case)
            sets = _rotating_sets(torch, d, case, with_state_slot0=K == 1)
            calls = [raw_forward_call(lib, case, s, s["state"], s["o"], K=None if K == 1 else K) for s in sets]
            t = _timing(*run_timed(torch, calls, steps, warmup), steps)
            nbytes = recurrent_bytes(B, T, 16, 128, K, False, True)
            gbs = nbytes / (t["us_per_launch"] * 1e-6) / 1e9
            out[f"{kind}_B{B}"] = dict(bytes=nbytes, achieved_gbs=gbs, frac_of_hbm_peak=gbs / HBM_PEAK_GBS,
                                       tokens_per_s=B * T / (t["us_per_launch"] * 1e-6), **t)
            del sets, calls, d
            torch.cuda.empty_cache()
    out["workload"] = (f"GDA H=16 d=128 bf16 q/k/v: decode (T=1) and verify (T=4, K=4) at B in {SMALL_BATCHES}")
    return out


def bench_verify(torch, lib, cfg, steps, warmup):
    """Speculative verify (K=4 snapshots, no final state), then rollback."""
    import gdn_inputs as gi
    case = gi.workload_case(cfg)
    d = upload_case(torch, case)
    sets = _rotating_sets(torch, d, case)
    acc = torch.from_numpy(case.accepted).to("cuda")
    fwd = [raw_forward_call(lib, case, s, s["state"], s["o"], K=case.K) for s in sets]
    vp = lambda t: ctypes.c_void_p(t.data_ptr())

    def rb_call(s):
        args = (case.B, case.H, case.K, case.d_k, case.d_v, vp(acc), vp(s["state"]), None)

        def call(stream):
            st = lib.gdn_rollback_select(*args, stream)
            if st != 0:
                raise RuntimeError(f"libgdn status {st}")
        return call
    rbs = [rb_call(s) for s in sets]

    def both(f, r):
        def call(stream):
            f(stream)
            r(stream)
        return call
    pair = [both(f, r) for f, r in zip(fwd, rbs)]

    def fused_call(s):
        # the rollback of the previous draft fused into the next verification
        dt = 1 if case.qkv_dtype == "bf16" else 0
        args = (case.B, case.T, case.H, case.H, 0, case.d_k, case.d_v, dt, 1 if case.gate == "kda" else 0, case.K,
                vp(acc), vp(s["q"]), vp(s["k"]), vp(s["v"]), vp(s["g"]), vp(s["beta"]), vp(s["state"]), None,
                vp(s["o"]), None)

        def call(stream):
            st = lib.gdn_forward_snapshots_after_rollback(*args, stream)
            if st != 0:
                raise RuntimeError(f"libgdn status {st}")
        return call
    fused = [fused_call(s) for s in sets]
    kda = case.gate == "kda"
    vt = _timing(*run_timed(torch, fwd, steps, warmup), steps)
    rt = _timing(*run_timed(torch, rbs, steps, warmup), steps)
    # one event pair per eager launch, 100 launches (the graph mean is the figure)
    vt["launch_us_p10_p50_p90"] = [round(x, 3) for x in launch_spread(torch, fwd)]
    rt["launch_us_p10_p50_p90"] = [round(x, 3) for x in launch_spread(torch, rbs)]
    bt = _timing(*run_timed(torch, pair, steps, warmup), steps)
    ft = _timing(*run_timed(torch, fused, steps, warmup), steps)
    vbytes = recurrent_bytes(case.B, case.T, case.H, case.d_k, case.K, kda, True)
    moved = int(np.count_nonzero(case.accepted > 0))
    rbytes = 2 * moved * case.H * 4 * case.d_k * case.d_v
    tokens = case.B * case.T
    vg = vbytes / (vt["us_per_launch"] * 1e-6) / 1e9
    rg = rbytes / (rt["us_per_launch"] * 1e-6) / 1e9
    out = dict(
        workload=gi.WORKLOADS[cfg]["name"],
        verify=dict(bytes=vbytes, achieved_gbs=vg, frac_of_hbm_peak=vg / HBM_PEAK_GBS,
                    tokens_per_s=tokens / (vt["us_per_launch"] * 1e-6), **vt),
        rollback=dict(bytes=rbytes, sequences_rolled=moved, achieved_gbs=rg,
                      frac_of_hbm_peak=rg / HBM_PEAK_GBS, **rt),
        verify_plus_rollback=dict(tokens_per_s=tokens / (bt["us_per_launch"] * 1e-6), **bt),
        # gdn_forward_snapshots_after_rollback: the same two steps in one launch
        rollback_fused_into_verify=dict(tokens_per_s=tokens / (ft["us_per_launch"] * 1e-6),
                                        bytes=vbytes + rbytes // 2, **ft),
        rotating_sets=len(sets),
    )
    del sets, fwd, rbs, pair, fused
    torch.cuda.empty_cache()
    return out


def _nbytes(ts) -> int:
    return sum(t.numel() * t.element_size() for t in ts)


def _prefill_sets(torch, tensors, extra_bytes):
    """Independent copies of a prefill's device tensors (inputs, state, o and
    workspace), as many as make up >= 1 GiB, so that no timed launch finds its
    data in the 256 MB Infinity Cache.  `tensors` maps names to the tensors
    of one set; `extra_bytes` maps the names of buffers allocated per set
    (o, workspace) to their sizes in bytes."""
    per_set = _nbytes(tensors.values()) + sum(extra_bytes.values())
    n_sets = max(2, -(-ROTATE_BYTES // per_set))
    sets = []
    for _ in range(n_sets):
        ds = {k: v.clone() for k, v in tensors.items()}
        for k, nb in extra_bytes.items():
            ds[k] = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
        sets.append(ds)
    return sets, per_set


def _prefill_result(name, case, t, nb, fl, ws_bytes, n_sets, per_set):
    sec = t["us_per_launch"] * 1e-6
    return dict(
        workload=name, bytes=nb, flops=fl, tokens_per_s=case.B * case.T / sec,
        achieved_gbs=nb / sec / 1e9, frac_of_hbm_peak=nb / sec / 1e9 / HBM_PEAK_GBS,
        achieved_tflops=fl / sec / 1e12, frac_of_bf16_peak=fl / sec / 1e12 / BF16_PEAK_TFLOPS,
        workspace_bytes=int(ws_bytes), rotating_sets=n_sets, bytes_per_set=int(per_set), **t,
    )


def _bench_prefill_leg(torch, lib, case, entry, ws_bytes, steps, warmup):
    """Time one single-sequence prefill entry point over rotating sets.
    `entry(s)` returns the argument tuple (without the stream) and the C
    function for set s."""
    d = upload_case(torch, case)
    base = {k: v for k, v in d.items() if k != "state"}
    base["state"] = d["state"][:, :, 0].contiguous()
    o_bytes = case.B * case.T * case.H * case.d_v * 4
    sets, per_set = _prefill_sets(torch, base, {"o": o_bytes, "ws": ws_bytes})
    del d, base

    def mk(s):
        fn, args = entry(s)

        def call(stream):
            st = fn(*args, stream)
            if st != 0:
                raise RuntimeError(f"libgdn status {st}")
        return call
    calls = [mk(s) for s in sets]
    t = _timing(*run_timed(torch, calls, steps, warmup), steps)
    # the same launches on the first set only, whose data the 256 MB Infinity
    # Cache then holds: for comparison with single-set timings, never `value`
    warm = _timing(*run_timed(torch, calls[:1], steps, warmup), steps)
    t["single_set_us_per_launch"] = warm["us_per_launch"]
    # one event pair per eager launch, 100 launches (the graph mean is the figure)
    t["launch_us_p10_p50_p90"] = [round(x, 3) for x in launch_spread(torch, calls)]
    n_sets = len(sets)
    del sets, calls
    torch.cuda.empty_cache()
    return t, n_sets, per_set


def _vp(t):
    return ctypes.c_void_p(t.data_ptr())


def bench_prefill(torch, lib, steps, warmup):
    import gdn_inputs as gi
    case = gi.workload_case(4)
    ws_bytes = lib.gdn_prefill_workspace_size(case.B, case.T, case.H, case.d_k, case.d_v, 64)

    def entry(s):
        return lib.gdn_prefill_chunked, (
            case.B, case.T, case.H, case.d_k, case.d_v, 64, _vp(s["q"]), _vp(s["k"]), _vp(s["v"]),
            _vp(s["g"]), _vp(s["beta"]), _vp(s["state"]), _vp(s["o"]), _vp(s["ws"]), ws_bytes)
    t, n_sets, per_set = _bench_prefill_leg(torch, lib, case, entry, ws_bytes, steps, warmup)
    return _prefill_result(gi.WORKLOADS[4]["name"], case, t, prefill_bytes(case.B, case.T, case.H, case.d_k),
                           prefill_flops(case.B, case.T, case.H, case.d_k), ws_bytes, n_sets, per_set)


VARLEN_WORKLOAD = dict(name="prefill GDA, 8192 tokens packed as 16 sequences of mixed length "
                            "(seeded log-uniform mix), H=16 d=128 chunk 64", total=8192, N=16, H=16,
                       d=128, seed=21)


def bench_prefill_varlen(torch, lib, steps, warmup):
    """The prefill token count split into many sequences (gdn_prefill_chunked_varlen)."""
    import gdn_inputs as gi
    w = VARLEN_WORKLOAD
    lens = gi.varlen_lengths(w["total"], w["N"], seed=w["seed"])
    vc = gi.make_varlen_case(lens, w["H"], w["d"], seed=w["seed"])
    bf = torch.bfloat16
    t = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dt)
    q, k, v = t(vc.q, bf), t(vc.k, bf), t(vc.v, bf)
    g, beta, st = t(vc.g), t(vc.beta), t(vc.state)
    cu = torch.from_numpy(vc.cu_seqlens).to("cuda")
    ws_bytes = lib.gdn_prefill_varlen_workspace_size(vc.N, vc.total, vc.H, vc.d, vc.d, 64)
    sets, per_set = _prefill_sets(torch, dict(q=q, k=k, v=v, g=g, beta=beta, state=st, cu=cu),
                                  {"o": vc.total * vc.H * vc.d * 4, "ws": ws_bytes})
    del q, k, v, g, beta, st, cu

    def mk(s):
        args = (vc.N, vc.total, vc.H, vc.H, 0, vc.d, vc.d, 64, _vp(s["cu"]), _vp(s["q"]), _vp(s["k"]),
                _vp(s["v"]), _vp(s["g"]), _vp(s["beta"]), _vp(s["state"]), _vp(s["o"]), _vp(s["ws"]),
                ws_bytes)

        def call(stream):
            st_ = lib.gdn_prefill_chunked_varlen(*args, stream)
            if st_ != 0:
                raise RuntimeError(f"libgdn status {st_}")
        return call
    vcalls = [mk(s) for s in sets]
    tm = _timing(*run_timed(torch, vcalls, steps, warmup), steps)
    tm["launch_us_p10_p50_p90"] = [round(x, 3) for x in launch_spread(torch, vcalls)]
    n_sets = len(sets)
    del sets, vcalls
    torch.cuda.empty_cache()
    sec = tm["us_per_launch"] * 1e-6
    # per sequence: tokens as in the single-sequence prefill, plus its own state in and out
    nb = prefill_bytes(1, vc.total, vc.H, vc.d) + (vc.N - 1) * 2 * vc.H * 4 * vc.d * vc.d
    fl = prefill_flops(1, vc.total, vc.H, vc.d)
    return dict(workload=w["name"], lengths=lens, bytes=nb, flops=fl,
                tokens_per_s=vc.total / sec, achieved_gbs=nb / sec / 1e9,
                frac_of_hbm_peak=nb / sec / 1e9 / HBM_PEAK_GBS, achieved_tflops=fl / sec / 1e12,
                frac_of_bf16_peak=fl / sec / 1e12 / BF16_PEAK_TFLOPS, workspace_bytes=int(ws_bytes),
                rotating_sets=n_sets, bytes_per_set=int(per_set), **tm)


SNAP_WORKLOAD = dict(name="verify of a 16-token draft through the chunked path: GDA B=32 H=16 d=128 "
                          "T=16, K=17 snapshots (one per token), no final state", B=32, T=16, H=16, d=128,
                     K=17)


def bench_prefill_snapshots(torch, lib, steps, warmup):
    """gdn_prefill_chunked_snapshots on a long draft, with the recurrent
    snapshot kernel timed on the same inputs beside it."""
    import gdn_inputs as gi
    w = SNAP_WORKLOAD
    case = gi.make_case(w["B"], w["T"], w["H"], w["d"], K=w["K"], qkv_dtype="bf16", seed=13, with_accepted=True)
    d = upload_case(torch, case)
    sets = _rotating_sets(torch, d, case)
    acc = torch.from_numpy(case.accepted).to("cuda")
    ws_bytes = lib.gdn_prefill_workspace_size(case.B, case.T, case.H, case.d_k, case.d_v, 64)
    for s in sets:
        s["ws"] = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    vp = lambda t: ctypes.c_void_p(t.data_ptr())

    def chunked(s):
        args = (case.B, case.T, case.H, case.H, 0, case.d_k, case.d_v, 64, case.K, vp(s["q"]),
                vp(s["k"]), vp(s["v"]), vp(s["g"]), vp(s["beta"]), vp(s["state"]), None, vp(s["o"]),
                vp(s["ws"]), ws_bytes)

        def call(stream):
            st = lib.gdn_prefill_chunked_snapshots(*args, stream)
            if st != 0:
                raise RuntimeError(f"libgdn status {st}")
        return call
    def rolled_then_chunked(s):
        rb = (case.B, case.H, case.K, case.d_k, case.d_v, vp(acc), vp(s["state"]), None)
        ch = chunked(s)

        def call(stream):
            st = lib.gdn_rollback_select(*rb, stream)
            if st != 0:
                raise RuntimeError(f"libgdn status {st}")
            ch(stream)
        return call

    def fused(s):
        # the rollback of the previous draft fused into the chunked verification
        args = (case.B, case.T, case.H, case.H, 0, case.d_k, case.d_v, 64, 1, 0, case.K, vp(acc), vp(s["q"]),
                vp(s["k"]), vp(s["v"]), vp(s["g"]), vp(s["beta"]), vp(s["state"]), None, vp(s["o"]),
                vp(s["ws"]), ws_bytes, None)

        def call(stream):
            st = lib.gdn_prefill_chunked_ex_after_rollback(*args, stream)
            if st != 0:
                raise RuntimeError(f"libgdn status {st}")
        return call
    ct = _timing(*run_timed(torch, [chunked(s) for s in sets], steps, warmup), steps)
    bt = _timing(*run_timed(torch, [rolled_then_chunked(s) for s in sets], steps, warmup), steps)
    ft = _timing(*run_timed(torch, [fused(s) for s in sets], steps, warmup), steps)
    rec = [raw_forward_call(lib, case, s, s["state"], s["o"], K=case.K) for s in sets]
    rt = _timing(*run_timed(torch, rec, steps, warmup), steps)
    nb = recurrent_bytes(case.B, case.T, case.H, case.d_k, case.K, False, True)
    tokens = case.B * case.T
    out = dict(workload=w["name"], bytes=nb, rotating_sets=len(sets), workspace_bytes=int(ws_bytes))
    for key, t in (("chunked", ct), ("recurrent", rt)):
        gbs = nb / (t["us_per_launch"] * 1e-6) / 1e9
        out[key] = dict(tokens_per_s=tokens / (t["us_per_launch"] * 1e-6), achieved_gbs=gbs,
                        frac_of_hbm_peak=gbs / HBM_PEAK_GBS, **t)
    # rollback (accepted lengths drawn with the inputs) then the chunked call,
    # as two launches and as gdn_prefill_chunked_ex_after_rollback
    out["rollback_then_chunked"] = dict(tokens_per_s=tokens / (bt["us_per_launch"] * 1e-6), **bt)
    out["rollback_fused_into_chunked"] = dict(tokens_per_s=tokens / (ft["us_per_launch"] * 1e-6), **ft)
    del sets, rec
    torch.cuda.empty_cache()
    return out


def bench_prefill_f32(torch, lib, steps, warmup):
    """The prefill workload with float32 q/k/v (gdn_prefill_chunked_ex; rounded
    to bf16 inside the kernels for the MFMA products)."""
    import gdn_inputs as gi
    case = gi.workload_case(4, qkv_dtype="f32")
    ws_bytes = lib.gdn_prefill_workspace_size_ex(case.B, case.T, case.H, case.d_k, case.d_v, 64, 0, 0)

    def entry(s):
        return lib.gdn_prefill_chunked_ex, (
            case.B, case.T, case.H, case.H, 0, case.d_k, case.d_v, 64, 0, 0, 1, _vp(s["q"]), _vp(s["k"]),
            _vp(s["v"]), _vp(s["g"]), _vp(s["beta"]), _vp(s["state"]), None, _vp(s["o"]), _vp(s["ws"]),
            ws_bytes)
    t, n_sets, per_set = _bench_prefill_leg(torch, lib, case, entry, ws_bytes, steps, warmup)
    B, T, H, dd = case.B, case.T, case.H, case.d_k
    nb = B * T * H * (3 * 4 * dd + 8 + 4 * dd) + 2 * B * H * 4 * dd * dd
    return _prefill_result("prefill GDA B=1 T=8192 H=16 d=128 chunk 64 with float32 q/k/v", case, t, nb,
                           prefill_flops(B, T, H, dd), ws_bytes, n_sets, per_set)


def bench_prefill_kda(torch, lib, steps, warmup):
    """The prefill workload's shape with KDA gates (gdn_prefill_chunked_kda)."""
    import gdn_inputs as gi
    case = gi.workload_case(4, gate="kda")
    ws_bytes = lib.gdn_prefill_kda_workspace_size(case.B, case.T, case.H, case.d_k, case.d_v, 64)

    def entry(s):
        return lib.gdn_prefill_chunked_kda, (
            case.B, case.T, case.H, case.H, 0, case.d_k, case.d_v, 64, _vp(s["q"]), _vp(s["k"]),
            _vp(s["v"]), _vp(s["g"]), _vp(s["beta"]), _vp(s["state"]), _vp(s["o"]), _vp(s["ws"]), ws_bytes)
    t, n_sets, per_set = _bench_prefill_leg(torch, lib, case, entry, ws_bytes, steps, warmup)
    return _prefill_result("prefill KDA B=1 T=8192 H=16 d=128 chunk 64 (the prefill workload with one "
                           "log-gate per key row)", case, t,
                           prefill_kda_bytes(case.B, case.T, case.H, case.d_k),
                           prefill_flops(case.B, case.T, case.H, case.d_k), ws_bytes, n_sets, per_set)


# ----------------------------------------------------------------------------
# CPU baseline: the float64 oracle on the host cores
# ----------------------------------------------------------------------------
def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_runs(fn, tokens_per_call, run_s, runs=3):
    """`runs` runs of `fn`, each repeated for at least `run_s` seconds;
    returns the tokens/s of each run (input generation excluded)."""
    rates = []
    for _ in range(runs):
        reps, t0 = 0, time.perf_counter()
        while True:
            fn()
            reps += 1
            el = time.perf_counter() - t0
            if el >= run_s:
                break
        rates.append(tokens_per_call * reps / el)
    return rates


def cpu_baseline(run_s: float = 3.5):
    """The float64 oracle (plain per-token loop, OpenMP over independent
    (sequence, head) pairs) on the host cores: the decode workload and the
    prefill workload, each the median of 3 runs of >= run_s seconds."""
    import gdn_inputs as gi
    import oracle
    threads = oracle.num_threads()
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    # decode: B=64 H=16 d=128 T=1, 1024 independent (sequence, head) pairs
    case = gi.workload_case(1)
    args = [case.f64(n) for n in ("q", "k", "v", "g", "beta")]
    st = case.f64("state")
    oracle.forward(*args, st)  # load / warm
    dec = _oracle_runs(lambda: oracle.forward(*args, st), case.B * case.T, run_s)
    # prefill: B=1 T=8192 H=16 d=128 from a zero state, 16 (sequence, head) pairs
    pc = gi.workload_case(4)
    pargs = [pc.f64(n) for n in ("q", "k", "v", "g", "beta")]
    pst = pc.f64("state")
    pre = _oracle_runs(lambda: oracle.forward(*pargs, pst), pc.B * pc.T, run_s)
    busy = min(threads, pc.B * pc.H)
    return dict(
        value=float(np.median(dec)), unit="tokens/s", cores=threads, kind="oracle",
        sample=f"full decode workload (B=64 H=16 d=128 T=1), fp64 per-token loop, OpenMP over the "
               f"1024 (sequence, head) pairs; median of 3 runs of >= {run_s:.1f} s",
        runs_tokens_per_s=[round(x, 1) for x in dec],
        nproc=os.cpu_count(), affinity_cpus=affinity, threads=threads, cpu_model=_cpu_model(),
        prefill=dict(
            value=float(np.median(pre)), unit="tokens/s", threads_busy=busy, kind="oracle",
            sample=f"full prefill workload (B=1 T=8192 H=16 d=128, zero initial state), fp64 per-token "
                   f"loop; {busy} threads busy, since the workload has only {pc.B * pc.H} independent "
                   f"(sequence, head) pairs; median of 3 runs of >= {run_s:.1f} s",
            runs_tokens_per_s=[round(x, 1) for x in pre]),
    )


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run 20 device copies of 64 MiB (a plain copy kernel of known "
                         "size, for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--only", choices=["decode", "verify", "prefill", "prefill_kda", "prefill_f32", "broadcast", "varlen",
                             "snapshots", "small", "all"], default="all",
                    help="run one workload only (the JSON line then omits the others)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the GDN path is "
              "benchmarked on a single MI355X", file=sys.stderr)
        sys.exit(2)

    import torch
    from linear_attention_recurrence_net_amd import _binding
    if not os.path.exists(_binding.library_path()):
        from linear_attention_recurrence_net_amd import build
        build.build()
    lib = _binding.library()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    log("device:", torch.cuda.get_device_name(0))

    dec = None
    if args.only in ("decode", "all"):
        log("decode ...")
        dec = bench_decode(torch, lib, args.steps, args.warmup)
        log(f"decode: {dec['us_per_launch']:.2f} us/launch, {dec['achieved_gbs']:.0f} GB/s "
            f"(eager {dec['eager_us_per_launch']:.2f} us)")
        copy_ctx = bench_copy_context(torch, min(args.steps, 100), min(args.warmup, 10))
        log(f"copy context: {copy_ctx['us_per_copy']:.2f} us per 64 MiB copy, {copy_ctx['achieved_gbs']:.0f} GB/s")
    if args.copy_calibration:
        log("copy calibration: 20 x 64 MiB device copies ...")
        src = torch.randn(16 * 1024 * 1024, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(20):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    paths = {}
    if args.only in ("verify", "all"):
        for cfg in (2, 3):
            log(f"verify config {cfg} ...")
            r = bench_verify(torch, lib, cfg, args.steps, args.warmup)
            paths[f"verify_rollback_{'gda' if cfg == 2 else 'kda'}"] = r
            log(f"  verify {r['verify']['us_per_launch']:.2f} us {r['verify']['achieved_gbs']:.0f} GB/s; "
                f"rollback {r['rollback']['us_per_launch']:.2f} us {r['rollback']['achieved_gbs']:.0f} GB/s; "
                f"both {r['verify_plus_rollback']['us_per_launch']:.2f} us, "
                f"fused {r['rollback_fused_into_verify']['us_per_launch']:.2f} us")
    if args.only in ("broadcast", "all"):
        log("decode with shared q/k heads ...")
        paths["decode_qk_broadcast_gda"] = r = bench_decode_broadcast(torch, lib, args.steps, args.warmup)
        log(f"  {r['us_per_launch']:.2f} us/launch, {r['achieved_gbs']:.0f} GB/s")
    if args.only in ("small", "all"):
        log("small batches ...")
        paths["small_batch_gda"] = r = bench_small_batch(torch, lib, args.steps, args.warmup)
        log("  " + ", ".join(f"{k} {v['us_per_launch']:.2f} us" for k, v in r.items() if isinstance(v, dict)))
    if args.only in ("prefill", "all"):
        log("prefill ...")
        steps = args.steps if args.only == "prefill" else max(5, args.steps // 10)
        warm = args.warmup if args.only == "prefill" else max(2, args.warmup // 10)
        paths["prefill_chunked_gda"] = r = bench_prefill(torch, lib, steps, warm)
        log(f"  prefill {r['us_per_launch']:.1f} us, {r['achieved_tflops']:.1f} TFLOP/s, "
            f"{r['achieved_gbs']:.0f} GB/s")
    if args.only in ("prefill_kda", "all"):
        log("prefill KDA ...")
        steps = args.steps if args.only == "prefill_kda" else max(5, args.steps // 10)
        warm = args.warmup if args.only == "prefill_kda" else max(2, args.warmup // 10)
        paths["prefill_chunked_kda"] = r = bench_prefill_kda(torch, lib, steps, warm)
        log(f"  prefill KDA {r['us_per_launch']:.1f} us, {r['achieved_tflops']:.1f} TFLOP/s, "
            f"{r['achieved_gbs']:.0f} GB/s")
    if args.only in ("prefill_f32", "all"):
        log("prefill with float32 q/k/v ...")
        steps = args.steps if args.only == "prefill_f32" else max(5, args.steps // 10)
        warm = args.warmup if args.only == "prefill_f32" else max(2, args.warmup // 10)
        paths["prefill_chunked_f32_inputs"] = r = bench_prefill_f32(torch, lib, steps, warm)
        log(f"  prefill f32 inputs {r['us_per_launch']:.1f} us, {r['achieved_tflops']:.1f} TFLOP/s")
    if args.only in ("varlen", "all"):
        log("varlen prefill ...")
        steps = args.steps if args.only == "varlen" else max(5, args.steps // 10)
        warm = args.warmup if args.only == "varlen" else max(2, args.warmup // 10)
        paths["prefill_chunked_varlen_gda"] = r = bench_prefill_varlen(torch, lib, steps, warm)
        log(f"  varlen prefill {r['us_per_launch']:.1f} us, {r['tokens_per_s'] / 1e6:.1f} M tokens/s, "
            f"{r['achieved_tflops']:.1f} TFLOP/s")
    if args.only in ("snapshots", "all"):
        log("chunked verify with snapshots ...")
        steps = args.steps if args.only == "snapshots" else max(5, args.steps // 4)
        warm = args.warmup if args.only == "snapshots" else max(2, args.warmup // 4)
        paths["prefill_snapshots_draft16_gda"] = r = bench_prefill_snapshots(torch, lib, steps, warm)
        log(f"  chunked {r['chunked']['us_per_launch']:.1f} us ({r['chunked']['achieved_gbs']:.0f} GB/s), "
            f"recurrent {r['recurrent']['us_per_launch']:.1f} us ({r['recurrent']['achieved_gbs']:.0f} GB/s); "
            f"rollback then chunked {r['rollback_then_chunked']['us_per_launch']:.1f} us, "
            f"fused {r['rollback_fused_into_chunked']['us_per_launch']:.1f} us")
    if dec is None:
        print(json.dumps({"partial_run": args.only, "paths": paths}), flush=True)
        return
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline()
        if "prefill_chunked_gda" in paths:  # the prefill path's own baseline, beside it
            paths["prefill_chunked_gda"]["cpu_baseline"] = cpu["prefill"]

    case = dec["case"]
    line = {
        "metric": METRIC,
        "value": dec["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "decode GDA B=64 H=16 d_k=d_v=128 T=1, bf16 q/k/v, fp32 gates/state "
                        "(state 64 MiB in place)",
            "B": case.B, "H": case.H, "d_k": case.d_k, "d_v": case.d_v, "T": case.T,
            "qkv": "bf16", "state": "f32", "rotating_sets": dec["n_sets"],
        },
        "roofline": {
            "bound": "hbm",
            "achieved": dec["achieved_gbs"],
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": dec["achieved_gbs"] / HBM_PEAK_GBS,
            "traffic": decode_traffic_bytes(),
            "kernel": "gdn::recurrent_kernel<d_k=128, d_v=128, GDA, bf16, single token>",
            "bytes_per_launch": dec["bytes"],
            "us_per_launch": dec["us_per_launch"],
            "eager_us_per_launch": dec["eager_us_per_launch"],
            # one event pair per eager launch, 100 launches
            "launch_us_p10_p50_p90": [round(x, 3) for x in dec["spread_us"]],
        },
        "cpu_baseline": cpu,
        "copy_context": copy_ctx,
        "paths": paths,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
