"""float64 CPU oracle for the gated delta net recurrence -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its Python
binding) never imports, links or calls it, and it shares no code with them.

The arithmetic lives in ``gdn_oracle.c`` (plain loops, float64, see its
header for the definition and the passages it follows); this module only
compiles it with gcc when needed and marshals numpy arrays through ctypes.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")

GCC_CMD = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
           "-o", _LIB, _SRC, "-lm"]

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle (gcc -O2, no fast-math) unless already built."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        subprocess.run(GCC_CMD, check=True)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int32)
        i = ctypes.c_int
        lib.oracle_gdn_forward.argtypes = [i, i, i, i, i, i, i, i, i, dp, dp, dp, dp, dp, dp, dp, dp]
        lib.oracle_gdn_forward.restype = i
        lib.oracle_gdn_rollback.argtypes = [i, i, i, i, i, ip, dp]
        lib.oracle_gdn_rollback.restype = i
        lib.oracle_gdn_chunked.argtypes = [i, i, i, i, i, i, i, dp, dp, dp, dp, dp, dp, dp]
        lib.oracle_gdn_chunked.restype = i
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = i
        _lib = lib
    return _lib


def _d(a: np.ndarray, shape=None) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float64)
    if shape is not None and a.shape != tuple(shape):
        raise ValueError(f"shape {a.shape} != {tuple(shape)}")
    return a


def _p(a: np.ndarray | None):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def num_threads() -> int:
    return _load().oracle_num_threads()


def forward(q, k, v, g, beta, state, *, kda: bool = False, want_final: bool = False,
            head_map: str = "grouped"):
    """Sequential recurrence.  ``state`` is [B,H,K,dk,dv] (slot 0 = input).

    q and k may have fewer heads (H_qk, a divisor of v's H) than v; value
    head h then reads q/k head h // (H // H_qk) (head_map 'grouped') or
    h % H_qk ('tiled').
    Returns ``(o, state_out, final_state_or_None)``; the input arrays are
    not modified.
    """
    q = _d(q)
    B, T, Hq, dk = q.shape
    v = _d(v)
    H, dv = v.shape[2], v.shape[3]
    st = np.array(state, dtype=np.float64, copy=True, order="C")
    K = st.shape[2]
    if st.shape != (B, H, K, dk, dv):
        raise ValueError(f"state shape {st.shape}")
    if head_map not in ("grouped", "tiled"):
        raise ValueError(head_map)
    k = _d(k, (B, T, Hq, dk))
    v = _d(v, (B, T, H, dv))
    g = _d(g, (B, T, H, dk) if kda else (B, T, H))
    beta = _d(beta, (B, T, H))
    o = np.zeros((B, T, H, dv), dtype=np.float64)
    fin = np.zeros((B, H, dk, dv), dtype=np.float64) if want_final else None
    rc = _load().oracle_gdn_forward(B, T, H, Hq, int(head_map == "tiled"), dk, dv, K, int(kda),
                                    _p(q), _p(k), _p(v), _p(g), _p(beta), _p(st), _p(fin), _p(o))
    if rc != 0:
        raise RuntimeError("oracle_gdn_forward failed")
    return o, st, fin


def rollback(accepted, state):
    """Returns ``(state_out, n_invalid)``; the input is not modified."""
    st = np.array(state, dtype=np.float64, copy=True, order="C")
    B, H, K, dk, dv = st.shape
    acc = np.ascontiguousarray(accepted, dtype=np.int32)
    if acc.shape != (B,):
        raise ValueError("accepted must be [B]")
    n = _load().oracle_gdn_rollback(B, H, K, dk, dv,
                                   acc.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), _p(st))
    return st, n


def chunked(q, k, v, g, beta, state, *, chunk: int = 64, kda: bool = False):
    """Chunked (WY/UT) form, GDA or KDA.  ``state`` is [B,H,dk,dv].

    Returns ``(o, state_out)``.
    """
    q = _d(q)
    B, T, H, dk = q.shape
    st = np.array(state, dtype=np.float64, copy=True, order="C")
    dv = st.shape[3]
    if st.shape != (B, H, dk, dv):
        raise ValueError(f"state shape {st.shape}")
    k = _d(k, (B, T, H, dk))
    v = _d(v, (B, T, H, dv))
    g = _d(g, (B, T, H, dk) if kda else (B, T, H))
    beta = _d(beta, (B, T, H))
    o = np.zeros((B, T, H, dv), dtype=np.float64)
    rc = _load().oracle_gdn_chunked(B, T, H, dk, dv, chunk, int(kda), _p(q), _p(k), _p(v), _p(g),
                                    _p(beta), _p(st), _p(o))
    if rc != 0:
        raise RuntimeError("oracle_gdn_chunked failed")
    return o, st
