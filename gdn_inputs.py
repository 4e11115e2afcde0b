"""Seeded synthetic inputs for the gated delta net (GDN) recurrence.

This module is shared by the tests, the benchmark and the smoke check.  It
draws random numbers and rounds them to the storage types the kernels read;
it performs none of the recurrence's arithmetic.

Recipe (the workloads of the GDN pages: per head, q and k drawn N(0,1) and
L2-normalised, q scaled by 1/sqrt(d_k), v ~ N(0,1), beta = sigmoid(N(0,1)),
log-gate g = -softplus(N(0,1)) so the decay is exp(g), initial state
S0 ~ N(0, 0.1) read as standard deviation 0.1):

* draws come from ``numpy.random.default_rng(seed)`` in the fixed order
  S0, q, k, v, beta_raw, g_raw, accepted;
* the L2 norm is taken over the key axis, in float64, before the q scale;
* the values are then rounded to float32, and q/k/v further to bfloat16 with
  round-to-nearest-even when the case is a bf16 case;
* g, beta and the state are always float32.

Every consumer receives the rounded values; the float64 oracle receives exact
float64 upcasts of them, so input rounding is not a source of disagreement.

Layouts (row-major, last axis contiguous):
  q, k  [B, T, H, d_k]      v, o  [B, T, H, d_v]
        (q, k [B, T, H_qk, d_k] for a case whose value heads share H_qk q/k heads)
  g     [B, T, H]  (GDA: one log-gate per head and token)
        [B, T, H, d_k]  (KDA: one log-gate per key row)
  beta  [B, T, H]
  state [B, H, K, d_k, d_v]  (slot 0 is the input state)
  accepted [B] int32 in 0..K-1
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "Case",
    "make_case",
    "bf16_round",
    "bf16_bits",
    "bf16_from_bits",
    "WORKLOADS",
    "workload_case",
    "VarlenCase",
    "make_varlen_case",
    "varlen_lengths",
]


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even) and
    return the 16-bit patterns as uint16."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    r = ((u + bias) >> np.uint64(16)).astype(np.uint16)
    return r


def bf16_from_bits(bits: np.ndarray) -> np.ndarray:
    """Exact float32 value of bfloat16 bit patterns."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 value, returned as float32."""
    return bf16_from_bits(bf16_bits(x))


@dataclasses.dataclass
class Case:
    """One seeded input set.

    ``q``, ``k``, ``v`` hold float32 values (already bf16-representable when
    ``qkv_dtype == 'bf16'``); ``*_bits`` give the bf16 patterns for upload.
    """

    B: int
    T: int
    H: int  # value heads (v, g, beta, state, o)
    d_k: int
    d_v: int
    K: int
    gate: str  # "gda" | "kda"
    qkv_dtype: str  # "bf16" | "f32"
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    state: np.ndarray  # [B,H,K,d_k,d_v] float32, slot 0 = S0, other slots 0
    accepted: np.ndarray | None  # [B] int32

    @property
    def H_qk(self) -> int:
        """Heads of q and k (H unless the value heads share q/k heads)."""
        return self.q.shape[2]

    def qkv_bits(self, name: str) -> np.ndarray:
        assert self.qkv_dtype == "bf16"
        return bf16_bits(getattr(self, name))

    def f64(self, name: str) -> np.ndarray:
        """Exact float64 copy of an input (what the oracle consumes)."""
        return np.ascontiguousarray(getattr(self, name), dtype=np.float64)

    @property
    def tokens(self) -> int:
        return self.B * self.T


def _l2n(x: np.ndarray) -> np.ndarray:
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def make_case(
    B: int,
    T: int,
    H: int,
    d_k: int,
    d_v: int | None = None,
    *,
    K: int = 1,
    gate: str = "gda",
    qkv_dtype: str = "bf16",
    seed: int = 0,
    zero_state: bool = False,
    with_accepted: bool = False,
    q_scale: bool = True,
    H_qk: int | None = None,
) -> Case:
    """Draw one seeded case (see the module docstring for the recipe).

    H_qk: number of q/k heads (default H); the value heads then share them.
    """
    if d_v is None:
        d_v = d_k
    if H_qk is None:
        H_qk = H
    if H_qk < 1 or H % H_qk != 0:
        raise ValueError(f"H_qk={H_qk} must divide H={H}")
    if gate not in ("gda", "kda"):
        raise ValueError(gate)
    if qkv_dtype not in ("bf16", "f32"):
        raise ValueError(qkv_dtype)
    rng = np.random.default_rng(seed)
    s0 = rng.normal(0.0, 0.1, size=(B, H, d_k, d_v))
    if zero_state:
        s0 = np.zeros_like(s0)
    q = _l2n(rng.standard_normal((B, T, H_qk, d_k)))
    if q_scale:
        q = q * (1.0 / math.sqrt(d_k))
    k = _l2n(rng.standard_normal((B, T, H_qk, d_k)))
    v = rng.standard_normal((B, T, H, d_v))
    beta_raw = rng.standard_normal((B, T, H))
    gshape = (B, T, H) if gate == "gda" else (B, T, H, d_k)
    g_raw = rng.standard_normal(gshape)
    accepted = None
    if with_accepted:
        accepted = rng.integers(0, K, size=B).astype(np.int32)

    beta = 1.0 / (1.0 + np.exp(-beta_raw))
    g = -np.log1p(np.exp(g_raw))

    def f32(a):
        return np.ascontiguousarray(a, dtype=np.float32)

    q, k, v = f32(q), f32(k), f32(v)
    if qkv_dtype == "bf16":
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    state = np.zeros((B, H, K, d_k, d_v), dtype=np.float32)
    state[:, :, 0] = s0
    return Case(B, T, H, d_k, d_v, K, gate, qkv_dtype, q, k, v, f32(g), f32(beta),
                state, accepted)


# The five synthetic workloads (name and make_case arguments; the seed is the index).
WORKLOADS = {
    0: dict(name="tiny GDA B=1 H=2 d=64 T=16 fp32 K=1",
            B=1, T=16, H=2, d_k=64, K=1, gate="gda", qkv_dtype="f32"),
    1: dict(name="decode GDA B=64 H=16 d=128 T=1",
            B=64, T=1, H=16, d_k=128, K=1, gate="gda", qkv_dtype="bf16"),
    2: dict(name="verify GDA B=32 H=16 d=128 T=4 K=4 + rollback",
            B=32, T=4, H=16, d_k=128, K=4, gate="gda", qkv_dtype="bf16",
            with_accepted=True),
    3: dict(name="verify KDA B=32 H=32 d=64 T=4 K=4 + rollback",
            B=32, T=4, H=32, d_k=64, K=4, gate="kda", qkv_dtype="bf16",
            with_accepted=True),
    4: dict(name="prefill GDA B=1 T=8192 H=16 d=128 chunk 64",
            B=1, T=8192, H=16, d_k=128, K=1, gate="gda", qkv_dtype="bf16",
            zero_state=True),
}


def workload_case(i: int, seed: int | None = None, **override) -> Case:
    """Case for workload ``i`` of WORKLOADS (seed defaults to the workload index)."""
    kw = dict(WORKLOADS[i])
    kw.pop("name")
    kw.update(override)
    return make_case(seed=i if seed is None else seed, **kw)


@dataclasses.dataclass
class VarlenCase:
    """Sequences of different lengths packed along the token axis.  q, k
    [total, H_qk, d]; v [total, H, d]; g [total, H] (GDA) or [total, H, d]
    (KDA); beta [total, H]; state [N, H, d, d] (one initial state per
    sequence); cu_seqlens [N+1]; q/k/v values bf16-representable unless
    qkv_dtype is "f32"."""

    lengths: list
    H: int
    d: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    state: np.ndarray
    cu_seqlens: np.ndarray
    gate: str = "gda"
    qkv_dtype: str = "bf16"

    @property
    def N(self) -> int:
        return len(self.lengths)

    @property
    def total(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def H_qk(self) -> int:
        return self.q.shape[1]

    def sequence(self, i: int) -> Case:
        """Sequence i alone as a B = 1 case (its rows of the packed arrays)."""
        a, b = int(self.cu_seqlens[i]), int(self.cu_seqlens[i + 1])
        st = self.state[i][None, :, None].copy()
        return Case(1, b - a, self.H, self.d, self.d, 1, self.gate, self.qkv_dtype, self.q[None, a:b].copy(),
                    self.k[None, a:b].copy(), self.v[None, a:b].copy(), self.g[None, a:b].copy(),
                    self.beta[None, a:b].copy(), st, None)


def make_varlen_case(lengths, H: int, d: int, *, H_qk: int | None = None, seed: int = 0,
                     gate: str = "gda", qkv_dtype: str = "bf16") -> VarlenCase:
    """Packed sequences with the recipe of make_case: one make_case draw over
    all tokens (B = 1), cut at the sequence boundaries, and N initial states
    drawn after it from the same generator stream."""
    total = int(sum(lengths))
    c = make_case(1, total, H, d, seed=seed, H_qk=H_qk, gate=gate, qkv_dtype=qkv_dtype)
    rng = np.random.default_rng(seed + 1)
    s0 = np.ascontiguousarray(rng.normal(0.0, 0.1, size=(len(lengths), H, d, d)), dtype=np.float32)
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    return VarlenCase(list(lengths), H, d, c.q[0], c.k[0], c.v[0], c.g[0], c.beta[0], s0, cu, gate, qkv_dtype)


def varlen_lengths(total: int, n: int, seed: int = 0, max_len: int | None = None) -> list:
    """n seeded sequence lengths summing to ``total``: a wide mix (log-uniform
    weights) so that short, ragged and multi-chunk sequences all occur."""
    rng = np.random.default_rng(seed)
    w = np.exp(rng.uniform(0.0, np.log(64.0), size=n))
    lens = np.floor(w / w.sum() * total).astype(np.int64)
    lens[int(np.argmax(lens))] += total - int(lens.sum())
    if max_len is not None and lens.max() > max_len:
        raise ValueError("length mix exceeds max_len")
    return [int(x) for x in lens]
