"""Chunked prefill of one sequence at the largest length the boundary takes
(T * H * d * 4 bytes just under 2^31), checked through state resets.

A log-gate of -200 at a token scales the carried state by exp(-200), which
is zero in float32 and below 1e-86 in float64: the recurrence restarts
there from the zero state.  The sequence here is one seeded segment of
P = 4096 tokens (a whole number of chunks) repeated, with that gate on the
first token of every repeat but the first, and cut at the length limit, so
that it ends with a tail of P - 1 tokens.  So:

* the first segment starts from the input state S0;
* every later segment, the tail included, starts from zero;
* on the chunked path every later full segment goes through the same
  arithmetic as the second (the carried state enters its products only
  through factors exp(G) that are exactly zero), so its outputs equal the
  second segment's value for value.

The float64 oracle runs three short sequences: the segment from S0, the
reset segment from zero, and the tail from zero.  The GPU's first and
second segments, its tail and its final state must match them within the
prefill bar (1e-2), and every other segment must equal the second.  This
covers the kernels' 32-bit row offsets and buffer ranges up to their limit,
for GDA gates and for KDA gates.
"""

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
from helpers import ensure_built, rel_err

pytestmark = pytest.mark.gpu

TOL = 1e-2
RESET = -200.0


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()
    assert torch.cuda.is_available()


def _tile(x: np.ndarray, T: int, dtype=None) -> torch.Tensor:
    """[1, P, ...] -> [1, T, ...] on the GPU, repeating along the token axis."""
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)  # exact for the bf16 cases: the values are bf16-representable
    t = t.to("cuda")
    reps = -(-T // t.shape[1])
    return t.repeat(1, reps, *([1] * (t.dim() - 2)))[:, :T].contiguous()


@pytest.mark.parametrize("gate", ["gda", "kda"])
def test_prefill_longest_sequence_through_resets(gate):
    import linear_attention_recurrence_net_amd as gdn

    H, d, P = 2, 128, 4096
    T = (1 << 31) // (H * d * 4) - 1  # the longest sequence the entry point takes
    nfull, tail = divmod(T, P)        # 511 whole segments and a tail of P - 1 tokens
    assert tail == P - 1 and nfull > 2
    kda = gate == "kda"
    seg = gi.make_case(1, P, H, d, gate=gate, qkv_dtype="bf16", seed=4242 + kda)
    g_reset = seg.g.copy()
    g_reset[:, 0] = RESET

    # the oracle: the segment from S0, the reset segment from zero, the tail from zero
    f64 = lambda a: np.ascontiguousarray(a, dtype=np.float64)
    qkv = [seg.f64(n) for n in ("q", "k", "v")]
    zero = np.zeros_like(seg.f64("state"))
    ro0, _, _ = oracle.forward(*qkv, seg.f64("g"), seg.f64("beta"), seg.f64("state"), kda=kda)
    ro1, _, _ = oracle.forward(*qkv, f64(g_reset), seg.f64("beta"), zero, kda=kda)
    _, rst, _ = oracle.forward(*[a[:, :tail] for a in qkv], f64(g_reset)[:, :tail],
                               seg.f64("beta")[:, :tail], zero, kda=kda)

    q = _tile(seg.q, T, torch.bfloat16)
    k = _tile(seg.k, T, torch.bfloat16)
    v = _tile(seg.v, T, torch.bfloat16)
    g = _tile(g_reset, T)
    g[:, 0] = torch.from_numpy(np.ascontiguousarray(seg.g[:, 0])).to("cuda")  # no reset before S0
    beta = _tile(seg.beta, T)
    s = torch.from_numpy(np.ascontiguousarray(seg.state[:, :, 0])).to("cuda")
    print(f"{gate} T={T} H={H} d={d}: {nfull} segments of {P} tokens and a tail of {tail}", flush=True)
    o = gdn.gdn_prefill_chunked_ex(q, k, v, g, beta, s)
    torch.cuda.synchronize()
    del q, k, v, g, beta

    e0 = rel_err(o[:, :P], ro0, "first segment o")
    e1 = rel_err(o[:, P:2 * P], ro1, "second segment o")
    et = rel_err(o[:, nfull * P:], ro1[:, :tail], "tail o")
    es = rel_err(s, rst[:, :, 0], "final state")
    print(f"o: first {e0:.3e} second {e1:.3e} tail {et:.3e}; final state {es:.3e}", flush=True)
    assert max(e0, e1, et, es) <= TOL, (e0, e1, et, es)
    later = o[:, 2 * P:nfull * P].view(nfull - 2, P, H, d)
    same = (later == o[:, P:2 * P]).view(nfull - 2, -1).all(dim=1)
    bad = torch.nonzero(~same).flatten().tolist()
    assert not bad, f"segments differing from the second: {[2 + i for i in bad][:8]}"
    del o, later, same
    torch.cuda.empty_cache()
