"""Seeded sweep of the chunked prefill's configurations against the float64 oracle.

Each case draws a shape and a mode at random (fixed seed, so the list is the
same on every run): batch, tokens (around and across chunk edges), value and
q/k heads with either head map, key and value head sizes 64 or 128 in any
pairing, GDA or KDA gates, bf16 or float32 q/k/v, K state slots (snapshots
within one chunk and across two) with or without a final state, and a zero
or random initial state.  The call goes through gdn_prefill_chunked_ex, the
entry point that every other prefill entry point reaches.  Checked per
output tensor at the prefill bar (max|gpu - ref| / max|ref| <= 1e-2): o,
every written snapshot slot, and the final state (or the in-place state for
K = 1); slots the call must not write keep their NaN sentinel bit for bit,
and so does slot 0 when K > 1.
"""

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
from helpers import bits, ensure_built, oracle_args, rel_err, upload

pytestmark = pytest.mark.gpu

TOL = 1e-2


def _cases(n=32, seed=20261):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        hq = int(rng.choice([1, 2, 3]))
        group = int(rng.choice([1, 2, 4]))
        out.append(dict(
            B=int(rng.integers(1, 4)),
            T=int(rng.choice([1, 17, 63, 64, 65, 100, 130, 200])),
            H=hq * group,
            Hq=hq,
            dk=int(rng.choice([64, 128])),
            dv=int(rng.choice([64, 128])),
            K=int(rng.choice([1, 1, 2, 5, 17, 70])),
            gate=str(rng.choice(["gda", "kda"])),
            dt=str(rng.choice(["bf16", "f32"])),
            head_map=str(rng.choice(["grouped", "tiled"])),
            final=bool(rng.integers(0, 2)),
            zero=bool(rng.integers(0, 2)),
            seed=5000 + i,
        ))
    return out


CASES = _cases()


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()
    import linear_attention_recurrence_net_amd as gdn
    gdn.library()
    assert torch.cuda.is_available()


@pytest.mark.parametrize("cfg", CASES, ids=[
    "B{B}T{T}H{H}q{Hq}k{dk}v{dv}K{K}-{gate}-{dt}-{head_map}-{f}-{z}".format(
        f="fin" if c["final"] else "nofin", z="s0" if c["zero"] else "rand", **c)
    for c in CASES])
def test_prefill_sweep(cfg):
    import linear_attention_recurrence_net_amd as gdn
    B, T, H, Hq, dk, dv, K = (cfg[n] for n in ("B", "T", "H", "Hq", "dk", "dv", "K"))
    c = gi.make_case(B, T, H, dk, dv, K=K, gate=cfg["gate"], qkv_dtype=cfg["dt"], seed=cfg["seed"], H_qk=Hq,
                     zero_state=cfg["zero"])
    if K > 1:
        c.state[:, :, 1:] = np.float32(np.nan)
    u = upload(c)
    st = u["state"] if K > 1 else u["state"][:, :, 0].contiguous()
    fin = torch.full((B, H, dk, dv), float("nan"), device="cuda") if cfg["final"] and K > 1 else None
    o = gdn.gdn_prefill_chunked_ex(u["q"], u["k"], u["v"], u["g"], u["beta"], st, head_map=cfg["head_map"],
                                   final_state=fin)
    torch.cuda.synchronize()
    ro, rst, rfin = oracle.forward(*oracle_args(c), c.f64("state"), kda=cfg["gate"] == "kda",
                                   want_final=True, head_map=cfg["head_map"])
    errs = {"o": rel_err(o, ro, "o")}
    if K == 1:
        errs["state"] = rel_err(st, rst[:, :, 0], "state")
    else:
        n_snap = min(T, K - 1)
        for s in range(1, n_snap + 1):
            errs[f"slot{s}"] = rel_err(st[:, :, s], rst[:, :, s], f"slot{s}")
        got = bits(st)
        want = c.state.view(np.int32)
        # slot 0 keeps the input and slots past the tokens keep their sentinel
        assert np.array_equal(got[:, :, 0], want[:, :, 0])
        assert np.array_equal(got[:, :, n_snap + 1:], want[:, :, n_snap + 1:])
    if fin is not None:
        errs["final"] = rel_err(fin, rfin, "final")
    worst = max(errs, key=errs.get)
    print(cfg, f"worst {worst} {errs[worst]:.2e}", flush=True)
    for name, e in errs.items():
        assert e <= TOL, (name, e)
