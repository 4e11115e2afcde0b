"""A speculative-decoding loop of several rounds against the float64 oracle.

Each round verifies a new draft with the previous round's rollback fused in
(accepted lengths drawn per round, an invalid one among them in one round),
on the state the previous round left, as an engine would (koboldcpp commit
log, tag v1.113.1, bullets "metal: add GDN partial rollback" and "llama:
allow partial seq_rm for GDN models for speculative decoding").  The oracle
runs the same rounds as its rollback followed by its token loop.  Checked
every round: o and every written slot, at 2e-4 through the token kernel
(gdn_forward_snapshots_after_rollback, the oracle carrying its own state over
all rounds) and at the prefill bar 1e-2 through the chunked path
(gdn_prefill_chunked_ex_after_rollback, drafts longer than a chunk; each
round from the state the GPU holds, since its bf16 products set the bar);
and the error flag of the round with the invalid length.
"""

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
from helpers import ensure_built, oracle_args, rel_err, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()
    assert torch.cuda.is_available()


@pytest.mark.parametrize("path,B,T,H,d,K,gate,tol", [
    ("token", 6, 4, 4, 128, 5, "gda", 2e-4),
    ("token", 5, 3, 8, 64, 4, "kda", 2e-4),
    ("chunked", 3, 70, 2, 64, 71, "kda", 1e-2),
    ("chunked", 2, 100, 2, 128, 9, "gda", 1e-2),
])
def test_speculative_rounds_match_oracle(path, B, T, H, d, K, gate, tol):
    import linear_attention_recurrence_net_amd as gdn
    rounds = 4
    rng = np.random.default_rng(4000 + T + d)
    c0 = gi.make_case(B, T, H, d, K=K, gate=gate, qkv_dtype="bf16", seed=4100 + T)
    state = upload(c0)["state"]                # slot 0: the prompt's state
    ref = c0.f64("state")
    acc = np.zeros(B, dtype=np.int32)          # nothing to roll back before the first round
    for r in range(rounds):
        c = gi.make_case(B, T, H, d, K=K, gate=gate, qkv_dtype="bf16", seed=4200 + 10 * r + T)
        u = upload(c)
        acc_t = torch.from_numpy(acc).cuda()
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        if path == "chunked":
            # bf16 products: each round is checked from the state the GPU holds
            ref = state.double().cpu().numpy()
        if path == "token":
            o = gdn.gdn_forward_snapshots_after_rollback(acc_t, u["q"], u["k"], u["v"], u["g"], u["beta"], state,
                                                         err_flag=err)
        else:
            o = gdn.gdn_prefill_chunked_ex_after_rollback(acc_t, u["q"], u["k"], u["v"], u["g"], u["beta"], state,
                                                          err_flag=err)
        torch.cuda.synchronize()
        rolled, n_bad = oracle.rollback(acc, ref)
        ro, rst, _ = oracle.forward(*oracle_args(c), rolled, kda=gate == "kda", want_final=True)
        errs = {"o": rel_err(o, ro, "o")}
        for s in range(min(T, K - 1) + 1):
            errs[f"slot{s}"] = rel_err(state[:, :, s], rst[:, :, s], f"slot{s}")
        worst = max(errs, key=errs.get)
        print(path, "round", r, f"o {errs['o']:.1e}, worst {worst} {errs[worst]:.1e}", flush=True)
        for name, e in errs.items():
            assert e <= tol, (r, name, e)
        assert int(err.item()) == (1 if n_bad else 0), r
        ref = rst
        # the next accepted lengths; those verified in the third speculative round include an invalid one
        acc = rng.integers(0, min(T, K - 1) + 1, size=B).astype(np.int32)
        if r == 1:
            acc[-1] = K + 3
