"""Concurrent calls on separate streams and host threads, and an aliased
output refused through the binding.

The library keeps no state between calls apart from a per-device compute-unit
count (and the allocation-free prefill's fixed scratch array, which is not
used here), so independent problems launched at the same time on different
HIP streams, from different host threads, must give the bits of the same
calls made one after another: a decode, a verification with the previous
draft's rollback fused in, a KDA chunked prefill, and a variable-length
prefill, each run three times concurrently with the others.
"""

import threading

import numpy as np
import pytest
import torch

import gdn_inputs as gi
from helpers import bits, ensure_built, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()
    assert torch.cuda.is_available()


def _problems():
    """Functions that each run one problem on the current stream and return
    its output tensors."""
    import linear_attention_recurrence_net_amd as gdn
    probs = []

    c = gi.make_case(8, 1, 16, 128, K=1, gate="gda", qkv_dtype="bf16", seed=3001)
    u = upload(c)
    st0 = u["state"][:, :, 0].contiguous()

    def decode(u=u, st0=st0):
        st = st0.clone()
        o = gdn.gdn_forward(u["q"], u["k"], u["v"], u["g"], u["beta"], st)
        return [o, st]
    probs.append(decode)

    c = gi.make_case(16, 4, 32, 64, K=4, gate="kda", qkv_dtype="bf16", seed=3002)
    c.state[:, :, 1:] = np.random.default_rng(3003).standard_normal(c.state[:, :, 1:].shape).astype(np.float32) * 0.1
    u2 = upload(c)
    acc = torch.from_numpy(np.random.default_rng(3004).integers(0, 5, size=16).astype(np.int32)).cuda()

    def verify(u=u2, acc=acc):
        st = u["state"].clone()
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        o = gdn.gdn_forward_snapshots_after_rollback(acc, u["q"], u["k"], u["v"], u["g"], u["beta"], st, err_flag=err)
        return [o, st, err]
    probs.append(verify)

    c = gi.make_case(1, 700, 4, 128, K=1, gate="kda", qkv_dtype="f32", seed=3005)
    u3 = upload(c)
    st3 = u3["state"][:, :, 0].contiguous()

    def prefill(u=u3, st0=st3):
        st = st0.clone()
        o = gdn.gdn_prefill_chunked_ex(u["q"], u["k"], u["v"], u["g"], u["beta"], st)
        return [o, st]
    probs.append(prefill)

    lens = [130, 0, 64, 257, 1]
    c = gi.make_case(1, sum(lens), 4, 64, K=1, gate="gda", qkv_dtype="bf16", seed=3006)
    u4 = upload(c)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), device="cuda")
    st4 = torch.from_numpy(np.random.default_rng(3007).standard_normal((len(lens), 4, 64, 64)).astype(np.float32)).cuda()

    def varlen(u=u4, cu=cu, st0=st4):
        st = st0.clone()
        o = gdn.gdn_prefill_chunked_varlen(cu, u["q"][0], u["k"][0], u["v"][0], u["g"][0], u["beta"][0], st)
        return [o, st]
    probs.append(varlen)
    return probs


def test_concurrent_streams_and_threads_match_sequential():
    probs = _problems()
    # one after another on the default stream
    ref = []
    for p in probs:
        ref.append([bits(x) for x in p()])
        torch.cuda.synchronize()

    results = {}
    errors = []
    streams = [torch.cuda.Stream() for _ in probs]

    def worker(i):
        try:
            outs = []
            with torch.cuda.stream(streams[i]):
                for _ in range(3):
                    outs.append(probs[i]())
            streams[i].synchronize()
            results[i] = [[bits(x) for x in o] for o in outs]
        except Exception as e:  # reported below, with the problem's index
            errors.append((i, repr(e)))

    torch.cuda.synchronize()
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(probs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    torch.cuda.synchronize()
    assert not errors, errors
    for i, r in enumerate(ref):
        assert i in results, i
        for rep, outs in enumerate(results[i]):
            for j, (a, b) in enumerate(zip(outs, r)):
                assert np.array_equal(a, b), (i, rep, j)


def test_overlapping_output_raises_before_any_launch():
    """A final state that is a view of the state's own memory is refused with
    GDN_ERR_ALIAS (raised as GdnError) and nothing is written."""
    import linear_attention_recurrence_net_amd as gdn
    c = gi.make_case(2, 3, 2, 64, K=4, gate="gda", qkv_dtype="bf16", seed=3010)
    u = upload(c)
    st = u["state"]
    before = bits(st)
    fin = st.view(-1)[: 2 * 2 * 64 * 64].view(2, 2, 64, 64)  # slot 0 of the first heads
    with pytest.raises(gdn.GdnError, match="overlaps"):
        gdn.gdn_forward_snapshots(u["q"], u["k"], u["v"], u["g"], u["beta"], st, fin)
    torch.cuda.synchronize()
    assert np.array_equal(bits(st), before)
