"""Pins for the float64 oracle (CPU only).

The pages print no worked values for the GDN recurrence, so the oracle is
pinned by facts the mathematics fixes, each chosen so that a plausible slip
in the oracle (decay after the update instead of before, a transposed state,
a dropped beta, a readout of the old state, an off-by-one snapshot slot, a
KDA gate applied to columns, a wrong chunk-form term) fails at least one:

* beta = 0 with gate 1 leaves S unchanged (bit-exact) and reads S0^T q;
* gate 1, beta = 1, unit-norm k: after the update S^T k = v;
* basis keys write rows: closed form of one token with k = e_i;
* beta = 0 closed form with decay: S_T = exp(sum g) S0 (row-wise for KDA);
* K = 1 equals the single-slot behaviour; snapshot slot i equals the state
  after the first i tokens; slots above T and slot 0 are not written;
* two-token brute force in the product form
  S_t = (I - beta_t k_t k_t^T) D_t S_{t-1} + beta_t k_t v_t^T;
* KDA with equal row gates equals GDA; a prefix split equals one run;
  outputs are linear in V from a zero state;
* the chunked form equals the sequential form at several lengths and tails,
  for GDA and for KDA (whose chunk form with equal row gates is GDA's);
* rollback copies slot a to slot 0 byte for byte.
"""

import math

import numpy as np
import pytest

import gdn_inputs as gi
import oracle


def _rand_case(B, T, H, d, K=1, gate="gda", seed=0, zero_state=False, d_v=None):
    c = gi.make_case(B, T, H, d, d_v, K=K, gate=gate, qkv_dtype="f32", seed=seed,
                     zero_state=zero_state)
    return (c.f64("q"), c.f64("k"), c.f64("v"), c.f64("g"), c.f64("beta"),
            c.f64("state"))


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


# ---------------------------------------------------------------- invariant 1
@pytest.mark.parametrize("kda", [False, True])
def test_beta0_gate1_leaves_state_unchanged(kda):
    q, k, v, g, beta, st = _rand_case(2, 5, 3, 16, gate="kda" if kda else "gda", seed=11)
    g[:] = 0.0
    beta[:] = 0.0
    o, st_out, fin = oracle.forward(q, k, v, g, beta, st, kda=kda, want_final=True)
    assert np.array_equal(st_out, st)  # bit-exact: 1*S + k*0 == S
    assert np.array_equal(fin, st[:, :, 0])
    S0 = st[:, :, 0]
    for t in range(q.shape[1]):
        ref = np.einsum("bhij,bhi->bhj", S0, q[:, t])
        np.testing.assert_allclose(o[:, t], ref, rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- invariant 2
def test_unit_key_beta1_gate1_stores_value():
    rng = np.random.default_rng(5)
    B, T, H, dk, dv = 2, 7, 2, 8, 5
    k = _unit(rng.standard_normal((B, T, H, dk)))
    q = k.copy()  # read back along the key just written: o_t = S_t^T k_t
    v = rng.standard_normal((B, T, H, dv))
    g = np.zeros((B, T, H))
    beta = np.ones((B, T, H))
    st = np.zeros((B, H, 1, dk, dv))
    st[:, :, 0] = rng.normal(0, 1.0, (B, H, dk, dv))
    o, _, _ = oracle.forward(q, k, v, g, beta, st)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-12)


def test_basis_key_closed_form_and_layout():
    """k = e_i, q = e_r: only row i of S moves, to (1-beta) a S[i,:] + beta v;
    every other row is scaled by a; the readout returns row r.  This fixes the
    state layout (row = key index) and the order decay -> update -> readout."""
    rng = np.random.default_rng(9)
    dk, dv = 6, 4
    S0 = rng.standard_normal((dk, dv))
    for i, r, beta_v, gv in [(2, 2, 0.3, -0.7), (0, 5, 0.9, -0.1), (5, 1, 0.5, -2.0)]:
        k = np.zeros((1, 1, 1, dk)); k[..., i] = 1.0
        q = np.zeros((1, 1, 1, dk)); q[..., r] = 1.0
        v = rng.standard_normal((1, 1, 1, dv))
        st = S0.reshape(1, 1, 1, dk, dv).copy()
        o, st_out, _ = oracle.forward(q, k, v, np.full((1, 1, 1), gv),
                                      np.full((1, 1, 1), beta_v), st)
        a = math.exp(gv)
        ref = a * S0
        ref[i] = (1 - beta_v) * a * S0[i] + beta_v * v[0, 0, 0]
        np.testing.assert_allclose(st_out[0, 0, 0], ref, rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(o[0, 0, 0], ref[r], rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------- closed form
@pytest.mark.parametrize("kda", [False, True])
def test_beta0_decay_closed_form(kda):
    q, k, v, g, beta, st = _rand_case(2, 6, 2, 8, gate="kda" if kda else "gda", seed=21)
    beta[:] = 0.0
    o, st_out, _ = oracle.forward(q, k, v, g, beta, st, kda=kda)
    S0 = st[:, :, 0]
    G = np.cumsum(g, axis=1)  # [B,T,H] or [B,T,H,dk]
    if kda:
        ST = np.exp(G[:, -1])[..., None] * S0
    else:
        ST = np.exp(G[:, -1])[..., None, None] * S0
    np.testing.assert_allclose(st_out[:, :, 0], ST, rtol=1e-13, atol=1e-16)
    for t in range(q.shape[1]):
        if kda:
            St = np.exp(G[:, t])[..., None] * S0
        else:
            St = np.exp(G[:, t])[..., None, None] * S0
        np.testing.assert_allclose(o[:, t], np.einsum("bhij,bhi->bhj", St, q[:, t]),
                                   rtol=1e-12, atol=1e-16)


# ---------------------------------------------------------------- invariant 6
@pytest.mark.parametrize("kda", [False, True])
def test_two_token_brute_force_product_form(kda):
    q, k, v, g, beta, st = _rand_case(2, 2, 3, 8, gate="kda" if kda else "gda", seed=3)
    o, st_out, _ = oracle.forward(q, k, v, g, beta, st, kda=kda)
    B, T, H, dk = q.shape
    for b in range(B):
        for h in range(H):
            S = st[b, h, 0].copy()
            for t in range(T):
                kt = k[b, t, h][:, None]
                D = np.diag(np.exp(g[b, t, h])) if kda else math.exp(g[b, t, h]) * np.eye(dk)
                P = np.eye(dk) - beta[b, t, h] * (kt @ kt.T)
                S = P @ D @ S + beta[b, t, h] * kt @ v[b, t, h][None, :]
                np.testing.assert_allclose(o[b, t, h], S.T @ q[b, t, h], rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(st_out[b, h, 0], S, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("kda", [False, True])
@pytest.mark.parametrize("dk,dv", [(6, 10), (10, 6)])
def test_two_token_brute_force_unequal_head_sizes(kda, dk, dv):
    """The same product form with a d_k x d_v state, d_k != d_v (q, k, the
    gates and the state rows on the key axis; v, o and the columns on the
    value axis)."""
    q, k, v, g, beta, st = _rand_case(2, 2, 3, dk, gate="kda" if kda else "gda", seed=13, d_v=dv)
    assert st.shape[-2:] == (dk, dv) and v.shape[-1] == dv
    o, st_out, _ = oracle.forward(q, k, v, g, beta, st, kda=kda)
    assert o.shape[-1] == dv
    B, T, H, _ = q.shape
    for b in range(B):
        for h in range(H):
            S = st[b, h, 0].copy()
            for t in range(T):
                kt = k[b, t, h][:, None]
                D = np.diag(np.exp(g[b, t, h])) if kda else math.exp(g[b, t, h]) * np.eye(dk)
                P = np.eye(dk) - beta[b, t, h] * (kt @ kt.T)
                S = P @ D @ S + beta[b, t, h] * kt @ v[b, t, h][None, :]
                np.testing.assert_allclose(o[b, t, h], S.T @ q[b, t, h], rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(st_out[b, h, 0], S, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("kda", [False, True])
def test_chunked_equals_sequential_unequal_head_sizes(kda):
    q, k, v, g, beta, st = _rand_case(1, 90, 2, 16, gate="kda" if kda else "gda", seed=29, d_v=24)
    o, s, _ = oracle.forward(q, k, v, g, beta, st, kda=kda)
    oc, sc = oracle.chunked(q, k, v, g, beta, st[:, :, 0], chunk=32, kda=kda)
    assert np.abs(oc - o).max() <= 1e-10 * np.abs(o).max()
    assert np.abs(sc - s[:, :, 0]).max() <= 1e-10 * np.abs(s).max()


# ---------------------------------------------------------------- invariants 3, 4
@pytest.mark.parametrize("kda", [False, True])
def test_k1_is_single_slot_and_snapshots_are_prefix_states(kda):
    gate = "kda" if kda else "gda"
    T, K = 5, 4
    q, k, v, g, beta, st1 = _rand_case(3, T, 2, 8, K=1, gate=gate, seed=7)
    o1, out1, fin1 = oracle.forward(q, k, v, g, beta, st1, kda=kda, want_final=True)
    # K = 1: the state after T tokens lands in slot 0, the same as final_state
    assert np.array_equal(out1[:, :, 0], fin1)
    # K = 4 with sentinel-filled slots 1..3
    stK = np.full(st1.shape[:2] + (K,) + st1.shape[3:], np.nan)
    stK[:, :, 0] = st1[:, :, 0]
    oK, outK, finK = oracle.forward(q, k, v, g, beta, stK, kda=kda, want_final=True)
    assert np.array_equal(oK, o1)
    assert np.array_equal(finK, fin1)
    assert np.array_equal(outK[:, :, 0], st1[:, :, 0])  # slot 0 keeps the input
    for i in range(1, K):
        sl = (slice(None), slice(0, i))
        _, pre, _ = oracle.forward(q[sl], k[sl], v[sl], g[sl], beta[sl], st1, kda=kda)
        assert np.array_equal(outK[:, :, i], pre[:, :, 0]), i


def test_snapshot_slots_above_T_untouched():
    q, k, v, g, beta, st = _rand_case(2, 2, 2, 8, K=1, seed=8)
    K = 5
    stK = np.full((2, 2, K, 8, 8), 7.25)
    stK[:, :, 0] = st[:, :, 0]
    _, out, _ = oracle.forward(q, k, v, g, beta, stK)
    assert np.all(out[:, :, 3:] == 7.25)
    assert not np.any(out[:, :, 1:3] == 7.25)


# ---------------------------------------------------------------- extras
def test_kda_with_equal_row_gates_is_gda():
    q, k, v, g, beta, st = _rand_case(2, 4, 2, 8, seed=13)
    gk = np.repeat(g[..., None], 8, axis=-1)
    o_g, s_g, _ = oracle.forward(q, k, v, g, beta, st)
    o_k, s_k, _ = oracle.forward(q, k, v, gk, beta, st, kda=True)
    assert np.array_equal(o_g, o_k) and np.array_equal(s_g, s_k)


@pytest.mark.parametrize("kda", [False, True])
def test_prefix_split_equals_one_run(kda):
    q, k, v, g, beta, st = _rand_case(2, 9, 2, 8, gate="kda" if kda else "gda", seed=17)
    o, s, _ = oracle.forward(q, k, v, g, beta, st, kda=kda)
    a, b = slice(0, 4), slice(4, 9)
    sl = lambda x, r: x[:, r]
    o1, s1, _ = oracle.forward(sl(q, a), sl(k, a), sl(v, a), sl(g, a), sl(beta, a), st, kda=kda)
    o2, s2, _ = oracle.forward(sl(q, b), sl(k, b), sl(v, b), sl(g, b), sl(beta, b), s1, kda=kda)
    assert np.array_equal(np.concatenate([o1, o2], axis=1), o)
    assert np.array_equal(s2, s)


def test_linear_in_values_from_zero_state():
    q, k, v, g, beta, st = _rand_case(2, 6, 2, 8, seed=19, zero_state=True)
    v2 = np.random.default_rng(1).standard_normal(v.shape)
    oa, sa, _ = oracle.forward(q, k, v, g, beta, st)
    ob, sb, _ = oracle.forward(q, k, v2, g, beta, st)
    oc, sc, _ = oracle.forward(q, k, v + v2, g, beta, st)
    np.testing.assert_allclose(oc, oa + ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(sc, sa + sb, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- invariant 5
@pytest.mark.parametrize("T,C", [(1, 64), (63, 64), (64, 64), (65, 64), (200, 64), (37, 8), (16, 16)])
def test_chunked_equals_sequential(T, C):
    q, k, v, g, beta, st = _rand_case(1, T, 2, 16, seed=T)
    o, s, _ = oracle.forward(q, k, v, g, beta, st)
    oc, sc = oracle.chunked(q, k, v, g, beta, st[:, :, 0], chunk=C)
    scale_o = np.abs(o).max()
    assert np.abs(oc - o).max() <= 1e-10 * scale_o
    assert np.abs(sc - s[:, :, 0]).max() <= 1e-10 * np.abs(s).max()


def test_chunked_equals_sequential_prefill_shape_sample():
    """The prefill workload's shape (d = 128, chunk 64, zero initial state)
    on a shorter sequence with a ragged tail."""
    c = gi.make_case(1, 150, 2, 128, qkv_dtype="bf16", seed=4, zero_state=True)
    args = [c.f64(n) for n in ("q", "k", "v", "g", "beta")]
    o, s, _ = oracle.forward(*args, c.f64("state"))
    oc, sc = oracle.chunked(*args, c.f64("state")[:, :, 0], chunk=64)
    assert np.abs(oc - o).max() <= 1e-10 * np.abs(o).max()
    assert np.abs(sc - s[:, :, 0]).max() <= 1e-10 * np.abs(s).max()


@pytest.mark.parametrize("T,C", [(1, 64), (63, 64), (65, 64), (150, 64), (37, 8), (16, 16)])
def test_chunked_kda_equals_sequential(T, C):
    """KDA chunk form (per-row decays inside A, QKm, the decayed K and Q and
    the state carry) against the KDA token loop."""
    q, k, v, g, beta, st = _rand_case(1, T, 2, 16, gate="kda", seed=40 + T)
    o, s, _ = oracle.forward(q, k, v, g, beta, st, kda=True)
    oc, sc = oracle.chunked(q, k, v, g, beta, st[:, :, 0], chunk=C, kda=True)
    assert np.abs(oc - o).max() <= 1e-10 * np.abs(o).max()
    assert np.abs(sc - s[:, :, 0]).max() <= 1e-10 * np.abs(s).max()


def test_chunked_kda_with_equal_row_gates_is_gda():
    """Every key row decaying by the token's one gate is the GDA chunk form."""
    q, k, v, g, beta, st = _rand_case(2, 100, 2, 16, seed=23)
    gk = np.repeat(g[..., None], 16, axis=-1)
    o1, s1 = oracle.chunked(q, k, v, g, beta, st[:, :, 0])
    o2, s2 = oracle.chunked(q, k, v, gk, beta, st[:, :, 0], kda=True)
    assert np.abs(o2 - o1).max() <= 1e-13 * np.abs(o1).max()
    assert np.abs(s2 - s1).max() <= 1e-13 * np.abs(s1).max()


def test_chunked_kda_prefill_shape_strong_decay():
    """d = 128, chunk 64, a ragged tail, and gates about four times stronger
    than the workload's, so that decays across a chunk reach exp(-200)."""
    c = gi.make_case(1, 130, 2, 128, gate="kda", qkv_dtype="bf16", seed=8)
    args = [c.f64(n) for n in ("q", "k", "v", "g", "beta")]
    args[3] = 4.0 * args[3]
    o, s, _ = oracle.forward(*args, c.f64("state"), kda=True)
    oc, sc = oracle.chunked(*args, c.f64("state")[:, :, 0], chunk=64, kda=True)
    assert np.abs(oc - o).max() <= 1e-10 * np.abs(o).max()
    assert np.abs(sc - s[:, :, 0]).max() <= 1e-10 * np.abs(s).max()


# ---------------------------------------------------------------- rollback
def test_rollback_copies_accepted_slot():
    rng = np.random.default_rng(2)
    B, H, K, d = 6, 3, 4, 4
    st = rng.standard_normal((B, H, K, d, d))
    acc = np.array([0, 1, 2, 3, 3, 0], dtype=np.int32)
    out, n = oracle.rollback(acc, st)
    assert n == 0
    for b in range(B):
        assert np.array_equal(out[b, :, 0], st[b, :, acc[b]])
        assert np.array_equal(out[b, :, 1:], st[b, :, 1:])


def test_rollback_rejects_out_of_range():
    rng = np.random.default_rng(3)
    st = rng.standard_normal((4, 2, 3, 2, 2))
    acc = np.array([-1, 3, 2, 99], dtype=np.int32)
    out, n = oracle.rollback(acc, st)
    assert n == 3
    assert np.array_equal(out[0], st[0]) and np.array_equal(out[1], st[1])
    assert np.array_equal(out[3], st[3])
    assert np.array_equal(out[2, :, 0], st[2, :, 2])


def test_verify_then_rollback_equals_running_accepted_prefix():
    """Speculative verify: run T draft tokens with K slots, roll back to a
    accepted tokens -> slot 0 equals a plain run of the first a tokens."""
    T, K = 4, 4
    c = gi.make_case(5, T, 2, 16, K=K, qkv_dtype="bf16", seed=23, with_accepted=True)
    args = [c.f64(n) for n in ("q", "k", "v", "g", "beta")]
    _, st, _ = oracle.forward(*args, c.f64("state"))
    rolled, n = oracle.rollback(c.accepted, st)
    assert n == 0
    for b in range(c.B):
        a = int(c.accepted[b])
        sl = slice(0, a)
        one = [x[b:b + 1, sl] for x in args]
        _, pre, _ = oracle.forward(*one, c.f64("state")[b:b + 1, :, :1])
        assert np.array_equal(rolled[b, :, 0], pre[0, :, 0])


# --- q/k shared between value heads (head broadcast) --------------------------
# The definition of sharing: the result equals the plain recurrence on q and k
# repeated to H heads -- by numpy's repeat (consecutive value heads share a
# q/k head) or tile (value head h uses q/k head h % H_qk).  The comparison is
# bitwise: the oracle runs the same arithmetic on the same values.


@pytest.mark.parametrize("H,H_qk", [(6, 2), (6, 3), (4, 1)])
@pytest.mark.parametrize("kda", [False, True])
def test_qk_broadcast_equals_materialised_repeat(H, H_qk, kda):
    c = gi.make_case(2, 5, H, 8, K=3, gate="kda" if kda else "gda", qkv_dtype="f32", seed=40 + H_qk,
                     H_qk=H_qk)
    args = dict(kda=kda, want_final=True)
    R = H // H_qk
    for head_map, rep in (("grouped", lambda a: np.repeat(a, R, axis=2)),
                          ("tiled", lambda a: np.tile(a, (1, 1, R, 1)))):
        o, st, fin = oracle.forward(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("g"), c.f64("beta"),
                                    c.f64("state"), head_map=head_map, **args)
        o2, st2, fin2 = oracle.forward(rep(c.f64("q")), rep(c.f64("k")), c.f64("v"), c.f64("g"),
                                       c.f64("beta"), c.f64("state"), **args)
        assert np.array_equal(o, o2) and np.array_equal(st, st2) and np.array_equal(fin, fin2), head_map


def test_grouped_and_tiled_orders_differ():
    # with 2 q/k heads and 4 value heads the two orders pair heads 1 and 2
    # differently, so the outputs of those heads must differ
    c = gi.make_case(1, 4, 4, 8, qkv_dtype="f32", seed=5, H_qk=2)
    a = [c.f64(n) for n in ("q", "k", "v", "g", "beta")]
    og, _, _ = oracle.forward(*a, c.f64("state"), head_map="grouped")
    ot, _, _ = oracle.forward(*a, c.f64("state"), head_map="tiled")
    assert np.array_equal(og[:, :, 0], ot[:, :, 0]) and np.array_equal(og[:, :, 3], ot[:, :, 3])
    assert not np.allclose(og[:, :, 1], ot[:, :, 1]) and not np.allclose(og[:, :, 2], ot[:, :, 2])


def test_qk_broadcast_rejects_non_divisor():
    c = gi.make_case(1, 2, 4, 8, qkv_dtype="f32", seed=1, H_qk=2)
    q3 = np.repeat(c.f64("q"), 3, axis=2)[:, :, :3]  # 3 q/k heads for 4 value heads
    with pytest.raises(RuntimeError):
        oracle.forward(q3, q3, c.f64("v"), c.f64("g"), c.f64("beta"), c.f64("state"))
