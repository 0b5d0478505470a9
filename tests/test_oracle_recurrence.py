"""Pins of the oracle's forward recurrence against closed forms, an independent matrix
statement of the update, and exact structural invariants.

The update (gated delta rule; GDN scalar gate, KDA per key channel gate), as stated for
the linear-attention state-QAT work, in value-by-key orientation:
    S_t = S_{t-1} diag(a_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t.
The oracle stores the transpose (key rows, value columns) and evaluates it step by step
through u = S~^T k and delta = beta (v - u); the matrix statement below is a different
evaluation of the same map.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _rand_inputs(rng, B, T, H, dk, dv, gate="scalar", s0=0.3):
    q = rng.standard_normal((B, T, H, dk)) / math.sqrt(dk)
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    gs = (B, T, H, dk) if gate == "key" else (B, T, H)
    g = -np.log1p(np.exp(rng.standard_normal(gs)))
    beta = 1 / (1 + np.exp(-rng.standard_normal((B, T, H))))
    S0 = rng.standard_normal((B, H, dk, dv)) * s0
    return q, k, v, g, beta, S0


def _matrix_form(q, k, v, g, beta, S0, gate):
    """Value-by-key matrix statement of the recurrence (no quantization)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    ST = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            M = S0[b, h].T.copy()  # dv x dk
            for t in range(T):
                a = np.exp(g[b, t, h]) * np.ones(dk) if gate == "scalar" else np.exp(g[b, t, h])
                kk = k[b, t, h]
                M = M @ np.diag(a) @ (np.eye(dk) - beta[b, t, h] * np.outer(kk, kk)) + \
                    beta[b, t, h] * np.outer(v[b, t, h], kk)
                o[b, t, h] = M @ q[b, t, h]
            ST[b, h] = M.T
    return o, ST


@pytest.mark.parametrize("gate", ["scalar", "key"])
def test_matches_matrix_form(oracle_mod, gate):
    rng = np.random.default_rng(1 if gate == "scalar" else 2)
    q, k, v, g, beta, S0 = _rand_inputs(rng, 2, 7, 3, 8, 6, gate)
    o, ST, _ = oracle.fwd(q, k, v, g, beta, S0, gate=oracle.GATE_KEY if gate == "key" else 0)
    o2, ST2 = _matrix_form(q, k, v, g, beta, S0, gate)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ST, ST2, rtol=0, atol=1e-12)


def test_two_token_hand_algebra_exact(oracle_mod):
    """S_0 = 0, GDN, no QDQ, worked by hand:
    S_1 = b1 k1 v1^T; o_1 = b1 (k1.q1) v1;
    delta_2 = b2 (v2 - a2 b1 (k1.k2) v1); o_2 = a2 b1 (k1.q2) v1 + (k2.q2) delta_2.
    Inputs are dyadic so float64 evaluation is exact and matches rational arithmetic."""
    F = Fraction
    dk, dv = 4, 3
    k1 = [F(1, 2), F(-1, 2), F(1, 2), F(1, 2)]
    k2 = [F(1, 2), F(1, 2), F(1, 2), F(-1, 2)]
    q1 = [F(1, 4), F(0), F(-3, 4), F(1, 2)]
    q2 = [F(-1, 2), F(1, 4), F(1, 8), F(1)]
    v1 = [F(1), F(-2), F(3, 4)]
    v2 = [F(-1, 2), F(5, 4), F(2)]
    b1, b2, a2 = F(3, 4), F(1, 2), F(1, 2)
    dot = lambda x, y: sum(i * j for i, j in zip(x, y))
    o1 = [b1 * dot(k1, q1) * x for x in v1]
    d2 = [b2 * (y - a2 * b1 * dot(k1, k2) * x) for x, y in zip(v1, v2)]
    o2 = [a2 * b1 * dot(k1, q2) * x + dot(k2, q2) * d for x, d in zip(v1, d2)]
    S2 = [[a2 * b1 * k1[i] * v1[j] + k2[i] * d2[j] for j in range(dv)] for i in range(dk)]
    arr = lambda L: np.array([[float(x) for x in L]])
    q = np.stack([arr(q1), arr(q2)])[None]   # [1, 2, 1, dk]
    k = np.stack([arr(k1), arr(k2)])[None]
    v = np.stack([arr(v1), arr(v2)])[None]
    g = np.array([[[0.0], [math.log(0.5)]]])
    beta = np.array([[[0.75], [0.5]]])
    o, ST, _ = oracle.fwd(q, k, v, g, beta, None)
    np.testing.assert_allclose(o[0, 0, 0], [float(x) for x in o1], rtol=0, atol=1e-15)
    np.testing.assert_allclose(o[0, 1, 0], [float(x) for x in o2], rtol=0, atol=1e-15)
    np.testing.assert_allclose(ST[0, 0], [[float(x) for x in r] for r in S2], rtol=0, atol=1e-15)


@pytest.mark.parametrize("mode,group,had", [(oracle.QDQ_NONE, 32, False), (oracle.QDQ_INT8, 32, False),
                                            (oracle.QDQ_E4M3, 64, False), (oracle.QDQ_INT8, 32, True)])
def test_noop_step_keeps_state(oracle_mod, mode, group, had):
    """beta = 0, g = 0: S' = S_{t-1} exactly and o_t = S_{t-1}^T q_t.  With QDQ on, S_0 is
    chosen exactly representable (so Q(S_0) = S_0)."""
    rng = np.random.default_rng(3)
    B, T, H, dk, dv = 1, 5, 2, 64, 64
    q, k, v, g, beta, _ = _rand_inputs(rng, B, T, H, dk, dv)
    g[:] = 0.0
    beta[:] = 0.0
    codes = rng.integers(-127, 128, size=(B, H, dk, dv))
    if mode == oracle.QDQ_E4M3:
        S0 = np.zeros((B, H, dk, dv))
        for b in range(B):
            for h in range(H):
                c = rng.integers(0, 126, size=(dk, dv))
                S0[b, h] = np.vectorize(oracle.e4m3_value)(c) * 2.0 ** -7
                S0[b, h, 0, 0] = S0[b, h, 0, 63] = 448 * 2.0 ** -7
    elif mode == oracle.QDQ_INT8 and had:
        codes[..., ::group] = 127
        Hn = np.array([[(-1) ** bin(i & j).count("1") for j in range(dk)] for i in range(dk)]) / 8.0
        S0 = np.einsum("ij,bhjk->bhik", Hn, codes * 2.0 ** -8).astype(np.float32).astype(np.float64)
    else:
        codes[..., ::group] = 127
        S0 = codes * 2.0 ** -8
    o, ST, _ = oracle.fwd(q, k, v, g, beta, S0, qdq_mode=mode, group=group, hadamard=had)
    expect_o = np.einsum("bhij,bthi->bthj", S0, q)
    np.testing.assert_allclose(o, expect_o, rtol=0, atol=1e-14)
    tol = 8 * 2.0 ** -24 * np.abs(S0).max() if had else 0.0
    np.testing.assert_allclose(ST, S0, rtol=0, atol=tol)


def test_unit_key_overwrites(oracle_mod):
    """beta = 1, g = 0, k = e_i: row i of S' becomes v (to one rounding of s + (v - s)), other
    rows are unchanged bit for bit; and for any unit-norm k, k^T S' = v^T."""
    rng = np.random.default_rng(4)
    dk, dv = 16, 8
    S0 = rng.standard_normal((1, 1, dk, dv))
    v = rng.standard_normal((1, 1, 1, dv))
    q = rng.standard_normal((1, 1, 1, dk))
    g = np.zeros((1, 1, 1))
    beta = np.ones((1, 1, 1))
    k = np.zeros((1, 1, 1, dk))
    k[..., 5] = 1.0
    _, ST, _ = oracle.fwd(q, k, v, g, beta, S0)
    exp = S0[0, 0].copy()
    exp[5] = v[0, 0, 0]
    np.testing.assert_array_equal(np.delete(ST[0, 0], 5, 0), np.delete(exp, 5, 0))
    np.testing.assert_allclose(ST[0, 0, 5], exp[5], rtol=2.0 ** -52, atol=2.0 ** -52 * 4)
    k = rng.standard_normal((1, 1, 1, dk))
    k /= np.linalg.norm(k)
    _, ST, _ = oracle.fwd(q, k, v, g, beta, S0)
    np.testing.assert_allclose(k[0, 0, 0] @ ST[0, 0], v[0, 0, 0], rtol=0, atol=1e-14)


QCASES = [(oracle.QDQ_INT8, 32, False, 1), (oracle.QDQ_INT8, 16, False, 1),
          (oracle.QDQ_INT8, 64, False, 1), (oracle.QDQ_E4M3, 64, False, 64),
          (oracle.QDQ_E4M3, 64, False, 1), (oracle.QDQ_INT8, 32, True, 1),
          (oracle.QDQ_INT8, 32, False, 16)]


@pytest.mark.parametrize("mode,group,had,interval", QCASES)
@pytest.mark.parametrize("gate", ["scalar", "key"])
def test_power_of_two_and_sign_equivariance(oracle_mod, mode, group, had, interval, gate):
    """The recurrence is jointly linear in (S_0, v) and every quantizer commutes with 2^m
    scaling and with negation, so (2^m v, 2^m S_0) gives exactly 2^m o and 2^m S."""
    rng = np.random.default_rng(10 + mode + group)
    q, k, v, g, beta, S0 = _rand_inputs(rng, 1, 70, 2, 64, 64, gate)
    kw = dict(gate=1 if gate == "key" else 0, qdq_mode=mode, group=group, hadamard=had,
              qdq_interval=interval)
    o, ST, _ = oracle.fwd(q, k, v, g, beta, S0, **kw)
    o2, ST2, _ = oracle.fwd(q, k, v * 2.0 ** 5, g, beta, S0 * 2.0 ** 5, **kw)
    np.testing.assert_array_equal(o2, o * 2.0 ** 5)
    np.testing.assert_array_equal(ST2, ST * 2.0 ** 5)
    o3, ST3, _ = oracle.fwd(q, k, -v, g, beta, -S0, **kw)
    np.testing.assert_array_equal(o3, -o)
    np.testing.assert_array_equal(ST3, -ST)


@pytest.mark.parametrize("mode,group,had,interval", QCASES)
def test_structure_batch_split_checkpoints(oracle_mod, mode, group, had, interval):
    """Units are independent; a call split at a quantization point resumes exactly;
    checkpoint c equals the state after c * n tokens; interval-1 QDQ equals chained
    single-token calls."""
    rng = np.random.default_rng(20 + mode)
    B, T, H, dk, dv = 2, 128, 3, 64, 64
    q, k, v, g, beta, S0 = _rand_inputs(rng, B, T, H, dk, dv)
    kw = dict(qdq_mode=mode, group=group, hadamard=had, qdq_interval=interval)
    o, ST, ck = oracle.fwd(q, k, v, g, beta, S0, ckpt_interval=32, **kw)
    # batch independence
    o1, ST1, _ = oracle.fwd(q[1:2, :, 2:3], k[1:2, :, 2:3], v[1:2, :, 2:3], g[1:2, :, 2:3],
                            beta[1:2, :, 2:3], S0[1:2, 2:3], **kw)
    np.testing.assert_array_equal(o1[0, :, 0], o[1, :, 2])
    np.testing.assert_array_equal(ST1[0, 0], ST[1, 2])
    # split at token 64 (a quantization point for every interval used here)
    sl1, sl2 = slice(0, 64), slice(64, 128)
    oa, Sa, _ = oracle.fwd(q[:, sl1], k[:, sl1], v[:, sl1], g[:, sl1], beta[:, sl1], S0, **kw)
    ob, Sb, _ = oracle.fwd(q[:, sl2], k[:, sl2], v[:, sl2], g[:, sl2], beta[:, sl2], Sa, **kw)
    np.testing.assert_array_equal(np.concatenate([oa, ob], axis=1), o)
    np.testing.assert_array_equal(Sb, ST)
    # checkpoints: state entering tokens 0, 32, 64, 96
    np.testing.assert_array_equal(ck[:, :, 0], S0)
    np.testing.assert_array_equal(ck[:, :, 2], Sa)
    _, S96, _ = oracle.fwd(q[:, :96], k[:, :96], v[:, :96], g[:, :96], beta[:, :96], S0, **kw)
    if interval in (1, 16, 32):
        np.testing.assert_array_equal(ck[:, :, 3], S96)
    if interval == 1:
        S = S0
        for t in range(8):
            sl = slice(t, t + 1)
            ot, S, _ = oracle.fwd(q[:, sl], k[:, sl], v[:, sl], g[:, sl], beta[:, sl], S, **kw)
            np.testing.assert_array_equal(ot[:, 0], o[:, t])
        S8 = oracle.fwd(q[:, :8], k[:, :8], v[:, :8], g[:, :8], beta[:, :8], S0, **kw)[1]
        np.testing.assert_array_equal(S, S8)


def test_qdq_points_and_output_reads_unrounded_state(oracle_mod):
    """o_t is computed from S' before rounding; the carried state is Q(S') at the
    quantization points: after tokens n, 2n, ... and after the last token."""
    rng = np.random.default_rng(30)
    B, T, H, dk, dv = 1, 21, 1, 64, 64
    q, k, v, g, beta, S0 = _rand_inputs(rng, B, T, H, dk, dv)
    o_ref, S_ref, ck = oracle.fwd(q, k, v, g, beta, S0, ckpt_interval=1)
    o, ST, ckq = oracle.fwd(q, k, v, g, beta, S0, qdq_mode=oracle.QDQ_INT8, group=32,
                            qdq_interval=8, ckpt_interval=1)
    # tokens before the first quantization point match the unquantized run exactly
    np.testing.assert_array_equal(o[:, :8], o_ref[:, :8])
    np.testing.assert_array_equal(ckq[:, :, :8], ck[:, :, :8])
    # the state entering token 8 is Q of the unquantized state after token 7
    S8 = oracle.fwd(q[:, :8], k[:, :8], v[:, :8], g[:, :8], beta[:, :8], S0)[1]
    np.testing.assert_array_equal(ckq[0, 0, 8], oracle.qdq(S8[0, 0], oracle.QDQ_INT8, 32)[0])
    # the last token (21 is not a multiple of 8) is a quantization point
    last = oracle.fwd(q[:, 16:], k[:, 16:], v[:, 16:], g[:, 16:], beta[:, 16:], ckq[:, :, 16])
    np.testing.assert_array_equal(ST[0, 0], oracle.qdq(last[1][0, 0], oracle.QDQ_INT8, 32)[0])
    np.testing.assert_array_equal(o[:, 16:], last[0])


def test_decode_slots_padding_noop_and_permutation(oracle_mod):
    """Slot-pool decode: entries naming slot 0 or an index outside the pool give o = 0 and touch
    no slot; with beta = 0, g = 0 and exactly representable INT8 states, each live entry returns
    S^T q of the slot it names (a matrix product, not the recurrence) and leaves the pool as it
    was; permuting the entries together with their slots permutes the outputs and gives the
    same pool."""
    rng = np.random.default_rng(31)
    B, H, dk, dv, n = 6, 2, 32, 32, 5
    q, k, v, g, beta, _ = _rand_inputs(rng, B, 1, H, dk, dv)
    codes = rng.integers(-127, 128, size=(n, H, dk, dv))
    codes[..., ::32] = 127
    pool = codes * 2.0 ** -8
    slots = np.array([3, 0, 1, 7, -2, 4])
    g0, b0 = np.zeros_like(g), np.zeros_like(beta)
    o, pool2 = oracle.decode_slots(q, k, v, g0, b0, pool, slots, qdq_mode=oracle.QDQ_INT8, group=32)
    np.testing.assert_array_equal(pool2, pool)
    for b in range(B):
        if 1 <= slots[b] < n:
            np.testing.assert_allclose(o[b, 0], np.einsum("hij,hi->hj", pool[slots[b]], q[b, 0]), rtol=0, atol=1e-14)
        else:
            assert np.all(o[b] == 0)
    # a real step: padding entries and unnamed slots (0 and 2) keep their states
    o, pool3 = oracle.decode_slots(q, k, v, g, beta, pool, slots, qdq_mode=oracle.QDQ_INT8, group=32)
    for sl in (0, 2):
        np.testing.assert_array_equal(pool3[sl], pool[sl])
    for sl in (1, 3, 4):
        assert np.any(pool3[sl] != pool[sl])
    assert np.all(o[1] == 0) and np.all(o[3] == 0) and np.all(o[4] == 0)
    perm = np.array([5, 2, 0, 4, 1, 3])
    op, poolp = oracle.decode_slots(q[perm], k[perm], v[perm], g[perm], beta[perm], pool, slots[perm],
                                    qdq_mode=oracle.QDQ_INT8, group=32)
    np.testing.assert_array_equal(op, o[perm])
    np.testing.assert_array_equal(poolp, pool3)


def test_fwd_varlen_structure(oracle_mod):
    """Packed sequences: an empty sequence hands its S_0 through; a sequence's outputs and final
    state depend on its own tokens only (changing another sequence's tokens changes nothing);
    reordering the sequences in the packing reorders the results; with one sequence per call
    and equal lengths, the rows of the packed result are the batched forward's rows (the packing
    moves data only)."""
    rng = np.random.default_rng(41)
    H, dk, dv = 2, 16, 16
    lens = [5, 0, 3, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    q, k, v, g, beta, _ = _rand_inputs(rng, 1, T, H, dk, dv)
    q, k, v, g, beta = q[0], k[0], v[0], g[0], beta[0]
    S0 = rng.standard_normal((4, H, dk, dv)) * 0.3
    kw = dict(qdq_mode=oracle.QDQ_INT8, group=16, qdq_interval=2)
    o, ST = oracle.fwd_varlen(q, k, v, g, beta, cu, S0, **kw)
    np.testing.assert_array_equal(ST[1], S0[1])
    v2 = v.copy()
    v2[cu[2]:cu[3]] += 1.0  # sequence 2's values
    o2, ST2 = oracle.fwd_varlen(q, k, v2, g, beta, cu, S0, **kw)
    for b in (0, 1, 3):
        np.testing.assert_array_equal(ST2[b], ST[b])
        np.testing.assert_array_equal(o2[cu[b]:cu[b + 1]], o[cu[b]:cu[b + 1]])
    assert np.any(ST2[2] != ST[2])
    order = [3, 0, 2, 1]
    idx = np.concatenate([np.arange(cu[b], cu[b + 1]) for b in order]).astype(int)
    cu_p = np.concatenate([[0], np.cumsum([lens[b] for b in order])])
    op, STp = oracle.fwd_varlen(q[idx], k[idx], v[idx], g[idx], beta[idx], cu_p, S0[order], **kw)
    np.testing.assert_array_equal(op, o[idx])
    np.testing.assert_array_equal(STp, ST[order])
    # equal lengths: the packing is the batched layout with the batch axis folded into time
    L = 6
    qb, kb, vb, gb, bb, S0b = _rand_inputs(rng, 3, L, H, dk, dv)
    ob, STb, _ = oracle.fwd(qb, kb, vb, gb, bb, S0b, **kw)
    fold = lambda x: x.reshape((3 * L,) + x.shape[2:])
    ov, STv = oracle.fwd_varlen(fold(qb), fold(kb), fold(vb), fold(gb), fold(bb), np.arange(4) * L, S0b, **kw)
    np.testing.assert_array_equal(ov, fold(ob))
    np.testing.assert_array_equal(STv, STb)
