"""Pins of the oracle's replay windows.

Reading ("Torch GDN/KDA decode QAT + INT8", What does this PR do?: a one-token window
checkpoints every token, longer windows store BF16 key/update entries and refresh at the window
boundary; "Fused Triton GDN/KDA decode QAT", What does this PR do?: replay with encode-once
factors): with a window of W tokens the rounding points are those of qdq_interval = W; at every
other token the carried state takes the token's rank-1 update from its key and delta, each
encoded once to BF16 (nearest, ties to even, from the FP32 value); outputs read the token's
own unencoded update; the backward passes straight through the encoding.

The pins: the encoding against torch's float32 -> bfloat16 conversion; a window of one token
equals rounding after every token; the carried state inside a window equals the checkpoint
decayed plus the sum of the decayed BF16 entries (the serving side's reconstruction, a
non-recursive evaluation); a two-token case worked by hand in exact dyadic arithmetic;
power-of-two and sign equivariance; teacher forcing by given entries; the backward against
torch float64 autograd of the value-by-key matrix statement with straight-through encodings.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle



def _rand_inputs(rng, B, T, H, dk, dv, gate="scalar", s0=0.3):
    q = rng.standard_normal((B, T, H, dk)) / math.sqrt(dk)
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    k = torch.from_numpy(k).float().bfloat16().double().numpy()  # keys enter as bf16 values
    v = rng.standard_normal((B, T, H, dv))
    gs = (B, T, H, dk) if gate == "key" else (B, T, H)
    g = -np.log1p(np.exp(rng.standard_normal(gs)))
    beta = 1 / (1 + np.exp(-rng.standard_normal((B, T, H))))
    S0 = rng.standard_normal((B, H, dk, dv)) * s0
    return q, k, v, g, beta, S0


def torch_bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float64)).float().bfloat16().double().numpy()


def test_bf16_encoding_matches_torch(oracle_mod):
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        # exact ties of 8-bit significands and their neighbours
                        (np.arange(256, 512) + 0.5) * 2.0 ** -8, (np.arange(256, 512) + 0.5) * 2.0 ** 20,
                        -(np.arange(256, 512) + 0.5) * 2.0 ** -100])
    ours = np.array([oracle.bf16(v) for v in x])
    np.testing.assert_array_equal(ours, torch_bf16(x))
    # ties go to the even significand
    assert oracle.bf16(1 + 2 ** -8) == 1.0 and oracle.bf16(1 + 3 * 2 ** -8) == 1 + 2 ** -6


@pytest.mark.parametrize("mode,group,had,gate", [(oracle.QDQ_INT8, 32, True, 0), (oracle.QDQ_INT8, 64, False, 1),
                                                 (oracle.QDQ_E4M3, 64, False, 0)])
def test_window_of_one_is_rounding_every_token(oracle_mod, mode, group, had, gate):
    rng = np.random.default_rng(2)
    inp = _rand_inputs(rng, 2, 11, 2, 32, 64, "key" if gate else "scalar")
    kw = dict(gate=gate, qdq_mode=mode, group=group, hadamard=had, qdq_interval=1, ckpt_interval=1)
    o1, S1, c1 = oracle.fwd(*inp, replay=True, **kw)
    o2, S2, c2 = oracle.fwd(*inp, **kw)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(S1, S2)
    np.testing.assert_array_equal(c1, c2)


@pytest.mark.parametrize("gate,W", [(0, 4), (1, 5), (0, 16)])
def test_carried_state_is_checkpoint_plus_decayed_entries(oracle_mod, gate, W):
    """Inside a window the carried state entering token t is the window's checkpoint C decayed
    by every gate since, plus each earlier token's BF16 entries decayed by the gates after it:
    S = (prod a) C + sum_i (prod_{j>i} a_j) bf16(k_i) bf16(delta_i)^T (summed directly)."""
    rng = np.random.default_rng(3 + gate)
    B, T, H, dk, dv = 1, 37, 2, 16, 64
    q, k, v, g, beta, S0 = _rand_inputs(rng, B, T, H, dk, dv, "key" if gate else "scalar")
    o, ST, ck, deltas = oracle.fwd(q, k, v, g, beta, S0, gate=gate, qdq_mode=oracle.QDQ_INT8, group=32,
                                   qdq_interval=W, ckpt_interval=1, replay=True, return_deltas=True)
    states = np.concatenate([ck, ST[:, :, None]], axis=2)  # state entering t = 0 .. T
    a = np.exp(g)
    checked = 0
    for h in range(H):
        for t in range(T):
            w0 = (t // W) * W          # the window's first token: its checkpoint is states[w0]
            if t == w0 or t == T:
                continue
            C = states[0, h, w0]
            S = C.copy()
            gain = np.ones(dk)
            for j in range(w0, t):
                aj = a[0, j, h] if gate else np.full(dk, a[0, j, h])
                gain = gain * aj
            S = gain[:, None] * C
            for i in range(w0, t):
                di = np.ones(dk)
                for j in range(i + 1, t):
                    di = di * (a[0, j, h] if gate else np.full(dk, a[0, j, h]))
                S = S + di[:, None] * np.outer(torch_bf16(k[0, i, h]), torch_bf16(deltas[0, i, h]))
            np.testing.assert_allclose(states[0, h, t], S, rtol=0, atol=1e-12 * max(1.0, np.abs(S).max()))
            checked += 1
    assert checked > 20


def _bf16_frac(x: Fraction) -> Fraction:
    """Nearest value with an 8-bit significand (ties to even), for a dyadic rational."""
    if x == 0:
        return x
    sgn = -1 if x < 0 else 1
    a = abs(x)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    m = a * 128                       # significand in [128, 256)
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sgn * Fraction(fl, 128) * Fraction(2) ** e


def test_two_token_window_hand_algebra(oracle_mod):
    """S_0 = 0, GDN, one window of two tokens (INT8 rounding only after the second):
    delta_1 = b1 v1;  S_1 = bf16(k1) bf16(delta_1)^T (the first token is inside the window);
    o_1 = (k1 . q1) delta_1 (the unencoded update);
    delta_2 = b2 (v2 - a2 S_1^T k2);  o_2 = a2 S_1^T q2 + (k2 . q2) delta_2 (read before rounding).
    Dyadic inputs with more than eight significant bits in b1 v1, so the encoding matters and
    float64 evaluation is exact."""
    F = Fraction
    dk, dv = 4, 3
    k1 = [F(1, 2), F(-1, 2), F(1, 2), F(1, 2)]
    k2 = [F(1, 2), F(1, 2), F(1, 2), F(-1, 2)]
    q1 = [F(1, 4), F(0), F(-3, 4), F(1, 2)]
    q2 = [F(-1, 2), F(1, 4), F(1, 8), F(1)]
    v1 = [F(1) + F(3, 2 ** 11), F(-2) + F(5, 2 ** 10), F(3, 4) + F(1, 2 ** 9)]
    v2 = [F(-1, 2), F(5, 4), F(2)]
    b1, b2, a2 = F(3, 4), F(1, 2), F(1, 2)
    dot = lambda x, y: sum(i * j for i, j in zip(x, y))
    d1 = [b1 * x for x in v1]
    d1h = [_bf16_frac(x) for x in d1]
    assert d1h != d1
    S1 = [[k1[i] * d1h[j] for j in range(dv)] for i in range(dk)]
    o1 = [dot(k1, q1) * x for x in d1]
    u2 = [a2 * sum(S1[i][j] * k2[i] for i in range(dk)) for j in range(dv)]
    d2 = [b2 * (y - u) for y, u in zip(v2, u2)]
    o2 = [a2 * sum(S1[i][j] * q2[i] for i in range(dk)) + dot(k2, q2) * d2[j] for j in range(dv)]
    arr = lambda L: np.array([[float(x) for x in L]])
    q = np.stack([arr(q1), arr(q2)], axis=1)[:, :, None, :].reshape(1, 2, 1, dk)
    k = np.stack([arr(k1), arr(k2)], axis=1).reshape(1, 2, 1, dk)
    v = np.stack([arr(v1), arr(v2)], axis=1).reshape(1, 2, 1, dv)
    g = np.array([[[0.0], [math.log(float(a2))]]])  # a1 = 1 (S_0 = 0 makes it irrelevant)
    beta = np.array([[[float(b1)], [float(b2)]]])
    # INT8 groups of three columns (the whole row)
    o, _, ck = oracle.fwd(q, k, v, g, beta, None, qdq_mode=oracle.QDQ_INT8, group=3, qdq_interval=2,
                          ckpt_interval=1, replay=True)
    np.testing.assert_array_equal(o[0, 0, 0], [float(x) for x in o1])
    np.testing.assert_array_equal(ck[0, 0, 1], np.array([[float(x) for x in row] for row in S1]))
    np.testing.assert_allclose(o[0, 1, 0], [float(x) for x in o2], rtol=0, atol=1e-15)
    # without replay the first token's update is carried unencoded: a different second output
    o_n, _, _ = oracle.fwd(q, k, v, g, beta, None, qdq_mode=oracle.QDQ_INT8, group=3, qdq_interval=2)
    assert np.abs(o_n[0, 1, 0] - o[0, 1, 0]).max() > 1e-6


@pytest.mark.parametrize("gate", [0, 1])
def test_power_of_two_and_sign_equivariance(oracle_mod, gate):
    """BF16 encoding and the codecs commute with 2^m and negation, and the map is jointly
    linear in (v, S_0): scaling both scales every output and state exactly."""
    rng = np.random.default_rng(7 + gate)
    q, k, v, g, beta, S0 = _rand_inputs(rng, 1, 23, 2, 32, 64, "key" if gate else "scalar")
    kw = dict(gate=gate, qdq_mode=oracle.QDQ_INT8, group=32, hadamard=True, qdq_interval=6, replay=True)
    o, ST, _ = oracle.fwd(q, k, v, g, beta, S0, **kw)
    o2, ST2, _ = oracle.fwd(q, k, v * 2.0 ** 5, g, beta, S0 * 2.0 ** 5, **kw)
    np.testing.assert_array_equal(o2, o * 2.0 ** 5)
    np.testing.assert_array_equal(ST2, ST * 2.0 ** 5)
    o3, ST3, _ = oracle.fwd(q, k, -v, g, beta, -S0, **kw)
    np.testing.assert_array_equal(o3, -o)
    np.testing.assert_array_equal(ST3, -ST)


def test_given_entries_teacher_force_the_window(oracle_mod):
    """Entries passed in replace the oracle's own at the tokens inside windows: perturbing one
    entry changes the later states by exactly that entry's decayed rank-1 term."""
    rng = np.random.default_rng(9)
    q, k, v, g, beta, S0 = _rand_inputs(rng, 1, 8, 1, 16, 64)
    kw = dict(qdq_mode=oracle.QDQ_INT8, group=32, qdq_interval=8, replay=True, ckpt_interval=1)
    o, ST, ck, deltas = oracle.fwd(q, k, v, g, beta, S0, return_deltas=True, **kw)
    dhat = np.full_like(deltas, np.nan)
    dhat[0, 2, 0] = torch_bf16(deltas[0, 2, 0]) + 2.0 ** -5
    o2, _, ck2 = oracle.fwd(q, k, v, g, beta, S0, dhat=dhat, **kw)
    np.testing.assert_array_equal(ck2[0, 0, :3], ck[0, 0, :3])
    np.testing.assert_array_equal(o2[0, :3], o[0, :3])
    diff = ck2[0, 0, 3] - ck[0, 0, 3]
    np.testing.assert_allclose(diff, np.outer(k[0, 2, 0], np.full(64, 2.0 ** -5)), rtol=0, atol=1e-14)


def _torch_replay_forward(q, k, v, g, beta, S0, gate, mode, group, had, W):
    """Value-by-key matrix statement with straight-through encodings (torch, float64): at a
    rounding point M <- M + (Q(M) - M).detach(); inside a window
    M <- M + (M~ + bf16(delta) bf16(k)^T - M).detach() with M~ the decayed state."""
    B, T, H, dk = q.shape
    outs, finals = [], []
    for b in range(B):
        for h in range(H):
            M = S0[b, h].T
            ob = []
            for t in range(T):
                a = torch.exp(g[b, t, h]) * torch.ones(dk, dtype=torch.float64) if gate == 0 else torch.exp(g[b, t, h])
                kk = k[b, t, h]
                Mt = M @ torch.diag(a)
                delta = beta[b, t, h] * (v[b, t, h] - Mt @ kk)
                M = Mt + torch.outer(delta, kk)
                ob.append(M @ q[b, t, h])
                if (t + 1) % W == 0 or t == T - 1:
                    Xh = oracle.qdq(M.detach().numpy().T, mode, group, had)[0]
                    M = M + (torch.from_numpy(Xh.T.copy()) - M).detach()
                else:
                    enc = Mt.detach() + torch.outer(delta.detach().float().bfloat16().double(),
                                                    kk.detach().float().bfloat16().double())
                    M = M + (enc - M).detach()
            outs.append(torch.stack(ob))
            finals.append(M.T)
    o = torch.stack(outs).reshape(B, H, T, -1).permute(0, 2, 1, 3)
    ST = torch.stack(finals).reshape(B, H, dk, -1)
    return o, ST


@pytest.mark.parametrize("gate,mode,group,had,W", [(0, oracle.QDQ_INT8, 32, True, 4), (1, oracle.QDQ_INT8, 64, False, 3),
                                                   (0, oracle.QDQ_E4M3, 64, False, 5)])
def test_backward_matches_torch_autograd_ste(oracle_mod, gate, mode, group, had, W):
    rng = np.random.default_rng(11 + W)
    B, T, H, dk, dv = 1, 11, 2, 32, 64
    inp = _rand_inputs(rng, B, T, H, dk, dv, "key" if gate else "scalar", s0=0.4)
    do = rng.standard_normal((B, T, H, dv))
    dST = rng.standard_normal((B, H, dk, dv))
    kw = dict(gate=gate, qdq_mode=mode, group=group, hadamard=had, qdq_interval=W, replay=True)
    r = oracle.bwd(*inp, do, dST, **kw)
    ts = [torch.tensor(x, requires_grad=True) for x in inp]
    o, ST = _torch_replay_forward(*ts, gate, mode, group, had, W)
    o_or, _, _ = oracle.fwd(*inp, **kw)
    np.testing.assert_allclose(o.detach().numpy(), o_or, atol=1e-10)
    L = (o * torch.from_numpy(do)).sum() + (ST * torch.from_numpy(dST)).sum()
    L.backward()
    for name, t in zip(["dq", "dk", "dv", "dg", "dbeta", "dS0"], ts):
        np.testing.assert_allclose(r[name], t.grad.numpy(), rtol=1e-9, atol=1e-10, err_msg=name)
    # and the backward fed with the forward's per-token states equals its own recompute
    _, _, ck = oracle.fwd(*inp, ckpt_interval=1, **kw)
    r2 = oracle.bwd(*inp, do, dST, states=ck, **kw)
    for name in r:
        np.testing.assert_array_equal(r[name], r2[name])
