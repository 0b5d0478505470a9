"""Pins of the oracle's packed-sequence backward and its per-sequence prefix/suffix boundary
("Torch GDN/KDA decode QAT + INT8", What does this PR do?: an explicit per-sequence boundary
selects a chunked prefill prefix and a recurrent suffix, and the suffix's gradients flow
through the handoff into the prefill; "Experimental GDN/KDA approximate-inverse QAT", Testing:
packed sequence tails).

The pins: without rounding at the boundary the handoff is exact, so a split call equals one
uncut call of each sequence (forward and backward); rounding after every token puts a rounding
point at every boundary, so the same holds with the quantizer on; central finite differences
of a loss through the split forward (no quantizer); torch float64 autograd of the two parts
chained with straight-through rounding, E4M3 prefix and INT8 suffix (the gradient reaching
the prefix through the handoff state); empty prefixes, empty suffixes and tokens outside
every sequence.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests.test_oracle_backward import _torch_ste_forward

LENS = [7, 0, 8, 1, 5]
PRE = [3, 2, 8, 0, 2]   # prefix lengths: inside, beyond an empty sequence, whole, none, inside


def _inputs(rng, T, H, dk, dv, gate="scalar"):
    q = rng.standard_normal((T, H, dk)) / math.sqrt(dk)
    k = rng.standard_normal((T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    gs = (T, H, dk) if gate == "key" else (T, H)
    g = -np.log1p(np.exp(rng.standard_normal(gs)))
    beta = 1 / (1 + np.exp(-rng.standard_normal((T, H))))
    return q, k, v, g, beta


def _cu(lens, tail=0):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64), int(sum(lens)) + tail


@pytest.mark.parametrize("gate", [0, 1])
def test_split_without_rounding_is_one_call(oracle_mod, gate):
    rng = np.random.default_rng(1 + gate)
    cu, T = _cu(LENS, tail=2)
    H, dk, dv = 2, 8, 16
    inp = _inputs(rng, T, H, dk, dv, "key" if gate else "scalar")
    S0 = rng.standard_normal((len(LENS), H, dk, dv)) * 0.3
    kw = dict(qdq_mode=oracle.QDQ_NONE)
    o, S_mid, S_T = oracle.fwd_split(*inp, cu, PRE, S0, kw, kw, gate=gate)
    o1, S_T1 = oracle.fwd_varlen(*inp, cu, S0, gate=gate)
    np.testing.assert_allclose(o, o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(S_T, S_T1, rtol=0, atol=1e-13)
    do = rng.standard_normal((T, H, dv))
    dST = rng.standard_normal(S0.shape)
    r = oracle.bwd_split(*inp, cu, PRE, S0, S_mid, do, dST, kw, kw, gate=gate)
    r1 = oracle.bwd_varlen(*inp, cu, S0, do, dST, gate=gate)
    for n in ("dq", "dk", "dv", "dg", "dbeta", "dS0"):
        np.testing.assert_allclose(r[n], r1[n], rtol=0, atol=1e-12, err_msg=n)
    # tokens outside every sequence: zero gradients
    for n in ("dq", "dk", "dv", "dg", "dbeta"):
        assert np.all(r[n][T - 2:] == 0)


def test_split_rounding_every_token_is_one_call(oracle_mod):
    rng = np.random.default_rng(3)
    cu, T = _cu(LENS)
    H, dk, dv = 2, 16, 32
    inp = _inputs(rng, T, H, dk, dv)
    S0 = rng.standard_normal((len(LENS), H, dk, dv)) * 0.3
    kw = dict(qdq_mode=oracle.QDQ_INT8, group=16, qdq_interval=1, hadamard=True)
    o, S_mid, S_T = oracle.fwd_split(*inp, cu, PRE, S0, kw, kw)
    o1, S_T1 = oracle.fwd_varlen(*inp, cu, S0, **kw)
    np.testing.assert_array_equal(o, o1)
    np.testing.assert_array_equal(S_T, S_T1)


def test_split_handoff_states(oracle_mod):
    """An empty prefix hands S0 to the suffix (S_mid = S0); a whole-sequence prefix leaves the
    suffix empty (S_T = S_mid); the handoff equals the prefix run alone."""
    rng = np.random.default_rng(4)
    cu, T = _cu(LENS)
    H, dk, dv = 1, 8, 16
    inp = _inputs(rng, T, H, dk, dv)
    S0 = rng.standard_normal((len(LENS), H, dk, dv)) * 0.3
    pk = dict(qdq_mode=oracle.QDQ_E4M3, group=16, qdq_interval=4)
    sk = dict(qdq_mode=oracle.QDQ_INT8, group=16, qdq_interval=1)
    o, S_mid, S_T = oracle.fwd_split(*inp, cu, PRE, S0, pk, sk)
    np.testing.assert_array_equal(S_mid[3], S0[3])            # prefix 0
    np.testing.assert_array_equal(S_T[2], S_mid[2])           # prefix = the whole sequence
    np.testing.assert_array_equal(S_mid[1], S0[1])            # empty sequence
    t0 = int(cu[0])
    _, S_p, _ = oracle.fwd(*[x[None, t0:t0 + PRE[0]] for x in inp], S0[0:1], **pk)
    np.testing.assert_array_equal(S_mid[0], S_p[0])


def test_split_backward_finite_differences(oracle_mod):
    rng = np.random.default_rng(5)
    lens, pre = [4, 3], [2, 1]
    cu, T = _cu(lens)
    H, dk, dv = 1, 3, 2
    inp = list(_inputs(rng, T, H, dk, dv))
    S0 = rng.standard_normal((2, H, dk, dv)) * 0.4
    do = rng.standard_normal((T, H, dv))
    dST = rng.standard_normal(S0.shape)
    kw = dict(qdq_mode=oracle.QDQ_NONE)

    def loss(*a):
        o, _, S_T = oracle.fwd_split(*a[:5], cu, pre, a[5], kw, kw)
        return float(np.sum(o * do) + np.sum(S_T * dST))
    _, S_mid, _ = oracle.fwd_split(*inp, cu, pre, S0, kw, kw)
    r = oracle.bwd_split(*inp, cu, pre, S0, S_mid, do, dST, kw, kw)
    eps = 1e-6
    for idx, name in enumerate(["dq", "dk", "dv", "dg", "dbeta", "dS0"]):
        base = (inp + [S0])[idx]
        num = np.zeros_like(base)
        for pos in np.ndindex(base.shape):
            xp, xm = base.copy(), base.copy()
            xp[pos] += eps
            xm[pos] -= eps
            ap, am = list(inp + [S0]), list(inp + [S0])
            ap[idx], am[idx] = xp, xm
            num[pos] = (loss(*ap) - loss(*am)) / (2 * eps)
        np.testing.assert_allclose(r[name], num, rtol=1e-6, atol=1e-7, err_msg=name)


@pytest.mark.parametrize("gate", [0, 1])
def test_split_backward_matches_torch_autograd(oracle_mod, gate):
    """One sequence: E4M3 prefix rounding every 4 tokens, then an INT8 (Hadamard) suffix
    rounding every token, chained through the handoff state; torch float64 autograd with
    straight-through rounding in both parts."""
    rng = np.random.default_rng(6 + gate)
    T, pre, H, dk, dv = 11, 6, 2, 16, 32
    q, k, v, g, beta = _inputs(rng, T, H, dk, dv, "key" if gate else "scalar")
    S0 = rng.standard_normal((1, H, dk, dv)) * 0.3
    do = rng.standard_normal((T, H, dv))
    dST = rng.standard_normal(S0.shape)
    pk = dict(qdq_mode=oracle.QDQ_E4M3, group=16, qdq_interval=4)
    sk = dict(qdq_mode=oracle.QDQ_INT8, group=16, qdq_interval=1, hadamard=True)
    cu = np.array([0, T])
    o, S_mid, S_T = oracle.fwd_split(q, k, v, g, beta, cu, [pre], S0, pk, sk, gate=gate)
    r = oracle.bwd_split(q, k, v, g, beta, cu, [pre], S0, S_mid, do, dST, pk, sk, gate=gate)
    ts = [torch.tensor(x[None], requires_grad=True) for x in (q, k, v, g, beta)]
    tS0 = torch.tensor(S0, requires_grad=True)
    o1, S1 = _torch_ste_forward(*[t[:, :pre] for t in ts], tS0, gate, oracle.QDQ_E4M3, 16, False, 4)
    o2, S2 = _torch_ste_forward(*[t[:, pre:] for t in ts], S1, gate, oracle.QDQ_INT8, 16, True, 1)
    np.testing.assert_allclose(torch.cat([o1, o2], dim=1).detach().numpy()[0], o, atol=1e-10)
    L = (torch.cat([o1, o2], dim=1)[0] * torch.from_numpy(do)).sum() + (S2 * torch.from_numpy(dST)).sum()
    L.backward()
    for name, t in zip(["dq", "dk", "dv", "dg", "dbeta"], ts):
        np.testing.assert_allclose(r[name], t.grad.numpy()[0], rtol=1e-9, atol=1e-10, err_msg=name)
    np.testing.assert_allclose(r["dS0"], tS0.grad.numpy(), rtol=1e-9, atol=1e-10)
