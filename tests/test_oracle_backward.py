"""Pins of the oracle's straight-through backward.

The pages ("Torch GDN/KDA decode QAT + INT8", "GDN state/W QAT foundation", "Fused Triton
GDN/KDA decode QAT", each under "What does this PR do?") specify identity straight-through
gradients through the state QDQ, a differentiable adjoint and a differentiable carry of
the initial state.  Pinned here by: a one-token closed form derived by hand, central
finite differences (QDQ off, where the map is smooth), and torch float64 autograd of an
independent matrix statement of the recurrence with the straight-through rounding
written as x + (Q(x) - x).detach().
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests.test_oracle_recurrence import _rand_inputs


def test_one_token_closed_form(oracle_mod):
    """T = 1, GDN, no QDQ, L = <do, o>:
    dS_0 = a (I - b k k^T) q do^T;  dv = b (k.q) do;  db = (k.q) <do, v - a S_0^T k>;
    dq = S' do;  dg = a <do, S_0^T q - b (k.q) S_0^T k>."""
    rng = np.random.default_rng(40)
    dk, dv = 8, 6
    q, k, v, g, beta, S0 = _rand_inputs(rng, 1, 1, 1, dk, dv, s0=0.7)
    do = rng.standard_normal((1, 1, 1, dv))
    r = oracle.bwd(q, k, v, g, beta, S0, do)
    a, b = math.exp(g[0, 0, 0]), beta[0, 0, 0]
    kk, qq, vv, dd, S = k[0, 0, 0], q[0, 0, 0], v[0, 0, 0], do[0, 0, 0], S0[0, 0]
    kq = kk @ qq
    dS0 = a * np.outer((np.eye(dk) - b * np.outer(kk, kk)) @ qq, dd)
    np.testing.assert_allclose(r["dS0"][0, 0], dS0, atol=1e-13)
    np.testing.assert_allclose(r["dv"][0, 0, 0], b * kq * dd, atol=1e-13)
    np.testing.assert_allclose(r["dbeta"][0, 0, 0], kq * dd @ (vv - a * S.T @ kk), atol=1e-13)
    Sp = a * S + np.outer(kk, b * (vv - a * S.T @ kk))
    np.testing.assert_allclose(r["dq"][0, 0, 0], Sp @ dd, atol=1e-13)
    np.testing.assert_allclose(r["dg"][0, 0, 0], a * dd @ (S.T @ qq - b * kq * (S.T @ kk)), atol=1e-13)


def _loss(q, k, v, g, beta, S0, do, dST, gate):
    o, ST, _ = oracle.fwd(q, k, v, g, beta, S0, gate=gate)
    return float(np.sum(o * do) + np.sum(ST * dST))


@pytest.mark.parametrize("gate", [oracle.GATE_SCALAR, oracle.GATE_KEY])
def test_finite_differences(oracle_mod, gate):
    """Central differences of L = <do, o> + <dS_T, S_T> (QDQ off) at T = 4."""
    rng = np.random.default_rng(41 + gate)
    B, T, H, dk, dv = 1, 4, 1, 6, 5
    inp = list(_rand_inputs(rng, B, T, H, dk, dv, "key" if gate else "scalar", s0=0.5))
    do = rng.standard_normal((B, T, H, dv))
    dST = rng.standard_normal((B, H, dk, dv))
    r = oracle.bwd(*inp, do, dST, gate=gate)
    names = ["dq", "dk", "dv", "dg", "dbeta", "dS0"]
    eps = 1e-6
    for idx, name in enumerate(names):
        x = inp[idx]
        num = np.zeros_like(x)
        for pos in np.ndindex(x.shape):
            xp = x.copy(); xp[pos] += eps
            xm = x.copy(); xm[pos] -= eps
            a1 = list(inp); a1[idx] = xp
            a2 = list(inp); a2[idx] = xm
            num[pos] = (_loss(*a1, do, dST, gate) - _loss(*a2, do, dST, gate)) / (2 * eps)
        np.testing.assert_allclose(r[name], num, rtol=1e-6, atol=1e-7, err_msg=name)


def _torch_ste_forward(q, k, v, g, beta, S0, gate, mode, group, had, interval):
    """Value-by-key matrix statement with straight-through rounding (torch, float64)."""
    B, T, H, dk = q.shape
    outs, finals = [], []
    for b in range(B):
        for h in range(H):
            M = S0[b, h].T
            ob = []
            for t in range(T):
                a = torch.exp(g[b, t, h]) * torch.ones(dk, dtype=torch.float64) if gate == 0 \
                    else torch.exp(g[b, t, h])
                kk = k[b, t, h]
                M = M @ torch.diag(a) @ (torch.eye(dk, dtype=torch.float64) - beta[b, t, h] * torch.outer(kk, kk)) \
                    + beta[b, t, h] * torch.outer(v[b, t, h], kk)
                ob.append(M @ q[b, t, h])
                if mode != oracle.QDQ_NONE and ((t + 1) % interval == 0 or t == T - 1):
                    Xh = oracle.qdq(M.detach().numpy().T, mode, group, had)[0]
                    M = M + (torch.from_numpy(Xh.T.copy()) - M).detach()
            outs.append(torch.stack(ob))
            finals.append(M.T)
    o = torch.stack(outs).reshape(B, H, T, -1).permute(0, 2, 1, 3)
    ST = torch.stack(finals).reshape(B, H, dk, -1)
    return o, ST


@pytest.mark.parametrize("gate,mode,group,had,interval", [
    (0, oracle.QDQ_NONE, 32, False, 1),
    (0, oracle.QDQ_INT8, 32, False, 1),
    (1, oracle.QDQ_INT8, 64, False, 1),
    (0, oracle.QDQ_E4M3, 64, False, 4),
    (0, oracle.QDQ_INT8, 32, True, 1),
    (1, oracle.QDQ_INT8, 32, True, 1),
])
def test_matches_torch_autograd_ste(oracle_mod, gate, mode, group, had, interval):
    rng = np.random.default_rng(50 + mode)
    B, T, H, dk, dv = 1, 9, 2, 64, 64
    inp = _rand_inputs(rng, B, T, H, dk, dv, "key" if gate else "scalar", s0=0.4)
    do = rng.standard_normal((B, T, H, dv))
    dST = rng.standard_normal((B, H, dk, dv))
    r = oracle.bwd(*inp, do, dST, gate=gate, qdq_mode=mode, group=group, hadamard=had,
                   qdq_interval=interval)
    ts = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in inp]
    o, ST = _torch_ste_forward(*ts, gate, mode, group, had, interval)
    # the torch forward follows the same quantized trajectory
    o_or, ST_or, _ = oracle.fwd(*inp, gate=gate, qdq_mode=mode, group=group, hadamard=had,
                                qdq_interval=interval)
    np.testing.assert_allclose(o.detach().numpy(), o_or, atol=1e-10)
    L = (o * torch.from_numpy(do)).sum() + (ST * torch.from_numpy(dST)).sum()
    L.backward()
    for name, t in zip(["dq", "dk", "dv", "dg", "dbeta", "dS0"], ts):
        np.testing.assert_allclose(r[name], t.grad.numpy(), rtol=1e-9, atol=1e-10, err_msg=name)


def test_given_states_equal_recompute(oracle_mod):
    """The backward fed with the per-token carried states equals the one that recomputes."""
    rng = np.random.default_rng(60)
    B, T, H, dk, dv = 2, 12, 2, 64, 64
    inp = _rand_inputs(rng, B, T, H, dk, dv)
    do = rng.standard_normal((B, T, H, dv))
    kw = dict(qdq_mode=oracle.QDQ_INT8, group=32, qdq_interval=1)
    _, _, ck = oracle.fwd(*inp, ckpt_interval=1, **kw)
    r1 = oracle.bwd(*inp, do, **kw)
    r2 = oracle.bwd(*inp, do, states=ck, **kw)
    for name in r1:
        np.testing.assert_array_equal(r1[name], r2[name])
