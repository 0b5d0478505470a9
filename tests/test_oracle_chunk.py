"""Pins of the chunked oracle (oracle/chunk.py): the 64-token chunk form with the exact
triangular solve or the Neumann approximate inverse ("GDN state/W QAT foundation", What does
this PR do?: 64-token chunks with the state rounded at each chunk boundary; "Experimental
GDN/KDA approximate-inverse QAT", What does this PR do?: an explicit Neumann degree, backward
through the actual polynomial; Testing: residual identities and polynomial gradients).

Pins, each independent of the chunk code's own formulas:
  * exact solve = the token recurrence (oracle.fwd / oracle.bwd, the C oracle), forward and
    backward, with and without rounding at chunk ends, both gates, ragged last chunk;
  * Neumann degree >= L - 1 is exact (A is nilpotent); degree d on a chunk of d + 2 tokens
    differs from the recurrence only at the last token, by the closed form
    -(A[1,0] A[2,1] ... A[L-1,L-2]) delta_0 built from the recurrence's own deltas;
  * the residual identity (I + A) P_d(A) = I - (-A)^(d+1) against numpy's matrix_power;
  * gradients: central finite differences of the polynomial and of the whole chunked map,
    and torch float64 autograd through a chunked forward with straight-through rounding.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import chunk as oc

G_SCALAR, G_KEY = oracle.GATE_SCALAR, oracle.GATE_KEY


def _inputs(rng, B, T, H, dk, dv, gate, s0=0.3):
    q = rng.standard_normal((B, T, H, dk)) / math.sqrt(dk)
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    gs = (B, T, H, dk) if gate == G_KEY else (B, T, H)
    g = -np.log1p(np.exp(rng.standard_normal(gs))) * 0.3
    beta = 1 / (1 + np.exp(-rng.standard_normal((B, T, H))))
    S0 = rng.standard_normal((B, H, dk, dv)) * s0
    return q, k, v, g, beta, S0


def _err(x, ref):
    return float(np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-300))


CASES = [
    # gate, quantizer kw (rounding at chunk ends), T
    (G_SCALAR, dict(qdq_mode=oracle.QDQ_NONE), 150),
    (G_KEY, dict(qdq_mode=oracle.QDQ_NONE), 150),
    (G_SCALAR, dict(qdq_mode=oracle.QDQ_E4M3, group=64, qdq_interval=64), 150),
    (G_KEY, dict(qdq_mode=oracle.QDQ_E4M3, group=64, qdq_interval=64), 130),
    (G_SCALAR, dict(qdq_mode=oracle.QDQ_INT8, group=32, qdq_interval=128), 200),
    (G_KEY, dict(qdq_mode=oracle.QDQ_INT8, group=16, qdq_interval=64, hadamard=True), 140),
]


@pytest.mark.parametrize("gate,kw,T", CASES)
def test_exact_solve_is_the_recurrence(oracle_mod, gate, kw, T):
    rng = np.random.default_rng(10 + T + gate)
    q, k, v, g, beta, S0 = _inputs(rng, 1, T, 2, 16, 64, gate)
    o, ST, ck = oc.fwd(q, k, v, g, beta, S0, gate=gate, solve=oc.SOLVE_EXACT, ckpt_interval=64, **kw)
    o_r, ST_r, ck_r = oracle.fwd(q, k, v, g, beta, S0, gate=gate, ckpt_interval=64, **kw)
    assert _err(o, o_r) < 1e-12
    assert _err(ST, ST_r) < 1e-12
    assert _err(ck, ck_r) < 1e-12


@pytest.mark.parametrize("gate,kw,T", CASES)
def test_exact_solve_backward_is_the_recurrence_backward(oracle_mod, gate, kw, T):
    rng = np.random.default_rng(20 + T + gate)
    q, k, v, g, beta, S0 = _inputs(rng, 1, T, 2, 16, 64, gate)
    do = rng.standard_normal(v.shape)
    dST = rng.standard_normal(S0.shape)
    r = oc.bwd(q, k, v, g, beta, S0, do, dST, gate=gate, solve=oc.SOLVE_EXACT, **kw)
    r_r = oracle.bwd(q, k, v, g, beta, S0, do, dST, gate=gate, **kw)
    for n in ("dq", "dk", "dv", "dg", "dbeta", "dS0"):
        assert _err(r[n], r_r[n]) < 1e-11, n


@pytest.mark.parametrize("gate", [G_SCALAR, G_KEY])
def test_neumann_of_full_degree_is_exact(oracle_mod, gate):
    rng = np.random.default_rng(30 + gate)
    q, k, v, g, beta, S0 = _inputs(rng, 1, 150, 1, 16, 64, gate)
    kw = dict(gate=gate, qdq_mode=oracle.QDQ_E4M3, group=64, qdq_interval=64)
    o, ST, _ = oc.fwd(q, k, v, g, beta, S0, solve=oc.SOLVE_NEUMANN, degree=63, **kw)
    o_r, ST_r, _ = oracle.fwd(q, k, v, g, beta, S0, **kw)
    assert _err(o, o_r) < 1e-11 and _err(ST, ST_r) < 1e-11
    # a single short chunk of L <= d + 1 tokens
    for d in (3, 7, 15, 31):
        L = d + 1
        args = [x[:, :L] for x in (q, k, v, g, beta)]
        o, ST, _ = oc.fwd(*args, S0, gate=gate, solve=oc.SOLVE_NEUMANN, degree=d)
        o_r, ST_r, _ = oracle.fwd(*args, S0, gate=gate)
        assert _err(o, o_r) < 1e-11 and _err(ST, ST_r) < 1e-11, d


def _correlated_inputs(rng, L, dk, dv, gate):
    """Consecutive keys strongly aligned and beta near one, so that the subdiagonal of A is
    near one and its product over the chunk is far above rounding."""
    base = rng.standard_normal(dk)
    k = base[None, :] + 0.25 * rng.standard_normal((L, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q = rng.standard_normal((L, dk)) / math.sqrt(dk)
    v = rng.standard_normal((L, dv))
    g = -0.01 * rng.random((L, dk) if gate == G_KEY else (L,))
    beta = 0.85 + 0.15 * rng.random(L)
    S0 = rng.standard_normal((dk, dv)) * 0.3
    return q[None, :, None], k[None, :, None], v[None, :, None], g[None, :, None], beta[None, :, None], S0[None, None]


@pytest.mark.parametrize("gate", [G_SCALAR, G_KEY])
@pytest.mark.parametrize("d", [3, 7, 15, 31])
def test_neumann_deviation_closed_form(oracle_mod, gate, d):
    rng = np.random.default_rng(40 + d + gate)
    L, dk, dv = d + 2, 16, 8
    q, k, v, g, beta, S0 = _correlated_inputs(rng, L, dk, dv, gate)
    o, ST, _ = oc.fwd(q, k, v, g, beta, S0, gate=gate, solve=oc.SOLVE_NEUMANN, degree=d)
    o_r, ST_r, _, deltas = oracle.fwd(q, k, v, g, beta, S0, gate=gate, return_deltas=True)
    kk, bb = k[0, :, 0], beta[0, :, 0]
    a = np.exp(g[0, :, 0]) if gate == G_KEY else np.exp(g[0, :, 0])[:, None] * np.ones(dk)
    sub = [bb[j + 1] * np.sum(kk[j + 1] * a[j + 1] * kk[j]) for j in range(L - 1)]
    pi = float(np.prod(sub))
    corr = pi * deltas[0, 0, 0]                       # delta_d[L-1] = delta[L-1] - pi delta_0
    # the float64 power sum of degree 31 carries rounding noise near 1e-9 here; the deviation
    # it must show is at least 1e-3, four decades above the tolerance
    tol = 1e-8
    scale = np.max(np.abs(o_r))
    assert np.max(np.abs(corr)) > 1e4 * tol * scale
    qk = float(np.dot(q[0, L - 1, 0], kk[L - 1]))
    np.testing.assert_allclose(o[0, :L - 1], o_r[0, :L - 1], rtol=0, atol=tol * scale)
    np.testing.assert_allclose(o[0, L - 1, 0] - o_r[0, L - 1, 0], -qk * corr, rtol=1e-5, atol=tol * scale)
    np.testing.assert_allclose(ST[0, 0] - ST_r[0, 0], -np.outer(kk[L - 1], corr), rtol=1e-5,
                               atol=tol * np.max(np.abs(ST_r)))


@pytest.mark.parametrize("d", [0, 1, 3, 7, 15, 31])
def test_neumann_residual_identity(d):
    rng = np.random.default_rng(50 + d)
    A = np.tril(rng.standard_normal((64, 64)) * 0.1, -1)
    P = oc.neumann(A, d)
    rhs = np.eye(64) - np.linalg.matrix_power(-A, d + 1)
    np.testing.assert_allclose((np.eye(64) + A) @ P, rhs, rtol=0, atol=1e-13)


@pytest.mark.parametrize("d", [1, 3, 7])
def test_polynomial_and_inverse_gradients_finite_differences(d):
    rng = np.random.default_rng(60 + d)
    n = 6
    A = np.tril(rng.standard_normal((n, n)) * 0.4, -1)
    dP = rng.standard_normal((n, n))
    eps = 1e-6
    for solve, f in ((oc.SOLVE_NEUMANN, lambda X: oc.neumann(X, d)),
                     (oc.SOLVE_EXACT, lambda X: np.linalg.inv(np.eye(n) + X))):
        P = f(A)
        got = oc._solve_grad(A, P, dP, solve, d) * np.tril(np.ones((n, n)), -1)
        num = np.zeros((n, n))
        for i in range(n):
            for j in range(i):
                Ap, Am = A.copy(), A.copy()
                Ap[i, j] += eps
                Am[i, j] -= eps
                num[i, j] = (np.sum(dP * f(Ap)) - np.sum(dP * f(Am))) / (2 * eps)
        np.testing.assert_allclose(got, num, rtol=1e-7, atol=1e-8)


@pytest.mark.parametrize("gate", [G_SCALAR, G_KEY])
def test_chunked_backward_finite_differences(oracle_mod, gate):
    """Neumann degree 3 over a full chunk and a 6-token tail (no rounding): every gradient
    against central differences of the chunked forward itself."""
    rng = np.random.default_rng(70 + gate)
    T, dk, dv = 70, 3, 2
    q, k, v, g, beta, S0 = _inputs(rng, 1, T, 1, dk, dv, gate, s0=0.5)
    do = rng.standard_normal(v.shape)
    dST = rng.standard_normal(S0.shape)
    kw = dict(gate=gate, solve=oc.SOLVE_NEUMANN, degree=3)
    r = oc.bwd(q, k, v, g, beta, S0, do, dST, **kw)

    def loss(args):
        o, ST, _ = oc.fwd(*args, **kw)
        return float(np.sum(o * do) + np.sum(ST * dST))
    base = [q, k, v, g, beta, S0]
    eps = 1e-6
    for idx, name in enumerate(["dq", "dk", "dv", "dg", "dbeta", "dS0"]):
        x = base[idx]
        num = np.zeros_like(x)
        for pos in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[pos] += eps
            xm[pos] -= eps
            ap, am = list(base), list(base)
            ap[idx], am[idx] = xp, xm
            num[pos] = (loss(ap) - loss(am)) / (2 * eps)
        np.testing.assert_allclose(r[name], num, rtol=1e-6, atol=1e-7, err_msg=name)


def _torch_chunked_ste(q, k, v, g, beta, S0, gate, degree, mode, group, interval, chunk=64):
    """Chunk form in torch float64 with straight-through rounding at chunk ends (autograd
    supplies the gradients; the values are checked against the oracle first)."""
    B, T, H, dk = q.shape
    outs, finals = [], []
    for b in range(B):
        for h in range(H):
            S = S0[b, h]
            ob = []
            for t0 in range(0, T, chunk):
                t1 = min(T, t0 + chunk)
                L = t1 - t0
                qc, kc, vc, bc = q[b, t0:t1, h], k[b, t0:t1, h], v[b, t0:t1, h], beta[b, t0:t1, h]
                gc = g[b, t0:t1, h] if gate == G_KEY else g[b, t0:t1, h][:, None].expand(L, dk)
                G = torch.cumsum(gc, 0)
                low = torch.tril(torch.ones(L, L, dtype=torch.float64), -1)
                lowd = torch.tril(torch.ones(L, L, dtype=torch.float64))
                diff = (G[:, None, :] - G[None, :, :]) * lowd[:, :, None]
                D = torch.exp(diff) * lowd[:, :, None]
                A = bc[:, None] * torch.einsum("rk,ik,rik->ri", kc, kc, D) * low
                M = torch.einsum("rk,ik,rik->ri", qc, kc, D) * lowd
                P = torch.eye(L, dtype=torch.float64)
                term = torch.eye(L, dtype=torch.float64)
                for _ in range(degree):
                    term = term @ (-A)
                    P = P + term
                E = torch.exp(G)
                F = torch.exp(G[-1][None, :] - G)
                Delta = P @ (bc[:, None] * (vc - (kc * E) @ S))
                ob.append((qc * E) @ S + M @ Delta)
                S = E[-1][:, None] * S + (kc * F).T @ Delta
                if mode != oracle.QDQ_NONE and (t1 % interval == 0 or t1 == T):
                    Xh = oracle.qdq(S.detach().numpy(), mode, group)[0]
                    S = S + (torch.from_numpy(Xh) - S).detach()
            outs.append(torch.cat(ob))
            finals.append(S)
    o = torch.stack(outs).reshape(B, H, T, -1).permute(0, 2, 1, 3)
    return o, torch.stack(finals).reshape(B, H, dk, -1)


@pytest.mark.parametrize("gate", [G_SCALAR, G_KEY])
def test_chunked_backward_matches_torch_autograd_ste(oracle_mod, gate):
    rng = np.random.default_rng(80 + gate)
    T, dk, dv, d = 100, 16, 64, 7
    inp = _inputs(rng, 1, T, 2, dk, dv, gate, s0=0.4)
    do = rng.standard_normal(inp[2].shape)
    dST = rng.standard_normal(inp[5].shape)
    kw = dict(qdq_mode=oracle.QDQ_E4M3, group=64, qdq_interval=64)
    r = oc.bwd(*inp, do, dST, gate=gate, solve=oc.SOLVE_NEUMANN, degree=d, **kw)
    o_or, ST_or, _ = oc.fwd(*inp, gate=gate, solve=oc.SOLVE_NEUMANN, degree=d, **kw)
    ts = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in inp]
    o, ST = _torch_chunked_ste(*ts, gate, d, oracle.QDQ_E4M3, 64, 64)
    np.testing.assert_allclose(o.detach().numpy(), o_or, atol=1e-10)
    np.testing.assert_allclose(ST.detach().numpy(), ST_or, atol=1e-10)
    L = (o * torch.from_numpy(do)).sum() + (ST * torch.from_numpy(dST)).sum()
    L.backward()
    for name, t in zip(["dq", "dk", "dv", "dg", "dbeta", "dS0"], ts):
        np.testing.assert_allclose(r[name], t.grad.numpy(), rtol=1e-9, atol=1e-10, err_msg=name)


def test_given_chunk_states_equal_recompute(oracle_mod):
    rng = np.random.default_rng(90)
    inp = _inputs(rng, 1, 140, 1, 16, 64, G_KEY)
    do = rng.standard_normal(inp[2].shape)
    kw = dict(gate=G_KEY, solve=oc.SOLVE_NEUMANN, degree=15, qdq_mode=oracle.QDQ_E4M3, group=64, qdq_interval=64)
    cks = oc.fwd(*inp, return_chunk_states=True, **kw)[3]
    r1 = oc.bwd(*inp, do, **kw)
    r2 = oc.bwd(*inp, do, chunk_states=cks, **kw)
    for n in r1:
        np.testing.assert_array_equal(r1[n], r2[n])


def test_rounding_points_must_fall_on_chunk_ends(oracle_mod):
    rng = np.random.default_rng(91)
    inp = _inputs(rng, 1, 70, 1, 8, 64, G_SCALAR)
    with pytest.raises(ValueError):
        oc.fwd(*inp, qdq_mode=oracle.QDQ_E4M3, group=64, qdq_interval=32)
    with pytest.raises(ValueError):
        oc.fwd(*inp, ckpt_interval=16)
