"""CPU oracle (float64, NumPy) of the 64-token chunked form of the gated delta rule, with the
exact triangular solve or the Neumann approximate inverse inside each chunk.

TEST INFRASTRUCTURE ONLY: imported by the tests, by ``__graft_entry__.smoke()`` and by the
bench's CPU-baseline leg, never by the library.  It shares no code with the GPU path; the
rounding of the state at chunk ends calls this package's own codec (``oracle.qdq``).

What is computed ("GDN state/W QAT foundation", What does this PR do?: state QDQ on 64-token
chunks, rounding at each chunk boundary; "Experimental GDN/KDA approximate-inverse QAT", What
does this PR do?: an explicit Neumann polynomial degree replaces the chunk's exact triangular
solve, and the backward differentiates that polynomial).  Per sequence b and head h the tokens
are cut into chunks of 64 from the start of the call (the last one may be shorter).  For one
chunk of L tokens entering with the carried state S (d_k x d_v), with per-key log decays g_r
(a scalar gate is the same value on every key) and the cumulative sums G_r = g_0 + ... + g_r:

    D_ri[k] = exp(G_r[k] - G_i[k])                     (i <= r; the decay from token i to r)
    A_ri    = beta_r sum_k k_r[k] k_i[k] D_ri[k]        (i < r, else 0: strictly lower)
    M_ri    = sum_k q_r[k] k_i[k] D_ri[k]               (i <= r, else 0)
    P       = (I + A)^-1              exact solve
            = sum_{n=0}^{d} (-A)^n    Neumann polynomial of degree d
    U       = V - (K o E) S,  E_r = exp(G_r)            R = diag(beta) U
    Delta   = P R                                       (the chunk's deltas)
    O       = (Q o E) S + M Delta                       (outputs, read before rounding)
    S_end   = diag(E_{L-1}) S + (K o F)^T Delta,  F_i = exp(G_{L-1} - G_i)

then S_end is rounded when the chunk ends on a rounding point (every qdq_interval tokens, a
multiple of 64, and the last token of the call).  With the exact solve this is the token
recurrence regrouped: (I + A) Delta = R is the recurrence's delta_r = beta_r (v_r - S~_r^T k_r)
written for all tokens of the chunk at once.  A is strictly lower triangular, so A^L = 0 and
the Neumann polynomial of degree d >= L - 1 is the exact inverse.
"""
from __future__ import annotations

import numpy as np

from . import GATE_KEY, GATE_SCALAR, QDQ_NONE, qdq

SOLVE_EXACT, SOLVE_NEUMANN = 0, 1
CHUNK = 64


def neumann(A: np.ndarray, degree: int) -> np.ndarray:
    """sum_{n=0}^{degree} (-A)^n, the power sum written out term by term."""
    n = A.shape[0]
    X = -A
    term = np.eye(n)
    P = np.eye(n)
    for _ in range(degree):
        term = term @ X
        P = P + term
    return P


def neumann_grad(A: np.ndarray, degree: int, dP: np.ndarray) -> np.ndarray:
    """Gradient with respect to A of <dP, neumann(A, degree)>: with X = -A and Y = X^T, the
    derivative of X^n contracted with dP is W_n = sum_{a<n} Y^a dP Y^(n-1-a), which obeys
    W_1 = dP, W_{n+1} = Y W_n + dP Y^n; the result is -(W_1 + ... + W_degree)."""
    Y = -A.T
    W = dP.copy()
    Yn = Y.copy()
    acc = np.zeros_like(dP)
    for n in range(1, degree + 1):
        acc += W
        if n < degree:
            W = Y @ W + dP @ Yn
            Yn = Yn @ Y
    return -acc


def _solve(A, solve, degree):
    if solve == SOLVE_EXACT:
        return np.linalg.inv(np.eye(A.shape[0]) + A)
    return neumann(A, degree)


def _solve_grad(A, P, dP, solve, degree):
    if solve == SOLVE_EXACT:
        return -P.T @ dP @ P.T          # d(I + A)^-1 = -P dA P
    return neumann_grad(A, degree, dP)


def _key_gates(g, gate, dk):
    """Per-key log decays [B, T, H, d_k]: a scalar gate repeated over the keys."""
    g = np.asarray(g, dtype=np.float64)
    if gate == GATE_KEY:
        return g
    return np.repeat(g[..., None], dk, axis=-1)


def _chunk_forward(qc, kc, vc, gc, bc, S, solve, degree):
    """One chunk's terms (see the module docstring); returns the outputs, the end state before
    rounding and the intermediates the backward needs."""
    L = len(bc)
    low = np.tril(np.ones((L, L)), -1)
    lowd = np.tril(np.ones((L, L)))
    G = np.cumsum(gc, axis=0)
    diff = np.where(lowd[:, :, None] > 0, G[:, None, :] - G[None, :, :], 0.0)
    D = np.exp(diff) * lowd[:, :, None]
    Bm = np.einsum("rk,ik,rik->ri", kc, kc, D) * low
    A = bc[:, None] * Bm
    M = np.einsum("rk,ik,rik->ri", qc, kc, D) * lowd
    P = _solve(A, solve, degree)
    E = np.exp(G)
    F = np.exp(G[-1][None, :] - G)
    Kp, Qp, Kd = kc * E, qc * E, kc * F
    U = vc - Kp @ S
    R = bc[:, None] * U
    Delta = P @ R
    O = Qp @ S + M @ Delta
    S_end = E[-1][:, None] * S + Kd.T @ Delta
    return O, S_end, dict(G=G, D=D, Bm=Bm, A=A, M=M, P=P, E=E, F=F, Kp=Kp, Qp=Qp, Kd=Kd, U=U, R=R, Delta=Delta,
                          low=low, lowd=lowd)


def _chunk_backward(qc, kc, bc, S, dS_end, dO, t, solve, degree):
    """Chain rule through one chunk (t: the forward's intermediates); returns the gradients of
    the chunk's q, k, v, per-key g, beta and of its entering state S."""
    L = len(bc)
    dDelta = t["Kd"] @ dS_end + t["M"].T @ dO
    dR = t["P"].T @ dDelta
    dU = bc[:, None] * dR
    dS = t["E"][-1][:, None] * dS_end + t["Qp"].T @ dO - t["Kp"].T @ dU
    dv = dU
    dbeta = np.sum(dR * t["U"], axis=1)
    dKp = -dU @ S.T
    dQp = dO @ S.T
    dKd = t["Delta"] @ dS_end.T
    dEL = np.sum(dS_end * S, axis=1)
    dP = dDelta @ t["R"].T
    dM = (dO @ t["Delta"].T) * t["lowd"]
    dA = _solve_grad(t["A"], t["P"], dP, solve, degree) * t["low"]
    dbeta += np.sum(dA * t["Bm"], axis=1)
    dBm = bc[:, None] * dA
    D = t["D"]
    dq = np.einsum("ri,ik,rik->rk", dM, kc, D) + dQp * t["E"]
    dk = (np.einsum("ri,ik,rik->rk", dBm, kc, D) + np.einsum("ri,rk,rik->ik", dBm, kc, D)
          + np.einsum("ri,rk,rik->ik", dM, qc, D) + dKp * t["E"] + dKd * t["F"])
    # d/dG through D_ri = exp(G_r - G_i): + at r, - at i
    dDD = (dBm[:, :, None] * kc[:, None, :] * kc[None, :, :] + dM[:, :, None] * qc[:, None, :] * kc[None, :, :]) * D
    dG = dDD.sum(axis=1) - dDD.sum(axis=0)
    dG += dKp * t["Kp"] + dQp * t["Qp"]            # E_r = exp(G_r)
    dG -= dKd * t["Kd"]                            # F_i = exp(G_{L-1} - G_i)
    dG[L - 1] += np.sum(dKd * t["Kd"], axis=0) + dEL * t["E"][-1]
    dg = np.cumsum(dG[::-1], axis=0)[::-1]        # G_r = g_0 + ... + g_r
    return dq, dk, dv, dg, dbeta, dS


def _check(T, qdq_mode, qdq_interval, ckpt_interval, chunk):
    if qdq_mode != QDQ_NONE and (qdq_interval < 1 or qdq_interval % chunk != 0):
        raise ValueError("rounding points must fall on chunk ends: qdq_interval a multiple of the chunk")
    if ckpt_interval and ckpt_interval % chunk != 0:
        raise ValueError("checkpoints must fall on chunk starts")


def _rounds(c_end, T, qdq_mode, qdq_interval):
    return qdq_mode != QDQ_NONE and (c_end % qdq_interval == 0 or c_end == T)


def fwd(q, k, v, g, beta, S0=None, *, gate=GATE_SCALAR, solve=SOLVE_EXACT, degree=3, qdq_mode=QDQ_NONE, group=64,
        hadamard=False, qdq_interval=CHUNK, ckpt_interval=0, chunk=CHUNK, return_chunk_states=False):
    """Chunked forward.  q, k [B, T, H, d_k]; v [B, T, H, d_v]; g [B, T, H] (scalar gate) or
    [B, T, H, d_k] (per-key); beta [B, T, H]; S0 [B, H, d_k, d_v] or None (zeros).  Returns
    (o, S_T, ckpts or None) in float64, and the carried state entering every chunk
    [B, H, n_chunks, d_k, d_v] as a fourth item when return_chunk_states."""
    q, k, v, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    _check(T, qdq_mode, qdq_interval, ckpt_interval, chunk)
    gk = _key_gates(g, gate, dk)
    nch = (T + chunk - 1) // chunk
    o = np.zeros((B, T, H, dv))
    ST = np.zeros((B, H, dk, dv))
    cks = np.zeros((B, H, nch, dk, dv))
    ck = np.zeros((B, H, (T + ckpt_interval - 1) // ckpt_interval, dk, dv)) if ckpt_interval else None
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else np.asarray(S0[b, h], dtype=np.float64).copy()
            for c in range(nch):
                t0, t1 = c * chunk, min(T, (c + 1) * chunk)
                cks[b, h, c] = S
                if ck is not None and t0 % ckpt_interval == 0:
                    ck[b, h, t0 // ckpt_interval] = S
                O, S, _ = _chunk_forward(q[b, t0:t1, h], k[b, t0:t1, h], v[b, t0:t1, h], gk[b, t0:t1, h],
                                         beta[b, t0:t1, h], S, solve, degree)
                o[b, t0:t1, h] = O
                if _rounds(t1, T, qdq_mode, qdq_interval):
                    S = qdq(S, qdq_mode, group, hadamard)[0]
            ST[b, h] = S
    out = (o, ST, ck)
    return out + (cks,) if return_chunk_states else out


def bwd(q, k, v, g, beta, S0, dout, dST=None, *, gate=GATE_SCALAR, solve=SOLVE_EXACT, degree=3, qdq_mode=QDQ_NONE,
        group=64, hadamard=False, qdq_interval=CHUNK, chunk=CHUNK, chunk_states=None):
    """Straight-through backward of fwd: identity gradient through every rounding, the chain
    rule through each chunk's terms (through the Neumann polynomial itself, not the inverse it
    approximates).  chunk_states [B, H, n_chunks, d_k, d_v]: the carried state entering each
    chunk (teacher forcing); recomputed by fwd when None.  Returns dq, dk, dv, dg (shaped like
    g), dbeta, dS0, all float64."""
    q, k, v, beta, dout = (np.asarray(x, dtype=np.float64) for x in (q, k, v, beta, dout))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    _check(T, qdq_mode, qdq_interval, 0, chunk)
    gk = _key_gates(g, gate, dk)
    nch = (T + chunk - 1) // chunk
    if chunk_states is None:
        chunk_states = fwd(q, k, v, g, beta, S0, gate=gate, solve=solve, degree=degree, qdq_mode=qdq_mode,
                           group=group, hadamard=hadamard, qdq_interval=qdq_interval, chunk=chunk,
                           return_chunk_states=True)[3]
    out = {"dq": np.zeros_like(q), "dk": np.zeros_like(k), "dv": np.zeros_like(v), "dgk": np.zeros_like(gk),
           "dbeta": np.zeros_like(beta), "dS0": np.zeros((B, H, dk, dv))}
    for b in range(B):
        for h in range(H):
            dS = np.zeros((dk, dv)) if dST is None else np.asarray(dST[b, h], dtype=np.float64).copy()
            for c in reversed(range(nch)):
                t0, t1 = c * chunk, min(T, (c + 1) * chunk)
                S = np.asarray(chunk_states[b, h, c], dtype=np.float64)
                qc, kc, bc = q[b, t0:t1, h], k[b, t0:t1, h], beta[b, t0:t1, h]
                _, _, t = _chunk_forward(qc, kc, v[b, t0:t1, h], gk[b, t0:t1, h], bc, S, solve, degree)
                dq, dk_, dv_, dg, db, dS = _chunk_backward(qc, kc, bc, S, dS, dout[b, t0:t1, h], t, solve, degree)
                out["dq"][b, t0:t1, h] = dq
                out["dk"][b, t0:t1, h] = dk_
                out["dv"][b, t0:t1, h] = dv_
                out["dgk"][b, t0:t1, h] = dg
                out["dbeta"][b, t0:t1, h] = db
            out["dS0"][b, h] = dS
    dgk = out.pop("dgk")
    out["dg"] = dgk if gate == GATE_KEY else dgk.sum(axis=-1)
    return out
