"""CPU oracle (float64) for the gated delta rule recurrence with state fake-quantization.

TEST INFRASTRUCTURE ONLY: this package may be imported by the tests, by
``__graft_entry__.smoke()`` and by the bench's CPU-baseline leg, never by the
library.  It wraps ``oracle.c`` (plain C, built with gcc) through ctypes and
shares no code with the GPU path.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_DIR, "oracle.c")
_LIB = os.path.join(_DIR, "liboracle.so")

GATE_SCALAR, GATE_KEY = 0, 1
QDQ_NONE, QDQ_INT8, QDQ_E4M3 = 0, 1, 2


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < max(
        os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_DIR, "oracle.h"))
    ):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-fPIC", "-shared", "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True, cwd=_DIR)
        os.replace(tmp, _LIB)
    return _LIB


class _Cfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in
                ("B", "T", "H", "dk", "dv", "gate", "qdq", "group", "hadamard", "qdq_interval",
                 "ckpt_interval", "replay")]


_lib = None


def _load():
    global _lib
    if _lib is None:
        path = build()
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_set_num_threads.restype = None
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.oracle_e4m3_value.restype = ctypes.c_double
        lib.oracle_e4m3_value.argtypes = [ctypes.c_int]
        lib.oracle_e4m3_code.restype = ctypes.c_int
        lib.oracle_e4m3_code.argtypes = [ctypes.c_double]
        lib.oracle_hadamard.restype = None
        lib.oracle_hadamard.argtypes = [ctypes.c_int, ctypes.c_int, dp, dp]
        lib.oracle_qdq.restype = ctypes.c_int
        lib.oracle_qdq.argtypes = [ctypes.c_int] * 5 + [dp, dp, ctypes.c_void_p, ctypes.c_void_p,
                                                       ctypes.c_void_p]
        lib.oracle_fwd.restype = ctypes.c_int
        lib.oracle_fwd.argtypes = [ctypes.POINTER(_Cfg)] + [ctypes.c_void_p] * 9
        lib.oracle_fwd_ex.restype = ctypes.c_int
        lib.oracle_fwd_ex.argtypes = [ctypes.POINTER(_Cfg)] + [ctypes.c_void_p] * 11
        lib.oracle_bf16.restype = ctypes.c_double
        lib.oracle_bf16.argtypes = [ctypes.c_double]
        lib.oracle_bwd.restype = ctypes.c_int
        lib.oracle_bwd.argtypes = [ctypes.POINTER(_Cfg)] + [ctypes.c_void_p] * 15
        _lib = lib
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _d(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def num_threads() -> int:
    """Threads the oracle's parallel loops over (sequence, head) units use."""
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads for later calls (OpenMP); the CPU baseline times the oracle at 1 and at all."""
    _load().oracle_set_num_threads(int(n))


def e4m3_value(code: int) -> float:
    return _load().oracle_e4m3_value(int(code))


def e4m3_code(y: float) -> int:
    return _load().oracle_e4m3_code(float(y))


def hadamard(X: np.ndarray) -> np.ndarray:
    """Hn X along the first (key) axis of a d_k x d_v matrix."""
    X = _d(X)
    Y = np.empty_like(X)
    dp = ctypes.POINTER(ctypes.c_double)
    _load().oracle_hadamard(X.shape[0], X.shape[1], X.ctypes.data_as(dp), Y.ctypes.data_as(dp))
    return Y


def qdq(X: np.ndarray, mode: int, group: int, hadamard: bool = False):
    """Fake-quantize one d_k x d_v state; returns (Xhat, codes, scales, ypre)."""
    X = _d(X)
    dk, dv = X.shape
    Xh = np.empty_like(X)
    codes = np.zeros((dk, dv), dtype=np.int32)
    nsc = (dk * (dv // group)) if mode == QDQ_INT8 else (dv // group)
    scales = np.zeros(nsc, dtype=np.float32)
    ypre = np.zeros((dk, dv), dtype=np.float32)
    dp = ctypes.POINTER(ctypes.c_double)
    rc = _load().oracle_qdq(mode, group, int(hadamard), dk, dv, X.ctypes.data_as(dp),
                            Xh.ctypes.data_as(dp), _p(codes), _p(scales), _p(ypre))
    if rc:
        raise ValueError("oracle_qdq rejected its arguments")
    return Xh, codes, scales, ypre


def _cfg(B, T, H, dk, dv, gate, qdq_mode, group, hadamard, qdq_interval, ckpt_interval, replay=False):
    return _Cfg(B, T, H, dk, dv, gate, qdq_mode, group, int(hadamard), qdq_interval, ckpt_interval, int(replay))


def bf16(x: float) -> float:
    """Nearest BF16 value to fl32(x) (ties to even), the replay windows' entry encoding."""
    return _load().oracle_bf16(float(x))


def fwd(q, k, v, g, beta, S0=None, *, gate=GATE_SCALAR, qdq_mode=QDQ_NONE, group=32,
        hadamard=False, qdq_interval=1, ckpt_interval=0, replay=False, dhat=None, return_deltas=False):
    """Forward recurrence.  Returns (o, S_T, ckpts or None), all float64, and the deltas of
    every token [B, T, H, d_v] as a fourth item when return_deltas.  replay: replay windows of
    qdq_interval tokens (BF16 key and update entries between rounding points); dhat
    [B, T, H, d_v]: the update entries to use at the tokens that are not rounding points (NaN:
    encode the oracle's own delta), for teacher forcing."""
    q, k, v, g, beta = map(_d, (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S0 = None if S0 is None else _d(S0)
    dhat = None if dhat is None else _d(dhat)
    o = np.zeros((B, T, H, dv))
    ST = np.zeros((B, H, dk, dv))
    deltas = np.zeros((B, T, H, dv)) if return_deltas else None
    ck = None
    if ckpt_interval > 0:
        ck = np.zeros((B, H, (T + ckpt_interval - 1) // ckpt_interval, dk, dv))
    c = _cfg(B, T, H, dk, dv, gate, qdq_mode, group, hadamard, qdq_interval, ckpt_interval, replay)
    rc = _load().oracle_fwd_ex(ctypes.byref(c), _p(q), _p(k), _p(v), _p(g), _p(beta), _p(S0), _p(o),
                               _p(ST), _p(ck), _p(dhat), _p(deltas))
    if rc:
        raise ValueError("oracle_fwd rejected its configuration")
    return (o, ST, ck, deltas) if return_deltas else (o, ST, ck)


def fwd_varlen(q, k, v, g, beta, cu_seqlens, S0=None, *, gate=GATE_SCALAR, qdq_mode=QDQ_NONE, group=32,
               hadamard=False, qdq_interval=1):
    """Forward over packed sequences (the pages' packed sequence tails): q, k, v, g, beta hold the
    tokens of all sequences one after another ([T, H, ...], no batch axis), sequence b being
    tokens cu_seqlens[b] .. cu_seqlens[b + 1] - 1 (boundaries clamped to [0, T], an inverted
    pair is an empty sequence).  Each sequence is the forward above on its own tokens, from
    S0[b] (zeros when S0 is None), with its own rounding points.  Returns (o [T, H, d_v],
    S_T [B, H, d_k, d_v]), float64; tokens outside every sequence give o = 0."""
    q, k, v, g, beta = map(_d, (q, k, v, g, beta))
    T, H, dk = q.shape
    dv = v.shape[-1]
    B = len(cu_seqlens) - 1
    o = np.zeros((T, H, dv))
    ST = np.zeros((B, H, dk, dv))
    for b in range(B):
        t0 = min(max(int(cu_seqlens[b]), 0), T)
        t1 = min(max(int(cu_seqlens[b + 1]), t0), T)
        S0b = None if S0 is None else _d(S0)[b:b + 1]
        if t1 == t0:
            ST[b] = 0.0 if S0b is None else S0b[0]
            continue
        ob, STb, _ = fwd(q[None, t0:t1], k[None, t0:t1], v[None, t0:t1], g[None, t0:t1], beta[None, t0:t1], S0b,
                         gate=gate, qdq_mode=qdq_mode, group=group, hadamard=hadamard, qdq_interval=qdq_interval)
        o[t0:t1] = ob[0]
        ST[b] = STb[0]
    return o, ST


def decode_slots(q, k, v, g, beta, S_pool, slots, *, gate=GATE_SCALAR, qdq_mode=QDQ_NONE, group=32,
                 hadamard=False):
    """One decode token over a pool of state slots (the serving adapter's paged cache with index
    zero reserved; linear-attention state-QAT pages, "Torch/Triton GDN/KDA decode QAT").  Entry
    b of the batch (q, k, v, g, beta of shape [B, 1, H, ...]) advances pool slot slots[b] by the
    forward step above with a rounding point at its token; slot 0 and indices outside the pool
    are padding: o[b] = 0 and the pool is left as it was.  Returns (o [B, 1, H, d_v], new pool),
    float64.  Entries are taken one at a time, in order."""
    q, k, v, g, beta = map(_d, (q, k, v, g, beta))
    pool = _d(S_pool).copy()
    B, T, H, dk = q.shape
    assert T == 1
    dv = v.shape[-1]
    o = np.zeros((B, 1, H, dv))
    for b in range(B):
        sl = int(slots[b])
        if sl <= 0 or sl >= pool.shape[0]:
            continue
        ob, Sb, _ = fwd(q[b:b + 1], k[b:b + 1], v[b:b + 1], g[b:b + 1], beta[b:b + 1], pool[sl:sl + 1],
                        gate=gate, qdq_mode=qdq_mode, group=group, hadamard=hadamard, qdq_interval=1)
        o[b] = ob[0]
        pool[sl] = Sb[0]
    return o, pool


def bwd(q, k, v, g, beta, S0, dout, dST=None, states=None, *, gate=GATE_SCALAR,
        qdq_mode=QDQ_NONE, group=32, hadamard=False, qdq_interval=1, replay=False):
    """Straight-through backward.  Returns dict of dq, dk, dv, dg, dbeta, dS0 (float64)."""
    q, k, v, g, beta, dout = map(_d, (q, k, v, g, beta, dout))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S0 = None if S0 is None else _d(S0)
    dST = None if dST is None else _d(dST)
    states = None if states is None else _d(states)
    out = {
        "dq": np.zeros_like(q), "dk": np.zeros_like(k), "dv": np.zeros_like(v),
        "dg": np.zeros_like(g), "dbeta": np.zeros_like(beta), "dS0": np.zeros((B, H, dk, dv)),
    }
    c = _cfg(B, T, H, dk, dv, gate, qdq_mode, group, hadamard, qdq_interval, 0, replay)
    rc = _load().oracle_bwd(ctypes.byref(c), _p(q), _p(k), _p(v), _p(g), _p(beta), _p(S0),
                            _p(states), _p(dout), _p(dST), _p(out["dq"]), _p(out["dk"]),
                            _p(out["dv"]), _p(out["dg"]), _p(out["dbeta"]), _p(out["dS0"]))
    if rc:
        raise ValueError("oracle_bwd rejected its configuration")
    return out


def _seq_range(cu_seqlens, b, T):
    t0 = min(max(int(cu_seqlens[b]), 0), T)
    t1 = min(max(int(cu_seqlens[b + 1]), t0), T)
    return t0, t1


def bwd_varlen(q, k, v, g, beta, cu_seqlens, S0, dout, dST=None, *, gate=GATE_SCALAR, qdq_mode=QDQ_NONE, group=32,
               hadamard=False, qdq_interval=1, replay=False, states=None):
    """Straight-through backward of fwd_varlen: each sequence's backward on its own tokens
    ([T, H, ...] packing, sequence b = tokens cu_seqlens[b] .. cu_seqlens[b + 1] - 1, clamped),
    from S0[b] and dST[b].  states: optional [T, H, d_k, d_v], the carried state entering each
    packed token (teacher forcing).  Tokens outside every sequence get zero gradients; an empty
    sequence hands dST through as dS0.  Returns the gradients (packed) and dS0 [B, H, d_k, d_v]."""
    q, k, v, g, beta, dout = map(_d, (q, k, v, g, beta, dout))
    T, H, dk = q.shape
    dv = v.shape[-1]
    B = len(cu_seqlens) - 1
    out = {"dq": np.zeros_like(q), "dk": np.zeros_like(k), "dv": np.zeros_like(v), "dg": np.zeros_like(g),
           "dbeta": np.zeros_like(beta), "dS0": np.zeros((B, H, dk, dv))}
    for b in range(B):
        t0, t1 = _seq_range(cu_seqlens, b, T)
        S0b = None if S0 is None else _d(S0)[b:b + 1]
        dSTb = None if dST is None else _d(dST)[b:b + 1]
        if t1 == t0:
            out["dS0"][b] = 0.0 if dSTb is None else dSTb[0]
            continue
        st = None if states is None else _d(states)[None, t0:t1].transpose(0, 2, 1, 3, 4)
        r = bwd(q[None, t0:t1], k[None, t0:t1], v[None, t0:t1], g[None, t0:t1], beta[None, t0:t1], S0b,
                dout[None, t0:t1], dSTb, states=st, gate=gate, qdq_mode=qdq_mode, group=group, hadamard=hadamard,
                qdq_interval=qdq_interval, replay=replay)
        for n in ("dq", "dk", "dv", "dg", "dbeta"):
            out[n][t0:t1] = r[n][0]
        out["dS0"][b] = r["dS0"][0]
    return out


def _split_ranges(cu_seqlens, prefix_len, T):
    B = len(cu_seqlens) - 1
    pre, suf = [], []
    for b in range(B):
        t0, t1 = _seq_range(cu_seqlens, b, T)
        mid = min(max(t0 + int(prefix_len[b]), t0), t1)
        pre.append((t0, mid))
        suf.append((mid, t1))
    return pre, suf


def _ranges_to_cu(ranges, T):
    """Packing of sub-ranges into a token index list and a cumulative offset array."""
    idx = np.concatenate([np.arange(a, b) for a, b in ranges]) if ranges else np.zeros(0, dtype=np.int64)
    cu = np.concatenate([[0], np.cumsum([b - a for a, b in ranges])]).astype(np.int64)
    return idx.astype(np.int64), cu


def fwd_split(q, k, v, g, beta, cu_seqlens, prefix_len, S0, prefix_kw, suffix_kw, *, gate=GATE_SCALAR):
    """Packed sequences cut at a per-sequence boundary (the pages' chunked-prefill prefix and
    recurrent suffix with the state handed over between them): sequence b's first
    prefix_len[b] tokens (clamped) run fwd with prefix_kw from S0[b], the rest with suffix_kw
    from the prefix's final state S_mid[b].  Returns (o [T, H, d_v], S_mid, S_T), float64."""
    q, k, v, g, beta = map(_d, (q, k, v, g, beta))
    T, H, dk = q.shape
    pre, suf = _split_ranges(cu_seqlens, prefix_len, T)
    o = np.zeros((T, H, v.shape[-1]))
    ip, cp = _ranges_to_cu(pre, T)
    o_p, S_mid = fwd_varlen(q[ip], k[ip], v[ip], g[ip], beta[ip], cp, S0, gate=gate, **prefix_kw)
    o[ip] = o_p
    is_, cs = _ranges_to_cu(suf, T)
    o_s, S_T = fwd_varlen(q[is_], k[is_], v[is_], g[is_], beta[is_], cs, S_mid, gate=gate, **suffix_kw)
    o[is_] = o_s
    return o, S_mid, S_T


def bwd_split(q, k, v, g, beta, cu_seqlens, prefix_len, S0, S_mid, dout, dST, prefix_kw, suffix_kw, *,
              gate=GATE_SCALAR, states=None):
    """Straight-through backward of fwd_split: the suffixes' backward from S_mid for dout and
    dST, whose dS0 is the gradient at the handoff; then the prefixes' backward from S0 with it
    as their dST.  states: optional [T, H, d_k, d_v] carried states entering each token
    (teacher forcing).  Returns the packed gradients and dS0."""
    q, k, v, g, beta, dout = map(_d, (q, k, v, g, beta, dout))
    T = q.shape[0]
    pre, suf = _split_ranges(cu_seqlens, prefix_len, T)
    out = {"dq": np.zeros_like(q), "dk": np.zeros_like(k), "dv": np.zeros_like(v), "dg": np.zeros_like(g),
           "dbeta": np.zeros_like(beta)}
    is_, cs = _ranges_to_cu(suf, T)
    st_s = None if states is None else _d(states)[is_]
    r_s = bwd_varlen(q[is_], k[is_], v[is_], g[is_], beta[is_], cs, S_mid, dout[is_], dST, gate=gate, states=st_s,
                     **suffix_kw)
    ip, cp = _ranges_to_cu(pre, T)
    st_p = None if states is None else _d(states)[ip]
    r_p = bwd_varlen(q[ip], k[ip], v[ip], g[ip], beta[ip], cp, S0, dout[ip], r_s["dS0"], gate=gate, states=st_p,
                     **prefix_kw)
    for n in out:
        out[n][is_] = r_s[n]
        out[n][ip] = r_p[n]
    out["dS0"] = r_p["dS0"]
    out["dS_mid"] = r_s["dS0"]
    return out
