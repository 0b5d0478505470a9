"""Helpers for the GPU parity tests: device transfer of generated inputs, calls through the
C ABI, the error metric and the quantization-code comparison protocol.

Error metric: e(x, ref) = max|x - ref| / max|ref| over a whole tensor.
Code protocol (teacher forced): at a quantization point the GPU's carried state and the
oracle's must agree code for code; the only allowed differences are +-1 at near-ties
(where the oracle's pre-rounding value lies within TIE_WINDOW of a rounding boundary; for
E4M3, neighbouring grid values of one sign with the oracle's x/s within E4M3_TIE_WINDOW of
their midpoint), on at most 1e-4 of the codes of a whole test (of
CODE_MIN_SAMPLE codes for smaller tests).
"""
from __future__ import annotations

import math

import numpy as np

import oracle
import quantized_state_qat_amd as la
import synth

TIE_WINDOW = 2e-3          # distance of x/s to a rounding boundary, in code units
# The same window for E4M3, as a distance of x/s to the midpoint of two grid values: x/s
# spans +-448 where an INT8 code spans +-127, so this is the same distance relative to the
# largest magnitude of the tile (1.6e-5 amax).  A window relative to the local grid step
# would shrink 64-fold in the subnormal range, where fp32-against-float64 differences of a
# state relative to its largest element are the same as anywhere else.
E4M3_TIE_WINDOW = TIE_WINDOW * 448.0 / 127.0
CODE_MISMATCH_MAX = 1e-4   # fraction of codes allowed to differ (by one, at near-ties)
# A fraction of 1e-4 cannot resolve a handful of near-tie flips on a small sample, so a
# tally of fewer codes than this is held to the budget of this many (ten mismatches); every
# mismatch must still be one step at a near-tie.
CODE_MIN_SAMPLE = 100_000
TOL_BF16 = 2e-3            # output/state error bound with bf16 inputs
TOL_F32 = 1e-5             # output/state error bound with fp32 inputs


def torch_mod():
    import torch
    return torch


def dev(t: synth.Tensor):
    """Device tensor with the storage dtype of a generated tensor."""
    torch = torch_mod()
    if t.dtype == "bf16":
        return torch.from_numpy(t.bits.astype(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(t.f32)).cuda()


def dtype_code(t: synth.Tensor) -> int:
    return la.LA_BF16 if t.dtype == "bf16" else la.LA_F32


def err(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max()
    if den == 0:
        return float(np.abs(x).max())
    return float(np.abs(x - ref).max() / den)


def cfg_for(w: synth.Workload, d, **kw) -> la.Config:
    c = la.Config(B=w.B, T=w.T, H=w.H, d_k=w.d_k, d_v=w.d_v,
                  gate=la.LA_GATE_KEY if w.gate == "key" else la.LA_GATE_SCALAR,
                  qkv_dtype=dtype_code(d["q"]), gate_dtype=dtype_code(d["g"]))
    for k_, v_ in kw.items():
        setattr(c, k_, v_)
    return c


def nan_like(torch, shape, dtype=None):
    return torch.full(shape, float("nan"), dtype=dtype or torch.float32, device="cuda")


def run_fwd(c: la.Config, d, S0=None, ckpt_interval=0, dev_inputs=None):
    """GPU forward; returns numpy (o, S_T, ckpts or None)."""
    torch = torch_mod()
    c.ckpt_interval = ckpt_interval
    di = dev_inputs or {k: dev(d[k]) for k in ("q", "k", "v", "g", "beta")}
    S0d = None
    if S0 is not None:
        S0d = torch.from_numpy(np.ascontiguousarray(S0, dtype=np.float32)).cuda()
    o = nan_like(torch, (c.B, c.T, c.H, c.d_v), torch.float32 if c.out_dtype == la.LA_F32 else torch.bfloat16)
    ST = nan_like(torch, (c.B, c.H, c.d_k, c.d_v))
    ck = None
    if ckpt_interval > 0:
        nck = (c.T + ckpt_interval - 1) // ckpt_interval
        ck = nan_like(torch, (c.B, c.H, nck, c.d_k, c.d_v))
    la.la_recurrent_fwd(c, di["q"], di["k"], di["v"], di["g"], di["beta"], S0d, o, ST, ck)
    torch.cuda.synchronize()
    return (o.float().cpu().numpy(), ST.cpu().numpy(), None if ck is None else ck.cpu().numpy())


def run_bwd(c: la.Config, d, dout, S0=None, dST=None, ckpts=None, dev_inputs=None):
    torch = torch_mod()
    di = dev_inputs or {k: dev(d[k]) for k in ("q", "k", "v", "g", "beta")}
    f = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    gshape = (c.B, c.T, c.H, c.d_k) if c.gate == la.LA_GATE_KEY else (c.B, c.T, c.H)
    out = {
        "dq": nan_like(torch, (c.B, c.T, c.H, c.d_k)), "dk": nan_like(torch, (c.B, c.T, c.H, c.d_k)),
        "dv": nan_like(torch, (c.B, c.T, c.H, c.d_v)), "dg": nan_like(torch, gshape),
        "dbeta": nan_like(torch, (c.B, c.T, c.H)), "dS0": nan_like(torch, (c.B, c.H, c.d_k, c.d_v)),
    }
    nbytes = la.la_bwd_workspace_bytes(c)
    ws = torch.full((nbytes // 4 + 1,), float("nan"), dtype=torch.float32, device="cuda")
    la.la_recurrent_bwd_ste(c, di["q"], di["k"], di["v"], di["g"], di["beta"], f(S0), f(ckpts), f(dout),
                            f(dST), out["dq"], out["dk"], out["dv"], out["dg"], out["dbeta"], out["dS0"],
                            ws, nbytes)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def int8_codes_from_state(X: np.ndarray, group: int):
    """Recover (codes, scales) from a dequantized INT8-group state [.., d_k, d_v]: the
    largest magnitude in a group is 127 * s (to one fp32 rounding)."""
    X = np.asarray(X, dtype=np.float64)
    G = X.reshape(*X.shape[:-1], X.shape[-1] // group, group)
    amax = np.abs(G).max(axis=-1, keepdims=True)
    s = np.where(amax > 0, amax / 127.0, 1.0)
    c = np.rint(G / s)
    return c.reshape(X.shape).astype(np.int32), s[..., 0]


def e4m3_codes_from_state(X: np.ndarray, tile: int = 64):
    """Recover E4M3 grid values (codes as values y) from a dequantized tile state [d_k, d_v]."""
    X = np.asarray(X, dtype=np.float64)
    dk, dv = X.shape[-2:]
    out = np.zeros_like(X)
    for t in range(dv // tile):
        sl = X[..., t * tile:(t + 1) * tile]
        amax = np.abs(sl).max()
        s = amax / 448.0 if amax > 0 else 1.0
        y = sl / s
        out[..., t * tile:(t + 1) * tile] = np.vectorize(lambda z: oracle.e4m3_value(oracle.e4m3_code(z)))(y)
    return out


# Non-negative E4M3FN values in increasing order, from the format's definition: subnormals
# m 2^-9 (m = 0..7), normals (1 + m/8) 2^(e-7) for e = 1..15 (e = 15, m = 7 is NaN; max 448).
E4M3_GRID = np.array([m * 2.0 ** -9 for m in range(8)]
                     + [(1 + m / 8) * 2.0 ** (e - 7) for e in range(1, 16) for m in range(8) if (e, m) != (15, 7)])


def compare_e4m3_values(yg: np.ndarray, yo: np.ndarray, tally: "CodeTally") -> None:
    """Add one quantization point's E4M3 grid values (GPU yg, oracle yo) to the tally; every
    mismatch must be a pair of neighbouring grid values of one sign (a near-tie decided the
    other way), or zero against the smallest subnormal."""
    yg = np.asarray(yg, dtype=np.float64)
    yo = np.asarray(yo, dtype=np.float64)
    bad = yg != yo
    tally.add(int(bad.sum()), yg.size)
    if bad.any():
        a, b = yg[bad], yo[bad]
        same_side = (np.sign(a) == np.sign(b)) | (a == 0) | (b == 0)
        ia = np.searchsorted(E4M3_GRID, np.abs(a))
        ib = np.searchsorted(E4M3_GRID, np.abs(b))
        assert np.all(E4M3_GRID[ia] == np.abs(a)) and np.all(E4M3_GRID[ib] == np.abs(b)), "values off the grid"
        assert np.all(same_side & (np.abs(ia - ib) == 1)), list(zip(a[:8], b[:8]))


_E4M3_TABLE = None


def e4m3_table() -> np.ndarray:
    """Value of every E4M3FN code 0..255 from the oracle's code table (0x7F/0xFF, NaN in the
    format, are never produced and map to the table's own value)."""
    global _E4M3_TABLE
    if _E4M3_TABLE is None:
        _E4M3_TABLE = np.array([oracle.e4m3_value(c) for c in range(256)])
    return _E4M3_TABLE


def e4m3_grid_of_state(X: np.ndarray, tile: int = 64) -> np.ndarray:
    """Grid values y (E4M3 values, float64) of a dequantized E4M3 tile state [..., d_k, d_v]:
    per tile of all d_k rows x `tile` columns the largest magnitude is 448 s, so X/s lies
    within fp32 rounding of a grid value; asserts that it does and returns that value."""
    X = np.asarray(X, dtype=np.float64)
    dk, dv = X.shape[-2:]
    T = X.reshape(*X.shape[:-1], dv // tile, tile)
    amax = np.abs(T).max(axis=(-3, -1), keepdims=True)
    s = np.where(amax > 0, amax / 448.0, 1.0)
    y = (T / s).reshape(X.shape)
    a = np.abs(y)
    i = np.clip(np.searchsorted(E4M3_GRID, a), 1, len(E4M3_GRID) - 1)
    lo, hi = E4M3_GRID[i - 1], E4M3_GRID[i]
    near = np.where(a - lo <= hi - a, lo, hi)
    assert np.all(np.abs(a - near) <= 1e-5 * np.maximum(near, 2.0 ** -9)), "state is not on the E4M3 grid"
    return np.copysign(near, y)


def compare_e4m3_point(gpu_state, ora_codes, ora_ypre, tally: "CodeTally", tile: int = 64) -> None:
    """Teacher-forced comparison of one E4M3 quantization point: the GPU's dequantized state
    [.., d_k, d_v] against the oracle's codes and pre-rounding values y = x/s for the same
    entering state.  Every mismatch must be a pair of neighbouring grid values of one sign
    (or zero against the smallest subnormal) with the oracle's y within E4M3_TIE_WINDOW of
    their midpoint; counts go to `tally`."""
    yg = e4m3_grid_of_state(gpu_state, tile)
    yo = e4m3_table()[np.asarray(ora_codes, dtype=np.int64) & 0xFF]
    bad = yg != yo
    tally.add(int(bad.sum()), yg.size)
    if bad.any():
        compare_e4m3_values(yg, yo, CodeTally())
        a, b = np.abs(yg[bad]), np.abs(yo[bad])
        y = np.abs(np.asarray(ora_ypre, dtype=np.float64)[bad])
        dist = np.abs(y - 0.5 * (a + b))
        assert dist.max() <= E4M3_TIE_WINDOW, f"E4M3 mismatch away from a tie (x/s {dist.max()} from the midpoint)"


def hadamard_n(n: int) -> np.ndarray:
    H = np.array([[1.0]])
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H / math.sqrt(n)


class CodeTally:
    """Counts compared codes and mismatches over a whole test; the 1e-4 budget applies to
    the total, each individual mismatch must be +-1 at a near-tie."""

    def __init__(self):
        self.mismatches = 0
        self.total = 0

    def add(self, mism: int, total: int) -> None:
        self.mismatches += int(mism)
        self.total += int(total)

    @property
    def fraction(self) -> float:
        return self.mismatches / self.total if self.total else 0.0

    def check(self) -> float:
        allowed = CODE_MISMATCH_MAX * max(self.total, CODE_MIN_SAMPLE)
        assert self.mismatches <= allowed, \
            f"code mismatch fraction {self.fraction} ({self.mismatches} of {self.total}, {allowed:.0f} allowed)"
        return self.fraction


def rotated_to_state(Y: np.ndarray) -> np.ndarray:
    """S = Hu Y / d_k (float64) for a state held rotated (Hadamard mode)."""
    Y = np.asarray(Y, dtype=np.float64)
    Hn = hadamard_n(Y.shape[-2])
    return np.einsum("ij,...jk->...ik", Hn, Y) / math.sqrt(Y.shape[-2])


def compare_int8_codes(gpu_state, ora_codes, ora_ypre, group, hadamard=False, tally=None):
    """Teacher-forced code comparison for one INT8 quantization point.
    gpu_state [.., d_k, d_v] is the GPU's dequantized carried state (hadamard=True: the
    unrotated S, rotated here to Hn S; a state already held rotated is passed with
    hadamard=False).  Every mismatch must be +-1 at a near-tie; counts go to `tally`."""
    X = np.asarray(gpu_state, dtype=np.float64)
    if hadamard:
        Hn = hadamard_n(X.shape[-2])
        X = np.einsum("ij,...jk->...ik", Hn, X)
    codes, _ = int8_codes_from_state(X, group)
    diff = codes != ora_codes
    nmis = int(diff.sum())
    if nmis:
        d = np.abs(codes[diff] - ora_codes[diff])
        assert d.max() == 1, f"code mismatch larger than one: {d.max()}"
        y = np.asarray(ora_ypre, dtype=np.float64)[diff]
        dist = np.abs(np.abs(y - np.floor(y)) - 0.5)
        assert dist.max() <= TIE_WINDOW, f"mismatch away from a tie (distance {dist.max()})"
    if tally is not None:
        tally.add(nmis, codes.size)
    return nmis / codes.size
