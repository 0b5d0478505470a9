"""The state codecs on the GPU against the oracle's, bit for bit, through the C ABI.

With beta = 0 and g = 0 a token leaves the state unchanged (a = exp(0) = 1, delta = 0), so
a call that ends on a quantization point returns Q(S0): the bare codec of every kernel, fed
the same FP32 values the oracle's codec reads.  Both sides then decide in FP32 from identical
inputs ("GDN state/W QAT foundation", What does this PR do?: E4M3 per full-key x 64-column
tile, scale amax/448 with a zero guard; "Torch GDN/KDA decode QAT + INT8", What does this PR
do?: INT8 groups along the value axis), so codes, scales and dequantized states must agree
exactly, with no near-tie allowance.

Kernels (la_fwd_kernel_name, and the decode step): the per-token kernel (one token), the
eight-wave kernel (two tokens, rounding every two), the single-wave kernel (eight tokens),
the block kernel (one 16-token block on the matrix cores) and decode.  The wave, block and
per-token kernels round E4M3 with the hardware conversion, decode and the eight-wave kernel
with exact power-of-two scaling; all of them use the division-free scale, reciprocal and
quotient of the INT8 and E4M3 codecs.

* E4M3, every fp32 value: per binade [2^e, 2^(e+1)) of x/s for e = -11 .. 8 (below 2^-10
  everything rounds to zero; 448 is the largest value), every fp32 significand, both signs,
  with s = 1 exactly (each tile's largest magnitude is 448).  This covers every midpoint of
  the grid, the subnormal ties and the top binade.
* E4M3 across scales: tile maxima with random significands from 2^-90 to 2^100 (about half
  of them make amax/448 round down, so the largest x/s lies just above 448 and saturates),
  values at and next to scaled midpoints.
* INT8, every scale significand: every fp32 significand of amax in [1, 2) (eight chunks of
  2^20 groups of 16), the other values of each group at and next to code midpoints.
* INT8 across scales: group maxima from 2^-110 to 2^100 (scales below 2^-100 take the
  division path), groups of 16, 32 and 64; decode's codes and scales outputs compared too.
"""
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
import quantized_state_qat_amd as la
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

# kernel -> (tokens, rounding interval, q/k/v dtype)
KERNELS = {"token": (1, 1, la.LA_F32), "fast": (2, 2, la.LA_F32), "wave": (8, 8, la.LA_F32),
           "block": (16, 16, la.LA_BF16), "decode": (1, 1, la.LA_BF16)}
POOL = ThreadPoolExecutor(max_workers=8)


def oracle_codec(S0, mode, group):
    """(Xhat as float32, codes, scales) of the oracle's codec for every unit of S0 [U, d_k, d_v]."""
    res = list(POOL.map(lambda u: oracle.qdq(S0[u].astype(np.float64), mode, group, False), range(S0.shape[0])))
    Xh = np.stack([r[0] for r in res])
    assert np.all(Xh.astype(np.float32).astype(np.float64) == Xh)  # dequantized values are fp32 values
    return Xh.astype(np.float32), np.stack([r[1] for r in res]), np.stack([r[2] for r in res])


def gpu_codec(kernel, S0, mode, group):
    """Q(S0) computed by `kernel` from S0 [U, d_k, d_v] (U heads of one sequence): returns
    (state, codes, scales); codes and scales only for decode."""
    torch = gu.torch_mod()
    U, dk, dv = S0.shape
    T, interval, qdt = KERNELS[kernel]
    tdt = torch.bfloat16 if qdt == la.LA_BF16 else torch.float32
    rng = np.random.default_rng(7)
    q = torch.from_numpy(rng.standard_normal((1, T, U, dk)).astype(np.float32) / math.sqrt(dk)).to(tdt).cuda()
    k = torch.zeros((1, T, U, dk), dtype=tdt, device="cuda")      # with beta = 0 the key only
    v = torch.from_numpy(rng.standard_normal((1, T, U, dv)).astype(np.float32)).to(tdt).cuda()
    g = torch.zeros((1, T, U), dtype=tdt, device="cuda")          # a = exp(0) = 1
    beta = torch.zeros((1, T, U), dtype=tdt, device="cuda")       # delta = 0
    c = la.Config(B=1, T=T, H=U, d_k=dk, d_v=dv, qdq=mode, group=group, qdq_interval=interval,
                  qkv_dtype=qdt, gate_dtype=qdt)
    S = torch.from_numpy(np.ascontiguousarray(S0)).cuda()
    o = gu.nan_like(torch, (1, T, U, dv))
    if kernel == "decode":
        codes = torch.full((1, U, dk, dv), 99, dtype=torch.int8 if mode == la.LA_QDQ_INT8_GROUP else torch.uint8,
                           device="cuda")
        nsc = (1, U, dk, dv // group) if mode == la.LA_QDQ_INT8_GROUP else (1, U, dv // 64)
        scales = gu.nan_like(torch, nsc)
        la.la_decode_step(c, q, k, v, g, beta, S, o, codes, scales)
        torch.cuda.synchronize()
        return S.cpu().numpy(), codes.cpu().numpy()[0], scales.cpu().numpy()[0]
    assert la.la_fwd_kernel_name(c) == kernel
    ST = gu.nan_like(torch, (1, U, dk, dv))
    la.la_recurrent_fwd(c, q, k, v, g, beta, S, o, ST, None)
    torch.cuda.synchronize()
    return ST.cpu().numpy()[0], None, None


def check_all_kernels(S0, mode, group):
    Xh, codes_r, scales_r = oracle_codec(S0, mode, group)
    for kernel in KERNELS:
        S, codes, scales = gpu_codec(kernel, S0, mode, group)
        # equal values (the sign of a zero that a negative value rounds to is not compared)
        bad = ~(S == Xh)
        assert not bad.any(), (kernel, int(bad.sum()), S0[bad][:4], S[bad][:4], Xh[bad][:4])
        if codes is not None:
            if mode == la.LA_QDQ_INT8_GROUP:
                np.testing.assert_array_equal(codes.astype(np.int32), codes_r)
            else:
                # a zero code's sign bit is not compared: the update S' = 1 S + k delta adds
                # +0 to a state element -0 (IEEE sum +0), so the kernel codes +0 where the
                # oracle's codec, fed S0 itself, codes -0
                cg = codes.astype(np.int32)
                co = codes_r & 0xFF
                cg = np.where((cg & 0x7F) == 0, 0, cg)
                co = np.where((co & 0x7F) == 0, 0, co)
                np.testing.assert_array_equal(cg, co)
            np.testing.assert_array_equal(scales.reshape(-1), scales_r.reshape(-1).astype(np.float32))


def f32_from_bits(bits):
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


def e4m3_binade_state(e):
    """Every fp32 value of |y| in [2^e, 2^(e+1)) (capped at 448), random signs, packed into
    tiles of 128 rows x 64 columns whose first element is the anchor 448 (so s = 1)."""
    lo = np.float32(2.0 ** e).view(np.uint32)
    hi = np.float32(min(2.0 ** (e + 1), 448.0)).view(np.uint32) + (1 if 2.0 ** (e + 1) > 448.0 else 0)
    vals = f32_from_bits(np.arange(lo, hi, dtype=np.uint32))
    rng = np.random.default_rng(1000 + e)
    vals = np.where(rng.random(vals.size) < 0.5, -vals, vals).astype(np.float32)
    per = 128 * 64 - 1
    n_tiles = -(-vals.size // per)
    pad = np.resize(vals, n_tiles * per)
    S0 = np.empty((n_tiles, 128 * 64), dtype=np.float32)
    S0[:, 0] = 448.0
    S0[:, 1:] = pad.reshape(n_tiles, per)
    return S0.reshape(n_tiles, 128, 64)


@pytest.mark.parametrize("e", list(range(-11, 9)), ids=[f"binade_2^{e}" for e in range(-11, 9)])
def test_e4m3_every_value_in_binade(e):
    S0 = e4m3_binade_state(e)
    check_all_kernels(S0, la.LA_QDQ_E4M3_TILE, 64)


def near_midpoints(mids, rng):
    """fp32 values at and up to two ulps either side of each (float64) midpoint."""
    m = mids.astype(np.float32)
    step = rng.integers(-2, 3, size=m.size).astype(np.int64)
    b = m.view(np.uint32).astype(np.int64)
    mag = (b & 0x7FFFFFFF) + step
    mag = np.clip(mag, 0, 0x7F7FFFFF)
    return ((b & 0x80000000) | mag).astype(np.uint32).view(np.float32)


def test_e4m3_across_scales():
    rng = np.random.default_rng(11)
    n_tiles = 2048
    exps = rng.integers(-90, 101, size=n_tiles)
    amax = (1.0 + rng.random(n_tiles)) * np.exp2(exps.astype(np.float64))
    amax = amax.astype(np.float32)
    s64 = amax.astype(np.float64) / 448.0
    grid = gu.E4M3_GRID
    mids = 0.5 * (grid[1:] + grid[:-1])
    per = 128 * 64
    S0 = np.empty((n_tiles, per), dtype=np.float32)
    for t in range(n_tiles):
        kind = rng.integers(0, 3, size=per)
        y = np.where(kind == 0, rng.choice(mids, size=per), np.where(kind == 1, rng.choice(grid, size=per),
                                                                      rng.random(per) * 448.0))
        y = np.where(rng.random(per) < 0.5, -y, y)
        x = near_midpoints(y * s64[t], rng)
        x = np.clip(x, -amax[t], amax[t])
        S0[t] = x
        S0[t, rng.integers(0, per)] = amax[t] * (1 if rng.random() < 0.5 else -1)
    S0[0] = 0.0  # an all-zero tile (zero guard)
    check_all_kernels(S0.reshape(n_tiles, 128, 64), la.LA_QDQ_E4M3_TILE, 64)


def int8_groups(amax, group, rng):
    """Groups [n, group]: element 0 holds +-amax, the others sit at or next to code
    midpoints (c + 1/2) s of the group's scale, or are uniform in [-amax, amax]."""
    n = amax.size
    s64 = amax.astype(np.float64) / 127.0
    c = rng.integers(-127, 127, size=(n, group - 1)) + 0.5
    y = np.where(rng.random((n, group - 1)) < 0.7, c, rng.uniform(-127, 127, size=(n, group - 1)))
    x = near_midpoints((y * s64[:, None]).reshape(-1), rng).reshape(n, group - 1)
    x = np.clip(x, -amax[:, None], amax[:, None])
    G = np.empty((n, group), dtype=np.float32)
    G[:, 0] = np.where(rng.random(n) < 0.5, -amax, amax)
    G[:, 1:] = x
    perm = rng.permuted(np.tile(np.arange(group), (n, 1)), axis=1)
    return np.take_along_axis(G, perm, axis=1)


@pytest.mark.parametrize("chunk", list(range(8)), ids=[f"chunk{i}" for i in range(8)])
def test_int8_every_scale_significand(chunk):
    """amax = every fp32 value in [1, 2), 2^20 of them per chunk, one group of 16 each."""
    lo = np.float32(1.0).view(np.uint32) + chunk * (1 << 20)
    amax = f32_from_bits(np.arange(lo, lo + (1 << 20), dtype=np.uint32))
    rng = np.random.default_rng(2000 + chunk)
    G = int8_groups(amax, 16, rng)                        # [2^20, 16]
    S0 = G.reshape(-1, 128, 64)                           # 4 groups per row, 2048 heads
    check_all_kernels(S0, la.LA_QDQ_INT8_GROUP, 16)


@pytest.mark.parametrize("group", [16, 32, 64])
def test_int8_across_scales(group):
    rng = np.random.default_rng(3000 + group)
    heads = 512
    n = heads * 128 * 64 // group
    exps = rng.integers(-110, 101, size=n)
    amax = ((1.0 + rng.random(n)) * np.exp2(exps.astype(np.float64))).astype(np.float32)
    G = int8_groups(amax, group, rng)
    S0 = G.reshape(heads, 128, 64)
    S0[0, 0, :group] = 0.0  # an all-zero group (zero guard)
    check_all_kernels(S0, la.LA_QDQ_INT8_GROUP, group)
