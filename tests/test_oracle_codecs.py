"""Pins of the oracle's state codecs against the format definitions and library routines.

INT8 group QDQ (linear-attention state-QAT pages, "Torch GDN/KDA decode QAT + INT8",
"What does this PR do?": symmetric dynamic groups of 16/32/64 along the value axis)
and FP8 E4M3 tile QDQ ("GDN state/W QAT foundation", "What does this PR do?": per
full-key x 64-value-column tile, scale amax/448 with a zero guard) and the normalized
Walsh-Hadamard rotation used around INT8.
"""
import math

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle

pytestmark = []


# ----------------------------------------------------------------------------- E4M3 table
def test_e4m3_format_facts(oracle_mod):
    """OCP E4M3FN: bias 7, 3 mantissa bits, max 448, min normal 2^-6, min subnormal 2^-9."""
    val = oracle.e4m3_value
    assert val(0x00) == 0.0
    assert val(0x01) == 2.0 ** -9          # smallest subnormal
    assert val(0x07) == 7 * 2.0 ** -9      # largest subnormal
    assert val(0x08) == 2.0 ** -6          # smallest normal
    assert val(0x38) == 1.0
    assert val(0x77) == 240.0
    assert val(0x7E) == 448.0              # largest finite (0x7F is NaN)
    assert val(0xB8) == -1.0
    vals = [val(c) for c in range(256) if (c & 0x7F) != 0x7F]
    assert len(vals) == 254
    assert len(set(vals)) == 253           # +0 and -0 coincide
    pos = [val(c) for c in range(127)]
    assert all(b > a for a, b in zip(pos, pos[1:]))  # codes 0..126 increase


def _brute_nearest_code(y: float) -> int:
    """Linear scan over all 127 non-negative finite codes, ties to the even code."""
    a = abs(y)
    best, bestd = None, None
    for c in range(127):
        d = abs(oracle.e4m3_value(c) - a)
        if bestd is None or d < bestd or (d == bestd and c % 2 == 0):
            best, bestd = c, d
    if a >= 448.0:
        best = 0x7E
    return (0x80 if (y < 0 or (y == 0 and math.copysign(1, y) < 0)) else 0) | best


def test_e4m3_rounding_matches_brute_force(oracle_mod):
    rng = np.random.default_rng(7)
    ys = list(rng.uniform(-460, 460, 400)) + list(rng.uniform(-1, 1, 200)) + \
        list(rng.uniform(-0.02, 0.02, 200))
    # every midpoint between neighbouring codes (the ties) and their fp32 neighbours
    pos = [oracle.e4m3_value(c) for c in range(127)]
    for a, b in zip(pos, pos[1:]):
        m = (a + b) / 2
        m32 = np.float32(m)
        ys += [m, -m, float(np.nextafter(m32, np.float32(0))), float(np.nextafter(m32, np.float32(1e9)))]
    for y in ys:
        assert oracle.e4m3_code(y) == _brute_nearest_code(y), y


def test_e4m3_special_ties(oracle_mod):
    c = oracle.e4m3_code
    v = oracle.e4m3_value
    assert v(c(2.0 ** -10)) == 0.0                 # tie 0 | 2^-9 -> even code 0
    assert v(c(3 * 2.0 ** -10)) == 2.0 ** -8        # tie 2^-9 | 2^-8 -> even code 2
    assert v(c(1.0 + 1.0 / 16)) == 1.0              # tie 1 | 1.125 -> even mantissa
    assert v(c(1.0 + 3.0 / 16)) == 1.25             # tie 1.125 | 1.25 -> even mantissa
    assert v(c(449.0)) == 448.0 and v(c(470.0)) == 448.0 and v(c(1e6)) == 448.0
    assert v(c(-470.0)) == -448.0


def test_e4m3_matches_torch_float8(oracle_mod):
    """torch.float8_e4m3fn conversion (round to nearest even) agrees on |y| < 464."""
    rng = np.random.default_rng(11)
    y = np.concatenate([rng.uniform(-463.9, 463.9, 20000), rng.uniform(-2, 2, 20000),
                        rng.uniform(-0.03, 0.03, 20000)]).astype(np.float32)
    t = torch.from_numpy(y).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = np.array([oracle.e4m3_value(oracle.e4m3_code(float(x))) for x in y])
    np.testing.assert_array_equal(mine, t)


# ----------------------------------------------------------------------------- INT8 groups
@pytest.mark.parametrize("group", [16, 32, 64])
def test_int8_identity_on_representable_state(oracle_mod, group):
    """X = c * 2^m with integer |c| <= 127 and one |c| = 127 per group: s = 2^m, Q(X) = X."""
    rng = np.random.default_rng(group)
    dk, dv = 8, 128
    codes = rng.integers(-127, 128, size=(dk, dv))
    codes[:, ::group] = 127 * np.sign(rng.standard_normal((dk, dv // group)))
    m = rng.integers(-20, 5, size=(dk, dv // group))
    X = codes * np.exp2(np.repeat(m, group, axis=1))
    Xh, c, s, _ = oracle.qdq(X, oracle.QDQ_INT8, group)
    np.testing.assert_array_equal(Xh, X)
    np.testing.assert_array_equal(c, codes)
    np.testing.assert_array_equal(s, np.exp2(m).astype(np.float32).ravel())


def test_int8_round_half_even_and_zero_guard(oracle_mod):
    dv = 32
    X = np.zeros((3, dv))
    X[0, :8] = [127, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5]
    X[1, 0] = -127 * 2.0 ** -3
    X[1, 1:4] = np.array([0.5, 1.5, 126.5]) * 2.0 ** -3
    # row 2 all zero: zero guard -> scale 1, codes 0, output 0
    Xh, c, s, _ = oracle.qdq(X, oracle.QDQ_INT8, dv)
    assert list(c[0, :8]) == [127, 0, 2, 2, 0, -2, -2, 4]
    assert list(c[1, :4]) == [-127, 0, 2, 126]
    assert s[0] == 1.0 and s[1] == 2.0 ** -3 and s[2] == 1.0
    assert np.all(Xh[2] == 0) and np.all(c[2] == 0)


@pytest.mark.parametrize("group", [16, 32, 64])
def test_int8_invariants(oracle_mod, group):
    """Error <= s/2 (+ fp32 rounding), amax element codes to +-127, sign and 2^m equivariance,
    and groups never mix across rows or across value-axis groups."""
    rng = np.random.default_rng(100 + group)
    dk, dv = 16, 128
    X = rng.standard_normal((dk, dv)).astype(np.float32).astype(np.float64) * 0.3
    Xh, c, s, y = oracle.qdq(X, oracle.QDQ_INT8, group)
    S = np.repeat(s.reshape(dk, dv // group), group, axis=1).astype(np.float64)
    assert np.all(np.abs(Xh - X) <= S * (0.5 + 1e-6) + np.abs(X) * 2 ** -23)
    G = X.reshape(dk, dv // group, group)
    arg = np.abs(G).argmax(axis=2)
    cg = c.reshape(dk, dv // group, group)
    assert np.all(np.abs(np.take_along_axis(cg, arg[..., None], 2)) == 127)
    assert np.all(np.abs(c) <= 127)
    Xn, cn, sn, _ = oracle.qdq(-X, oracle.QDQ_INT8, group)
    np.testing.assert_array_equal(Xn, -Xh)
    X2, c2, s2, _ = oracle.qdq(X * 2.0 ** 7, oracle.QDQ_INT8, group)
    np.testing.assert_array_equal(X2, Xh * 2.0 ** 7)
    np.testing.assert_array_equal(c2, c)
    # locality: perturbing one element changes codes only inside its (row, group)
    Xp = X.copy()
    Xp[5, 3 * group // 2] *= 3.0
    _, cp, _, _ = oracle.qdq(Xp, oracle.QDQ_INT8, group)
    diff = np.argwhere(cp != c)
    g0 = (3 * group // 2) // group
    assert np.all(diff[:, 0] == 5)
    assert np.all(diff[:, 1] // group == g0)


# ----------------------------------------------------------------------------- E4M3 tiles
def test_e4m3_tile_identity_and_invariants(oracle_mod):
    rng = np.random.default_rng(5)
    dk, dv, tile = 32, 128, 64
    # values on the E4M3 grid times 2^m with max |y| = 448 in each tile -> identity
    codes = rng.integers(0, 126, size=(dk, dv))
    vals = np.array([oracle.e4m3_value(int(c)) for c in codes.ravel()]).reshape(dk, dv)
    vals *= np.where(rng.standard_normal((dk, dv)) < 0, -1, 1)
    vals[0, 0], vals[1, 64] = 448.0, -448.0
    X = vals * 2.0 ** -9
    Xh, _, s, _ = oracle.qdq(X, oracle.QDQ_E4M3, tile)
    np.testing.assert_array_equal(Xh, X)
    np.testing.assert_array_equal(s, [2.0 ** -9, 2.0 ** -9])
    # random tiles: relative error of each element <= 2^-4 of its magnitude (3 mantissa bits)
    # above the subnormal range, and the amax element is reproduced
    X = rng.standard_normal((dk, dv)).astype(np.float32).astype(np.float64)
    Xh, _, s, y = oracle.qdq(X, oracle.QDQ_E4M3, tile)
    for t in range(2):
        sl = slice(64 * t, 64 * t + 64)
        amax = np.abs(X[:, sl]).max()
        big = np.abs(X[:, sl]) >= 2.0 ** -6 * s[t]
        rel = np.abs(Xh[:, sl] - X[:, sl])[big] / np.abs(X[:, sl])[big]
        assert rel.max() <= 2.0 ** -4 + 1e-6
        assert np.abs(Xh[:, sl]).max() == pytest.approx(amax, rel=1e-6)
    # zero tile: scale 1 and zeros
    Z = np.zeros((dk, dv))
    Z[:, 64:] = X[:, 64:]
    Zh, _, sz, _ = oracle.qdq(Z, oracle.QDQ_E4M3, tile)
    assert sz[0] == 1.0 and np.all(Zh[:, :64] == 0)
    np.testing.assert_array_equal(Zh[:, 64:], Xh[:, 64:])


# ----------------------------------------------------------------------------- Hadamard
@pytest.mark.parametrize("n", [4, 64, 128])
def test_hadamard_matches_scipy_and_is_involution(oracle_mod, n):
    rng = np.random.default_rng(n)
    X = rng.standard_normal((n, 8))
    H = scipy.linalg.hadamard(n) / math.sqrt(n)
    Y = oracle.hadamard(X)
    np.testing.assert_allclose(Y, H @ X, rtol=0, atol=1e-12)
    np.testing.assert_allclose(oracle.hadamard(Y), X, rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.sum(Y * Y), np.sum(X * X), rtol=1e-12)  # Parseval


def test_hadamard_int8_identity_in_rotated_domain(oracle_mod):
    """If Hn X is exactly INT8-representable per group, the codes are recovered exactly and
    Q_H(X) = X up to the float32 rounding of the carried state."""
    rng = np.random.default_rng(9)
    n, dv, group = 128, 64, 32
    codes = rng.integers(-127, 128, size=(n, dv))
    codes[:, ::group] = 127
    Y = codes * 2.0 ** -8
    H = scipy.linalg.hadamard(n) / math.sqrt(n)
    X = (H @ Y).astype(np.float32).astype(np.float64)  # the carried state is fp32
    Xh, c, _, _ = oracle.qdq(X, oracle.QDQ_INT8, group, hadamard=True)
    np.testing.assert_array_equal(c, codes)
    np.testing.assert_allclose(Xh, H @ Y, atol=4 * 2.0 ** -24 * np.abs(H @ Y).max())
