"""GPU parity of la_decode_step against the CPU oracle.

One decode token reads the FP32 state, updates it, fake-quantizes it and writes it back in
place ("Torch GDN/KDA decode QAT + INT8", "What does this PR do?": the recurrent suffix with
token state QDQ; FP32 working values).  A single step is teacher forced by construction:
the oracle starts from the same state.  The batched-decode workload is B=256 sequences x
H=16 heads, d_k = d_v = 128, bf16 inputs, FP32 state ~ N(0, 0.05^2), INT8 groups of 32.
"""
import numpy as np
import pytest

import oracle
import quantized_state_qat_amd as la
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _run_decode(c, d, S_init, want_codes=True):
    torch = gu.torch_mod()
    di = {k: gu.dev(d[k]) for k in ("q", "k", "v", "g", "beta")}
    S = torch.from_numpy(np.ascontiguousarray(S_init, dtype=np.float32)).cuda()
    o = gu.nan_like(torch, (c.B, 1, c.H, c.d_v))
    codes = scales = None
    if want_codes and c.qdq != la.LA_QDQ_NONE:
        codes = torch.full((c.B, c.H, c.d_k, c.d_v), 99,
                           dtype=torch.int8 if c.qdq == la.LA_QDQ_INT8_GROUP else torch.uint8, device="cuda")
        nsc = (c.B, c.H, c.d_k, c.d_v // c.group) if c.qdq == la.LA_QDQ_INT8_GROUP else (c.B, c.H, c.d_v // 64)
        scales = gu.nan_like(torch, nsc)
    la.la_decode_step(c, di["q"], di["k"], di["v"], di["g"], di["beta"], S, o, codes, scales)
    torch.cuda.synchronize()
    return (S.cpu().numpy(), o.cpu().numpy(),
            None if codes is None else codes.cpu().numpy(), None if scales is None else scales.cpu().numpy())


def _oracle_step(d, S_init, gate, mode, group, had, rot=False):
    """o and S' (float64) of one token, then the codec per unit.  rot: S_init holds the
    rotated state Hu S."""
    S_phys = gu.rotated_to_state(S_init) if rot else S_init.astype(np.float64)
    o, Sp, _ = oracle.fwd(d["q"].f64, d["k"].f64, d["v"].f64, d["g"].f64, d["beta"].f64,
                          S_phys, gate=gate)
    B, H = Sp.shape[:2]
    Xh = np.zeros_like(Sp)
    codes = np.zeros(Sp.shape, dtype=np.int32)
    ypre = np.zeros(Sp.shape, dtype=np.float32)
    scales = []
    for b in range(B):
        for h in range(H):
            if mode == la.LA_QDQ_NONE:
                Xh[b, h] = Sp[b, h]
                continue
            Xh[b, h], codes[b, h], s, ypre[b, h] = oracle.qdq(Sp[b, h], mode, group, had)
            scales.append(s)
    return o, Sp, Xh, codes, ypre, (np.array(scales) if scales else None)


CASES = [
    # name, B, H, d_k, d_v, gate, qdq, group, had
    ("int8g32", 3, 2, 128, 128, "scalar", la.LA_QDQ_INT8_GROUP, 32, 0),
    ("int8g16_dk64", 2, 3, 64, 192, "scalar", la.LA_QDQ_INT8_GROUP, 16, 0),
    ("int8g64_kda", 2, 2, 128, 128, "key", la.LA_QDQ_INT8_GROUP, 64, 0),
    ("e4m3", 2, 3, 128, 128, "scalar", la.LA_QDQ_E4M3_TILE, 64, 0),
    ("wht_int8g32", 2, 2, 128, 128, "scalar", la.LA_QDQ_INT8_GROUP, 32, 1),
    ("wht_int8g64_kda", 2, 2, 128, 128, "key", la.LA_QDQ_INT8_GROUP, 64, 1),
    ("wht_int8g16_rotated_state", 2, 3, 128, 128, "scalar", la.LA_QDQ_INT8_GROUP, 16, 2),
    ("none_dk32", 2, 2, 32, 64, "scalar", la.LA_QDQ_NONE, 32, 0),
    ("int8g32_dk16", 1, 3, 16, 64, "scalar", la.LA_QDQ_INT8_GROUP, 32, 0),
]


@pytest.mark.parametrize("name,B,H,dk,dv,gate,mode,group,had", CASES, ids=[c[0] for c in CASES])
def test_decode_matches_oracle(name, B, H, dk, dv, gate, mode, group, had):
    w = synth.Workload(name, B=B, T=1, H=H, d_k=dk, d_v=dv, gate=gate, s0_sigma=0.05, config_id=11)
    d = synth.generate(w)
    rot = had == 2  # Hadamard with the state held rotated (Y = Hu S in and out)
    c = gu.cfg_for(w, d, qdq=mode, group=group, hadamard=int(had > 0), state_rotated=int(rot))
    S_init = d["S0"].f32
    S, o, codes, scales = _run_decode(c, d, S_init)
    o_r, Sp, Xh, codes_r, ypre, scales_r = _oracle_step(d, S_init, c.gate, mode, group, had > 0, rot)
    if rot:
        S = gu.rotated_to_state(S)  # compare states unrotated
    assert gu.err(o, o_r) <= gu.TOL_BF16
    assert gu.err(o, o_r) <= 1e-5  # same inputs, one token: fp32 rounding only
    if mode == la.LA_QDQ_NONE:
        assert gu.err(S, Sp) <= 1e-6
        return
    if mode == la.LA_QDQ_INT8_GROUP:
        frac = gu.compare_int8_codes(S, codes_r, ypre, group, hadamard=had > 0)
        mism = codes.astype(np.int32) != codes_r
        assert mism.mean() <= gu.CODE_MISMATCH_MAX and mism.mean() == pytest.approx(frac, abs=1e-12)
        if had == 0:
            # where every code of a group agrees, the scale and the dequantized state agree to an ulp
            sc = scales.reshape(-1)
            np.testing.assert_allclose(sc, scales_r.reshape(-1), rtol=2 ** -22)
        # one code step of difference moves one element by s = amax/127 of its group
        assert gu.err(S, Xh) <= (1e-5 if not mism.any() else 2.0 / 127)
    else:
        mism = codes.astype(np.int32) != (codes_r & 0xFF)
        assert mism.mean() <= gu.CODE_MISMATCH_MAX
        if mism.any():  # only neighbouring grid values, at near-ties of the oracle's x/s
            vg = np.vectorize(oracle.e4m3_value)(codes[mism].astype(np.int64))
            vo = np.vectorize(oracle.e4m3_value)(codes_r[mism].astype(np.int64))
            mid = (vg + vo) / 2
            assert np.all(np.abs(np.abs(ypre[mism]) - np.abs(mid)) <= gu.E4M3_TIE_WINDOW)
        np.testing.assert_allclose(scales.reshape(-1), scales_r.reshape(-1), rtol=2 ** -22)
        assert gu.err(S, Xh) <= (1e-5 if not mism.any() else 1.0 / 8)


@pytest.mark.parametrize("mode,group,had", [(la.LA_QDQ_INT8_GROUP, 16, 0), (la.LA_QDQ_INT8_GROUP, 32, 0),
                                            (la.LA_QDQ_INT8_GROUP, 64, 0), (la.LA_QDQ_E4M3_TILE, 64, 0)])
def test_codec_bit_exact(mode, group, had):
    """beta = 0 and g = 0 leave S' = S exactly, so the step is the bare codec: both sides
    decide in FP32 from identical inputs and must agree bit for bit."""
    w = synth.Workload("codec", B=4, T=1, H=4, d_k=128, d_v=128, s0_sigma=1.0, config_id=12)
    d = synth.generate(w)
    d["g"] = synth.cast(np.zeros((4, 1, 4)), "bf16")
    d["beta"] = synth.cast(np.zeros((4, 1, 4)), "bf16")
    S_init = d["S0"].f32.copy()
    # include an all-zero group / tile and a few exact ties
    S_init[0, 0, 3, :64] = 0.0
    S_init[1, 1, 5, :32] = np.float32(2.0 ** -3) * np.arange(32) / 2.0
    S_init[1, 1, 5, 7] = np.float32(127 * 2.0 ** -3)
    c = gu.cfg_for(w, d, qdq=mode, group=group, hadamard=had)
    S, _, codes, scales = _run_decode(c, d, S_init)
    for b in range(4):
        for h in range(4):
            Xh, cr, sr, _ = oracle.qdq(S_init[b, h].astype(np.float64), mode, group)
            np.testing.assert_array_equal(S[b, h], Xh.astype(np.float32))
            if mode == la.LA_QDQ_INT8_GROUP:
                np.testing.assert_array_equal(codes[b, h].astype(np.int32), cr)
                np.testing.assert_array_equal(scales[b, h].reshape(-1), sr)
            else:
                np.testing.assert_array_equal(codes[b, h].astype(np.int32), cr & 0xFF)
                np.testing.assert_array_equal(scales[b, h].reshape(-1), sr)


def test_decode_full_size_workload():
    """B=256, H=16, d=128 (the benchmark's decode batch): every unit checked."""
    w = synth.WORKLOADS[1]
    d = synth.generate(w)
    c = gu.cfg_for(w, d, qdq=la.LA_QDQ_INT8_GROUP, group=32)
    S_init = d["S0"].f32
    S, o, codes, scales = _run_decode(c, d, S_init)
    o_r, Sp = oracle.fwd(d["q"].f64, d["k"].f64, d["v"].f64, d["g"].f64, d["beta"].f64,
                         S_init.astype(np.float64))[:2]
    assert gu.err(o, o_r) <= 1e-5
    nmis = 0
    for b in range(w.B):
        for h in range(w.H):
            Xh, cr, sr, yp = oracle.qdq(Sp[b, h], la.LA_QDQ_INT8_GROUP, 32)
            diff = codes[b, h].astype(np.int32) != cr
            if diff.any():
                assert np.abs(codes[b, h][diff].astype(np.int32) - cr[diff]).max() == 1
                y = yp[diff].astype(np.float64)
                assert np.abs(np.abs(y - np.floor(y)) - 0.5).max() <= gu.TIE_WINDOW
                nmis += int(diff.sum())
    assert nmis / codes.size <= gu.CODE_MISMATCH_MAX
    assert gu.err(S, Sp) <= 1e-2  # QDQ error (half a step of 1/127 of each group's range)


def test_decode_deterministic_and_overwrites():
    w = synth.Workload("det", B=8, T=1, H=4, d_k=128, d_v=128, s0_sigma=0.05, config_id=13)
    d = synth.generate(w)
    c = gu.cfg_for(w, d, qdq=la.LA_QDQ_INT8_GROUP, group=32)
    r1 = _run_decode(c, d, d["S0"].f32)
    r2 = _run_decode(c, d, d["S0"].f32)
    for x, y in zip(r1, r2):
        np.testing.assert_array_equal(x, y)
    assert all(np.all(np.isfinite(x)) for x in r1[:2])


SLOT_CASES = [
    # name, B, H, d_k, d_v, gate, qdq, group, had
    ("int8g32", 6, 2, 128, 128, "scalar", la.LA_QDQ_INT8_GROUP, 32, 0),
    ("e4m3_kda_dk64", 5, 3, 64, 128, "key", la.LA_QDQ_E4M3_TILE, 64, 0),
    ("wht_int8g16_rotated_state", 4, 2, 128, 64, "scalar", la.LA_QDQ_INT8_GROUP, 16, 2),
    ("wht_int8g32_kda", 4, 2, 128, 128, "key", la.LA_QDQ_INT8_GROUP, 32, 1),
]


@pytest.mark.parametrize("name,B,H,dk,dv,gate,mode,group,had", SLOT_CASES, ids=[c[0] for c in SLOT_CASES])
def test_decode_slots(name, B, H, dk, dv, gate, mode, group, had):
    """Slot-pool decode: live entries advance the slot they name exactly as la_decode_step
    advances the gathered states (bit for bit, same kernel), and match the oracle's slot decode;
    padding entries (slot 0, indices outside the pool) write zeros to o and nothing else; slots
    no entry names keep their bits."""
    torch = gu.torch_mod()
    w = synth.Workload(name, B=B, T=1, H=H, d_k=dk, d_v=dv, gate=gate, s0_sigma=0.05, config_id=13)
    d = synth.generate(w)
    rot = had == 2
    c = gu.cfg_for(w, d, qdq=mode, group=group, hadamard=int(had > 0), state_rotated=int(rot))
    n_slots = B + 3
    rng = np.random.default_rng(7)
    pool = (rng.standard_normal((n_slots, H, dk, dv)) * 0.05).astype(np.float32)
    live = rng.permutation(np.arange(1, n_slots))[:B].astype(np.int32)
    slots = live.copy()
    slots[1] = 0            # padding
    slots[-1] = n_slots + 4  # outside the pool: padding too
    di = {k_: gu.dev(d[k_]) for k_ in ("q", "k", "v", "g", "beta")}
    P = torch.from_numpy(pool.copy()).cuda()
    sl = torch.from_numpy(slots).cuda()
    o = gu.nan_like(torch, (B, 1, H, dv))
    cdt = torch.int8 if mode == la.LA_QDQ_INT8_GROUP else torch.uint8
    codes = torch.full((B, H, dk, dv), 99, dtype=cdt, device="cuda")
    nsc = (B, H, dk, dv // group) if mode == la.LA_QDQ_INT8_GROUP else (B, H, dv // 64)
    scales = gu.nan_like(torch, nsc)
    la.la_decode_step_slots(c, di["q"], di["k"], di["v"], di["g"], di["beta"], P, sl, n_slots, o, codes, scales)
    torch.cuda.synchronize()
    P, o, codes, scales = P.cpu().numpy(), o.cpu().numpy(), codes.cpu().numpy(), scales.cpu().numpy()
    is_live = (slots >= 1) & (slots < n_slots)
    # padding entries
    assert np.all(o[~is_live] == 0)
    assert np.all(codes[~is_live] == 99) and np.all(np.isnan(scales[~is_live]))
    # slots nobody names keep their bits
    named = set(int(x) for x in slots[is_live])
    for s_ in range(n_slots):
        if s_ not in named:
            np.testing.assert_array_equal(P[s_], pool[s_])
    # live entries equal la_decode_step on the gathered states, bit for bit
    S_g, o_g, codes_g, scales_g = _run_decode(c, d, pool[np.where(is_live, slots, 0)])
    for b in np.nonzero(is_live)[0]:
        np.testing.assert_array_equal(P[slots[b]], S_g[b])
        np.testing.assert_array_equal(o[b], o_g[b])
        np.testing.assert_array_equal(codes[b], codes_g[b])
        np.testing.assert_array_equal(scales[b], scales_g[b])
    # and the oracle's slot decode (unrotated domain)
    pool_phys = gu.rotated_to_state(pool) if rot else pool.astype(np.float64)
    o_r, pool_r = oracle.decode_slots(d["q"].f64, d["k"].f64, d["v"].f64, d["g"].f64, d["beta"].f64,
                                      pool_phys, slots, gate=c.gate, qdq_mode=mode, group=group,
                                      hadamard=had > 0)
    assert gu.err(o, o_r) <= 1e-5
    P_phys = gu.rotated_to_state(P) if rot else P.astype(np.float64)
    for b in np.nonzero(is_live)[0]:
        # one code step of difference at a near-tie moves an element by at most one grid step
        assert gu.err(P_phys[slots[b]], pool_r[slots[b]]) <= (2.0 / 127 if mode == la.LA_QDQ_INT8_GROUP else 1.0 / 8)


SLOT_ORDER_CASES = [
    # name, B, n_slots: the slot-ordered map (B <= 1024, n_slots <= 16384) over several waves,
    # passes and bitmap words, and the identity map past either limit
    ("ordered_b700_pool2000", 700, 2000),
    ("ordered_b1024_pool16384", 1024, 16384),
    ("identity_b1100", 1100, 1500),
    ("identity_pool20000", 300, 20000),
]


@pytest.mark.parametrize("name,B,n_slots", SLOT_ORDER_CASES, ids=[c[0] for c in SLOT_ORDER_CASES])
def test_decode_slots_visit_order(name, B, n_slots):
    """Slot-pool decode of large shuffled batches with padding scattered among them (slot 0,
    negative indices, indices past the pool): whichever workgroup serves an entry, every live
    entry advances its own slot exactly as la_decode_step advances the gathered state (bit for
    bit), o is written in entry order and matches the oracle, padding entries write zeros, and
    slots no entry names keep their bits."""
    torch = gu.torch_mod()
    H, dk, dv = 1, 16, 64
    w = synth.Workload(name, B=B, T=1, H=H, d_k=dk, d_v=dv, gate="scalar", s0_sigma=0.05, config_id=17)
    d = synth.generate(w)
    c = gu.cfg_for(w, d, qdq=la.LA_QDQ_INT8_GROUP, group=16)
    rng = np.random.default_rng(11)
    pool = (rng.standard_normal((n_slots, H, dk, dv)) * 0.05).astype(np.float32)
    slots = rng.permutation(np.arange(1, n_slots))[:B].astype(np.int32)
    pad = rng.choice(B, size=B // 10, replace=False)
    slots[pad[0::3]] = 0
    slots[pad[1::3]] = -5
    slots[pad[2::3]] = n_slots + 7
    di = {k_: gu.dev(d[k_]) for k_ in ("q", "k", "v", "g", "beta")}
    P = torch.from_numpy(pool.copy()).cuda()
    o = gu.nan_like(torch, (B, 1, H, dv))
    la.la_decode_step_slots(c, di["q"], di["k"], di["v"], di["g"], di["beta"], P, torch.from_numpy(slots).cuda(),
                            n_slots, o)
    torch.cuda.synchronize()
    P, o = P.cpu().numpy(), o.cpu().numpy()
    is_live = (slots >= 1) & (slots < n_slots)
    assert np.all(o[~is_live] == 0)
    untouched = np.ones(n_slots, dtype=bool)
    untouched[slots[is_live]] = False
    np.testing.assert_array_equal(P[untouched], pool[untouched])
    S_g, o_g, _, _ = _run_decode(c, d, pool[np.where(is_live, slots, 0)], want_codes=False)
    live = np.nonzero(is_live)[0]
    np.testing.assert_array_equal(P[slots[live]], S_g[live])
    np.testing.assert_array_equal(o[live], o_g[live])
    o_r, _ = oracle.decode_slots(d["q"].f64, d["k"].f64, d["v"].f64, d["g"].f64, d["beta"].f64,
                                 pool, slots, gate=c.gate, qdq_mode=la.LA_QDQ_INT8_GROUP, group=16)
    assert gu.err(o, o_r) <= 1e-5
