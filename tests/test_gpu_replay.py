"""GPU parity of replay windows (la_config.replay) against the oracle.

Replay windows ("Torch GDN/KDA decode QAT + INT8", What does this PR do?: BF16 key/update
entries between checkpoints, refreshed at the window boundary; "Fused Triton GDN/KDA decode
QAT", What does this PR do?: encode-once factors): the rounding points are the window ends
(qdq_interval = W); every other token's update reaches the carried state through its delta
rounded once to BF16, while the output reads the unrounded update.

Teacher forcing per window: the GPU forward returns its carried state entering every token
and every token's BF16 entry (la_recurrent_fwd_entries); from the GPU state entering a window
the oracle runs the window with the GPU's entries forced, so both follow one trajectory.
Compared: outputs and the carried states inside the window (fp32 bound), every entry against
the oracle's own encoding of its delta (equal except one BF16 step at a near-tie of the
oracle's FP32 delta), and the codes of the refresh at the window end (near-tie protocol).
The backward: recompute equals the forward's checkpoints bit for bit, and matches the
oracle's backward on the GPU trajectory.
"""
import numpy as np
import pytest

import oracle
import quantized_state_qat_amd as la
import synth
from tests import gpu_util as gu
from tests.test_gpu_fwd import sl

pytestmark = pytest.mark.gpu

W_ = synth.Workload
INT8, E4M3 = la.LA_QDQ_INT8_GROUP, la.LA_QDQ_E4M3_TILE
# distance of the oracle's FP32 delta from the midpoint of two BF16 values, relative to the
# largest |delta| of its token: the INT8 window (2e-3 of a code) expressed for an 8-bit
# significand at the token's largest entry
BF16_TIE_WINDOW = gu.TIE_WINDOW * 2.0 ** -8


def bits_to_f64(b16):
    return synth.bf16_bits_to_f32(np.asarray(b16).view(np.uint16)).astype(np.float64).reshape(np.asarray(b16).shape)


def run_entries(c, d, S0):
    torch = gu.torch_mod()
    di = {k: gu.dev(d[k]) for k in ("q", "k", "v", "g", "beta")}
    o = gu.nan_like(torch, (c.B, c.T, c.H, c.d_v))
    ST = gu.nan_like(torch, (c.B, c.H, c.d_k, c.d_v))
    ck = gu.nan_like(torch, (c.B, c.H, c.T, c.d_k, c.d_v))
    ent = torch.full((c.B, c.T, c.H, c.d_v), -1, dtype=torch.int16, device="cuda")
    c.ckpt_interval = 1
    S0d = torch.from_numpy(np.ascontiguousarray(S0, dtype=np.float32)).cuda()
    la.la_recurrent_fwd_entries(c, di["q"], di["k"], di["v"], di["g"], di["beta"], S0d, o, ST, ck, ent)
    torch.cuda.synchronize()
    return o.cpu().numpy(), ST.cpu().numpy(), ck.cpu().numpy(), ent.cpu().numpy()


def compare_entries(e_gpu, delta_or, tally):
    """GPU BF16 entries against the oracle's encoding of its own delta, one token's vector per
    row of the last axis."""
    d32 = delta_or.astype(np.float32).astype(np.float64)
    e_or = np.vectorize(oracle.bf16)(d32)
    bad = e_gpu != e_or
    tally.add(int(bad.sum()), e_gpu.size)
    if bad.any():
        a, b = e_gpu[bad], e_or[bad]
        # neighbouring BF16 values of one sign: bit patterns one apart
        ba = (a.astype(np.float32).view(np.uint32) >> 16).astype(np.int64)
        bb = (b.astype(np.float32).view(np.uint32) >> 16).astype(np.int64)
        assert np.all(np.sign(a) == np.sign(b)) and np.all(np.abs(ba - bb) == 1), (a[:4], b[:4])
        scale = np.abs(delta_or).max(axis=-1, keepdims=True) * np.ones_like(delta_or)
        dist = np.abs(d32[bad] - 0.5 * (a + b)) / scale[bad]
        assert dist.max() <= BF16_TIE_WINDOW, f"entry mismatch away from a tie ({dist.max()})"


def window_teacher_forced(c, d, S0, o, ST, ck, ent, W):
    had = bool(c.hadamard)
    rc = had and c.gate == la.LA_GATE_SCALAR
    state = (lambda X: gu.rotated_to_state(X)) if rc else (lambda X: X.astype(np.float64))
    B, T, H = c.B, c.T, c.H
    e64 = bits_to_f64(ent)
    tally_c, tally_e = gu.CodeTally(), gu.CodeTally()
    worst_o = worst_s = 0.0
    for w0 in range(0, T, W):
        w1 = min(w0 + W, T)
        dd = sl(d, 0, B, w0, w1, 0, H)
        dhat = e64[:, w0:w1].copy()
        dhat[:, -1] = np.nan
        o_r, _, ck_r, dl_r = oracle.fwd(dd["q"].f64, dd["k"].f64, dd["v"].f64, dd["g"].f64, dd["beta"].f64,
                                        state(ck[:, :, w0]), gate=c.gate, qdq_mode=c.qdq, group=c.group,
                                        hadamard=had, qdq_interval=W, replay=True, dhat=dhat, ckpt_interval=1,
                                        return_deltas=True)
        worst_o = max(worst_o, gu.err(o[:, w0:w1], o_r))
        for t in range(w0 + 1, w1):
            worst_s = max(worst_s, gu.err(state(ck[:, :, t]), ck_r[:, :, t - w0]))
        if w1 - w0 > 1:
            compare_entries(e64[:, w0:w1 - 1], dl_r[:, :w1 - 1 - w0], tally_e)
        # the refresh at the window end, from the GPU state entering its last token
        tl = w1 - 1
        dl = sl(d, 0, B, tl, tl + 1, 0, H)
        _, Sp, _ = oracle.fwd(dl["q"].f64, dl["k"].f64, dl["v"].f64, dl["g"].f64, dl["beta"].f64,
                              state(ck[:, :, tl]), gate=c.gate)
        S_out = ck[:, :, w1] if w1 < T else ST
        out_rot = rc and w1 < T
        for b in range(B):
            for h in range(H):
                _, codes, _, ypre = oracle.qdq(Sp[b, h], c.qdq, c.group, had)
                if c.qdq == INT8:
                    gu.compare_int8_codes(S_out[b, h], codes, ypre, c.group, hadamard=had and not out_rot,
                                          tally=tally_c)
                else:
                    gu.compare_e4m3_point(S_out[b, h], codes, ypre, tally_c)
    assert worst_o <= gu.TOL_F32, worst_o
    assert worst_s <= gu.TOL_F32, worst_s
    tally_c.check()
    tally_e.check()
    return worst_o, worst_s, tally_c, tally_e


CASES = [
    # name, workload, quantizer, group, hadamard, window
    ("gdn_wht_int8g32_w4", W_("r1", B=2, T=70, H=2, d_k=128, d_v=128, s0_sigma=0.2, config_id=90), INT8, 32, 1, 4),
    ("gdn_int8g32_w16", W_("r2", B=2, T=70, H=2, d_k=128, d_v=128, s0_sigma=0.2, config_id=91), INT8, 32, 0, 16),
    ("kda_int8g64_w4", W_("r3", B=1, T=70, H=2, d_k=128, d_v=128, gate="key", s0_sigma=0.2, config_id=92),
     INT8, 64, 0, 4),
    ("kda_wht_int8g32_w16", W_("r4", B=1, T=70, H=2, d_k=128, d_v=128, gate="key", s0_sigma=0.2, config_id=93),
     INT8, 32, 1, 16),
    ("gdn_e4m3_w8_dk64", W_("r5", B=2, T=45, H=2, d_k=64, d_v=128, s0_sigma=0.2, config_id=94), E4M3, 64, 0, 8),
    ("gdn_wht_int8g16_w5_dk32", W_("r6", B=1, T=33, H=3, d_k=32, d_v=64, s0_sigma=0.2, config_id=95),
     INT8, 16, 1, 5),
]


@pytest.mark.parametrize("name,w,mode,group,had,W", CASES, ids=[c[0] for c in CASES])
def test_replay_forward_teacher_forced(name, w, mode, group, had, W):
    d = synth.generate(w)
    c = gu.cfg_for(w, d, qdq=mode, group=group, hadamard=had, qdq_interval=W, replay=1)
    assert la.la_fwd_kernel_name(c) == "token"
    S0 = d["S0"].f32
    o, ST, ck, ent = run_entries(c, d, S0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ST))
    # the plain forward runs the same kernel: bit-identical
    o2, ST2, _ = gu.run_fwd(c, d, S0=S0)
    np.testing.assert_array_equal(o2, o)
    np.testing.assert_array_equal(ST2, ST)
    # replay changes the trajectory: the same call without it differs
    c_n = gu.cfg_for(w, d, qdq=mode, group=group, hadamard=had, qdq_interval=W)
    o_n, _, _ = gu.run_fwd(c_n, d, S0=S0)
    assert np.abs(o_n - o).max() > 1e-6
    wo, ws, tc, te = window_teacher_forced(c, d, S0, o, ST, ck, ent, W)
    print(f"{name}: output {wo:.2e}, state {ws:.2e}, codes {tc.mismatches}/{tc.total}, "
          f"entries {te.mismatches}/{te.total}")


@pytest.mark.parametrize("mode,group,had,gate", [(INT8, 32, 1, "scalar"), (INT8, 64, 0, "key"), (E4M3, 64, 0, "scalar")])
def test_window_of_one_token_is_rounding_every_token(mode, group, had, gate):
    w = W_("r7", B=2, T=40, H=2, d_k=64, d_v=64, gate=gate, s0_sigma=0.2, config_id=96)
    d = synth.generate(w)
    c1 = gu.cfg_for(w, d, qdq=mode, group=group, hadamard=had, qdq_interval=1, replay=1)
    c0 = gu.cfg_for(w, d, qdq=mode, group=group, hadamard=had, qdq_interval=1)
    o1, S1, k1 = gu.run_fwd(c1, d, S0=d["S0"].f32, ckpt_interval=1)
    o0, S0_, k0 = gu.run_fwd(c0, d, S0=d["S0"].f32, ckpt_interval=1)
    np.testing.assert_array_equal(o1, o0)
    np.testing.assert_array_equal(S1, S0_)
    np.testing.assert_array_equal(k1, k0)


def test_replay_exact_properties():
    """Power-of-two scaling and negation of (v, S_0) scale outputs and states exactly (the
    BF16 encoding commutes with both); a call split at a window end resumes exactly; units are
    independent; repeated runs are bit-identical."""
    w = W_("r8", B=3, T=64, H=2, d_k=128, d_v=128, s0_sigma=0.2, config_id=97)
    d = synth.generate(w)
    c = gu.cfg_for(w, d, qdq=INT8, group=32, hadamard=1, qdq_interval=8, replay=1, state_rotated=1)
    S0 = d["S0"].f32
    o, ST, _ = gu.run_fwd(c, d, S0=S0)
    o_b, ST_b, _ = gu.run_fwd(c, d, S0=S0)
    np.testing.assert_array_equal(o_b, o)
    np.testing.assert_array_equal(ST_b, ST)
    d2 = dict(d)
    d2["v"] = synth.cast(d["v"].f64 * 2.0 ** 3, "bf16")
    o2, ST2, _ = gu.run_fwd(c, d2, S0=S0 * np.float32(8))
    np.testing.assert_array_equal(o2, o * 8)
    np.testing.assert_array_equal(ST2, ST * 8)
    d3 = dict(d)
    d3["v"] = synth.cast(-d["v"].f64, "bf16")
    o3, ST3, _ = gu.run_fwd(c, d3, S0=-S0)
    np.testing.assert_array_equal(o3, -o)
    np.testing.assert_array_equal(ST3, -ST)
    da, db = sl(d, 0, 3, 0, 24, 0, 2), sl(d, 0, 3, 24, 64, 0, 2)
    ca = gu.cfg_for(w, da, qdq=INT8, group=32, hadamard=1, qdq_interval=8, replay=1, state_rotated=1)
    ca.T = 24
    oa, Sa, _ = gu.run_fwd(ca, da, S0=S0)
    ca.T = 40
    ob, Sb, _ = gu.run_fwd(ca, db, S0=Sa)
    np.testing.assert_array_equal(np.concatenate([oa, ob], axis=1), o)
    np.testing.assert_array_equal(Sb, ST)
    d1 = sl(d, 1, 2, 0, 64, 1, 2)
    c1 = gu.cfg_for(w, d1, qdq=INT8, group=32, hadamard=1, qdq_interval=8, replay=1, state_rotated=1)
    c1.B, c1.H = 1, 1
    o1, S1, _ = gu.run_fwd(c1, d1, S0=S0[1:2, 1:2])
    np.testing.assert_array_equal(o1[0, :, 0], o[1, :, 1])
    np.testing.assert_array_equal(S1[0, 0], ST[1, 1])


BWD = [
    ("gdn_wht_int8g32_w8_ckpt16", W_("rb1", B=2, T=70, H=2, d_k=128, d_v=128, s0_sigma=0.2, config_id=98),
     INT8, 32, 1, 8, 16),
    ("kda_int8g64_w4_ckpt12", W_("rb2", B=1, T=50, H=2, d_k=128, d_v=128, gate="key", s0_sigma=0.2, config_id=99),
     INT8, 64, 0, 4, 12),
    ("kda_wht_int8g32_w16", W_("rb3", B=1, T=40, H=2, d_k=64, d_v=64, gate="key", s0_sigma=0.2, config_id=100),
     INT8, 32, 1, 16, 16),
]


@pytest.mark.parametrize("name,w,mode,group,had,W,ckpt", BWD, ids=[b[0] for b in BWD])
def test_replay_backward(name, w, mode, group, had, W, ckpt):
    from tests.test_gpu_bwd import GRADS, _check_against_oracle
    d = synth.generate(w, with_do=True, with_dST=True)
    c = gu.cfg_for(w, d, qdq=mode, group=group, hadamard=had, qdq_interval=W, replay=1)
    c.ckpt_interval = ckpt
    assert la.la_bwd_kernel_name(c) == "token"
    S0, dST = d["S0"].f32, d["dST"].f32
    g1 = gu.run_bwd(c, d, d["do"].f32, S0=S0, dST=dST)
    _, _, ck = gu.run_fwd(c, d, S0=S0, ckpt_interval=ckpt)
    c.ckpt_interval = ckpt
    g2 = gu.run_bwd(c, d, d["do"].f32, S0=S0, dST=dST, ckpts=ck)
    for n in GRADS:
        np.testing.assert_array_equal(g1[n], g2[n])
    errs = _check_against_oracle(c, d, S0, d["do"].f32, dST, g1, gu.TOL_F32)
    print(name, {k: f"{v:.2e}" for k, v in errs.items()})


DECODE = [
    # name, gate, quantizer, group, hadamard, window, d_k
    ("gdn_wht_int8g32_w4", "scalar", INT8, 32, 1, 4, 128),
    ("gdn_int8g32_w16", "scalar", INT8, 32, 0, 16, 128),
    ("kda_int8g64_w4", "key", INT8, 64, 0, 4, 128),
    ("kda_wht_int8g32_w16", "key", INT8, 32, 1, 16, 64),
    ("gdn_e4m3_w8", "scalar", E4M3, 64, 0, 8, 128),
    ("gdn_int8g16_w1", "scalar", INT8, 16, 0, 1, 64),
]


@pytest.mark.parametrize("name,gate,mode,group,had,W,dk", DECODE, ids=[x[0] for x in DECODE])
def test_replay_decode_against_oracle(name, gate, mode, group, had, W, dk):
    """Serving decode in replay mode, token after token over two windows and a half: every
    output against the oracle (the window run from the GPU's checkpoint with the GPU's logged
    entries forced), every appended entry against the oracle's encoding of its delta (near-tie
    protocol), the logged key and gate bits exactly, the checkpoint untouched inside a window,
    and at each window end the refreshed checkpoint's codes (near-tie protocol) and the codes
    and scales outputs."""
    torch = gu.torch_mod()
    B, H, dv = 3, 2, 128
    T = 2 * W + W // 2 + 1
    w = W_("rd", B=B, T=T, H=H, d_k=dk, d_v=dv, gate=gate, s0_sigma=0.05, config_id=101)
    d = synth.generate(w)
    dev = {n: gu.dev(d[n]) for n in ("q", "k", "v", "g", "beta")}
    c = gu.cfg_for(w, d, qdq=mode, group=group, hadamard=had, qdq_interval=W, replay=1)
    c.T = 1
    W1 = max(W - 1, 1)
    log_k = torch.zeros((B, H, W1, dk), dtype=torch.int16, device="cuda")
    log_d = torch.zeros((B, H, W1, dv), dtype=torch.int16, device="cuda")
    log_g = torch.zeros((B, H, W1) + ((dk,) if gate == "key" else ()), dtype=torch.float32, device="cuda")
    S = torch.from_numpy(d["S0"].f32.copy()).cuda()
    C_win = d["S0"].f32.copy()       # checkpoint entering the current window (host copy)
    tally_e, tally_c = gu.CodeTally(), gu.CodeTally()
    worst_o = 0.0
    for t in range(T):
        p = t % W
        w0 = t - p
        pos = torch.full((B,), p, dtype=torch.int32, device="cuda")
        o = gu.nan_like(torch, (B, 1, H, dv))
        codes = torch.full((B, H, dk, dv), 99, dtype=torch.int8 if mode == INT8 else torch.uint8, device="cuda")
        nsc = (B, H, dk, dv // group) if mode == INT8 else (B, H, dv // 64)
        scales = gu.nan_like(torch, nsc)
        tk = {n: dev[n][:, t:t + 1].contiguous() for n in dev}
        la.la_decode_step_replay(c, tk["q"], tk["k"], tk["v"], tk["g"], tk["beta"], S, log_k, log_d, log_g, pos,
                                 o, codes, scales)
        torch.cuda.synchronize()
        o = o.cpu().numpy()
        # oracle: the window so far from the GPU's checkpoint, the GPU's entries forced
        dd = sl(d, 0, B, w0, t + 1, 0, H)
        ents = bits_to_f64(log_d.cpu().numpy())                      # [B, H, W1, dv]
        dhat = np.full((B, p + 1, H, dv), np.nan)
        for i in range(p):
            dhat[:, i] = ents[:, :, i]
        o_r, _, ck_r, dl_r = oracle.fwd(dd["q"].f64, dd["k"].f64, dd["v"].f64, dd["g"].f64, dd["beta"].f64,
                                        C_win.astype(np.float64), gate=c.gate, qdq_mode=mode, group=group,
                                        hadamard=bool(had), qdq_interval=W, replay=True, dhat=dhat,
                                        ckpt_interval=1, return_deltas=True)
        worst_o = max(worst_o, gu.err(o[:, 0], o_r[:, p]))
        if p < W - 1:
            # an entry was appended; the checkpoint is unchanged
            np.testing.assert_array_equal(S.cpu().numpy(), C_win)
            compare_entries(ents[:, :, p], dl_r[:, p], tally_e)
            kb = log_k.cpu().numpy()[:, :, p].view(np.uint16)
            np.testing.assert_array_equal(kb, d["k"].bits[:, t])
            gl = log_g.cpu().numpy()[:, :, p]
            np.testing.assert_array_equal(gl, d["g"].f32[:, t])
        else:
            # window end: the refreshed checkpoint against the oracle's rounding of S'
            S_new = S.cpu().numpy()
            dl = sl(d, 0, B, t, t + 1, 0, H)
            _, Sp, _ = oracle.fwd(dl["q"].f64, dl["k"].f64, dl["v"].f64, dl["g"].f64, dl["beta"].f64,
                                  ck_r[:, :, p], gate=c.gate)
            cg, sg = codes.cpu().numpy(), scales.cpu().numpy()
            for b in range(B):
                for h in range(H):
                    _, cr, sr, ypre = oracle.qdq(Sp[b, h], mode, group, bool(had))
                    if mode == INT8:
                        gu.compare_int8_codes(S_new[b, h], cr, ypre, group, hadamard=bool(had), tally=tally_c)
                        mism = cg[b, h].astype(np.int32) != cr
                        if not mism.any() and not had:
                            # a scale is its group's largest magnitude over 127: it carries that
                            # element's fp32 error, accumulated over the window's reconstruction
                            np.testing.assert_allclose(sg[b, h].reshape(-1), sr, rtol=2e-6)
                    else:
                        gu.compare_e4m3_point(S_new[b, h], cr, ypre, tally_c)
            C_win = S_new.copy()
    assert worst_o <= gu.TOL_F32, worst_o
    tally_c.check()
    tally_e.check()
    print(f"{name}: output {worst_o:.2e}, codes {tally_c.mismatches}/{tally_c.total}, "
          f"entries {tally_e.mismatches}/{tally_e.total}")


def test_replay_decode_window_of_one_is_the_decode_step():
    torch = gu.torch_mod()
    w = W_("rd1", B=4, T=1, H=2, d_k=128, d_v=128, s0_sigma=0.05, config_id=102)
    d = synth.generate(w)
    dev = {n: gu.dev(d[n]) for n in ("q", "k", "v", "g", "beta")}
    c = gu.cfg_for(w, d, qdq=INT8, group=32, hadamard=1, qdq_interval=1, replay=1)
    S1 = torch.from_numpy(d["S0"].f32.copy()).cuda()
    S2 = S1.clone()
    o1, o2 = gu.nan_like(torch, (4, 1, 2, 128)), gu.nan_like(torch, (4, 1, 2, 128))
    pos = torch.zeros((4,), dtype=torch.int32, device="cuda")
    la.la_decode_step_replay(c, dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], S1, None, None, None, pos, o1)
    c0 = gu.cfg_for(w, d, qdq=INT8, group=32, hadamard=1, qdq_interval=1)
    la.la_decode_step(c0, dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], S2, o2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(o1.cpu().numpy(), o2.cpu().numpy())
    np.testing.assert_array_equal(S1.cpu().numpy(), S2.cpu().numpy())
