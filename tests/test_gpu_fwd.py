"""GPU parity of la_recurrent_fwd against the CPU oracle.

Per-token quantization (INT8 groups, optionally around a Hadamard rotation; "Torch GDN/KDA
decode QAT + INT8", "What does this PR do?") is checked teacher forced token by token: the
GPU returns its carried state entering every token (checkpoint interval 1), the oracle
advances each of those states by one token in float64 and rounds it with the FP32 codec,
and codes, outputs and states are compared.  Interval-64 quantization (E4M3 tiles, "GDN
state/W QAT foundation", "What does this PR do?") is teacher forced per 64-token segment
from the GPU's checkpoints.  Full-size workloads are checked on sampled units and windows,
and through properties that hold exactly at any size (determinism, checkpoint
independence, batch independence, split/resume, power-of-two equivariance).
"""
import numpy as np
import pytest

import oracle
import quantized_state_qat_amd as la
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def sl(d, b0, b1, t0, t1, h0, h1):
    """Slice generated inputs along (B, T, H)."""
    out = {}
    for key in ("q", "k", "v", "g", "beta"):
        x = d[key]
        idx = (slice(b0, b1), slice(t0, t1), slice(h0, h1))
        out[key] = synth.Tensor(f32=np.ascontiguousarray(x.f32[idx]), dtype=x.dtype,
                                bits=None if x.bits is None else np.ascontiguousarray(x.bits[idx]))
    return out


def _oracle_kw(c):
    return dict(gate=c.gate, group=c.group, hadamard=bool(c.hadamard))


def per_token_teacher_forced(c, d, ck, ST, o_gpu, tol, tally=None):
    """Compare every token: GPU state entering token t -> oracle one step -> GPU state after
    token t (codes) and o_t.  In Hadamard mode with the scalar gate the checkpoints hold the
    rotated state (c.state_rotated decides whether S_T does too); per-key gates carry and
    checkpoint the unrotated state.  Returns (max output error, tally)."""
    T = c.T
    had = bool(c.hadamard)
    rc = had and c.gate == la.LA_GATE_SCALAR
    tally = tally if tally is not None else gu.CodeTally()
    worst_o = 0.0
    for t in range(T):
        S_in = gu.rotated_to_state(ck[:, :, t]) if rc else ck[:, :, t].astype(np.float64)
        if t + 1 < T:
            S_out, out_rotated = ck[:, :, t + 1], rc
        else:
            S_out, out_rotated = ST, had and bool(c.state_rotated)
        o_t, Sp, _ = oracle.fwd(d["q"].f64[:, t:t + 1], d["k"].f64[:, t:t + 1], d["v"].f64[:, t:t + 1],
                                d["g"].f64[:, t:t + 1], d["beta"].f64[:, t:t + 1], S_in, gate=c.gate)
        worst_o = max(worst_o, gu.err(o_gpu[:, t], o_t[:, 0]))
        qpoint = c.qdq != la.LA_QDQ_NONE and ((t + 1) % c.qdq_interval == 0 or t == T - 1)
        if not qpoint:
            S_chk = gu.rotated_to_state(S_out) if out_rotated else S_out
            assert gu.err(S_chk, Sp) <= 1e-5
            continue
        for b in range(c.B):
            for h in range(c.H):
                Xh, codes, _, ypre = oracle.qdq(Sp[b, h], c.qdq, c.group, had)
                if c.qdq == la.LA_QDQ_INT8_GROUP:
                    gu.compare_int8_codes(S_out[b, h], codes, ypre, c.group,
                                          hadamard=had and not out_rotated, tally=tally)
                else:
                    gu.compare_e4m3_point(S_out[b, h], codes, ypre, tally)
    assert worst_o <= tol, worst_o
    return worst_o, tally


PER_TOKEN = [
    # id, workload, qdq, group, hadamard
    ("cfg0_gdn_fp32_int8g32", synth.WORKLOADS[0], la.LA_QDQ_INT8_GROUP, 32, 0),
    ("kda_int8g64_ragged", synth.Workload("kda", B=2, T=70, H=2, d_k=128, d_v=128, gate="key", config_id=21),
     la.LA_QDQ_INT8_GROUP, 64, 0),
    ("gdn_wht_int8g32_ragged", synth.Workload("wht", B=2, T=70, H=2, d_k=128, d_v=128, config_id=22),
     la.LA_QDQ_INT8_GROUP, 32, 1),
    # per-key gates with the rotation: the state is carried unrotated, rotated at each rounding
    ("kda_wht_int8g32_ragged", synth.Workload("kwh", B=2, T=70, H=2, d_k=128, d_v=128, gate="key", config_id=27),
     la.LA_QDQ_INT8_GROUP, 32, 1),
    ("kda_wht_int8g16_dk64", synth.Workload("kw6", B=1, T=33, H=2, d_k=64, d_v=128, gate="key", config_id=28),
     la.LA_QDQ_INT8_GROUP, 16, 1),
    ("gdn_int8g16_dk32_dv128", synth.Workload("g16", B=1, T=33, H=3, d_k=32, d_v=128, config_id=23),
     la.LA_QDQ_INT8_GROUP, 16, 0),
    ("kda_e4m3_tok_dk64", synth.Workload("e4t", B=1, T=20, H=2, d_k=64, d_v=64, gate="key", config_id=24),
     la.LA_QDQ_E4M3_TILE, 64, 0),
    ("gdn_noqdq_dk16_dv192", synth.Workload("nq", B=2, T=25, H=1, d_k=16, d_v=192, config_id=25),
     la.LA_QDQ_NONE, 32, 0),
]


@pytest.mark.parametrize("name,w,mode,group,had", PER_TOKEN, ids=[p[0] for p in PER_TOKEN])
def test_per_token_teacher_forced(name, w, mode, group, had):
    d = synth.generate(w)
    c = gu.cfg_for(w, d, qdq=mode, group=group, hadamard=had, qdq_interval=1)
    S0 = d["S0"].f32
    o, ST, ck = gu.run_fwd(c, d, S0=S0, ckpt_interval=1)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ST))
    # bf16 inputs widen exactly, so both sides read the same values and the fp32 bound holds
    # for them too (the 2e-3 bound for bf16 inputs is implied)
    worst_o, tally = per_token_teacher_forced(c, d, ck, ST, o, gu.TOL_F32)
    frac = tally.check()
    print(f"{name}: max output error {worst_o:.3e}, code mismatches {tally.mismatches}/{tally.total} ({frac:.2e})")


def seg_inputs(d, t0, t1):
    """float64 q, k, v, g, beta of tokens t0..t1-1 (sliced before widening)."""
    return [np.ascontiguousarray(d[n].f32[:, t0:t1]).astype(np.float64) for n in ("q", "k", "v", "g", "beta")]


def segment_teacher_forced(c, d, ck, ST, o_gpu, seg=64):
    """Interval-64 quantization, every unit and every segment: from the GPU checkpoints
    entering a segment the oracle runs the segment for all units at once in float64 and rounds
    each unit's state at its end; E4M3 grid values are compared with the near-tie protocol and
    tallied over the whole run (the 1e-4 budget applies to the total)."""
    from concurrent.futures import ThreadPoolExecutor
    T, B, H = c.T, c.B, c.H
    worst_o = 0.0
    tally = gu.CodeTally()
    with ThreadPoolExecutor(max_workers=8) as pool:
        for s_idx in range((T + seg - 1) // seg):
            t0, t1 = s_idx * seg, min(T, s_idx * seg + seg)
            S_in = ck[:, :, s_idx].astype(np.float64)
            o_r, Sp, _ = oracle.fwd(*seg_inputs(d, t0, t1), S_in, gate=c.gate)
            worst_o = max(worst_o, gu.err(o_gpu[:, t0:t1], o_r))
            S_out = ck[:, :, s_idx + 1] if t1 < T else ST
            res = list(pool.map(lambda u: oracle.qdq(Sp[u // H, u % H], c.qdq, c.group, False), range(B * H)))
            codes = np.stack([r[1] for r in res]).reshape(B, H, c.d_k, c.d_v)
            ypre = np.stack([r[3] for r in res]).reshape(B, H, c.d_k, c.d_v)
            gu.compare_e4m3_point(S_out, codes, ypre, tally)
    # bf16 inputs widen exactly: the fp32 bound applies (the bf16 bound is implied)
    assert worst_o <= gu.TOL_F32, worst_o
    frac = tally.check()
    print(f"E4M3 code mismatches {tally.mismatches}/{tally.total} ({frac:.2e}), max output error {worst_o:.2e}")
    return worst_o


def test_e4m3_interval64_small_ragged():
    w = synth.Workload("e4m3", B=2, T=200, H=3, d_k=128, d_v=128, gate_dtype="f32", config_id=26)
    d = synth.generate(w)
    c = gu.cfg_for(w, d, qdq=la.LA_QDQ_E4M3_TILE, group=64, qdq_interval=64)
    o, ST, ck = gu.run_fwd(c, d, ckpt_interval=64)
    worst = segment_teacher_forced(c, d, ck, ST, o)
    print(f"e4m3 small: max output error {worst:.3e}")


def test_e4m3_interval64_full_size():
    """B=8, H=16, T=4096, d=128, bf16 q/k/v, fp32 g/beta and state, E4M3 every 64 tokens:
    checkpoint independence at full size, then all 128 units and all 64 segments teacher
    forced per segment."""
    w = synth.WORKLOADS[2]
    d = synth.generate(w)
    c = gu.cfg_for(w, d, qdq=la.LA_QDQ_E4M3_TILE, group=64, qdq_interval=64)
    torch = gu.torch_mod()
    di = {k: gu.dev(d[k]) for k in ("q", "k", "v", "g", "beta")}
    o, ST, ck = gu.run_fwd(c, d, ckpt_interval=64, dev_inputs=di)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ST))
    # checkpointing does not change the arithmetic; a second run is bit-identical
    o2, ST2, _ = gu.run_fwd(c, d, ckpt_interval=0, dev_inputs=di)
    np.testing.assert_array_equal(o2, o)
    np.testing.assert_array_equal(ST2, ST)
    del di
    torch.cuda.empty_cache()
    worst = segment_teacher_forced(c, d, ck, ST, o)
    print(f"e4m3 full size: max output error {worst:.3e}")


def test_kda_e4m3_interval64_full_size():
    """KDA at the long-sequence shape (B=8, H=16, T=4096, d=128, bf16 q/k/v, fp32 per-key
    gates and beta, E4M3 every 64 tokens), served by the block kernel: checkpoint
    independence at full size, then every unit teacher forced per 64-token segment."""
    w = synth.Workload("kda_long_e4m3_64", B=8, T=4096, H=16, d_k=128, d_v=128, gate="key", gate_dtype="f32",
                       config_id=2)
    d = synth.generate(w)
    c = gu.cfg_for(w, d, qdq=la.LA_QDQ_E4M3_TILE, group=64, qdq_interval=64)
    assert la.la_fwd_kernel_name(c) == "block"
    torch = gu.torch_mod()
    di = {k: gu.dev(d[k]) for k in ("q", "k", "v", "g", "beta")}
    o, ST, ck = gu.run_fwd(c, d, ckpt_interval=64, dev_inputs=di)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ST))
    o2, ST2, _ = gu.run_fwd(c, d, ckpt_interval=0, dev_inputs=di)
    np.testing.assert_array_equal(o2, o)
    np.testing.assert_array_equal(ST2, ST)
    del di
    torch.cuda.empty_cache()
    worst = segment_teacher_forced(c, d, ck, ST, o)
    print(f"kda e4m3 full size: max output error {worst:.3e}")


@pytest.mark.parametrize("cid,mode,group,had", [(3, la.LA_QDQ_INT8_GROUP, 64, 0), (4, la.LA_QDQ_INT8_GROUP, 32, 1)],
                         ids=["kda_int8g64_full", "gdn_wht_int8g32_full"])
def test_per_token_full_size_windows(cid, mode, group, had):
    """Full-size per-token workloads (KDA B=4 H=32 T=2048; GDN+Hadamard B=4 H=16 T=2048):
    one run at full size with 64-token checkpoints; then the first and the last 64-token
    window of every unit are re-run from the checkpoint with per-token checkpoints (all units
    in one call: bit-identical to the full run by batch independence and exact resume) and
    teacher forced token by token against the oracle."""
    w = synth.WORKLOADS[cid]
    d = synth.generate(w)
    c = gu.cfg_for(w, d, qdq=mode, group=group, hadamard=had, qdq_interval=1, state_rotated=had)
    o, ST, ck = gu.run_fwd(c, d, ckpt_interval=64)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ST))
    worst = 0.0
    tally = gu.CodeTally()
    for s_idx in (0, w.T // 64 - 1):
        t0, t1 = 64 * s_idx, 64 * s_idx + 64
        dd = sl(d, 0, w.B, t0, t1, 0, w.H)
        cw = gu.cfg_for(w, dd, qdq=mode, group=group, hadamard=had, qdq_interval=1, state_rotated=had)
        cw.T = 64
        ow, STw, ckw = gu.run_fwd(cw, dd, S0=ck[:, :, s_idx], ckpt_interval=1)
        np.testing.assert_array_equal(ow, o[:, t0:t1])
        ref_end = ck[:, :, s_idx + 1] if t1 < w.T else ST
        np.testing.assert_array_equal(STw, ref_end)
        wo, _ = per_token_teacher_forced(cw, dd, ckw, STw, ow, gu.TOL_F32, tally)
        worst = max(worst, wo)
        del ckw
    frac = tally.check()
    print(f"config {cid}: max windowed output error {worst:.3e}, code mismatches "
          f"{tally.mismatches}/{tally.total} ({frac:.2e})")


@pytest.mark.parametrize("mode,group,had,gate,interval", [
    (la.LA_QDQ_INT8_GROUP, 32, 0, "scalar", 1), (la.LA_QDQ_INT8_GROUP, 64, 0, "key", 1),
    (la.LA_QDQ_INT8_GROUP, 32, 1, "scalar", 1), (la.LA_QDQ_E4M3_TILE, 64, 0, "scalar", 64),
    (la.LA_QDQ_INT8_GROUP, 16, 0, "scalar", 16)])
def test_exact_properties(mode, group, had, gate, interval):
    """Exact at any size: power-of-two scaling of (v, S_0) scales o and S_T exactly, and so
    does negation on the per-token path (to rounding on the block path); units are
    independent; a call split at a quantization point resumes exactly; repeated runs are
    bit-identical; T = 0 copies S_0."""
    w = synth.Workload("prop", B=3, T=128, H=2, d_k=128, d_v=128, gate=gate, s0_sigma=0.2, config_id=27)
    d = synth.generate(w)
    c = gu.cfg_for(w, d, qdq=mode, group=group, hadamard=had, qdq_interval=interval, state_rotated=had)
    S0 = d["S0"].f32
    o, ST, _ = gu.run_fwd(c, d, S0=S0)
    o_b, ST_b, _ = gu.run_fwd(c, d, S0=S0)
    np.testing.assert_array_equal(o, o_b)
    np.testing.assert_array_equal(ST, ST_b)
    d2 = dict(d)
    d2["v"] = synth.cast(d["v"].f64 * 2.0 ** 4, "bf16")
    o2, ST2, _ = gu.run_fwd(c, d2, S0=S0 * np.float32(2.0 ** 4))
    np.testing.assert_array_equal(o2, o * 2.0 ** 4)
    np.testing.assert_array_equal(ST2, ST * 2.0 ** 4)
    d3 = dict(d)
    d3["v"] = synth.cast(-d["v"].f64, "bf16")
    o3, ST3, _ = gu.run_fwd(c, d3, S0=-S0)
    if interval == 1:
        np.testing.assert_array_equal(o3, -o)
        np.testing.assert_array_equal(ST3, -ST)
    else:
        # Rounding every 16 tokens or more runs the block path, whose bf16 matrix-core sums
        # truncate their internal alignment (within an ulp, not symmetric in sign): negation
        # holds to rounding, and a code may flip where the state sits on a rounding tie.
        assert np.max(np.abs(o3 + o)) <= 1e-4 * np.max(np.abs(o))
        assert np.max(np.abs(ST3 + ST)) <= 1e-3 * np.max(np.abs(ST))
        assert np.mean(o3 != -o) < 0.5
    # unit (2, 1) alone
    d1 = sl(d, 2, 3, 0, 128, 1, 2)
    c1 = gu.cfg_for(w, d1, qdq=mode, group=group, hadamard=had, qdq_interval=interval, state_rotated=had)
    c1.B, c1.H = 1, 1
    o1, ST1, _ = gu.run_fwd(c1, d1, S0=S0[2:3, 1:2])
    np.testing.assert_array_equal(o1[0, :, 0], o[2, :, 1])
    np.testing.assert_array_equal(ST1[0, 0], ST[2, 1])
    # split at token 64
    da, db = sl(d, 0, 3, 0, 64, 0, 2), sl(d, 0, 3, 64, 128, 0, 2)
    ca = gu.cfg_for(w, da, qdq=mode, group=group, hadamard=had, qdq_interval=interval, state_rotated=had)
    ca.T = 64
    oa, Sa, _ = gu.run_fwd(ca, da, S0=S0)
    ob, Sb, _ = gu.run_fwd(ca, db, S0=Sa)
    np.testing.assert_array_equal(np.concatenate([oa, ob], axis=1), o)
    np.testing.assert_array_equal(Sb, ST)
    # T = 0: S_T = S_0
    c0 = gu.cfg_for(w, d, qdq=mode, group=group, hadamard=had, qdq_interval=interval, state_rotated=had)
    c0.T = 0
    _, ST0, _ = gu.run_fwd(c0, sl(d, 0, 3, 0, 0, 0, 2), S0=S0)
    np.testing.assert_array_equal(ST0, S0)


def test_bf16_output_is_rounded_fp32_output():
    w = synth.Workload("bf16o", B=2, T=40, H=2, d_k=64, d_v=128, config_id=28)
    d = synth.generate(w)
    c = gu.cfg_for(w, d, qdq=la.LA_QDQ_INT8_GROUP, group=32)
    o32, ST32, _ = gu.run_fwd(c, d)
    c.out_dtype = la.LA_BF16
    o16, ST16, _ = gu.run_fwd(c, d)
    np.testing.assert_array_equal(ST16, ST32)
    np.testing.assert_array_equal(o16, synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(o32.astype(np.float32))).reshape(o32.shape))
