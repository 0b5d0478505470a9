"""Every forward kernel against the float64 oracle, teacher forced per rounding interval.

la_recurrent_fwd selects one of four kernels from the configuration (la_fwd_kernel_name):
the block kernel (16-token blocks on the matrix cores, scalar or per-key gates), the
single-wave kernel (scalar or per-key gates), the eight-wave kernel and the per-token kernel.  Each case below is chosen to land on one of them
(asserted), runs with checkpoints at the rounding interval, and then, for every unit and every
interval, the oracle advances the GPU's checkpoint over that interval in float64 and rounds it
with the FP32 codec ("GDN state/W QAT foundation", "Torch GDN/KDA decode QAT + INT8": What
does this PR do?).  Both sides read the same input values (bf16 inputs widen exactly), so the
only difference is fp32 against float64 arithmetic over one interval: outputs and unrounded
carried states agree to 1e-5 of their largest magnitude, quantization codes exactly except
+-1 at near-ties (aggregate budget).
"""
import numpy as np
import pytest

import oracle
import quantized_state_qat_amd as la
import synth
from tests import gpu_util as gu
from tests.test_gpu_fwd import sl

pytestmark = pytest.mark.gpu

W = synth.Workload
INT8, E4M3, NONE = la.LA_QDQ_INT8_GROUP, la.LA_QDQ_E4M3_TILE, la.LA_QDQ_NONE

CASES = [
    # id, workload, quantizer, group, interval (= checkpoint spacing), kernel
    ("block_int8g32_i16", W("bi8", B=2, T=90, H=2, d_k=128, d_v=128, s0_sigma=0.2, config_id=40), INT8, 32, 16, "block"),
    ("block_e4m3_i32_dv192", W("be4", B=1, T=77, H=2, d_k=128, d_v=192, s0_sigma=0.2, config_id=41), E4M3, 64, 32, "block"),
    ("block_noqdq_i16", W("bnq", B=2, T=50, H=1, d_k=128, d_v=64, s0_sigma=0.2, config_id=42), NONE, 32, 16, "block"),
    ("wave_e4m3_dk64_i64", W("we4", B=2, T=150, H=2, d_k=64, d_v=128, s0_sigma=0.2, config_id=43), E4M3, 64, 64, "wave"),
    ("wave_fp32_int8g64_i8", W("wi8", B=1, T=45, H=3, d_k=128, d_v=128, qkv_dtype="f32", gate_dtype="f32",
                                s0_sigma=0.2, config_id=44), INT8, 64, 8, "wave"),
    ("wave_int8g16_dk32_i24", W("wdk32", B=2, T=60, H=1, d_k=32, d_v=64, s0_sigma=0.2, config_id=45), INT8, 16, 24, "wave"),
    ("fast_int8g16_i3", W("fi8", B=1, T=40, H=2, d_k=128, d_v=128, s0_sigma=0.2, config_id=46), INT8, 16, 3, "fast"),
    ("fast_e4m3_dk16_i5", W("fe4", B=2, T=33, H=2, d_k=16, d_v=64, s0_sigma=0.2, config_id=47), E4M3, 64, 5, "fast"),
    ("wave_kda_e4m3_dk64_i16", W("tk", B=1, T=40, H=2, d_k=64, d_v=64, gate="key", s0_sigma=0.2, config_id=48), E4M3, 64, 16, "wave"),
    ("block_kda_int8g32_i64", W("wk1", B=2, T=150, H=2, d_k=128, d_v=128, gate="key", s0_sigma=0.2, config_id=60),
     INT8, 32, 64, "block"),
    ("block_kda_e4m3_i16_dv192", W("bk2", B=1, T=77, H=2, d_k=128, d_v=192, gate="key", s0_sigma=0.2, config_id=67),
     E4M3, 64, 16, "block"),
    ("block_kda_noqdq_f32gate_i16", W("bk3", B=2, T=40, H=1, d_k=128, d_v=64, gate="key", gate_dtype="f32",
                                       s0_sigma=0.2, config_id=68), NONE, 32, 16, "block"),
    ("wave_kda_fp32_noqdq_dk128_i8", W("wk2", B=1, T=45, H=2, d_k=128, d_v=64, gate="key", qkv_dtype="f32",
                                        gate_dtype="f32", s0_sigma=0.2, config_id=61), NONE, 32, 8, "wave"),
    ("wave_kda_int8g16_dk32_i8", W("wk3", B=3, T=37, H=3, d_k=32, d_v=64, gate="key", s0_sigma=0.2, config_id=62),
     INT8, 16, 8, "wave"),
    ("wave_kda_e4m3_bf16gate_dk128_i24", W("wk4", B=1, T=70, H=3, d_k=128, d_v=192, gate="key", s0_sigma=0.1,
                                            config_id=63), E4M3, 64, 24, "wave"),
    ("token_kda_e4m3_i12", W("tk2", B=1, T=40, H=2, d_k=64, d_v=64, gate="key", s0_sigma=0.2, config_id=64), E4M3, 64, 12, "token"),
]


def _check_intervals(name, w, d, mode, group, interval, kernel):
    c = gu.cfg_for(w, d, qdq=mode, group=group, qdq_interval=interval if mode != NONE else 1)
    c.ckpt_interval = interval
    assert la.la_fwd_kernel_name(c) == kernel
    S0 = d["S0"].f32
    o, ST, ck = gu.run_fwd(c, d, S0=S0, ckpt_interval=interval)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ST)) and np.all(np.isfinite(ck))
    tally = gu.CodeTally()
    worst_o, worst_s = 0.0, 0.0
    nseg = (w.T + interval - 1) // interval
    for b in range(w.B):
        for h in range(w.H):
            for s in range(nseg):
                t0, t1 = s * interval, min(w.T, (s + 1) * interval)
                dd = sl(d, b, b + 1, t0, t1, h, h + 1)
                S_in = ck[b:b + 1, h:h + 1, s].astype(np.float64)
                o_r, Sp, _ = oracle.fwd(dd["q"].f64, dd["k"].f64, dd["v"].f64, dd["g"].f64, dd["beta"].f64,
                                        S_in, gate=c.gate)
                worst_o = max(worst_o, gu.err(o[b, t0:t1, h], o_r[0, :, 0]))
                S_out = ck[b, h, s + 1] if t1 < w.T else ST[b, h]
                if mode == NONE:
                    worst_s = max(worst_s, gu.err(S_out, Sp[0, 0]))
                    continue
                Xh, codes, _, ypre = oracle.qdq(Sp[0, 0], mode, group, False)
                if mode == INT8:
                    gu.compare_int8_codes(S_out, codes, ypre, group, tally=tally)
                else:
                    gu.compare_e4m3_point(S_out, codes, ypre, tally)
    assert worst_o <= gu.TOL_F32, worst_o
    assert worst_s <= gu.TOL_F32, worst_s
    frac = tally.check()
    print(f"{name} [{kernel}]: max output error {worst_o:.3e}, state error {worst_s:.2e}, "
          f"code mismatches {tally.mismatches}/{tally.total} ({frac:.2e})")


@pytest.mark.parametrize("name,w,mode,group,interval,kernel", CASES, ids=[c[0] for c in CASES])
def test_intervals_against_oracle(name, w, mode, group, interval, kernel):
    _check_intervals(name, w, synth.generate(w), mode, group, interval, kernel)


def steep_gates(d, w):
    """Log gates with stretches that leave the kernels' rescaling ranges: tokens 16..39 at
    g = -5 (eight tokens decay by about 2^-58, sixteen by 2^-115: the block kernel's
    token-by-token path and the wave kernel's per-token fold), tokens 40..69 at g = -1.5
    (a few tokens' product leaves [2^-30, 2^30]: the wave and eight-wave kernels fold the
    scale back into the state), token 75 at g = -200 (the gate underflows to zero in FP32 and
    erases the state; in float64 it is 1.4e-87), the rest as drawn.  Per-key gates get the
    same pattern on even keys only."""
    g = d["g"].f64.copy()
    t = np.arange(w.T)
    for lo, hi, val in ((16, 40, -5.0), (40, 70, -1.5), (75, 76, -200.0)):
        idx = (slice(None), (t >= lo) & (t < hi))
        if w.gate == "key":
            g[idx[0], idx[1], :, 0::2] = val
        else:
            g[idx] = val
    out = dict(d)
    out["g"] = synth.cast(g, w.gate_dtype)
    return out


STEEP = [
    ("block_int8g32_i16", W("sbi8", B=1, T=96, H=2, d_k=128, d_v=128, s0_sigma=0.2, config_id=50), INT8, 32, 16, "block"),
    ("block_noqdq_i16_f32gate", W("sbnq", B=1, T=90, H=1, d_k=128, d_v=64, gate_dtype="f32",
                                s0_sigma=0.2, config_id=51), NONE, 32, 16, "block"),
    ("wave_e4m3_dk64_i64", W("swe4", B=1, T=150, H=2, d_k=64, d_v=128, s0_sigma=0.2, config_id=52), E4M3, 64, 64, "wave"),
    ("wave_int8g64_i8", W("swi8", B=1, T=85, H=2, d_k=128, d_v=128, s0_sigma=0.2, config_id=53), INT8, 64, 8, "wave"),
    ("fast_int8g16_i3", W("sfi8", B=1, T=80, H=2, d_k=128, d_v=128, s0_sigma=0.2, config_id=54), INT8, 16, 3, "fast"),
    ("wave_kda_int8g32_i16", W("stk", B=1, T=80, H=2, d_k=64, d_v=64, gate="key", s0_sigma=0.2, config_id=55),
     INT8, 32, 16, "wave"),
    ("block_kda_e4m3_i64", W("swk", B=1, T=150, H=2, d_k=128, d_v=128, gate="key", gate_dtype="f32",
                              s0_sigma=0.2, config_id=65), E4M3, 64, 64, "block"),
    ("token_kda_int8g32_i12", W("stk2", B=1, T=80, H=2, d_k=64, d_v=64, gate="key", s0_sigma=0.2, config_id=66),
     INT8, 32, 12, "token"),
]


@pytest.mark.parametrize("name,w,mode,group,interval,kernel", STEEP, ids=[c[0] for c in STEEP])
def test_steep_gates_against_oracle(name, w, mode, group, interval, kernel):
    d = steep_gates(synth.generate(w), w)
    assert np.min(d["g"].f32) == -200.0
    _check_intervals("steep " + name, w, d, mode, group, interval, kernel)
