"""GPU parity of the block backward ("block" in la_bwd_kernel_name) against the CPU oracle.

The straight-through backward ("GDN state/W QAT foundation", under "What does this PR do?")
treats the state quantizer as the identity, so the gradient is the adjoint of the unrounded
recurrence evaluated on the rounded trajectory.  The block path recomputes that trajectory
with the block forward, whose rounding points fall on 16-token block ends.  Teacher forcing
therefore takes the block forward's state entering every block (its 16-token checkpoints)
and continues each block token by token in float64 with the oracle's forward (no rounding
inside a block); the oracle's backward then runs on those states.
"""
import numpy as np
import pytest

import oracle
import quantized_state_qat_amd as la
import synth
from tests import gpu_util as gu
from tests.test_gpu_fwd import sl
from tests.test_gpu_fwd_paths import steep_gates

pytestmark = pytest.mark.gpu

GRADS = ["dq", "dk", "dv", "dg", "dbeta", "dS0"]
W = synth.Workload
# bf16 inputs are exact in fp32 and every product of the block form is an fp32-accurate
# product (exact bf16 splits, fp32 MFMAs), so the bound is the fp32 one; teacher forcing is
# per block, so nothing in the comparison depends on a rounding decision
TOL = gu.TOL_F32
NONE, INT8, E4M3 = la.LA_QDQ_NONE, la.LA_QDQ_INT8_GROUP, la.LA_QDQ_E4M3_TILE


def block_states(c, d, S0):
    """State entering every token: the GPU block forward's state at each block start,
    continued in float64 through the block."""
    _, _, ck16 = gu.run_fwd(c, d, S0=S0, ckpt_interval=16)
    B, T, H = c.B, c.T, c.H
    states = np.zeros((B, H, T, c.d_k, c.d_v))
    for blk in range((T + 15) // 16):
        t0, t1 = 16 * blk, min(16 * blk + 16, T)
        args = [d[n].f64[:, t0:t1] for n in ("q", "k", "v", "g", "beta")]
        _, _, ck = oracle.fwd(*args, ck16[:, :, blk].astype(np.float64), gate=c.gate, ckpt_interval=1)
        states[:, :, t0:t1] = ck
    return states


def check_block_bwd(c, d, S0, dST, tol):
    do = d["do"].f32
    g1 = gu.run_bwd(c, d, do, S0=S0, dST=dST)
    _, _, ck = gu.run_fwd(c, d, S0=S0, ckpt_interval=c.ckpt_interval)
    g2 = gu.run_bwd(c, d, do, S0=S0, dST=dST, ckpts=ck)
    for n in GRADS:
        assert np.all(np.isfinite(g1[n])), n
        np.testing.assert_array_equal(g1[n], g2[n])   # the block path does not read the checkpoints
    g3 = gu.run_bwd(c, d, do, S0=S0, dST=dST)
    for n in GRADS:
        np.testing.assert_array_equal(g3[n], g1[n])   # deterministic
    states = block_states(c, d, S0)
    ref = oracle.bwd(d["q"].f64, d["k"].f64, d["v"].f64, d["g"].f64, d["beta"].f64,
                     None if S0 is None else S0.astype(np.float64), do.astype(np.float64),
                     None if dST is None else dST.astype(np.float64), states=states,
                     gate=c.gate, qdq_mode=c.qdq, group=c.group, qdq_interval=c.qdq_interval)
    errs = {n: gu.err(g1[n], ref[n]) for n in GRADS}
    assert max(errs.values()) <= tol, errs
    return errs


CASES = [
    # id, workload, qdq, group, interval, user checkpoint spacing, with dS_T
    ("noqdq_ragged_bf16gate", W("bn", B=2, T=150, H=3, d_k=128, d_v=128, s0_sigma=0.3, config_id=70),
     NONE, 32, 1, 64, True),
    ("e4m3_i16_dv64", W("be", B=1, T=96, H=2, d_k=128, d_v=64, gate_dtype="f32", config_id=71),
     E4M3, 64, 16, 16, False),
    ("int8g32_i32_dv192", W("bi", B=1, T=37, H=2, d_k=128, d_v=192, s0_sigma=0.2, config_id=72),
     INT8, 32, 32, 32, True),
    ("int8g64_i64_one_block", W("b1", B=2, T=16, H=1, d_k=128, d_v=128, s0_sigma=0.2, config_id=73),
     INT8, 64, 64, 64, True),
    ("int8g16_i48_one_token", W("bt", B=1, T=1, H=2, d_k=128, d_v=64, s0_sigma=0.2, config_id=74),
     INT8, 16, 48, 16, True),
    ("e4m3_i64_ckpt64", W("bl", B=2, T=300, H=2, d_k=128, d_v=128, gate_dtype="f32", s0_sigma=0.1, config_id=75),
     E4M3, 64, 64, 64, True),
]


@pytest.mark.parametrize("name,w,mode,group,interval,ckpt,with_dst", CASES, ids=[x[0] for x in CASES])
def test_block_bwd_matches_oracle(name, w, mode, group, interval, ckpt, with_dst):
    d = synth.generate(w, with_do=True, with_dST=with_dst)
    c = gu.cfg_for(w, d, qdq=mode, group=group, qdq_interval=interval, ckpt_interval=ckpt)
    assert la.la_bwd_kernel_name(c) == "block"
    S0 = d["S0"].f32 if w.s0_sigma > 0 else None
    dST = d["dST"].f32 if with_dst else None
    errs = check_block_bwd(c, d, S0, dST, TOL)
    print(name, {k: f"{v:.2e}" for k, v in errs.items()})


def test_block_bwd_steep_gates():
    """Decays of e^-5 per token over 24 tokens, e^-1.5 over 30 and a gate that underflows to
    zero in FP32 (the forward path tests' pattern): the block form's factors are exponentials
    of gate-sum differences, never a quotient of two products, so they stay finite."""
    w = W("bs", B=1, T=96, H=2, d_k=128, d_v=128, s0_sigma=0.2, config_id=76)
    d = steep_gates(synth.generate(w, with_do=True, with_dST=True), w)
    c = gu.cfg_for(w, d, qdq=INT8, group=32, qdq_interval=16, ckpt_interval=16)
    assert la.la_bwd_kernel_name(c) == "block"
    errs = check_block_bwd(c, d, d["S0"].f32, d["dST"].f32, TOL)
    print("steep", {k: f"{v:.2e}" for k, v in errs.items()})


def test_block_bwd_full_size_sampled_unit():
    """GDN B=8 H=16 T=4096 d=128, E4M3 tiles every 64 tokens (the long-sequence workload):
    the full-size backward, then four units spread over the batch and the heads re-run alone
    (bit-identical by batch independence) and compared with the oracle over all 4096 tokens."""
    w = synth.WORKLOADS[2]
    d = synth.generate(w, with_do=True)
    c = gu.cfg_for(w, d, qdq=E4M3, group=64, qdq_interval=64, ckpt_interval=64)
    assert la.la_bwd_kernel_name(c) == "block"
    g = gu.run_bwd(c, d, d["do"].f32)
    for n in GRADS:
        assert np.all(np.isfinite(g[n])), n
    units = [(5, 11), (0, 0), (7, 15), (3, 4)]
    sub = {(b, h): sl(d, b, b + 1, 0, w.T, h, h + 1) for (b, h) in units}
    for (b, h) in units:
        sub[(b, h)]["do"] = synth.Tensor(f32=np.ascontiguousarray(d["do"].f32[b:b + 1, :, h:h + 1]), dtype="f32")
    del d
    for (b, h) in units:
        dd = sub[(b, h)]
        cu = gu.cfg_for(w, dd, qdq=E4M3, group=64, qdq_interval=64, ckpt_interval=64)
        cu.B, cu.H = 1, 1
        gu1 = gu.run_bwd(cu, dd, dd["do"].f32)
        for n in ["dq", "dk", "dv", "dbeta", "dg"]:
            np.testing.assert_array_equal(gu1[n][0, :, 0], g[n][b, :, h])
        np.testing.assert_array_equal(gu1["dS0"][0, 0], g["dS0"][b, h])
        states = block_states(cu, dd, None)
        ref = oracle.bwd(dd["q"].f64, dd["k"].f64, dd["v"].f64, dd["g"].f64, dd["beta"].f64, None,
                         dd["do"].f32.astype(np.float64), None, states=states, qdq_mode=E4M3, group=64,
                         qdq_interval=64)
        del states
        errs = {n: gu.err(gu1[n], ref[n]) for n in GRADS}
        print(f"unit ({b},{h})", {k: f"{v:.2e}" for k, v in errs.items()})
        assert max(errs.values()) <= TOL, errs
