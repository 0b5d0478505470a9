"""GPU parity of la_recurrent_bwd_ste against the CPU oracle.

The backward uses identity straight-through gradients through the state quantizer with
checkpointed recompute ("GDN state/W QAT foundation" and "Fused Triton GDN/KDA decode QAT",
both under "What does this PR do?").  With the quantizer off the gradient map is a smooth
function of the GPU's FP32 trajectory; with it on, the gradient is the unquantized
adjoint evaluated on the quantized trajectory.  The oracle is therefore fed the GPU's own
carried state entering every token (forward with per-token checkpoints): teacher forcing
of the trajectory; everything after that is float64.
"""
import dataclasses

import numpy as np
import pytest

import oracle
from oracle import chunk as oc
import quantized_state_qat_amd as la
import synth
from tests import gpu_util as gu
from tests.test_gpu_fwd import sl

pytestmark = pytest.mark.gpu

GRADS = ["dq", "dk", "dv", "dg", "dbeta", "dS0"]


def _check_against_oracle(c, d, S0, do, dST, g_gpu, tol):
    """S0 and dST are given in the representation the call used (rotated when
    c.state_rotated); the oracle works on the unrotated state."""
    had, rot = bool(c.hadamard), bool(c.state_rotated)
    rc = had and c.gate == la.LA_GATE_SCALAR  # per-key gates carry the unrotated state
    _, ST, states = gu.run_fwd(c, d, S0=S0, ckpt_interval=1)
    states = gu.rotated_to_state(states) if rc else states.astype(np.float64)
    S0_phys = None if S0 is None else (gu.rotated_to_state(S0) if rot else S0.astype(np.float64))
    dST_phys = None
    if dST is not None:
        # dL/dS = Hu dL/dY for a state held rotated
        dST_phys = gu.rotated_to_state(dST) * c.d_k if rot else dST.astype(np.float64)
    ref = oracle.bwd(d["q"].f64, d["k"].f64, d["v"].f64, d["g"].f64, d["beta"].f64,
                     S0_phys, do.astype(np.float64), dST_phys, states=states,
                     gate=c.gate, qdq_mode=c.qdq, group=c.group, hadamard=had,
                     qdq_interval=c.qdq_interval)
    g_cmp = dict(g_gpu)
    if rot:
        g_cmp["dS0"] = gu.rotated_to_state(g_gpu["dS0"]) * c.d_k
    errs = {}
    for name in GRADS:
        assert np.all(np.isfinite(g_gpu[name])), name
        errs[name] = gu.err(g_cmp[name], ref[name])
    assert max(errs.values()) <= tol, errs
    return errs


CASES = [
    # id, workload, qdq, group, hadamard, qdq_interval, ckpt, with dS_T
    ("gdn_wht_int8g32_tok", synth.Workload("w", B=2, T=130, H=2, d_k=128, d_v=128, config_id=31),
     la.LA_QDQ_INT8_GROUP, 32, 1, 1, 64, True),
    ("gdn_wht_int8g32_rotated_state", synth.Workload("wr", B=1, T=70, H=2, d_k=64, d_v=128, s0_sigma=0.2,
                                                     config_id=36),
     la.LA_QDQ_INT8_GROUP, 32, 2, 1, 32, True),
    ("kda_int8g64_tok", synth.Workload("k", B=2, T=100, H=2, d_k=128, d_v=128, gate="key", config_id=32),
     la.LA_QDQ_INT8_GROUP, 64, 0, 1, 64, False),
    ("kda_wht_int8g32_tok", synth.Workload("kw", B=1, T=70, H=2, d_k=128, d_v=128, gate="key", s0_sigma=0.2,
                                           config_id=41),
     la.LA_QDQ_INT8_GROUP, 32, 1, 1, 32, True),
    ("kda_wht_int8g64_i2_ckpt12", synth.Workload("kw2", B=2, T=41, H=1, d_k=128, d_v=64, gate="key", s0_sigma=0.2,
                                                 config_id=42),
     la.LA_QDQ_INT8_GROUP, 64, 1, 2, 12, True),
    # checkpoints from the KDA block forward, used (or recomputed by that forward) by the chunk
    # backward: every rounding point is a checkpoint
    ("kda_e4m3_64_block_ckpts", synth.Workload("kb", B=1, T=150, H=2, d_k=128, d_v=128, gate="key", gate_dtype="f32",
                                               s0_sigma=0.1, config_id=40),
     la.LA_QDQ_E4M3_TILE, 64, 0, 64, 64, True),
    ("gdn_e4m3_64", synth.Workload("e", B=2, T=150, H=2, d_k=128, d_v=128, gate_dtype="f32", config_id=33),
     la.LA_QDQ_E4M3_TILE, 64, 0, 64, 64, True),
    ("gdn_fp32_noqdq_dk64", synth.Workload("n", B=1, T=50, H=3, d_k=64, d_v=64, qkv_dtype="f32",
                                           gate_dtype="f32", s0_sigma=0.3, config_id=34),
     la.LA_QDQ_NONE, 32, 0, 1, 16, True),
    ("kda_int8g16_dv192_ckpt16", synth.Workload("r", B=1, T=45, H=2, d_k=32, d_v=192, gate="key",
                                                s0_sigma=0.1, config_id=35),
     la.LA_QDQ_INT8_GROUP, 16, 0, 1, 16, True),
    # recompute chunks that are not whole blocks of eight or groups of four tokens
    ("gdn_int8g32_ckpt5", synth.Workload("c5", B=1, T=23, H=2, d_k=128, d_v=64, s0_sigma=0.2, config_id=37),
     la.LA_QDQ_INT8_GROUP, 32, 0, 1, 5, True),
    ("kda_e4m3_i3_ckpt12_dk16", synth.Workload("c12", B=2, T=37, H=1, d_k=16, d_v=64, gate="key", s0_sigma=0.2,
                                               config_id=38),
     la.LA_QDQ_E4M3_TILE, 64, 0, 3, 12, True),
    ("gdn_wht_int8g16_fp32_ckpt7_dk32", synth.Workload("c7", B=1, T=30, H=2, d_k=32, d_v=64, qkv_dtype="f32",
                                                       gate_dtype="f32", s0_sigma=0.2, config_id=39),
     la.LA_QDQ_INT8_GROUP, 16, 1, 1, 7, False),
    # rounding every 16 tokens with checkpoints every 32: the forward runs the per-token kernel
    # (a rounding point falls inside a checkpoint chunk), so the backward must recompute with
    # it too rather than with the block kernel
    ("gdn_int8g32_i16_ckpt32", synth.Workload("c32", B=1, T=100, H=2, d_k=128, d_v=128, s0_sigma=0.2,
                                              config_id=43),
     la.LA_QDQ_INT8_GROUP, 32, 0, 16, 32, True),
]


@pytest.mark.parametrize("name,w,mode,group,had,interval,ckpt,with_dst", CASES, ids=[x[0] for x in CASES])
def test_bwd_matches_oracle(name, w, mode, group, had, interval, ckpt, with_dst):
    d = synth.generate(w, with_do=True, with_dST=with_dst)
    # had == 2: Hadamard with the state tensors held rotated
    c = gu.cfg_for(w, d, qdq=mode, group=group, hadamard=int(had > 0), qdq_interval=interval,
                   state_rotated=int(had == 2))
    S0 = d["S0"].f32 if w.s0_sigma > 0 else None
    dST = d["dST"].f32 if with_dst else None
    c.ckpt_interval = ckpt
    if name == "gdn_int8g32_i16_ckpt32":
        assert la.la_fwd_kernel_name(c) == "token" and la.la_bwd_kernel_name(c) == "token"
    if name == "kda_e4m3_64_block_ckpts":
        assert la.la_fwd_kernel_name(c) == "block" and la.la_bwd_kernel_name(c) == "chunk"
    g1 = gu.run_bwd(c, d, d["do"].f32, S0=S0, dST=dST)            # recomputes checkpoints
    _, _, ck = gu.run_fwd(c, d, S0=S0, ckpt_interval=ckpt)
    c.ckpt_interval = ckpt
    g2 = gu.run_bwd(c, d, d["do"].f32, S0=S0, dST=dST, ckpts=ck)  # uses the forward's
    for name_ in GRADS:
        np.testing.assert_array_equal(g1[name_], g2[name_])
    g3 = gu.run_bwd(c, d, d["do"].f32, S0=S0, dST=dST, ckpts=ck)
    for name_ in GRADS:
        np.testing.assert_array_equal(g3[name_], g2[name_])   # deterministic
    # bf16 inputs widen exactly and the trajectory is teacher forced: the fp32 bound applies
    # to every case (the 2e-3 bound for bf16 inputs is implied)
    errs = _check_against_oracle(c, d, S0, d["do"].f32, dST, g1, gu.TOL_F32)
    print(name, {k: f"{v:.2e}" for k, v in errs.items()})


def test_bwd_kda_chunk_and_token_backward_agree():
    """KDA with E4M3 every 64 tokens from the block forward's checkpoints: the chunk backward
    (what the configuration runs) and the per-token backward (asked for by kernel = token) take
    every state from those checkpoints (each rounding point is one), so both meet the chunked
    oracle's exact-solve backward teacher forced with the same checkpoints at the FP32 bound,
    and each other within twice it."""
    w = synth.Workload("kt", B=2, T=200, H=2, d_k=128, d_v=128, gate="key", gate_dtype="f32", s0_sigma=0.1,
                       config_id=58)
    d = synth.generate(w, with_do=True, with_dST=True)
    c = gu.cfg_for(w, d, qdq=la.LA_QDQ_E4M3_TILE, group=64, qdq_interval=64)
    c.ckpt_interval = 64
    ct = dataclasses.replace(c, kernel=la.LA_KERNEL_TOKEN)
    assert la.la_bwd_kernel_name(c) == "chunk" and la.la_bwd_kernel_name(ct) == "token"
    S0, dST = d["S0"].f32, d["dST"].f32
    _, _, ck = gu.run_fwd(c, d, S0=S0, ckpt_interval=64)
    c.ckpt_interval = 64
    gc = gu.run_bwd(c, d, d["do"].f32, S0=S0, dST=dST, ckpts=ck)
    gt = gu.run_bwd(ct, d, d["do"].f32, S0=S0, dST=dST, ckpts=ck)
    ref = oc.bwd(d["q"].f64, d["k"].f64, d["v"].f64, d["g"].f64, d["beta"].f64, S0.astype(np.float64),
                 d["do"].f64, dST.astype(np.float64),
                 gate=c.gate, qdq_mode=c.qdq, group=c.group, qdq_interval=c.qdq_interval,
                 chunk_states=ck.astype(np.float64))
    errs = {}
    for name in GRADS:
        for tag, g in (("chunk", gc), ("token", gt)):
            assert np.all(np.isfinite(g[name])), (tag, name)
            errs[f"{tag}_{name}"] = gu.err(g[name], ref[name])
        assert gu.err(gc[name], gt[name].astype(np.float64)) <= 2 * gu.TOL_F32, name
    assert max(errs.values()) <= gu.TOL_F32, errs
    print({k: f"{v:.2e}" for k, v in errs.items()})


def test_bwd_full_size_sampled_units():
    """GDN + Hadamard + INT8 g32 per token, B=4 H=16 T=2048 d=128, checkpoints every 64:
    full-size backward, then six units spread over the batch and the heads re-run alone
    (bit-identical by batch independence) and compared with the oracle over all 2048 tokens on
    the GPU's trajectory."""
    w = synth.WORKLOADS[4]
    d = synth.generate(w, with_do=True)
    c = gu.cfg_for(w, d, qdq=la.LA_QDQ_INT8_GROUP, group=32, hadamard=1, qdq_interval=1)
    c.ckpt_interval = 64
    g = gu.run_bwd(c, d, d["do"].f32)
    for name in GRADS:
        assert np.all(np.isfinite(g[name])), name
    for (b, h) in [(0, 0), (3, 15), (1, 4), (2, 9), (0, 13), (3, 2)]:
        dd = sl(d, b, b + 1, 0, w.T, h, h + 1)
        dd["do"] = synth.Tensor(f32=np.ascontiguousarray(d["do"].f32[b:b + 1, :, h:h + 1]), dtype="f32")
        cu = gu.cfg_for(w, dd, qdq=la.LA_QDQ_INT8_GROUP, group=32, hadamard=1, qdq_interval=1)
        cu.B, cu.H, cu.ckpt_interval = 1, 1, 64
        gu1 = gu.run_bwd(cu, dd, dd["do"].f32)
        for name in ["dq", "dk", "dv", "dbeta", "dg"]:
            np.testing.assert_array_equal(gu1[name][0, :, 0], g[name][b, :, h])
        np.testing.assert_array_equal(gu1["dS0"][0, 0], g["dS0"][b, h])
        errs = _check_against_oracle(cu, dd, None, dd["do"].f32, None, gu1, gu.TOL_F32)
        print(f"unit ({b},{h})", {k: f"{v:.2e}" for k, v in errs.items()})


STEEP_CASES = [
    ("gdn_wht_int8g32_i1", synth.Workload("sb1", B=1, T=90, H=2, d_k=64, d_v=128, s0_sigma=0.2, config_id=56),
     la.LA_QDQ_INT8_GROUP, 32, 1, 1, 16),
    ("kda_e4m3_i16", synth.Workload("sb2", B=1, T=85, H=2, d_k=64, d_v=64, gate="key", s0_sigma=0.2, config_id=57),
     la.LA_QDQ_E4M3_TILE, 64, 0, 16, 32),
]


@pytest.mark.parametrize("name,w,mode,group,had,interval,ckpt", STEEP_CASES, ids=[x[0] for x in STEEP_CASES])
def test_bwd_steep_gates(name, w, mode, group, had, interval, ckpt):
    """Gates whose products leave every rescaling range, one of them underflowing to zero in
    FP32 (the forward path tests' pattern): the backward applies gates token by token, so
    these check that decays of 2^-7 per token and a zero gate keep the adjoint finite and
    on the oracle's."""
    from tests.test_gpu_fwd_paths import steep_gates
    d = steep_gates(synth.generate(w, with_do=True, with_dST=True), w)
    c = gu.cfg_for(w, d, qdq=mode, group=group, hadamard=had, qdq_interval=interval)
    c.ckpt_interval = ckpt
    g = gu.run_bwd(c, d, d["do"].f32, S0=d["S0"].f32, dST=d["dST"].f32)
    errs = _check_against_oracle(c, d, d["S0"].f32, d["do"].f32, d["dST"].f32, g, gu.TOL_F32)
    print(name, {k: f"{v:.2e}" for k, v in errs.items()})


CODED_CASES = [
    # id, workload, group, hadamard, ckpt
    ("gdn_wht_int8g32_c64_ragged", synth.Workload("cw1", B=2, T=300, H=2, d_k=128, d_v=128, s0_sigma=0.2,
                                                  config_id=61), 32, 1, 64),
    ("gdn_int8g16_c16", synth.Workload("cw2", B=1, T=96, H=2, d_k=64, d_v=64, s0_sigma=0.2, config_id=62),
     16, 0, 16),
    ("gdn_int8g32_c5", synth.Workload("cw3", B=1, T=23, H=2, d_k=128, d_v=64, s0_sigma=0.2, config_id=63),
     32, 0, 5),
    ("gdn_wht_int8g16_dk32_c8", synth.Workload("cw4", B=1, T=40, H=2, d_k=32, d_v=64, s0_sigma=0.2,
                                               config_id=64), 16, 1, 8),
    ("kda_int8g64_c64", synth.Workload("cw5", B=2, T=150, H=2, d_k=128, d_v=128, gate="key", s0_sigma=0.2,
                                       config_id=65), 64, 0, 64),
    ("kda_int8g32_c32", synth.Workload("cw6", B=1, T=130, H=2, d_k=128, d_v=128, gate="key", s0_sigma=0.2,
                                       config_id=66), 32, 0, 32),
    ("gdn_int8g64_c1", synth.Workload("cw7", B=1, T=20, H=2, d_k=128, d_v=128, s0_sigma=0.2, config_id=67),
     64, 0, 1),
]


@pytest.mark.parametrize("name,w,group,had,ckpt", CODED_CASES, ids=[x[0] for x in CODED_CASES])
def test_bwd_coded_walk_matches_recompute_walk(name, w, group, had, ckpt):
    """With INT8 rounding after every token the token backward keeps each token's codes during
    its chunk recompute and decodes them for the adjoint (the coded walk).  Replay windows of one
    token round after every token too, with the same arithmetic ("Torch GDN/KDA decode QAT +
    INT8", What does this PR do?: a window of one writes a checkpoint each token), and take the
    recompute-per-group walk; the two walks' gradients must agree bit for bit."""
    d = synth.generate(w, with_do=True, with_dST=True)
    c = gu.cfg_for(w, d, qdq=la.LA_QDQ_INT8_GROUP, group=group, hadamard=had, qdq_interval=1)
    S0, dST = d["S0"].f32, d["dST"].f32
    _, _, ck = gu.run_fwd(c, d, S0=S0, ckpt_interval=ckpt)
    c.ckpt_interval = ckpt
    cr = dataclasses.replace(c, replay=1)
    _, _, ckr = gu.run_fwd(cr, d, S0=S0, ckpt_interval=ckpt)
    np.testing.assert_array_equal(ck, ckr)  # the forwards agree too
    cr.ckpt_interval = ckpt
    assert la.la_bwd_workspace_bytes(c) != la.la_bwd_workspace_bytes(cr)  # the two walks' layouts
    g_coded = gu.run_bwd(c, d, d["do"].f32, S0=S0, dST=dST, ckpts=ck)
    g_group = gu.run_bwd(cr, d, d["do"].f32, S0=S0, dST=dST, ckpts=ck)
    for name_ in GRADS:
        assert np.all(np.isfinite(g_coded[name_])), name_
        np.testing.assert_array_equal(g_coded[name_].view(np.uint32), g_group[name_].view(np.uint32), err_msg=name_)
