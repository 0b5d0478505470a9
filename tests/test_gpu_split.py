"""GPU parity of the packed-sequence backward and of the per-sequence prefix/suffix boundary
("Torch GDN/KDA decode QAT + INT8", What does this PR do?: an explicit per-sequence boundary
selects a chunked prefill prefix and a recurrent suffix, suffix gradients flow through the
handoff into the prefill; "Experimental GDN/KDA approximate-inverse QAT", Testing: packed
sequence tails).

Every packed call runs the per-token kernel, as the single-sequence calls do when they ask for
it (kernel = LA_KERNEL_TOKEN): each packed sequence, and each part of a split one, must equal
those calls on its own tokens bit for bit, and tokens outside every sequence get zero
gradients.  The single-sequence calls are compared with the oracle teacher forced (the
per-token trajectory from checkpoints after every token), the split backward with the
oracle's split backward on that trajectory.
"""
import numpy as np
import pytest

import oracle
import quantized_state_qat_amd as la
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

LENS = [37, 0, 1, 30, 17, 9]
PRE = [20, 3, 0, 30, 40, 4]      # clamped to each sequence: 20, 0, 0, 30, 17, 4
TAIL = 3                          # packed tokens after the last sequence
GRADS = ["dq", "dk", "dv", "dg", "dbeta"]
INT8, E4M3 = la.LA_QDQ_INT8_GROUP, la.LA_QDQ_E4M3_TILE


def packed_inputs(H, dk, dv, gate, seed):
    T = sum(LENS) + TAIL
    w = synth.Workload("pk", B=1, T=T, H=H, d_k=dk, d_v=dv, gate=gate, config_id=seed)
    d = synth.generate(w, with_do=True)
    rng = np.random.default_rng(seed)
    B = len(LENS)
    S0 = (rng.standard_normal((B, H, dk, dv)) * 0.2).astype(np.float32)
    dST = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(LENS)]).astype(np.int32)
    return w, d, S0, dST, cu


def dev_all(d):
    return {n: gu.dev(d[n]) for n in ("q", "k", "v", "g", "beta")}


def seq_slice(d, t0, t1):
    out = {}
    for n in ("q", "k", "v", "g", "beta"):
        x = d[n]
        out[n] = synth.Tensor(f32=np.ascontiguousarray(x.f32[:, t0:t1]), dtype=x.dtype,
                              bits=None if x.bits is None else np.ascontiguousarray(x.bits[:, t0:t1]))
    out["do"] = synth.Tensor(f32=np.ascontiguousarray(d["do"].f32[:, t0:t1]), dtype="f32")
    return out


def packed_grads_gpu(torch, c, T, H, dk, dv, gate):
    gshape = (T, H, dk) if gate == "key" else (T, H)
    return {"dq": gu.nan_like(torch, (T, H, dk)), "dk": gu.nan_like(torch, (T, H, dk)),
            "dv": gu.nan_like(torch, (T, H, dv)), "dg": gu.nan_like(torch, gshape),
            "dbeta": gu.nan_like(torch, (T, H)), "dS0": gu.nan_like(torch, (c.B, H, dk, dv))}


def one_seq_cfg(w, d, L, **kw):
    c = gu.cfg_for(w, d, **kw)
    c.B, c.T, c.kernel = 1, L, la.LA_KERNEL_TOKEN
    return c


VARLEN_BWD = [
    # name, d_k, gate, quantizer kw, checkpoint spacing
    ("gdn_wht_int8g32_tok_ckpt16", 128, "scalar", dict(qdq=INT8, group=32, hadamard=1, qdq_interval=1), 16),
    ("kda_e4m3_i12_ckpt12", 64, "key", dict(qdq=E4M3, group=64, qdq_interval=12), 12),
    ("gdn_int8g16_replay_w4_ckpt8", 128, "scalar", dict(qdq=INT8, group=16, qdq_interval=4, replay=1), 8),
]


@pytest.mark.parametrize("name,dk,gate,qkw,ckpt", VARLEN_BWD, ids=[v[0] for v in VARLEN_BWD])
def test_varlen_backward(name, dk, gate, qkw, ckpt):
    from tests.test_gpu_bwd import _check_against_oracle
    torch = gu.torch_mod()
    H, dv = 2, 128
    w, d, S0, dST, cu = packed_inputs(H, dk, dv, gate, 71)
    T = int(cu[-1]) + TAIL
    c = gu.cfg_for(w, d, ckpt_interval=ckpt, **qkw)
    c.B, c.T = len(LENS), T
    di = dev_all(d)
    g = packed_grads_gpu(torch, c, T, H, dk, dv, gate)
    nbytes = la.la_bwd_varlen_workspace_bytes(c)
    ws = torch.full((nbytes // 4 + 1,), float("nan"), device="cuda")
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    la.la_recurrent_bwd_ste_varlen(c, f(cu), di["q"], di["k"], di["v"], di["g"], di["beta"], f(S0),
                                   f(d["do"].f32[0]), f(dST), g["dq"], g["dk"], g["dv"], g["dg"], g["dbeta"], g["dS0"],
                                   ws, nbytes)
    torch.cuda.synchronize()
    g = {n: x.cpu().numpy() for n, x in g.items()}
    for n in GRADS:
        assert np.all(g[n][T - TAIL:] == 0), n          # outside every sequence
    for b, L in enumerate(LENS):
        t0, t1 = int(cu[b]), int(cu[b + 1])
        if L == 0:
            np.testing.assert_array_equal(g["dS0"][b], dST[b])
            continue
        ds = seq_slice(d, t0, t1)
        cb = one_seq_cfg(w, ds, L, ckpt_interval=ckpt, **qkw)
        r = gu.run_bwd(cb, ds, ds["do"].f32, S0=S0[b:b + 1], dST=dST[b:b + 1])
        for n in GRADS:
            np.testing.assert_array_equal(g[n][t0:t1], r[n][0], err_msg=f"{n} seq {b}")
        np.testing.assert_array_equal(g["dS0"][b], r["dS0"][0])
        if L > 1:
            _check_against_oracle(cb, ds, S0[b:b + 1], ds["do"].f32, dST[b:b + 1], r, gu.TOL_F32)


PK = dict(qdq=E4M3, group=64, qdq_interval=64, ckpt_interval=64)      # chunked prefill prefix
SK = dict(qdq=INT8, group=32, hadamard=1, qdq_interval=1, ckpt_interval=16)  # recurrent suffix


@pytest.mark.parametrize("gate", ["scalar", "key"])
def test_split_forward_and_backward(gate):
    from tests.test_gpu_fwd import per_token_teacher_forced
    torch = gu.torch_mod()
    H, dk, dv = 2, 128, 128
    w, d, S0, dST, cu = packed_inputs(H, dk, dv, gate, 72)
    T = int(cu[-1]) + TAIL
    B = len(LENS)
    cp, cs = gu.cfg_for(w, d, **PK), gu.cfg_for(w, d, **SK)
    for c in (cp, cs):
        c.B, c.T = B, T
    di = dev_all(d)
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    cu_d, pre_d = f(cu), f(np.array(PRE, dtype=np.int32))
    o = gu.nan_like(torch, (T, H, dv))
    S_mid = gu.nan_like(torch, (B, H, dk, dv))
    S_T = gu.nan_like(torch, (B, H, dk, dv))
    la.la_recurrent_fwd_split(cp, cs, cu_d, pre_d, di["q"], di["k"], di["v"], di["g"], di["beta"], f(S0), o, S_mid, S_T)
    g = packed_grads_gpu(torch, cp, T, H, dk, dv, gate)
    nbytes = la.la_bwd_split_workspace_bytes(cp, cs)
    ws = torch.full((nbytes // 4 + 1,), float("nan"), device="cuda")
    la.la_recurrent_bwd_ste_split(cp, cs, cu_d, pre_d, di["q"], di["k"], di["v"], di["g"], di["beta"], f(S0), S_mid,
                                  f(d["do"].f32[0]), f(dST), g["dq"], g["dk"], g["dv"], g["dg"], g["dbeta"],
                                  g["dS0"], ws, nbytes)
    torch.cuda.synchronize()
    o, S_mid, S_T = o.cpu().numpy(), S_mid.cpu().numpy(), S_T.cpu().numpy()
    g = {n: x.cpu().numpy() for n, x in g.items()}
    for n in GRADS:
        assert np.all(g[n][T - TAIL:] == 0), n
    tally = gu.CodeTally()
    states = np.zeros((T, H, dk, dv))      # carried state entering each token, teacher forcing
    worst = 0.0
    for b, L in enumerate(LENS):
        t0, t1 = int(cu[b]), int(cu[b + 1])
        m = t0 + min(max(PRE[b], 0), L)
        # prefix alone, from S0 (the prefix rounds only at its end: lengths below 64)
        if m > t0:
            dp = seq_slice(d, t0, m)
            c1 = one_seq_cfg(w, dp, m - t0, **PK)
            o1, S1, ck1 = gu.run_fwd(c1, dp, S0=S0[b:b + 1], ckpt_interval=1)
            np.testing.assert_array_equal(o[t0:m], o1[0])
            np.testing.assert_array_equal(S_mid[b], S1[0])
            states[t0:m] = ck1[0].transpose(1, 0, 2, 3)
            o_r, Sp, _ = oracle.fwd(dp["q"].f64, dp["k"].f64, dp["v"].f64, dp["g"].f64, dp["beta"].f64,
                                    S0[b:b + 1].astype(np.float64), gate=c1.gate)
            worst = max(worst, gu.err(o1, o_r))
            for h in range(H):
                _, codes, _, ypre = oracle.qdq(Sp[0, h], E4M3, 64)
                gu.compare_e4m3_point(S1[0, h], codes, ypre, tally)
        else:
            np.testing.assert_array_equal(S_mid[b], S0[b])
        # suffix alone, from the handoff state, teacher forced token by token
        if t1 > m:
            ds = seq_slice(d, m, t1)
            c2 = one_seq_cfg(w, ds, t1 - m, **SK)
            o2, S2, ck2 = gu.run_fwd(c2, ds, S0=S_mid[b:b + 1], ckpt_interval=1)
            np.testing.assert_array_equal(o[m:t1], o2[0])
            np.testing.assert_array_equal(S_T[b], S2[0])
            wo, _ = per_token_teacher_forced(c2, ds, ck2, S2, o2, gu.TOL_F32, tally)
            worst = max(worst, wo)
            # the scalar gate carries the rotated state in Hadamard mode, per-key gates S itself
            st2 = gu.rotated_to_state(ck2[0]) if gate == "scalar" else ck2[0].astype(np.float64)
            states[m:t1] = st2.transpose(1, 0, 2, 3)
        else:
            np.testing.assert_array_equal(S_T[b], S_mid[b])
    assert worst <= gu.TOL_F32, worst
    tally.check()
    # backward on the GPU trajectory against the oracle's split backward
    to64 = lambda x: x.f64[0]
    pk_o = dict(qdq_mode=E4M3, group=64, qdq_interval=64)
    sk_o = dict(qdq_mode=INT8, group=32, hadamard=True, qdq_interval=1)
    ref = oracle.bwd_split(to64(d["q"]), to64(d["k"]), to64(d["v"]), to64(d["g"]), to64(d["beta"]), cu, PRE,
                           S0.astype(np.float64), S_mid.astype(np.float64), d["do"].f32[0].astype(np.float64),
                           dST.astype(np.float64), pk_o, sk_o, gate=cp.gate, states=states)
    errs = {n: gu.err(g[n][:T - TAIL], ref[n][:T - TAIL]) for n in GRADS}
    errs["dS0"] = gu.err(g["dS0"], ref["dS0"])
    assert max(errs.values()) <= gu.TOL_F32, errs
    print(gate, {k: f"{v:.2e}" for k, v in errs.items()}, f"codes {tally.mismatches}/{tally.total}")
