"""GPU parity of la_recurrent_fwd_varlen (packed sequences of different lengths; the pages'
packed sequence tails, GDN/KDA state QAT).

Every configuration is served by the per-token kernel.  Where la_recurrent_fwd serves the same
configuration with that kernel too (rounding after every token, per-key gates, the Hadamard
rotation), each packed sequence must equal la_recurrent_fwd on that sequence alone bit for bit.
The packed result is compared with the oracle's packed forward without a quantizer, and with
every quantizer teacher forced at each rounding point (chained packed calls).
"""
import numpy as np
import pytest

import oracle
import quantized_state_qat_amd as la
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

LENS = [37, 0, 1, 130, 64, 17]


def _packed(w, lens, seed):
    """Inputs of len(lens) sequences drawn as one sequence of the total length, then cut."""
    T = int(sum(lens))
    wp = synth.Workload(w.name, B=1, T=T, H=w.H, d_k=w.d_k, d_v=w.d_v, gate=w.gate, qkv_dtype=w.qkv_dtype,
                        gate_dtype=w.gate_dtype, s0_sigma=0.0, config_id=seed)
    d = synth.generate(wp)
    rng = np.random.default_rng(seed)
    S0 = (rng.standard_normal((len(lens), w.H, w.d_k, w.d_v)) * 0.2).astype(np.float32)
    return d, S0, np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def _run_varlen(c, d, S0, cu):
    torch = gu.torch_mod()
    di = {k: gu.dev(d[k]) for k in ("q", "k", "v", "g", "beta")}
    o = gu.nan_like(torch, (c.T, c.H, c.d_v))
    ST = gu.nan_like(torch, (c.B, c.H, c.d_k, c.d_v))
    la.la_recurrent_fwd_varlen(c, torch.from_numpy(cu).cuda(), di["q"], di["k"], di["v"], di["g"], di["beta"],
                               torch.from_numpy(S0).cuda(), o, ST)
    torch.cuda.synchronize()
    return o.cpu().numpy(), ST.cpu().numpy()


CASES = [
    # name, d_k, d_v, gate, qdq, group, hadamard, interval
    ("gdn_int8g32_tok", 128, 128, "scalar", la.LA_QDQ_INT8_GROUP, 32, 0, 1),
    # an interval that is not a multiple of 8 keeps the single-sequence calls on the token kernel
    ("kda_e4m3_i12", 64, 128, "key", la.LA_QDQ_E4M3_TILE, 64, 0, 12),
    ("gdn_wht_int8g16_tok", 128, 64, "scalar", la.LA_QDQ_INT8_GROUP, 16, 1, 1),
    ("kda_wht_int8g32_tok", 128, 128, "key", la.LA_QDQ_INT8_GROUP, 32, 1, 1),
]


@pytest.mark.parametrize("name,dk,dv,gate,mode,group,had,interval", CASES, ids=[c[0] for c in CASES])
def test_varlen_equals_single_sequences(name, dk, dv, gate, mode, group, had, interval):
    w = synth.Workload(name, B=1, T=1, H=2, d_k=dk, d_v=dv, gate=gate)
    d, S0, cu = _packed(w, LENS, 61)
    c = gu.cfg_for(w, d, qdq=mode, group=group, hadamard=had, qdq_interval=interval)
    c.B, c.T = len(LENS), int(cu[-1])
    o, ST = _run_varlen(c, d, S0, cu)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ST))
    for b, L in enumerate(LENS):
        t0, t1 = int(cu[b]), int(cu[b + 1])
        db = {k_: synth.Tensor(f32=np.ascontiguousarray(d[k_].f32[:, t0:t1]), dtype=d[k_].dtype,
                               bits=None if d[k_].bits is None else np.ascontiguousarray(d[k_].bits[:, t0:t1]))
              for k_ in ("q", "k", "v", "g", "beta")}
        cb = gu.cfg_for(w, db, qdq=mode, group=group, hadamard=had, qdq_interval=interval)
        cb.B, cb.T = 1, L
        if L > 0:
            assert la.la_fwd_kernel_name(cb) == "token"
        ob, STb, _ = gu.run_fwd(cb, db, S0=S0[b:b + 1])
        np.testing.assert_array_equal(ST[b], STb[0])
        if L > 0:
            np.testing.assert_array_equal(o[t0:t1], ob[0])


def test_varlen_matches_oracle_without_quantizer():
    w = synth.Workload("vn", B=1, T=1, H=3, d_k=128, d_v=128)
    d, S0, cu = _packed(w, LENS, 62)
    c = gu.cfg_for(w, d, qdq=la.LA_QDQ_NONE)
    c.B, c.T = len(LENS), int(cu[-1])
    o, ST = _run_varlen(c, d, S0, cu)
    o_r, ST_r = oracle.fwd_varlen(d["q"].f64[0], d["k"].f64[0], d["v"].f64[0], d["g"].f64[0], d["beta"].f64[0],
                                  cu, S0.astype(np.float64))
    assert gu.err(o, o_r) <= gu.TOL_F32
    assert gu.err(ST, ST_r) <= gu.TOL_F32


def test_varlen_clamps_boundaries_to_the_packed_length():
    """The last boundary beyond the packed length is clamped: the last sequence ends at T."""
    w = synth.Workload("vc", B=1, T=1, H=2, d_k=64, d_v=64)
    lens = [20, 12]
    d, S0, cu = _packed(w, lens, 63)
    c = gu.cfg_for(w, d, qdq=la.LA_QDQ_INT8_GROUP, group=32)
    c.B, c.T = 2, int(cu[-1])
    o, ST = _run_varlen(c, d, S0, cu)
    cu_far = cu.copy()
    cu_far[-1] = 10 ** 6
    o2, ST2 = _run_varlen(c, d, S0, cu_far)
    np.testing.assert_array_equal(o2, o)
    np.testing.assert_array_equal(ST2, ST)


CHAINED = [
    # name, d_k, d_v, gate, qdq, group, hadamard, interval
    ("gdn_int8g32_i4", 128, 128, "scalar", la.LA_QDQ_INT8_GROUP, 32, 0, 4),
    ("kda_e4m3_i6", 64, 128, "key", la.LA_QDQ_E4M3_TILE, 64, 0, 6),
    ("gdn_wht_int8g16_tok", 128, 64, "scalar", la.LA_QDQ_INT8_GROUP, 16, 1, 1),
    ("kda_wht_int8g32_i3", 128, 128, "key", la.LA_QDQ_INT8_GROUP, 32, 1, 3),
]


@pytest.mark.parametrize("name,dk,dv,gate,mode,group,had,interval", CHAINED, ids=[c[0] for c in CHAINED])
def test_varlen_quantized_against_oracle(name, dk, dv, gate, mode, group, had, interval):
    """The packed forward with a quantizer against the oracle's packed forward, teacher forced
    at every rounding point: each sequence is cut into pieces of at most `interval` tokens and
    the pieces are run as successive packed calls, each starting from the GPU's states after
    the previous call.  A call rounds only after each sequence's last token, so every output
    reads an unrounded state (fp32 bound), and each sequence's final state is compared code
    for code with the oracle's rounding of the same entering state (near-tie protocol)."""
    lens = [37, 0, 1, 30, 17, 9]
    w = synth.Workload(name, B=1, T=1, H=2, d_k=dk, d_v=dv, gate=gate)
    d, S0, cu = _packed(w, lens, 64)
    tally = gu.CodeTally()
    worst_o = 0.0
    S_prev = S0
    done = np.zeros(len(lens), dtype=np.int64)
    calls = 0
    while np.any(done < np.array(lens)):
        piece = np.minimum(np.array(lens) - done, interval)
        idx = np.concatenate([np.arange(cu[b] + done[b], cu[b] + done[b] + piece[b]) for b in range(len(lens))])
        dp = {n: synth.Tensor(f32=np.ascontiguousarray(d[n].f32[:, idx]), dtype=d[n].dtype,
                              bits=None if d[n].bits is None else np.ascontiguousarray(d[n].bits[:, idx]))
              for n in ("q", "k", "v", "g", "beta")}
        cu_p = np.concatenate([[0], np.cumsum(piece)]).astype(np.int32)
        c = gu.cfg_for(w, dp, qdq=mode, group=group, hadamard=had, qdq_interval=interval)
        c.B, c.T = len(lens), int(cu_p[-1])
        o, ST = _run_varlen(c, dp, S_prev, cu_p)
        o_r, Sp = oracle.fwd_varlen(dp["q"].f64[0], dp["k"].f64[0], dp["v"].f64[0], dp["g"].f64[0],
                                    dp["beta"].f64[0], cu_p, S_prev.astype(np.float64), gate=c.gate)
        worst_o = max(worst_o, gu.err(o, o_r))
        for b in range(len(lens)):
            if piece[b] == 0:
                np.testing.assert_array_equal(ST[b], S_prev[b])   # an empty piece hands S0 through
                continue
            for h in range(w.H):
                _, codes, _, ypre = oracle.qdq(Sp[b, h], c.qdq, c.group, bool(had))
                if mode == la.LA_QDQ_INT8_GROUP:
                    gu.compare_int8_codes(ST[b, h], codes, ypre, group, hadamard=bool(had), tally=tally)
                else:
                    gu.compare_e4m3_point(ST[b, h], codes, ypre, tally)
        S_prev = ST
        done += piece
        calls += 1
    assert worst_o <= gu.TOL_F32, worst_o
    frac = tally.check()
    print(f"{name}: {calls} chained packed calls, max output error {worst_o:.2e}, "
          f"code mismatches {tally.mismatches}/{tally.total} ({frac:.2e})")
