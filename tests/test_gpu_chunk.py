"""GPU parity of the 64-token chunk form (la_recurrent_fwd_chunk) against the chunked oracle
(oracle/chunk.py): the exact triangular solve and the Neumann approximate inverse of degree
3, 7, 15 and 31 ("Experimental GDN/KDA approximate-inverse QAT", What does this PR do?), GDN
and KDA gates, rounding at chunk ends ("GDN state/W QAT foundation", What does this PR do?).

Without a quantizer the GPU's outputs and final state are compared with the oracle's float64
forward of the whole call.  With one, the comparison is teacher forced per chunk: the GPU's
checkpoints (every 64 tokens) are the states entering each chunk; the oracle advances each
of them over the chunk's tokens in float64, and the GPU's outputs, the next checkpoint's
codes (near-tie protocol of tests/gpu_util.py) and the final state are checked against it.
Bars: outputs and states to 1e-5 of their largest magnitude (inputs widen exactly from bf16,
so the comparison is fp32 arithmetic against float64).
"""
import numpy as np
import pytest

import oracle
import quantized_state_qat_amd as la
import synth
from oracle import chunk as oc
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

INT8, E4M3 = la.LA_QDQ_INT8_GROUP, la.LA_QDQ_E4M3_TILE


def chunk_cfg(w, d, solve, degree, **kw):
    c = gu.cfg_for(w, d, kernel=la.LA_KERNEL_CHUNK, solve=solve, degree=degree, **kw)
    if solve == la.LA_SOLVE_EXACT:
        c.degree = 0
    return c


def run_chunk(c, d, S0=None, ckpt_interval=0, dev_inputs=None):
    torch = gu.torch_mod()
    c.ckpt_interval = ckpt_interval
    di = dev_inputs or {k: gu.dev(d[k]) for k in ("q", "k", "v", "g", "beta")}
    S0d = None if S0 is None else torch.from_numpy(np.ascontiguousarray(S0, dtype=np.float32)).cuda()
    o = gu.nan_like(torch, (c.B, c.T, c.H, c.d_v))
    ST = gu.nan_like(torch, (c.B, c.H, c.d_k, c.d_v))
    ck = None
    if ckpt_interval:
        ck = gu.nan_like(torch, (c.B, c.H, (c.T + ckpt_interval - 1) // ckpt_interval, c.d_k, c.d_v))
    nbytes = la.la_chunk_workspace_bytes(c)
    assert nbytes > 0
    ws = torch.full((nbytes // 4 + 1,), float("nan"), device="cuda")
    la.la_recurrent_fwd_chunk(c, di["q"], di["k"], di["v"], di["g"], di["beta"], S0d, o, ST, ck, ws, nbytes)
    torch.cuda.synchronize()
    return o.cpu().numpy(), ST.cpu().numpy(), None if ck is None else ck.cpu().numpy()


def oracle_kw(c):
    return dict(gate=c.gate, solve=c.solve, degree=c.degree)


def inputs(name, B, T, H, gate, seed, s0=0.3):
    w = synth.Workload(name, B=B, T=T, H=H, d_k=128, d_v=128, gate=gate, config_id=seed)
    d = synth.generate(w)
    S0 = (np.random.default_rng(seed).standard_normal((B, H, 128, 128)) * s0).astype(np.float32)
    return w, d, S0


SOLVES = [(la.LA_SOLVE_EXACT, 0), (la.LA_SOLVE_NEUMANN, 3), (la.LA_SOLVE_NEUMANN, 7), (la.LA_SOLVE_NEUMANN, 15),
          (la.LA_SOLVE_NEUMANN, 31)]


@pytest.mark.parametrize("gate", ["scalar", "key"])
@pytest.mark.parametrize("solve,degree", SOLVES, ids=["exact", "n3", "n7", "n15", "n31"])
def test_chunk_forward_without_rounding(gate, solve, degree):
    """Three chunks, the last one ragged (64 + 64 + 22 tokens), two value tiles."""
    w, d, S0 = inputs("chunk_plain", 2, 150, 2, gate, 300 + degree)
    c = chunk_cfg(w, d, solve, degree)
    o, ST, _ = run_chunk(c, d, S0)
    o_r, ST_r, _ = oc.fwd(d["q"].f64, d["k"].f64, d["v"].f64, d["g"].f64, d["beta"].f64, S0, **oracle_kw(c))
    assert gu.err(o, o_r) <= gu.TOL_F32, gu.err(o, o_r)
    assert gu.err(ST, ST_r) <= gu.TOL_F32, gu.err(ST, ST_r)
    if solve == la.LA_SOLVE_EXACT:
        # the exact chunk form is the token recurrence
        o_t, ST_t, _ = oracle.fwd(d["q"].f64, d["k"].f64, d["v"].f64, d["g"].f64, d["beta"].f64, S0, gate=c.gate)
        assert gu.err(o, o_t) <= gu.TOL_F32 and gu.err(ST, ST_t) <= gu.TOL_F32


def teacher_forced_chunks(c, d, ck, ST, o, tally, units=None):
    """Per chunk from the GPU's checkpoint: outputs, then the next state (codes at rounding
    points).  Returns the largest output and state errors."""
    B, T, H = c.B, c.T, c.H
    nch = (T + 63) // 64
    units = units or [(b, h) for b in range(B) for h in range(H)]
    worst_o = worst_s = 0.0
    for b, h in units:
        for j in range(nch):
            t0, t1 = 64 * j, min(T, 64 * j + 64)
            args = [d[n].f64[b:b + 1, t0:t1, h:h + 1] for n in ("q", "k", "v", "g", "beta")]
            S_in = ck[b:b + 1, h:h + 1, j].astype(np.float64)
            o_r, S_pre, _ = oc.fwd(*args, S_in, **oracle_kw(c))
            worst_o = max(worst_o, gu.err(o[b, t0:t1, h], o_r[0, :, 0]))
            S_gpu = ck[b, h, j + 1] if j + 1 < nch else ST[b, h]
            qpoint = c.qdq != la.LA_QDQ_NONE and (t1 % c.qdq_interval == 0 or t1 == T)
            if not qpoint:
                worst_s = max(worst_s, gu.err(S_gpu, S_pre[0, 0]))
                continue
            _, codes, _, ypre = oracle.qdq(S_pre[0, 0], c.qdq, c.group)
            if c.qdq == E4M3:
                gu.compare_e4m3_point(S_gpu, codes, ypre, tally)
            else:
                gu.compare_int8_codes(S_gpu, codes, ypre, c.group, tally=tally)
    return worst_o, worst_s


QCASES = [
    # name, gate, quantizer kw, solve, degree, T
    ("gdn_e4m3_exact", "scalar", dict(qdq=E4M3, group=64, qdq_interval=64), la.LA_SOLVE_EXACT, 0, 200),
    ("gdn_e4m3_n7", "scalar", dict(qdq=E4M3, group=64, qdq_interval=64), la.LA_SOLVE_NEUMANN, 7, 200),
    ("kda_e4m3_n3", "key", dict(qdq=E4M3, group=64, qdq_interval=64), la.LA_SOLVE_NEUMANN, 3, 170),
    ("kda_e4m3_exact", "key", dict(qdq=E4M3, group=64, qdq_interval=64), la.LA_SOLVE_EXACT, 0, 170),
    ("gdn_int8g32_i128_n31", "scalar", dict(qdq=INT8, group=32, qdq_interval=128), la.LA_SOLVE_NEUMANN, 31, 300),
    ("kda_int8g16_n15", "key", dict(qdq=INT8, group=16, qdq_interval=64), la.LA_SOLVE_NEUMANN, 15, 140),
    ("gdn_int8g64_exact", "scalar", dict(qdq=INT8, group=64, qdq_interval=64), la.LA_SOLVE_EXACT, 0, 100),
]


@pytest.mark.parametrize("name,gate,qkw,solve,degree,T", QCASES, ids=[q[0] for q in QCASES])
def test_chunk_forward_rounding_teacher_forced(name, gate, qkw, solve, degree, T):
    w, d, S0 = inputs(name, 2, T, 2, gate, 310 + degree + T)
    c = chunk_cfg(w, d, solve, degree, **qkw)
    o, ST, ck = run_chunk(c, d, S0, ckpt_interval=64)
    np.testing.assert_array_equal(ck[:, :, 0], S0)
    tally = gu.CodeTally()
    wo, ws = teacher_forced_chunks(c, d, ck, ST, o, tally)
    assert wo <= gu.TOL_F32 and ws <= gu.TOL_F32, (wo, ws)
    tally.check()
    # the checkpointed call and a call without checkpoints agree bit for bit
    o2, ST2, _ = run_chunk(c, d, S0)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(ST, ST2)


@pytest.mark.parametrize("gate,degree", [("scalar", 31), ("key", 7)])
def test_chunk_forward_long_sequence_sampled(gate, degree):
    """The long-sequence workload's shape (B=8 H=16 T=4096, E4M3 tiles every 64 tokens): every
    chunk of sampled units teacher forced; batch independence over the rest."""
    w = synth.Workload("chunk_long", B=8, T=4096, H=16, d_k=128, d_v=128, gate=gate, gate_dtype="f32", config_id=2)
    d = synth.generate(w)
    c = chunk_cfg(w, d, la.LA_SOLVE_NEUMANN, degree, qdq=E4M3, group=64, qdq_interval=64)
    o, ST, ck = run_chunk(c, d, None, ckpt_interval=64)
    tally = gu.CodeTally()
    units = [(0, 0), (3, 7), (7, 15)]
    wo, ws = teacher_forced_chunks(c, d, ck, ST, o, tally, units=units)
    assert wo <= gu.TOL_F32 and ws <= gu.TOL_F32, (wo, ws)
    tally.check()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ST))


@pytest.mark.parametrize("gate", ["scalar", "key"])
def test_chunk_split_and_resume(gate):
    """Two calls cut at a chunk end equal one call bit for bit (rounding every 64 tokens)."""
    w, d, S0 = inputs("chunk_split", 1, 256, 2, gate, 320)
    c = chunk_cfg(w, d, la.LA_SOLVE_NEUMANN, 7, qdq=E4M3, group=64, qdq_interval=64)
    o, ST, _ = run_chunk(c, d, S0)
    from tests.test_gpu_fwd import sl
    d1, d2 = sl(d, 0, 1, 0, 128, 0, 2), sl(d, 0, 1, 128, 256, 0, 2)
    c1 = chunk_cfg(w, d, la.LA_SOLVE_NEUMANN, 7, qdq=E4M3, group=64, qdq_interval=64)
    c1.T = 128
    o1, S1, _ = run_chunk(c1, d1, S0)
    o2, S2, _ = run_chunk(c1, d2, S1)
    np.testing.assert_array_equal(np.concatenate([o1, o2], axis=1), o)
    np.testing.assert_array_equal(S2, ST)


@pytest.mark.parametrize("T", [1, 5, 63, 64, 65])
def test_chunk_short_and_edge_lengths(T):
    w, d, S0 = inputs("chunk_edge", 1, T, 1, "key", 330 + T)
    c = chunk_cfg(w, d, la.LA_SOLVE_NEUMANN, 3, qdq=E4M3, group=64, qdq_interval=64)
    o, ST, ck = run_chunk(c, d, S0, ckpt_interval=64)
    tally = gu.CodeTally()
    wo, ws = teacher_forced_chunks(c, d, ck, ST, o, tally)
    assert wo <= gu.TOL_F32 and ws <= gu.TOL_F32, (wo, ws)
    tally.check()


def test_chunk_empty_call_hands_the_state_through():
    torch = gu.torch_mod()
    c = la.Config(B=2, T=0, H=2, d_k=128, d_v=64, kernel=la.LA_KERNEL_CHUNK)
    S0 = torch.randn(2, 2, 128, 64, device="cuda", dtype=torch.float32)
    ST = torch.full_like(S0, float("nan"))
    la.la_recurrent_fwd_chunk(c, None, None, None, None, None, S0, None, ST, None, None, 0)
    torch.cuda.synchronize()
    assert torch.equal(ST, S0)


# ---------------------------------------------------------------- backward

def run_chunk_bwd(c, d, S0, ck, do, dST, dev_inputs=None):
    torch = gu.torch_mod()
    di = dev_inputs or {k: gu.dev(d[k]) for k in ("q", "k", "v", "g", "beta")}
    f = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    gshape = (c.B, c.T, c.H, c.d_k) if c.gate == la.LA_GATE_KEY else (c.B, c.T, c.H)
    out = {"dq": gu.nan_like(torch, (c.B, c.T, c.H, c.d_k)), "dk": gu.nan_like(torch, (c.B, c.T, c.H, c.d_k)),
           "dv": gu.nan_like(torch, (c.B, c.T, c.H, c.d_v)), "dg": gu.nan_like(torch, gshape),
           "dbeta": gu.nan_like(torch, (c.B, c.T, c.H)), "dS0": gu.nan_like(torch, (c.B, c.H, c.d_k, c.d_v))}
    nbytes = la.la_bwd_workspace_bytes(c)
    assert nbytes > 0, la.la_last_error()
    ws = torch.full((nbytes // 4 + 1,), float("nan"), device="cuda")
    la.la_recurrent_bwd_ste(c, di["q"], di["k"], di["v"], di["g"], di["beta"], f(S0), f(ck), f(do), f(dST),
                            out["dq"], out["dk"], out["dv"], out["dg"], out["dbeta"], out["dS0"], ws, nbytes)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def oracle_bwd_units(c, d, S0, ck, do, dST, units):
    """The chunked oracle's backward of each (b, h) unit, teacher forced with the GPU's
    checkpoints (the states entering every chunk)."""
    out = {}
    for b, h in units:
        args = [d[n].f64[b:b + 1, :, h:h + 1] for n in ("q", "k", "v", "g", "beta")]
        r = oc.bwd(*args, None if S0 is None else S0[b:b + 1, h:h + 1], do[b:b + 1, :, h:h + 1],
                   None if dST is None else dST[b:b + 1, h:h + 1], qdq_mode=c.qdq, group=c.group,
                   qdq_interval=c.qdq_interval, chunk_states=ck[b:b + 1, h:h + 1].astype(np.float64),
                   **oracle_kw(c))
        out[(b, h)] = r
    return out


GRADS = ("dq", "dk", "dv", "dg", "dbeta")
BCASES = [
    # name, gate, quantizer kw, solve, degree, T, d_v
    ("gdn_plain_exact", "scalar", {}, la.LA_SOLVE_EXACT, 0, 150, 128),
    ("kda_plain_exact", "key", {}, la.LA_SOLVE_EXACT, 0, 150, 128),
    ("gdn_e4m3_n3", "scalar", dict(qdq=E4M3, group=64, qdq_interval=64), la.LA_SOLVE_NEUMANN, 3, 150, 128),
    ("kda_e4m3_n7", "key", dict(qdq=E4M3, group=64, qdq_interval=64), la.LA_SOLVE_NEUMANN, 7, 150, 128),
    ("gdn_int8g32_n31_dv192", "scalar", dict(qdq=INT8, group=32, qdq_interval=128), la.LA_SOLVE_NEUMANN, 31, 200, 192),
    ("kda_e4m3_n15_dv64", "key", dict(qdq=E4M3, group=64, qdq_interval=64), la.LA_SOLVE_NEUMANN, 15, 130, 64),
    ("kda_int8g16_exact", "key", dict(qdq=INT8, group=16, qdq_interval=64), la.LA_SOLVE_EXACT, 0, 100, 128),
]


@pytest.mark.parametrize("name,gate,qkw,solve,degree,T,dv", BCASES, ids=[b[0] for b in BCASES])
def test_chunk_backward_against_oracle(name, gate, qkw, solve, degree, T, dv):
    B, H = 2, 2
    w = synth.Workload(name, B=B, T=T, H=H, d_k=128, d_v=dv, gate=gate, config_id=400 + degree + T)
    d = synth.generate(w, with_do=True)
    rng = np.random.default_rng(400 + T)
    S0 = (rng.standard_normal((B, H, 128, dv)) * 0.3).astype(np.float32)
    dST = rng.standard_normal((B, H, 128, dv)).astype(np.float32)
    c = chunk_cfg(w, d, solve, degree, **qkw)
    o, ST, ck = run_chunk(c, d, S0, ckpt_interval=64)
    do = d["do"].f32
    r = run_chunk_bwd(c, d, S0, ck, do, dST)
    ref = oracle_bwd_units(c, d, S0, ck, do.astype(np.float64), dST.astype(np.float64),
                           [(b, h) for b in range(B) for h in range(H)])
    errs = {}
    for n in GRADS + ("dS0",):
        got = np.stack([r[n][b, :, h] if n != "dS0" else r[n][b, h] for (b, h) in ref])
        want = np.stack([ref[(b, h)][n][0, :, 0] if n != "dS0" else ref[(b, h)][n][0, 0] for (b, h) in ref])
        errs[n] = gu.err(got, want)
    assert max(errs.values()) <= gu.TOL_F32, errs
    # the backward without checkpoints recomputes the same ones: bit-identical gradients
    r2 = run_chunk_bwd(c, d, S0, None, do, dST)
    for n in r:
        np.testing.assert_array_equal(r[n], r2[n], err_msg=n)


@pytest.mark.parametrize("T", [1, 64, 65])
def test_chunk_backward_edge_lengths(T):
    w = synth.Workload("chunk_bwd_edge", B=1, T=T, H=2, d_k=128, d_v=128, gate="key", config_id=450 + T)
    d = synth.generate(w, with_do=True)
    c = chunk_cfg(w, d, la.LA_SOLVE_NEUMANN, 3, qdq=E4M3, group=64, qdq_interval=64)
    o, ST, ck = run_chunk(c, d, None, ckpt_interval=64)
    do = d["do"].f32
    r = run_chunk_bwd(c, d, None, ck, do, None)
    ref = oracle_bwd_units(c, d, None, ck, do.astype(np.float64), None, [(0, 0), (0, 1)])
    for (b, h), rr in ref.items():
        for n in GRADS:
            assert gu.err(r[n][b, :, h], rr[n][0, :, 0]) <= gu.TOL_F32, (n, T)
        assert gu.err(r["dS0"][b, h], rr["dS0"][0, 0]) <= gu.TOL_F32


@pytest.mark.parametrize("gate,degree", [("scalar", 7), ("key", 31)])
def test_chunk_backward_long_sequence_sampled(gate, degree):
    """B=8 H=16 T=4096 with E4M3 tiles every 64 tokens: sampled units against the oracle."""
    w = synth.Workload("chunk_long", B=8, T=4096, H=16, d_k=128, d_v=128, gate=gate, gate_dtype="f32", config_id=2)
    d = synth.generate(w, with_do=True)
    c = chunk_cfg(w, d, la.LA_SOLVE_NEUMANN, degree, qdq=E4M3, group=64, qdq_interval=64)
    o, ST, ck = run_chunk(c, d, None, ckpt_interval=64)
    do = d["do"].f32
    r = run_chunk_bwd(c, d, None, ck, do, None)
    units = [(0, 0), (5, 11)]
    ref = oracle_bwd_units(c, d, None, ck, do.astype(np.float64), None, units)
    for (b, h), rr in ref.items():
        for n in GRADS:
            assert gu.err(r[n][b, :, h], rr[n][0, :, 0]) <= gu.TOL_F32, n
    for n in r:
        assert np.all(np.isfinite(r[n])), n


def test_chunk_kda_steep_gates():
    """Steep decay: every gate about -3.5 (a token keeps e^-3.5 of the state, the workloads'
    gates about e^-0.8), so a 16-token block spans about 56 of log decay and the diagonal
    blocks' factors reach about e^28 on either side of the block's eighth token; the kernels
    keep the factored products.  Forward and backward against the chunked oracle at the fp32
    bar.  Steeper uniform decay runs into the float cumulative log decays: late in a chunk they
    are large numbers, and the decay of two nearby tokens keeps an absolute error of about
    |G| 2^-24 per step in its exponent; the gate gradient, a suffix sum of largely cancelling
    terms, shows it first (7.5e-6 of its largest magnitude at -4.5 per token, 3.9e-5 at -6)."""
    T, B, H = 150, 1, 2
    w = synth.Workload("chunk_steep", B=B, T=T, H=H, d_k=128, d_v=128, gate="key", gate_dtype="f32", config_id=472)
    d = synth.generate(w, with_do=True)
    rng = np.random.default_rng(473)
    g = -3.5 + 0.2 * rng.standard_normal((B, T, H, 128))
    d["g"] = synth.cast(g, "f32")
    S0 = (rng.standard_normal((B, H, 128, 128)) * 0.3).astype(np.float32)
    c = chunk_cfg(w, d, la.LA_SOLVE_EXACT, 0, qdq=E4M3, group=64, qdq_interval=64)
    c.gate_dtype = la.LA_F32
    o, ST, ck = run_chunk(c, d, S0, ckpt_interval=64)
    tally = gu.CodeTally()
    wo, ws = teacher_forced_chunks(c, d, ck, ST, o, tally)
    assert wo <= gu.TOL_F32 and ws <= gu.TOL_F32, (wo, ws)
    tally.check()
    do = d["do"].f32
    r = run_chunk_bwd(c, d, S0, ck, do, None)
    ref = oracle_bwd_units(c, d, S0, ck, do.astype(np.float64), None, [(0, 0), (0, 1)])
    for (b, h), rr in ref.items():
        for n in GRADS:
            assert np.all(np.isfinite(r[n][b, :, h])), n
            assert gu.err(r[n][b, :, h], rr[n][0, :, 0]) <= gu.TOL_F32, n
        assert gu.err(r["dS0"][b, h], rr["dS0"][0, 0]) <= gu.TOL_F32


@pytest.mark.parametrize("first_gate", [-20.0, -85.0], ids=["factored", "per_key_fallback"])
def test_chunk_kda_positive_gates(first_gate):
    """Gates above zero make the factored decays exceed one: with a cumulative range under 80 per
    chunk the kernels keep the factored products, above it (first_gate = -85, then small
    positive gates) they take the per-key sums for every block.  Forward and backward against
    the chunked oracle.  The gates alternate +0.5 and -1.0 (factors above one inside a block,
    a net decay like the workloads'), so the 1e-5 bar (fp32 against float64, relative to the
    largest magnitude) applies as for the other cases; with gates near zero over a whole
    chunk (no decay at all) A's entries grow and the solve's backward loses about one more
    bit."""
    T, B, H = 130, 1, 2
    w = synth.Workload("chunk_posgate", B=B, T=T, H=H, d_k=128, d_v=128, gate="key", gate_dtype="f32", config_id=470)
    d = synth.generate(w, with_do=True)
    rng = np.random.default_rng(471)
    alt = np.where(np.arange(T) % 2 == 0, 0.5, -1.0)[None, :, None, None]
    g = alt + 0.05 * rng.standard_normal((B, T, H, 128))
    g[:, ::64] = first_gate
    d["g"] = synth.cast(g, "f32")
    S0 = (rng.standard_normal((B, H, 128, 128)) * 0.3).astype(np.float32)
    c = chunk_cfg(w, d, la.LA_SOLVE_NEUMANN, 7, qdq=E4M3, group=64, qdq_interval=64)
    c.gate_dtype = la.LA_F32
    o, ST, ck = run_chunk(c, d, S0, ckpt_interval=64)
    tally = gu.CodeTally()
    wo, ws = teacher_forced_chunks(c, d, ck, ST, o, tally)
    assert wo <= gu.TOL_F32 and ws <= gu.TOL_F32, (wo, ws)
    tally.check()
    do = d["do"].f32
    r = run_chunk_bwd(c, d, S0, ck, do, None)
    ref = oracle_bwd_units(c, d, S0, ck, do.astype(np.float64), None, [(0, 0), (0, 1)])
    for (b, h), rr in ref.items():
        for n in GRADS:
            assert gu.err(r[n][b, :, h], rr[n][0, :, 0]) <= gu.TOL_F32, n
        assert gu.err(r["dS0"][b, h], rr["dS0"][0, 0]) <= gu.TOL_F32
