"""The allocation-free backward entry point (la_recurrent_bwd_ste_noalloc) against
la_recurrent_bwd_ste with a caller-allocated workspace: the same kernels on the same inputs,
so every gradient must agree bit for bit.  Two calls in a row on one GPU share the library's
device array, the second with a smaller problem than the first, for the per-token and the
block backward."""
import numpy as np
import pytest

import quantized_state_qat_amd as la
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

GRADS = ["dq", "dk", "dv", "dg", "dbeta", "dS0"]


def run_noalloc(c, d, dout, S0=None, dST=None, ckpts=None):
    torch = gu.torch_mod()
    di = {k: gu.dev(d[k]) for k in ("q", "k", "v", "g", "beta")}
    f = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    gshape = (c.B, c.T, c.H, c.d_k) if c.gate == la.LA_GATE_KEY else (c.B, c.T, c.H)
    out = {
        "dq": gu.nan_like(torch, (c.B, c.T, c.H, c.d_k)), "dk": gu.nan_like(torch, (c.B, c.T, c.H, c.d_k)),
        "dv": gu.nan_like(torch, (c.B, c.T, c.H, c.d_v)), "dg": gu.nan_like(torch, gshape),
        "dbeta": gu.nan_like(torch, (c.B, c.T, c.H)), "dS0": gu.nan_like(torch, (c.B, c.H, c.d_k, c.d_v)),
    }
    la.la_recurrent_bwd_ste_noalloc(c, di["q"], di["k"], di["v"], di["g"], di["beta"], f(S0), f(ckpts), f(dout),
                                    f(dST), out["dq"], out["dk"], out["dv"], out["dg"], out["dbeta"], out["dS0"])
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def case(w, mode, group, had, interval, ckpt):
    d = synth.generate(w, with_do=True, with_dST=True)
    c = gu.cfg_for(w, d, qdq=mode, group=group, hadamard=had, qdq_interval=interval, ckpt_interval=ckpt)
    S0 = d["S0"].f32 if w.s0_sigma > 0 else None
    return c, d, S0


PAIRS = [
    # (larger, smaller) per pair; both calls go through the same device array
    ("token", (synth.Workload("na1", B=2, T=130, H=2, d_k=128, d_v=128, s0_sigma=0.1, config_id=80),
               la.LA_QDQ_INT8_GROUP, 32, 1, 1, 64),
     (synth.Workload("na2", B=1, T=37, H=1, d_k=64, d_v=64, s0_sigma=0.2, config_id=81),
      la.LA_QDQ_INT8_GROUP, 16, 0, 1, 16)),
    ("block", (synth.Workload("na3", B=2, T=150, H=2, d_k=128, d_v=128, gate_dtype="f32", s0_sigma=0.1,
                              config_id=82), la.LA_QDQ_E4M3_TILE, 64, 0, 64, 64),
     (synth.Workload("na4", B=1, T=40, H=1, d_k=128, d_v=64, s0_sigma=0.2, config_id=83),
      la.LA_QDQ_INT8_GROUP, 32, 0, 16, 16)),
    ("kda", (synth.Workload("na5", B=1, T=100, H=2, d_k=128, d_v=128, gate="key", s0_sigma=0.1, config_id=84),
             la.LA_QDQ_INT8_GROUP, 64, 0, 1, 32),
     (synth.Workload("na6", B=1, T=9, H=1, d_k=32, d_v=64, gate="key", s0_sigma=0.2, config_id=85),
      la.LA_QDQ_E4M3_TILE, 64, 0, 3, 6)),
]


@pytest.mark.parametrize("name,big,small", PAIRS, ids=[p[0] for p in PAIRS])
def test_noalloc_matches_workspace_call(name, big, small):
    for spec in (big, small):
        c, d, S0 = case(*spec)
        assert la.la_bwd_workspace_bytes(c) <= la.la_noalloc_workspace_limit()
        ref = gu.run_bwd(c, d, d["do"].f32, S0=S0, dST=d["dST"].f32)
        got = run_noalloc(c, d, d["do"].f32, S0=S0, dST=d["dST"].f32)
        for n in GRADS:
            assert np.all(np.isfinite(got[n])), (name, n)
            np.testing.assert_array_equal(got[n], ref[n])
        if name == "block":
            assert la.la_bwd_kernel_name(c) == "block" or spec is small
        # with the forward's checkpoints
        _, _, ck = gu.run_fwd(c, d, S0=S0, ckpt_interval=c.ckpt_interval)
        got2 = run_noalloc(c, d, d["do"].f32, S0=S0, dST=d["dST"].f32, ckpts=ck)
        for n in GRADS:
            np.testing.assert_array_equal(got2[n], ref[n])


def test_noalloc_rejects_a_workspace_beyond_its_array():
    """A problem whose workspace exceeds the device array is rejected on the host, before any
    HIP call (the pointers below are never dereferenced)."""
    c = la.Config(B=8, T=4096, H=16, d_k=128, d_v=128, qdq=la.LA_QDQ_E4M3_TILE, group=64, qdq_interval=64,
                  ckpt_interval=64, gate_dtype=la.LA_F32)
    assert la.la_bwd_workspace_bytes(c) > la.la_noalloc_workspace_limit()
    fake = 0x10000
    with pytest.raises(la.LaError) as ei:
        la.la_recurrent_bwd_ste_noalloc(c, fake, fake, fake, fake, fake, None, None, fake, None, fake, fake, fake,
                                        fake, fake, fake, stream=0)
    assert ei.value.status == la.LA_ERR_WORKSPACE
    assert "allocation-free" in la.la_last_error()
