"""Benchmark: token-head state updates per second of the batched decode step.

Workload (one step): GDN single-token decode over B=256 sequences x H=16 heads, d_k = d_v =
128, bf16 q/k/v/g/beta, FP32 state (268 MB) read, updated, INT8 group-32 fake-quantized and
written back in place.  Inputs are resident in HBM before the timed region; three state
buffers (805 MB, above the 256 MB Infinity Cache) are rotated so each step streams its state
from HBM.  Prints one JSON line with the throughput, the decode kernel's roofline figures
(HBM-bound; algorithmic bytes per launch / mean launch time) and the CPU oracle's rate on the
host cores for the same step.

The default warm-up is long on purpose: back-to-back decode steps on a fresh process run about
5% slower for the first hundred or so launches (measured in kernel traces: about 95 us per
step, settling at 91 us after 100-150 launches), so the timed steps follow 150 untimed ones.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extra]
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP32_VALU_PEAK_TFLOPS = 157.3  # MI355X FP32 (vector, packed; equal to the FP32 matrix peak)
BF16_MFMA_PEAK_TFLOPS = 2500.0 # MI355X dense bf16 matrix peak
METRIC = "token·head state updates/s + % of HBM/VALU roofline, GDN/KDA d=128 QDQ"


def decode_algorithmic_bytes(B, H, dk, dv, in_bytes=2, out_bytes=4):
    """State read + write, q/k/v, g/beta, o: what one decode launch must move."""
    state = 2 * 4 * B * H * dk * dv
    qkv = B * H * (2 * dk + dv) * in_bytes
    gb = 2 * B * H * in_bytes
    o = B * H * dv * out_bytes
    return state + qkv + gb + o


def kernel_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "quantized_state_qat_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def pmc_traffic(summary_name, khash):
    """HBM bytes per launch from a committed rocprofv3 PMC summary, if it was taken on the
    current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", summary_name)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("kernel_source_hash") != khash:
        return None
    return rec.get("hbm_bytes_per_launch")


def decode_setup():
    """Inputs of the decode workload on the GPU (three state buffers in rotation, 805 MB, so that
    every launch streams its state from HBM rather than from the 256 MB Infinity Cache)."""
    import numpy as np
    import torch

    import quantized_state_qat_amd as la
    import synth

    w = synth.WORKLOADS[1]
    d = synth.generate(w)
    dev = {k: torch.from_numpy(d[k].bits.astype(np.int16)).view(torch.bfloat16).cuda()
           for k in ("q", "k", "v", "g", "beta")}
    S0 = torch.from_numpy(d["S0"].f32).cuda()
    states = [S0.clone() for _ in range(3)]
    o = torch.empty((w.B, 1, w.H, w.d_v), device="cuda")
    c = la.Config(B=w.B, T=1, H=w.H, d_k=w.d_k, d_v=w.d_v, qdq=la.LA_QDQ_INT8_GROUP, group=32)
    torch.cuda.synchronize()
    return {"w": w, "d": d, "dev": dev, "states": states, "o": o, "c": c}


def bench_decode(steps, warmup, setup=None):
    import torch

    import quantized_state_qat_amd as la

    st = setup if setup is not None else decode_setup()
    w, dev, states, o, c = st["w"], st["dev"], st["states"], st["o"], st["c"]
    stream = torch.cuda.current_stream()

    def step(i):
        la.la_decode_step(c, dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], states[i % 3], o,
                          stream=stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total = e0.elapsed_time(e1) * 1e-3
    mean_launch = total / steps  # back-to-back launches on one stream
    nbytes = decode_algorithmic_bytes(w.B, w.H, w.d_k, w.d_v)
    return {
        "w": w, "d": st["d"], "total_s": total, "wall_s": wall, "mean_launch_s": mean_launch,
        "updates": w.B * w.H * steps, "bytes_per_launch": nbytes,
    }


def bench_long_e4m3(steps=3, warmup=1):
    """GDN B=8 H=16 T=4096 d=128, E4M3 tile QDQ every 64 tokens: the forward alone, then the
    training pair (forward with 64-token checkpoints, straight-through backward)."""
    import numpy as np
    import torch

    import quantized_state_qat_amd as la
    import synth

    w = synth.WORKLOADS[2]
    d = synth.generate(w, with_do=True)
    dev = {}
    for k in ("q", "k", "v"):
        dev[k] = torch.from_numpy(d[k].bits.astype(np.int16)).view(torch.bfloat16).cuda()
    for k in ("g", "beta", "do"):
        dev[k] = torch.from_numpy(d[k].f32).cuda()
    del d
    o = torch.empty((w.B, w.T, w.H, w.d_v), device="cuda")
    ST = torch.empty((w.B, w.H, w.d_k, w.d_v), device="cuda")
    c = la.Config(B=w.B, T=w.T, H=w.H, d_k=w.d_k, d_v=w.d_v, qdq=la.LA_QDQ_E4M3_TILE, group=64,
                  qdq_interval=64, gate_dtype=la.LA_F32)
    stream = torch.cuda.current_stream()
    t = _time_calls(lambda: la.la_recurrent_fwd(c, dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], None, o,
                                                ST, stream=stream), steps, warmup, stream)
    unit = w.d_k * w.d_v * w.B * w.H * w.T
    workload = "gdn_long_e4m3_64 B=8 H=16 T=4096 d_k=d_v=128 bf16 q/k/v, fp32 g/beta/state, E4M3 tile QDQ every 64 tokens"
    # matrix-core work the block kernel issues per (workgroup, 16-token block): each of the four
    # column waves 24 bf16 16x16x32 (projections of the split state), 24 bf16 16x16x16 (the
    # rank-16 update of the split deltas) and 8 fp32 16x16x4 (deltas and outputs); the producer
    # 8 bf16 16x16x32 (Gram matrices) and 4 fp32 16x16x4 (the solve)
    mfma_per_wg_block = 4 * (24 * 2 * 16 * 16 * 32 + 24 * 2 * 16 * 16 * 16 + 8 * 2 * 16 * 16 * 4) \
        + 8 * 2 * 16 * 16 * 32 + 4 * 2 * 16 * 16 * 4
    mfma_flops = mfma_per_wg_block * w.B * w.H * (w.d_v // 64) * (w.T // 16)
    fwd = {
        "workload": workload,
        "kernel": la.la_fwd_kernel_name(c), "ms_per_call": t * 1e3, "updates_per_s": w.B * w.H * w.T / t,
        "roofline": _fp32_roofline(7.0 * unit, t, "the chunked (16-token block) form on the matrix cores: algorithmic "
                                                  "fp32 work of the recurrence (7 d_k d_v per token-head) against the "
                                                  "FP32 peak, formed from exact bf16 products with fp32 sums"),
        "mfma_pipe": {"issued_flops_per_call": mfma_flops, "achieved": mfma_flops / t / 1e12, "unit": "TFLOP/s",
                      "peak_bf16_dense": BF16_MFMA_PEAK_TFLOPS, "frac": mfma_flops / t / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                      "note": "matrix-core work actually issued (exact three-part bf16 splits of fp32 operands), "
                              "against the dense bf16 peak"},
    }
    # the same workload on the VALU-only recurrence (single-wave kernel: no matrix cores)
    cv = la.Config(**{**c.__dict__, "kernel": la.LA_KERNEL_WAVE})
    t_v = _time_calls(lambda: la.la_recurrent_fwd(cv, dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], None, o,
                                                  ST, stream=stream), steps, warmup, stream)
    valu = {
        "workload": workload,
        "kernel": la.la_fwd_kernel_name(cv), "ms_per_call": t_v * 1e3, "updates_per_s": w.B * w.H * w.T / t_v,
        "roofline": _fp32_roofline(7.0 * unit, t_v, "VALU recurrence, one token at a time: 7 d_k d_v flops per "
                                                    "token-head against the FP32 vector peak (which needs packed "
                                                    "FP32 FMAs; this build issues unpacked FP32, whose peak is half)"),
        "frac_of_unpacked_valu_peak": 7.0 * unit / t_v / 1e12 / (FP32_VALU_PEAK_TFLOPS / 2),
        "issue_floor": _issue_roofline(3.0 + 8.0 / 64, unit, t_v, "two FMA passes (projections) and one FMA update per "
                                                               "element and token, the E4M3 codec (8) every 64 tokens"),
    }

    c.ckpt_interval = 64
    ck = torch.empty((w.B, w.H, w.T // 64, w.d_k, w.d_v), device="cuda")
    grads = [torch.empty((w.B, w.T, w.H, n), device="cuda") for n in (w.d_k, w.d_k, w.d_v)]
    dg = torch.empty((w.B, w.T, w.H), device="cuda")
    dbeta = torch.empty((w.B, w.T, w.H), device="cuda")
    dS0 = torch.empty((w.B, w.H, w.d_k, w.d_v), device="cuda")
    nbytes = la.la_bwd_workspace_bytes(c)
    ws = torch.empty((nbytes + 255) // 4, dtype=torch.float32, device="cuda")
    t_f = _time_calls(lambda: la.la_recurrent_fwd(c, dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], None, o,
                                                  ST, ck, stream=stream), steps, warmup, stream)
    t_b = _time_calls(lambda: la.la_recurrent_bwd_ste(c, dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], None, ck,
                                                      dev["do"], None, grads[0], grads[1], grads[2], dg, dbeta, dS0,
                                                      ws, nbytes, stream=stream), steps, warmup, stream)
    fwdbwd = {
        "workload": "gdn_long_e4m3_64 training pair: forward with 64-token checkpoints, then the straight-through "
                    "backward (same inputs, fp32 upstream gradient of o)",
        "kernel_fwd": la.la_fwd_kernel_name(c), "kernel_bwd": la.la_bwd_kernel_name(c),
        "ms_fwd": t_f * 1e3, "ms_bwd": t_b * 1e3, "workspace_bytes": nbytes,
        "updates_per_s": w.B * w.H * w.T / (t_f + t_b),
        "roofline_bwd": _fp32_roofline(22.0 * unit, t_b, "backward only: recompute 7 + adjoint 15 d_k d_v flops per "
                                                         "token-head (the block path also recomputes every block's "
                                                         "entering state with the block forward, not counted)"),
    }
    return fwd, fwdbwd, valu


def bench_kda_long(steps=3, warmup=1):
    """KDA B=8 H=16 T=4096 d=128, bf16 q/k/v, fp32 per-key gates and beta, E4M3 tile QDQ every
    64 tokens: the forward (block kernel) and the straight-through backward from its checkpoints
    (the chunk kernel: every rounding point is a checkpoint), with the per-token backward on the
    same checkpoints beside it."""
    import torch

    import quantized_state_qat_amd as la
    import synth

    w = synth.Workload("kda_long_e4m3_64", B=8, T=4096, H=16, d_k=128, d_v=128, gate="key", gate_dtype="f32",
                       config_id=2)
    d = synth.generate(w, with_do=True)
    dev = {k: _dev(d[k]) for k in ("q", "k", "v", "g", "beta", "do")}
    del d
    c = la.Config(B=w.B, T=w.T, H=w.H, d_k=w.d_k, d_v=w.d_v, gate=la.LA_GATE_KEY, qdq=la.LA_QDQ_E4M3_TILE, group=64,
                  qdq_interval=64, ckpt_interval=64, gate_dtype=la.LA_F32)
    o = torch.empty((w.B, w.T, w.H, w.d_v), device="cuda")
    ST = torch.empty((w.B, w.H, w.d_k, w.d_v), device="cuda")
    ck = torch.empty((w.B, w.H, w.T // 64, w.d_k, w.d_v), device="cuda")
    grads = [torch.empty((w.B, w.T, w.H, w.d_k), device="cuda") for _ in range(4)]
    dv = torch.empty((w.B, w.T, w.H, w.d_v), device="cuda")
    dbeta = torch.empty((w.B, w.T, w.H), device="cuda")
    dS0 = torch.empty((w.B, w.H, w.d_k, w.d_v), device="cuda")
    nbytes = la.la_bwd_workspace_bytes(c)
    ws = torch.empty((nbytes + 255) // 4, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    t_f = _time_calls(lambda: la.la_recurrent_fwd(c, dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], None, o, ST,
                                                  ck, stream=stream), steps, warmup, stream)
    t_b = _time_calls(lambda: la.la_recurrent_bwd_ste(c, dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], None, ck,
                                                      dev["do"], None, grads[0], grads[1], dv, grads[2], dbeta, dS0,
                                                      ws, nbytes, stream=stream), steps, warmup, stream)
    ct = dataclasses.replace(c, kernel=la.LA_KERNEL_TOKEN)
    nbt = la.la_bwd_workspace_bytes(ct)
    wst = torch.empty((nbt + 255) // 4, dtype=torch.float32, device="cuda") if nbt > nbytes else ws
    t_bt = _time_calls(lambda: la.la_recurrent_bwd_ste(ct, dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], None,
                                                       ck, dev["do"], None, grads[0], grads[1], dv, grads[2], dbeta,
                                                       dS0, wst, nbt, stream=stream), steps, warmup, stream)
    unit = w.d_k * w.d_v * w.B * w.H * w.T
    return {
        "workload": "kda_long_e4m3_64 B=8 H=16 T=4096 d_k=d_v=128 bf16 q/k/v, fp32 per-key gates and beta, E4M3 tile "
                    "QDQ every 64 tokens, 64-token checkpoints",
        "kernel_fwd": la.la_fwd_kernel_name(c), "kernel_bwd": la.la_bwd_kernel_name(c),
        "ms_fwd": t_f * 1e3, "ms_bwd": t_b * 1e3, "ms_bwd_token_kernel": t_bt * 1e3,
        "workspace_bytes_bwd": nbytes, "updates_per_s_fwd": w.B * w.H * w.T / t_f,
        "roofline_fwd": _fp32_roofline(7.0 * unit, t_f, "forward: 7 d_k d_v flops per token-head (the per-key decay "
                                                        "adds d_k d_v multiplies, not counted)"),
        "roofline_bwd": _fp32_roofline(22.0 * unit, t_b, "backward: recompute 7 + adjoint 15 d_k d_v per token-head"),
    }


def bench_chunk(steps=3, warmup=1):
    """The 64-token chunk form on the long-sequence shape (B=8 H=16 T=4096 d=128, bf16 q/k/v, fp32
    gates and beta, E4M3 tile QDQ every 64 tokens, a checkpoint per chunk): forward and
    straight-through backward with the exact solve and with Neumann polynomials, GDN and KDA."""
    import torch

    import quantized_state_qat_amd as la
    import synth

    out = {"workload": "B=8 H=16 T=4096 d_k=d_v=128 bf16 q/k/v, fp32 gates and beta, E4M3 tile QDQ every 64 tokens, "
                       "64-token chunks and checkpoints",
           "flops_note": "fp32 matrix work counted per chunk and head: state pass 2 (2*64*128 + 2*64*64 + 128*64) per "
                         "value column; prep 2*2*(64*65/2)*128 for A and M, 2*64^3/3 for the exact solve or "
                         "2*(2 log2(d+1) - 2)*64^3 for the Neumann product"}
    for gate in ("scalar", "key"):
        w = synth.Workload("chunk_long", B=8, T=4096, H=16, d_k=128, d_v=128, gate=gate, gate_dtype="f32", config_id=2)
        d = synth.generate(w, with_do=True)
        dev = {k: _dev(d[k]) for k in ("q", "k", "v", "g", "beta", "do")}
        del d
        o = torch.empty((w.B, w.T, w.H, w.d_v), device="cuda")
        ST = torch.empty((w.B, w.H, w.d_k, w.d_v), device="cuda")
        ck = torch.empty((w.B, w.H, w.T // 64, w.d_k, w.d_v), device="cuda")
        gshape = (w.B, w.T, w.H, w.d_k) if gate == "key" else (w.B, w.T, w.H)
        dq, dk = (torch.empty((w.B, w.T, w.H, w.d_k), device="cuda") for _ in range(2))
        dv = torch.empty((w.B, w.T, w.H, w.d_v), device="cuda")
        dg = torch.empty(gshape, device="cuda")
        dbeta = torch.empty((w.B, w.T, w.H), device="cuda")
        dS0 = torch.empty((w.B, w.H, w.d_k, w.d_v), device="cuda")
        stream = torch.cuda.current_stream()
        for solve, degree in ((la.LA_SOLVE_EXACT, 0), (la.LA_SOLVE_NEUMANN, 3), (la.LA_SOLVE_NEUMANN, 31)):
            if gate == "key" and degree == 31:
                continue
            c = la.Config(B=w.B, T=w.T, H=w.H, d_k=w.d_k, d_v=w.d_v,
                          gate=la.LA_GATE_KEY if gate == "key" else la.LA_GATE_SCALAR, qdq=la.LA_QDQ_E4M3_TILE,
                          group=64, qdq_interval=64, ckpt_interval=64, gate_dtype=la.LA_F32,
                          kernel=la.LA_KERNEL_CHUNK, solve=solve, degree=degree)
            nf = la.la_chunk_workspace_bytes(c)
            nb = la.la_bwd_workspace_bytes(c)
            ws = torch.empty((max(nf, nb) + 255) // 4, dtype=torch.float32, device="cuda")
            t_f = _time_calls(lambda: la.la_recurrent_fwd_chunk(c, dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"],
                                                                None, o, ST, ck, ws, nf, stream=stream),
                              steps, warmup, stream)
            t_b = _time_calls(lambda: la.la_recurrent_bwd_ste(c, dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"],
                                                              None, ck, dev["do"], None, dq, dk, dv, dg, dbeta, dS0,
                                                              ws, nb, stream=stream), steps, warmup, stream)
            nch = w.T // 64
            m = (degree + 1).bit_length() - 1
            solve_fl = 2 * 64 ** 3 / 3 if degree == 0 else 2 * (2 * m - 2) * 64 ** 3
            per_chunk = 2 * (2 * 64 * 128 + 2 * 64 * 64 + 128 * 64) * w.d_v + 2 * 2 * (64 * 65 / 2) * 128 + solve_fl
            fl = per_chunk * nch * w.B * w.H
            key = f"{'kda' if gate == 'key' else 'gdn'}_{'exact' if degree == 0 else 'neumann%d' % degree}"
            out[key] = {"ms_fwd": t_f * 1e3, "ms_bwd": t_b * 1e3, "updates_per_s_fwd": w.B * w.H * w.T / t_f,
                        "workspace_bytes_fwd": nf, "workspace_bytes_bwd": nb,
                        "roofline_fwd": {"bound": "mfma", "achieved": fl / t_f / 1e12, "peak": FP32_VALU_PEAK_TFLOPS,
                                         "unit": "TFLOP/s", "frac": fl / t_f / 1e12 / FP32_VALU_PEAK_TFLOPS,
                                         "flops_per_call": fl, "note": "fp32 matrix cores (16x16x4 f32), dense peak"}}
            del ws
            torch.cuda.empty_cache()
        del dev
    return out


def _dev(t):
    """Device copy of a generated tensor in its storage dtype."""
    import numpy as np
    import torch
    if t.dtype == "bf16":
        return torch.from_numpy(t.bits.astype(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(t.f32)).cuda()


def _fp32_roofline(flops, t, what):
    return {"bound": "fp32", "achieved": flops / t / 1e12, "peak": FP32_VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": flops / t / 1e12 / FP32_VALU_PEAK_TFLOPS, "flops_per_call": flops, "note": what}


# VALU issue rate of the chip: one wave64 instruction per CU per cycle (four 16-lane SIMDs, four
# cycles per wave instruction), i.e. 64 element operations per CU per cycle.
VALU_ELEM_OPS_PEAK = 64 * 256 * 2.4e9


def _issue_roofline(ops_per_elem, elems, t, what):
    """Algorithmic VALU issue floor: ops_per_elem element operations per state element and token
    (the recurrence's decay, projections and update, plus the codec and the rotations where they
    run) over `elems` state-element-tokens, against the chip's VALU issue rate."""
    ops = ops_per_elem * elems
    return {"bound": "alu", "achieved": ops / t / 1e12, "peak": VALU_ELEM_OPS_PEAK / 1e12,
            "unit": "T element-ops/s", "frac": ops / t / VALU_ELEM_OPS_PEAK, "ops_per_element_token": ops_per_elem,
            "note": what}


def _time_calls(fn, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    times = []
    for _ in range(steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) * 1e-3)
    return sum(times) / len(times)


def bench_kda_tok(steps=3, warmup=1):
    """KDA B=4 H=32 T=2048 d=128, bf16 inputs, INT8 group-64 QDQ after every token."""
    import torch

    import quantized_state_qat_amd as la
    import synth

    w = synth.WORKLOADS[3]
    d = synth.generate(w)
    dev = {k: _dev(d[k]) for k in ("q", "k", "v", "g", "beta")}
    del d
    o = torch.empty((w.B, w.T, w.H, w.d_v), device="cuda")
    ST = torch.empty((w.B, w.H, w.d_k, w.d_v), device="cuda")
    c = la.Config(B=w.B, T=w.T, H=w.H, d_k=w.d_k, d_v=w.d_v, gate=la.LA_GATE_KEY, qdq=la.LA_QDQ_INT8_GROUP,
                  group=64, qdq_interval=1)
    stream = torch.cuda.current_stream()
    t = _time_calls(lambda: la.la_recurrent_fwd(c, dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], None, o,
                                                ST, stream=stream), steps, warmup, stream)
    # the training pair of the same workload: forward with 64-token checkpoints, then the
    # straight-through backward from them (upstream gradient ~ N(0, 1))
    c.ckpt_interval = 64
    ck = torch.empty((w.B, w.H, (w.T + 63) // 64, w.d_k, w.d_v), device="cuda")
    dout = torch.randn((w.B, w.T, w.H, w.d_v), device="cuda", generator=torch.Generator("cuda").manual_seed(3))
    grads = [torch.empty((w.B, w.T, w.H, w.d_k), device="cuda") for _ in range(3)]
    dv = torch.empty((w.B, w.T, w.H, w.d_v), device="cuda")
    dbeta = torch.empty((w.B, w.T, w.H), device="cuda")
    dS0 = torch.empty((w.B, w.H, w.d_k, w.d_v), device="cuda")
    nbytes = la.la_bwd_workspace_bytes(c)
    ws = torch.empty((nbytes + 255) // 4, dtype=torch.float32, device="cuda")
    t_f = _time_calls(lambda: la.la_recurrent_fwd(c, dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], None, o,
                                                  ST, ck, stream=stream), steps, warmup, stream)
    t_b = _time_calls(lambda: la.la_recurrent_bwd_ste(c, dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], None, ck,
                                                      dout, None, grads[0], grads[1], dv, grads[2], dbeta, dS0, ws,
                                                      nbytes, stream=stream), steps, warmup, stream)
    kernel_bwd = la.la_bwd_kernel_name(c)
    del ws, grads, dv, dout, ck
    c.ckpt_interval = 0
    c.hadamard = 1
    t_h = _time_calls(lambda: la.la_recurrent_fwd(c, dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], None, o,
                                                  ST, stream=stream), steps, warmup, stream)
    flops = 7.0 * w.d_k * w.d_v * w.B * w.H * w.T
    return {
        "workload": "kda_int8g64_tok B=4 H=32 T=2048 d_k=d_v=128 bf16 inputs, KDA gate, INT8 group-64 QDQ every token",
        "kernel": la.la_fwd_kernel_name(c), "ms_per_call": t * 1e3, "updates_per_s": w.B * w.H * w.T / t,
        "roofline": _fp32_roofline(flops, t, "algorithmic fp32 work of the recurrence (7 d_k d_v per token-head); "
                                             "the INT8 codec is not counted"),
        "issue_floor": _issue_roofline(12.0, w.d_k * w.d_v * w.B * w.H * w.T, t,
                                       "decay, two projections and the update (4) plus the INT8 codec (8) per element "
                                       "and token"),
        "training_pair": {
            "ms_fwd": t_f * 1e3, "ms_bwd": t_b * 1e3, "kernel_bwd": kernel_bwd, "workspace_bytes_bwd": nbytes,
            "issue_floor_bwd": _issue_roofline(23.0, w.d_k * w.d_v * w.B * w.H * w.T, t_b,
                                               "recompute with the codec once (12), decode of the kept codes (2) and "
                                               "adjoint (9) per element and token"),
            "note": "forward with 64-token checkpoints, then the straight-through backward from them",
        },
        "ms_per_call_hadamard": t_h * 1e3,
        "issue_floor_hadamard": _issue_roofline(26.0, w.d_k * w.d_v * w.B * w.H * w.T, t_h,
                                                "as above plus two 7-stage butterfly rotations of the state (14) per "
                                                "element and token"),
        "note_hadamard": "the same call with the key-axis Hadamard rotation around every rounding (per-key gates "
                         "carry the state unrotated: two rotations of the state per token)",
    }


def bench_decode_slots(steps=100, warmup=150):
    """Serving decode over a slot pool: the decode workload's B=256 x H=16 states in a pool of
    3 B + 1 slots (slot 0 reserved), each step naming a shuffled set of B slots, the three
    sets in rotation so that every step streams its states from HBM."""
    import numpy as np
    import torch

    import quantized_state_qat_amd as la
    import synth

    w = synth.WORKLOADS[1]
    d = synth.generate(w)
    dev = {k: torch.from_numpy(d[k].bits.astype(np.int16)).view(torch.bfloat16).cuda()
           for k in ("q", "k", "v", "g", "beta")}
    n_slots = 3 * w.B + 1
    pool = torch.from_numpy(d["S0"].f32).cuda().repeat(3, 1, 1, 1)
    pool = torch.cat([torch.zeros_like(pool[:1]), pool])
    rng = np.random.default_rng(5)
    sets = [torch.from_numpy((1 + i * w.B + rng.permutation(w.B)).astype(np.int32)).cuda() for i in range(3)]
    o = torch.empty((w.B, 1, w.H, w.d_v), device="cuda")
    c = la.Config(B=w.B, T=1, H=w.H, d_k=w.d_k, d_v=w.d_v, qdq=la.LA_QDQ_INT8_GROUP, group=32)
    stream = torch.cuda.current_stream()
    i = [0]

    def step():
        la.la_decode_step_slots(c, dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], pool, sets[i[0] % 3],
                                n_slots, o, stream=stream)
        i[0] += 1
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / steps
    nbytes = decode_algorithmic_bytes(w.B, w.H, w.d_k, w.d_v) + 4 * w.B
    return {
        "workload": "gdn_decode_int8g32 over a slot pool: B=256 entries x H=16, d=128, pool of 769 slots, "
                    "INT8 group-32, three shuffled slot sets in rotation",
        "kernel": "decode (slot pool)", "us_per_step": t * 1e6, "updates_per_s": w.B * w.H / t,
        "roofline": {"bound": "hbm", "achieved": nbytes / t / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": nbytes / t / 1e9 / HBM_PEAK_GBS, "bytes_per_launch": nbytes},
    }


def bench_decode_replay(windows=6, warmup_windows=4, W=16):
    """Serving decode in replay mode: the decode workload's B=256 x H=16 states as checkpoints
    with a log of BF16 entries, windows of 16 tokens (Hadamard + INT8 group-32 refresh at each
    window end, entries appended at the other steps), three (checkpoint, log) sets in rotation
    so that every step streams its checkpoint from HBM.  Reported per step, averaged over whole
    windows."""
    import numpy as np
    import torch

    import quantized_state_qat_amd as la
    import synth

    w = synth.WORKLOADS[1]
    d = synth.generate(w)
    dev = {k: torch.from_numpy(d[k].bits.astype(np.int16)).view(torch.bfloat16).cuda()
           for k in ("q", "k", "v", "g", "beta")}
    B, H, dk, dv = w.B, w.H, w.d_k, w.d_v
    sets = [dict(S=torch.from_numpy(d["S0"].f32).cuda(),
                 lk=torch.zeros((B, H, W - 1, dk), dtype=torch.int16, device="cuda"),
                 ld=torch.zeros((B, H, W - 1, dv), dtype=torch.int16, device="cuda"),
                 lg=torch.zeros((B, H, W - 1), dtype=torch.float32, device="cuda")) for _ in range(3)]
    pos = [torch.full((B,), p, dtype=torch.int32, device="cuda") for p in range(W)]
    o = torch.empty((B, 1, H, dv), device="cuda")
    c = la.Config(B=B, T=1, H=H, d_k=dk, d_v=dv, qdq=la.LA_QDQ_INT8_GROUP, group=32, hadamard=1, qdq_interval=W,
                  replay=1)
    stream = torch.cuda.current_stream()

    def step(i):
        st = sets[i % 3]
        la.la_decode_step_replay(c, dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], st["S"], st["lk"], st["ld"],
                                 st["lg"], pos[(i // 3) % W], o, stream=stream)
    n_warm, n = 3 * W * warmup_windows, 3 * W * windows
    for i in range(n_warm):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / n
    # algorithmic bytes per step, averaged over a window: the checkpoint read, the window's
    # entries read (on average (W - 1) / 2 per step), one entry written or (once per window)
    # the checkpoint written, the token's inputs and output
    entry = (dk + dv) * 2 + 4
    per_head = (4 * dk * dv + (W - 1) / 2 * entry + (W - 1) / W * entry + 4 * dk * dv / W
                + 2 * (2 * dk + dv) + 4 + 4 * dv)
    nbytes = per_head * B * H
    return {
        "workload": f"gdn_decode_int8g32 shape in replay mode: B={B} H={H} d={dk}, windows of {W} tokens, Hadamard "
                    "+ INT8 group-32 refresh at window ends, BF16 entries between, 3 (checkpoint, log) sets in rotation",
        "kernel": "decode (replay)", "us_per_step": t * 1e6, "updates_per_s": B * H / t,
        "roofline": {"bound": "hbm", "achieved": nbytes / t / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": nbytes / t / 1e9 / HBM_PEAK_GBS, "bytes_per_step_avg": nbytes},
    }


def bench_varlen(steps=3, warmup=1):
    """Packed prefill: 64 sequences of lengths drawn uniformly from 1..1024 (seeded), H=16,
    d=128, bf16 inputs, GDN with INT8 group-32 rounding after every token."""
    import numpy as np
    import torch

    import quantized_state_qat_amd as la
    import synth

    rng = np.random.default_rng(9)
    lens = rng.integers(1, 1025, size=64)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    w = synth.Workload("varlen", B=1, T=T, H=16, d_k=128, d_v=128, s0_sigma=0.0, config_id=9)
    d = synth.generate(w)
    dev = {k: _dev(d[k]) for k in ("q", "k", "v", "g", "beta")}
    del d
    o = torch.empty((T, w.H, w.d_v), device="cuda")
    ST = torch.empty((len(lens), w.H, w.d_k, w.d_v), device="cuda")
    cu_d = torch.from_numpy(cu).cuda()
    c = la.Config(B=len(lens), T=T, H=w.H, d_k=w.d_k, d_v=w.d_v, qdq=la.LA_QDQ_INT8_GROUP, group=32, qdq_interval=1)
    stream = torch.cuda.current_stream()
    t = _time_calls(lambda: la.la_recurrent_fwd_varlen(c, cu_d, dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"],
                                                       None, o, ST, stream=stream), steps, warmup, stream)
    flops = 7.0 * w.d_k * w.d_v * w.H * T
    # the packed straight-through backward (checkpoints every 64 tokens recomputed inside)
    c.ckpt_interval = 64
    dout = torch.randn((T, w.H, w.d_v), device="cuda")
    gq, gk, gv = (torch.empty((T, w.H, n), device="cuda") for n in (w.d_k, w.d_k, w.d_v))
    gg, gb = torch.empty((T, w.H), device="cuda"), torch.empty((T, w.H), device="cuda")
    dS0 = torch.empty((len(lens), w.H, w.d_k, w.d_v), device="cuda")
    nbytes = la.la_bwd_varlen_workspace_bytes(c)
    ws = torch.empty((nbytes + 255) // 4, dtype=torch.float32, device="cuda")
    t_b = _time_calls(lambda: la.la_recurrent_bwd_ste_varlen(c, cu_d, dev["q"], dev["k"], dev["v"], dev["g"],
                                                             dev["beta"], None, dout, None, gq, gk, gv, gg, gb, dS0,
                                                             ws, nbytes, stream=stream), steps, warmup, stream)
    return {
        "ms_bwd": t_b * 1e3,
        "workload": f"packed prefill, 64 GDN sequences of 1..1024 tokens ({T} in all), H=16, d=128, bf16 inputs, "
                    "INT8 group-32 every token",
        "kernel": "token (packed sequences)", "ms_per_call": t * 1e3, "updates_per_s": w.H * T / t,
        "roofline": _fp32_roofline(flops, t, "algorithmic fp32 work of the recurrence (7 d_k d_v per token-head); "
                                             "the INT8 codec is not counted; the longest sequence sets the time"),
        "issue_floor": _issue_roofline(12.0, w.d_k * w.d_v * w.H * T, t, "token step (4) and INT8 codec (8) per "
                                                                       "element and token"),
        "issue_floor_bwd": _issue_roofline(23.0, w.d_k * w.d_v * w.H * T, t_b,
                                           "recompute with the codec once (12), decode of the kept codes (2) and "
                                           "adjoint (9)"),
    }


def bench_wht_fwdbwd(steps=2, warmup=1):
    """GDN B=4 H=16 T=2048 d=128, bf16 inputs, Hadamard + INT8 group-32 every token: forward with
    64-token checkpoints, then the straight-through backward from them."""
    import torch

    import quantized_state_qat_amd as la
    import synth

    w = synth.WORKLOADS[4]
    d = synth.generate(w, with_do=True)
    dev = {k: _dev(d[k]) for k in ("q", "k", "v", "g", "beta")}
    dout = _dev(d["do"])
    del d
    c = la.Config(B=w.B, T=w.T, H=w.H, d_k=w.d_k, d_v=w.d_v, qdq=la.LA_QDQ_INT8_GROUP, group=32, hadamard=1,
                  qdq_interval=1, ckpt_interval=64)
    o = torch.empty((w.B, w.T, w.H, w.d_v), device="cuda")
    ST = torch.empty((w.B, w.H, w.d_k, w.d_v), device="cuda")
    ck = torch.empty((w.B, w.H, (w.T + 63) // 64, w.d_k, w.d_v), device="cuda")
    grads = [torch.empty((w.B, w.T, w.H, n), device="cuda") for n in (w.d_k, w.d_k, w.d_v)]
    dg = torch.empty((w.B, w.T, w.H), device="cuda")
    dbeta = torch.empty((w.B, w.T, w.H), device="cuda")
    dS0 = torch.empty((w.B, w.H, w.d_k, w.d_v), device="cuda")
    nbytes = la.la_bwd_workspace_bytes(c)
    ws = torch.empty((nbytes + 255) // 4, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def fwd():
        la.la_recurrent_fwd(c, dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], None, o, ST, ck, stream=stream)

    def bwd():
        la.la_recurrent_bwd_ste(c, dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], None, ck, dout, None,
                                grads[0], grads[1], grads[2], dg, dbeta, dS0, ws, nbytes, stream=stream)

    t_f = _time_calls(fwd, steps, warmup, stream)
    t_b = _time_calls(bwd, steps, warmup, stream)
    unit = w.d_k * w.d_v * w.B * w.H * w.T
    return {
        "workload": "gdn_fwdbwd_wht_int8g32 B=4 H=16 T=2048 d_k=d_v=128 bf16 inputs, Hadamard + INT8 group-32 every "
                    "token, forward with 64-token checkpoints + STE backward",
        "kernel": la.la_fwd_kernel_name(c), "ms_fwd": t_f * 1e3, "ms_bwd": t_b * 1e3,
        "updates_per_s": w.B * w.H * w.T / (t_f + t_b),
        "roofline": _fp32_roofline(29.0 * unit, t_f + t_b,
                                   "forward 7 + recompute 7 + adjoint 15 d_k d_v flops per token-head; the "
                                   "rotations and the codec are not counted"),
        "roofline_fwd": _fp32_roofline(7.0 * unit, t_f, "forward only"),
        "roofline_bwd": _fp32_roofline(22.0 * unit, t_b, "backward only (recompute + adjoint)"),
        "issue_floor_fwd": _issue_roofline(12.0, unit, t_f, "decay, projections, update (4) and the INT8 codec (8) "
                                                            "per element and token (the state is carried rotated)"),
        "issue_floor_bwd": _issue_roofline(23.0, unit, t_b, "the forward token step with its codec once (recompute "
                                                            "of the chunk keeping every token's codes: 12), the "
                                                            "decode of the kept codes (2) and the adjoint (9) per "
                                                            "element and token"),
    }


def bench_replay(steps=2, warmup=1):
    """Replay windows of 16 tokens on the Hadamard workload's shape (GDN B=4 H=16 T=2048 d=128,
    bf16 inputs, Hadamard + INT8 group-32 refresh every 16 tokens, BF16 update entries in
    between): forward with 64-token checkpoints, then the straight-through backward."""
    import torch

    import quantized_state_qat_amd as la
    import synth

    w = synth.WORKLOADS[4]
    d = synth.generate(w, with_do=True)
    dev = {k: _dev(d[k]) for k in ("q", "k", "v", "g", "beta")}
    dout = _dev(d["do"])
    del d
    c = la.Config(B=w.B, T=w.T, H=w.H, d_k=w.d_k, d_v=w.d_v, qdq=la.LA_QDQ_INT8_GROUP, group=32, hadamard=1,
                  qdq_interval=16, replay=1, ckpt_interval=64)
    o = torch.empty((w.B, w.T, w.H, w.d_v), device="cuda")
    ST = torch.empty((w.B, w.H, w.d_k, w.d_v), device="cuda")
    ck = torch.empty((w.B, w.H, (w.T + 63) // 64, w.d_k, w.d_v), device="cuda")
    grads = [torch.empty((w.B, w.T, w.H, n), device="cuda") for n in (w.d_k, w.d_k, w.d_v)]
    dg = torch.empty((w.B, w.T, w.H), device="cuda")
    dbeta = torch.empty((w.B, w.T, w.H), device="cuda")
    dS0 = torch.empty((w.B, w.H, w.d_k, w.d_v), device="cuda")
    nbytes = la.la_bwd_workspace_bytes(c)
    ws = torch.empty((nbytes + 255) // 4, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    t_f = _time_calls(lambda: la.la_recurrent_fwd(c, dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], None, o,
                                                  ST, ck, stream=stream), steps, warmup, stream)
    t_b = _time_calls(lambda: la.la_recurrent_bwd_ste(c, dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], None, ck,
                                                      dout, None, grads[0], grads[1], grads[2], dg, dbeta, dS0, ws,
                                                      nbytes, stream=stream), steps, warmup, stream)
    unit = w.d_k * w.d_v * w.B * w.H * w.T
    return {
        "workload": "gdn_fwdbwd_wht_int8g32 shape with replay windows of 16 tokens: Hadamard + INT8 group-32 "
                    "refresh every 16 tokens, BF16 update entries in between, 64-token checkpoints",
        "kernel": la.la_fwd_kernel_name(c), "ms_fwd": t_f * 1e3, "ms_bwd": t_b * 1e3,
        "updates_per_s": w.B * w.H * w.T / (t_f + t_b),
        "roofline_fwd": _fp32_roofline(7.0 * unit, t_f, "forward: 7 d_k d_v flops per token-head"),
        "roofline_bwd": _fp32_roofline(22.0 * unit, t_b, "backward: recompute 7 + adjoint 15 d_k d_v per token-head"),
    }


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _timed_oracle(run, units_per_run, threads, reps=3):
    """Median over `reps` runs of the oracle at `threads` OpenMP threads: units per second."""
    import oracle
    oracle.set_num_threads(threads)
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        run()
        times.append(time.perf_counter() - t0)
    times.sort()
    med = times[len(times) // 2]
    return {"threads": threads, "median_s": med, "runs_s": times, "value": units_per_run / med}


def cpu_baseline(d, w):
    """The float64 oracle's decode step on the host cores (same generated inputs): the full
    B x H batch, median of three runs at all threads (ten steps a run) and at one thread (one
    step a run)."""
    import oracle
    oracle.build()
    all_threads = oracle.num_threads()
    args = [d[k].f64 for k in ("q", "k", "v", "g", "beta")]
    S0 = d["S0"].f64

    def steps(n):
        return lambda: [oracle.fwd(*args, S0, qdq_mode=oracle.QDQ_INT8, group=32, qdq_interval=1) for _ in range(n)]

    r_all = _timed_oracle(steps(10), 10 * w.B * w.H, all_threads)
    r_one = _timed_oracle(steps(1), w.B * w.H, 1)
    oracle.set_num_threads(all_threads)
    return {"value": r_all["value"], "unit": "token·head updates/s", "cores": all_threads, "kind": "oracle",
            "cpu_model": cpu_model(), "threads_all": r_all, "threads_1": r_one,
            "sample": f"decode steps of the full B={w.B} H={w.H} d={w.d_k} batch, INT8 g32: median of 3 runs of "
                      f"10 steps at {all_threads} threads and of 3 runs of 1 step at 1 thread (float64 oracle, "
                      "OpenMP over (sequence, head) units)"}


def cpu_baseline_long():
    """The oracle on a bounded sample of the long-sequence E4M3 workload (same generator):
    all 128 units over the first 256 tokens at all threads, 8 units over the first 256 tokens
    at one thread; median of three runs each."""
    import numpy as np

    import oracle
    import synth
    oracle.build()
    all_threads = oracle.num_threads()
    w = synth.Workload("gdn_long_e4m3_64", B=8, T=256, H=16, d_k=128, d_v=128, gate_dtype="f32", config_id=2)
    d = synth.generate(w)
    args = [d[k].f64 for k in ("q", "k", "v", "g", "beta")]
    one = [np.ascontiguousarray(a[:1, :, :8]) for a in args]
    kw = dict(qdq_mode=oracle.QDQ_E4M3, group=64, qdq_interval=64)
    r_all = _timed_oracle(lambda: oracle.fwd(*args, None, **kw), w.B * w.H * w.T, all_threads)
    r_one = _timed_oracle(lambda: oracle.fwd(*one, None, **kw), 8 * w.T, 1)
    oracle.set_num_threads(all_threads)
    return {"value": r_all["value"], "unit": "token·head updates/s", "cores": all_threads, "kind": "oracle",
            "cpu_model": cpu_model(), "threads_all": r_all, "threads_1": r_one,
            "sample": "the long-sequence E4M3 workload's first 256 tokens (generator of B=8 H=16 T=4096 d=128, "
                      "E4M3 every 64 tokens): all 128 units at all threads, 8 units at 1 thread; median of 3 runs"}


def profile_mode(steps):
    import torch
    r = bench_decode(steps, 1)
    src = torch.empty(268435456 // 4, dtype=torch.float32, device="cuda").normal_()
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"profile mode: {steps} decode launches (mean {r['mean_launch_s'] * 1e6:.1f} us), "
          f"2 copies of {src.numel() * 4} bytes", flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=150)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the long-sequence, KDA and Hadamard forward/backward measurements")
    ap.add_argument("--only", default="",
                    help="comma-separated extra measurements to run alone (e.g. long_sequence_fwdbwd), "
                         "printing their JSON only: for profiling one workload")
    ap.add_argument("--profile", action="store_true",
                    help="counter-collection mode: a few decode launches and one plain copy of a "
                         "256 MiB state buffer (the calibration kernel for HBM byte counters); no JSON")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards over (sequence, head) with no collective; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    torch.cuda.set_device(0)
    import quantized_state_qat_amd as la
    la.load_library()

    if args.profile:
        profile_mode(min(args.steps, 5))
        return
    if args.only:
        extras = {
            "long_sequence_valu": lambda: bench_long_e4m3()[2], "long_sequence": lambda: bench_long_e4m3()[0],
            "long_sequence_fwdbwd": lambda: bench_long_e4m3()[1], "kda_long_e4m3": bench_kda_long,
            "kda_int8g64_tok": bench_kda_tok, "gdn_fwdbwd_wht_int8g32": bench_wht_fwdbwd,
            "replay_w16_wht_int8g32": bench_replay, "decode_slots": bench_decode_slots,
            "decode_replay_w16": bench_decode_replay, "varlen_prefill": bench_varlen, "chunk_prefill": bench_chunk,
        }
        out = {}
        for name in args.only.split(","):
            out[name] = extras[name]()
            print(f"done {name}", file=sys.stderr, flush=True)
        print(json.dumps(out), flush=True)
        return

    # The decode inputs are placed first; the other workloads run next, and the decode steps are
    # timed right after them, so that the timed steps see the GPU at its steady-state clocks (in a
    # fresh process the first ~150 back-to-back decode launches run about 3% slower).
    setup = decode_setup()
    extra = None
    long_valu = None
    if not args.no_extra:
        long_fwd, long_fwdbwd, long_valu = bench_long_e4m3()
        extra = {"long_sequence_valu": long_valu, "long_sequence": long_fwd,
                 "long_sequence_fwdbwd": long_fwdbwd, "kda_long_e4m3": bench_kda_long(),
                 "kda_int8g64_tok": bench_kda_tok(),
                 "gdn_fwdbwd_wht_int8g32": bench_wht_fwdbwd(), "replay_w16_wht_int8g32": bench_replay(),
                 "decode_slots": bench_decode_slots(), "decode_replay_w16": bench_decode_replay(),
                 "varlen_prefill": bench_varlen(), "chunk_prefill": bench_chunk()}
    r = bench_decode(args.steps, args.warmup, setup)
    w = r["w"]
    value = r["updates"] / r["total_s"]
    achieved = r["bytes_per_launch"] / r["mean_launch_s"] / 1e9
    khash = kernel_hash(["decode.hip", "la_device.hpp"])
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "token·head updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["total_s"] / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "gdn_decode_int8g32: single-token GDN decode, B=256 H=16 d_k=d_v=128, bf16 q/k/v/g/beta, "
                        "fp32 state updated in place with INT8 group-32 QDQ (3 rotating state buffers)",
            "B": w.B, "H": w.H, "d_k": w.d_k, "d_v": w.d_v, "qdq": "int8_group32_every_token",
        },
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": pmc_traffic("decode_int8g32_b256h16_pmc.json", khash),
            "bytes_per_launch": r["bytes_per_launch"], "mean_launch_us": r["mean_launch_s"] * 1e6,
            "kernel_source_hash": khash,
        },
    }
    if extra is not None:
        if not args.no_cpu:
            long_valu["cpu_baseline"] = cpu_baseline_long()
        line["extra"] = extra
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(r["d"], w)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
