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
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP32_VALU_PEAK_TFLOPS = 157.3  # MI355X FP32 (vector, packed; equal to the FP32 matrix peak)
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


def bench_decode(steps, warmup):
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
        "w": w, "d": d, "total_s": total, "wall_s": wall, "mean_launch_s": mean_launch,
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
    fwd = {
        "workload": "gdn_long_e4m3_64 B=8 H=16 T=4096 d_k=d_v=128 bf16 q/k/v, fp32 g/beta/state, E4M3 tile QDQ every 64 tokens",
        "kernel": la.la_fwd_kernel_name(c), "ms_per_call": t * 1e3, "updates_per_s": w.B * w.H * w.T / t,
        "roofline": _fp32_roofline(7.0 * unit, t, "algorithmic fp32 work of the recurrence (7 d_k d_v per token-head) "
                                                  "against the FP32 peak; the block kernel forms it on the matrix cores "
                                                  "from exact bf16 products with fp32 sums"),
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
    return fwd, fwdbwd


def bench_kda_long(steps=3, warmup=1):
    """KDA B=8 H=16 T=4096 d=128, bf16 q/k/v, fp32 per-key gates and beta, E4M3 tile QDQ every
    64 tokens: the forward (block kernel) and the straight-through backward (token kernel)."""
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
    unit = w.d_k * w.d_v * w.B * w.H * w.T
    return {
        "workload": "kda_long_e4m3_64 B=8 H=16 T=4096 d_k=d_v=128 bf16 q/k/v, fp32 per-key gates and beta, E4M3 tile "
                    "QDQ every 64 tokens, 64-token checkpoints",
        "kernel_fwd": la.la_fwd_kernel_name(c), "kernel_bwd": la.la_bwd_kernel_name(c),
        "ms_fwd": t_f * 1e3, "ms_bwd": t_b * 1e3, "updates_per_s_fwd": w.B * w.H * w.T / t_f,
        "roofline_fwd": _fp32_roofline(7.0 * unit, t_f, "forward: 7 d_k d_v flops per token-head (the per-key decay "
                                                        "adds d_k d_v multiplies, not counted)"),
        "roofline_bwd": _fp32_roofline(22.0 * unit, t_b, "backward: recompute 7 + adjoint 15 d_k d_v per token-head"),
    }


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
    c.hadamard = 1
    t_h = _time_calls(lambda: la.la_recurrent_fwd(c, dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], None, o,
                                                  ST, stream=stream), steps, warmup, stream)
    flops = 7.0 * w.d_k * w.d_v * w.B * w.H * w.T
    return {
        "workload": "kda_int8g64_tok B=4 H=32 T=2048 d_k=d_v=128 bf16 inputs, KDA gate, INT8 group-64 QDQ every token",
        "kernel": la.la_fwd_kernel_name(c), "ms_per_call": t * 1e3, "updates_per_s": w.B * w.H * w.T / t,
        "roofline": _fp32_roofline(flops, t, "algorithmic fp32 work of the recurrence (7 d_k d_v per token-head); "
                                             "the INT8 codec is not counted"),
        "ms_per_call_hadamard": t_h * 1e3,
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
    return {
        "workload": f"packed prefill, 64 GDN sequences of 1..1024 tokens ({T} in all), H=16, d=128, bf16 inputs, "
                    "INT8 group-32 every token",
        "kernel": "token (packed sequences)", "ms_per_call": t * 1e3, "updates_per_s": w.H * T / t,
        "roofline": _fp32_roofline(flops, t, "algorithmic fp32 work of the recurrence (7 d_k d_v per token-head); "
                                             "the INT8 codec is not counted; the longest sequence sets the time"),
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
    }


def cpu_baseline(d, w, budget_s=12.0):
    """The float64 oracle's decode step on the host cores (same generated inputs), repeated on
    the full batch until about budget_s seconds of CPU time."""
    import oracle
    oracle.build()
    args = [d[k].f64 for k in ("q", "k", "v", "g", "beta")]
    S0 = d["S0"].f64
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.fwd(*args, S0, qdq_mode=oracle.QDQ_INT8, group=32, qdq_interval=1)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 5000:
            break
    rate = reps * w.B * w.H / el
    return {"value": rate, "unit": "token·head updates/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{reps} full decode steps of the B={w.B} H={w.H} d={w.d_k} batch in {el:.1f} s "
                      "(float64 oracle, OpenMP over (sequence, head) units)"}


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

    r = bench_decode(args.steps, args.warmup)
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
    if not args.no_extra:
        long_fwd, long_fwdbwd = bench_long_e4m3()
        line["extra"] = {"long_sequence": long_fwd, "long_sequence_fwdbwd": long_fwdbwd, "kda_long_e4m3": bench_kda_long(),
                         "kda_int8g64_tok": bench_kda_tok(),
                         "gdn_fwdbwd_wht_int8g32": bench_wht_fwdbwd(), "decode_slots": bench_decode_slots(),
                         "varlen_prefill": bench_varlen()}
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(r["d"], w)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
