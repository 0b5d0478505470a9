"""Seeded synthetic inputs for the gated delta rule recurrence.

This module only draws random numbers and shapes them into the input
distributions of the workloads; it holds none of the recurrence or codec
arithmetic.  The GPU library, its tests, the CPU oracle's tests and the bench
all draw their inputs from here so that every side sees the same bits.

Random numbers come from a counter-based SplitMix64 stream (Steele, Lea and
Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014): value
number ``i`` of stream ``seed`` is the SplitMix64 finaliser applied to
``seed + (i + 1) * 0x9E3779B97F4A7C15``.  Uniforms take the top 53 bits plus a
half-step offset (so they lie strictly inside (0, 1)); normals use the cosine
branch of Box-Muller on the uniform pair (2i, 2i + 1).  Every tensor is a pure
function of (seed, stream id), independent of the order tensors are drawn in
and of any library version.

Distributions (the workloads of the linear-attention state-QAT pages, with the
shapes of the five benchmark configurations):

* q ~ N(0, 1) / sqrt(d_k)
* k ~ N(0, 1), L2-normalised per (b, t, h) in float64
* v ~ N(0, 1)
* g = -softplus(N(0, 1)) (scalar per token-head, or one per key channel)
* beta = sigmoid(N(0, 1))
* S_0 = 0, or N(0, sigma^2) for the decode workload (sigma = 0.05)
* do ~ N(0, 1) (upstream gradient of the outputs)

Casting to bfloat16 rounds float64 -> float32 -> bfloat16, each step to
nearest-even; bf16 tensors are returned as their uint16 bit patterns together
with the exactly widened float32 values.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

BASE_SEED = 20261203

# stream ids: one independent stream per tensor
STREAMS = {"q": 0, "k": 1, "v": 2, "g": 3, "beta": 4, "S0": 5, "do": 6, "dST": 7}

_CHUNK = 1 << 22  # values per generation chunk (bounds temporary memory)


def splitmix64(seed: int, start: int, n: int) -> np.ndarray:
    """Values start..start+n-1 of the SplitMix64 stream keyed by ``seed``."""
    idx = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + idx * _GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def uniform(seed: int, n: int, start: int = 0) -> np.ndarray:
    """n uniforms in the open interval (0, 1), float64."""
    z = splitmix64(seed, start, n)
    return ((z >> np.uint64(11)).astype(np.float64) + 0.5) * (1.0 / 9007199254740992.0)


def normal(seed: int, n: int) -> np.ndarray:
    """n standard normals (float64), Box-Muller cosine branch on uniform pairs."""
    out = np.empty(n, dtype=np.float64)
    for s in range(0, n, _CHUNK):
        m = min(_CHUNK, n - s)
        u = uniform(seed, 2 * m, start=2 * s)
        u1 = u[0::2]
        u2 = u[1::2]
        out[s:s + m] = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Tensor:
    """A generated tensor: ``f32`` holds the values the kernels see (exactly
    representable in the storage dtype); ``bits`` holds the bf16 bit patterns
    when the storage dtype is bf16."""

    f32: np.ndarray
    dtype: str  # "f32" or "bf16"
    bits: Optional[np.ndarray] = None

    @property
    def f64(self) -> np.ndarray:
        return self.f32.astype(np.float64)

    def storage(self) -> np.ndarray:
        """The array in its storage dtype (float32, or uint16 bf16 bits)."""
        return self.bits if self.dtype == "bf16" else self.f32


def cast(x64: np.ndarray, dtype: str) -> Tensor:
    x32 = np.asarray(x64, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return Tensor(f32=x32, dtype="f32")
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x32)
        return Tensor(f32=bf16_bits_to_f32(bits).reshape(x32.shape), dtype="bf16", bits=bits.reshape(x32.shape))
    raise ValueError(f"unknown dtype {dtype}")


def seed_for(config_id: int, stream: str) -> int:
    return BASE_SEED + 100 * config_id + STREAMS[stream]


def softplus(x: np.ndarray) -> np.ndarray:
    return np.where(x > 0, x + np.log1p(np.exp(-np.abs(x))), np.log1p(np.exp(x)))


def sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


@dataclasses.dataclass
class Workload:
    """Shape and dtype recipe of one synthetic workload."""

    name: str
    B: int
    T: int
    H: int
    d_k: int
    d_v: int
    gate: str = "scalar"       # "scalar" (GDN) | "key" (KDA)
    qkv_dtype: str = "bf16"
    gate_dtype: str = "bf16"   # dtype of g and beta
    s0_sigma: float = 0.0      # 0 -> S_0 = 0
    config_id: int = 0         # seed family


def generate(w: Workload, with_do: bool = False, with_dST: bool = False) -> Dict[str, Tensor]:
    """Draw q, k, v, g, beta, S0 (and do, dS_T) for workload ``w``."""
    B, T, H, dk, dv = w.B, w.T, w.H, w.d_k, w.d_v
    cid = w.config_id
    out: Dict[str, Tensor] = {}
    q = normal(seed_for(cid, "q"), B * T * H * dk).reshape(B, T, H, dk) / math.sqrt(dk)
    out["q"] = cast(q, w.qkv_dtype)
    del q
    k = normal(seed_for(cid, "k"), B * T * H * dk).reshape(B, T, H, dk)
    k /= np.sqrt(np.sum(k * k, axis=-1, keepdims=True))
    out["k"] = cast(k, w.qkv_dtype)
    del k
    out["v"] = cast(normal(seed_for(cid, "v"), B * T * H * dv).reshape(B, T, H, dv), w.qkv_dtype)
    gshape = (B, T, H, dk) if w.gate == "key" else (B, T, H)
    gn = normal(seed_for(cid, "g"), int(np.prod(gshape))).reshape(gshape)
    out["g"] = cast(-softplus(gn), w.gate_dtype)
    bn = normal(seed_for(cid, "beta"), B * T * H).reshape(B, T, H)
    out["beta"] = cast(sigmoid(bn), w.gate_dtype)
    if w.s0_sigma > 0:
        s0 = normal(seed_for(cid, "S0"), B * H * dk * dv).reshape(B, H, dk, dv) * w.s0_sigma
    else:
        s0 = np.zeros((B, H, dk, dv))
    out["S0"] = cast(s0, "f32")
    if with_do:
        out["do"] = cast(normal(seed_for(cid, "do"), B * T * H * dv).reshape(B, T, H, dv), "f32")
    if with_dST:
        out["dST"] = cast(normal(seed_for(cid, "dST"), B * H * dk * dv).reshape(B, H, dk, dv), "f32")
    return out


# The five benchmark workloads of the state-QAT study (shapes and dtypes).
WORKLOADS = {
    0: Workload("gdn_fp32_int8g32_tok", B=1, T=64, H=2, d_k=64, d_v=64, qkv_dtype="f32", gate_dtype="f32", config_id=0),
    1: Workload("gdn_decode_int8g32", B=256, T=1, H=16, d_k=128, d_v=128, s0_sigma=0.05, config_id=1),
    2: Workload("gdn_long_e4m3_64", B=8, T=4096, H=16, d_k=128, d_v=128, gate_dtype="f32", config_id=2),
    3: Workload("kda_int8g64_tok", B=4, T=2048, H=32, d_k=128, d_v=128, gate="key", config_id=3),
    4: Workload("gdn_fwdbwd_wht_int8g32", B=4, T=2048, H=16, d_k=128, d_v=128, config_id=4),
}
