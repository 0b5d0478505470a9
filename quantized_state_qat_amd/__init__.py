"""Python binding of liblaqat.so: gated delta rule recurrence with fused dynamic state
fake-quantization on AMD MI355X (gfx950).

The functions here carry the C ABI's names (include/la.h) and only marshal arguments:
torch tensors supply device memory and the current HIP stream; every step of the
computation runs in the library's HIP kernels.  There is no fallback: if the library is
missing, or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblaqat.so")

LA_OK, LA_ERR_INVALID_ARG, LA_ERR_UNSUPPORTED, LA_ERR_ALIGNMENT, LA_ERR_WORKSPACE, LA_ERR_HIP = range(6)
LA_F32, LA_BF16 = 0, 1
LA_GATE_SCALAR, LA_GATE_KEY = 0, 1
LA_QDQ_NONE, LA_QDQ_INT8_GROUP, LA_QDQ_E4M3_TILE = 0, 1, 2


class LaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"la status {status}: {detail}")
        self.status = status


class la_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "T", "H", "d_k", "d_v", "gate", "qdq", "group", "hadamard", "qdq_interval",
                 "ckpt_interval", "qkv_dtype", "gate_dtype", "out_dtype", "state_rotated")]


@dataclasses.dataclass
class Config:
    B: int
    T: int
    H: int
    d_k: int
    d_v: int
    gate: int = LA_GATE_SCALAR
    qdq: int = LA_QDQ_NONE
    group: int = 32
    hadamard: int = 0
    qdq_interval: int = 1
    ckpt_interval: int = 0
    qkv_dtype: int = LA_BF16
    gate_dtype: int = LA_BF16
    out_dtype: int = LA_F32
    state_rotated: int = 0

    def c(self) -> la_config:
        return la_config(*[int(getattr(self, f.name)) for f in dataclasses.fields(self)])


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load liblaqat.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                               "(hipcc, gfx950); there is no fallback path")
        # torch carries its own HIP runtime, whose soname matches the one the library needs.
        # Loaded first, it is the runtime the library binds to; loaded after the library,
        # torch would bring a second runtime into the process, and the two cannot share
        # devices, pointers or streams.
        import torch  # noqa: F401
        lib = ctypes.CDLL(path)
        vp, cp = ctypes.c_void_p, ctypes.POINTER(la_config)
        lib.la_recurrent_fwd.restype = ctypes.c_int
        lib.la_recurrent_fwd.argtypes = [cp] + [vp] * 10
        lib.la_decode_step.restype = ctypes.c_int
        lib.la_decode_step.argtypes = [cp] + [vp] * 10
        lib.la_recurrent_bwd_ste.restype = ctypes.c_int
        lib.la_recurrent_bwd_ste.argtypes = [cp] + [vp] * 16 + [ctypes.c_size_t, vp]
        lib.la_recurrent_fwd_varlen.restype = ctypes.c_int
        lib.la_recurrent_fwd_varlen.argtypes = [cp] + [vp] * 10
        lib.la_decode_step_slots.restype = ctypes.c_int
        lib.la_decode_step_slots.argtypes = [cp] + [vp] * 7 + [ctypes.c_int32] + [vp] * 4
        lib.la_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.la_bwd_workspace_bytes.argtypes = [cp]
        lib.la_status_string.restype = ctypes.c_char_p
        lib.la_status_string.argtypes = [ctypes.c_int]
        lib.la_last_error.restype = ctypes.c_char_p
        lib.la_last_error.argtypes = []
        lib.la_fwd_kernel_name.restype = ctypes.c_char_p
        lib.la_fwd_kernel_name.argtypes = [cp]
        lib.la_bwd_kernel_name.restype = ctypes.c_char_p
        lib.la_bwd_kernel_name.argtypes = [cp]
        _lib = lib
    return _lib


def _ptr(t) -> Optional[int]:
    """Device address of a tensor (None stays NULL); the tensor must be contiguous."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(status: int) -> None:
    if status != LA_OK:
        lib = load_library()
        raise LaError(status, lib.la_last_error().decode() or lib.la_status_string(status).decode())


def la_recurrent_fwd(cfg: Config, q, k, v, g, beta, S0, o, S_T=None, ckpts=None, stream=None) -> None:
    lib = load_library()
    c = cfg.c()
    _check(lib.la_recurrent_fwd(ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                _ptr(S0), _ptr(o), _ptr(S_T), _ptr(ckpts), _stream(stream)))


def la_recurrent_fwd_varlen(cfg: Config, cu_seqlens, q, k, v, g, beta, S0, o, S_T=None, stream=None) -> None:
    lib = load_library()
    c = cfg.c()
    _check(lib.la_recurrent_fwd_varlen(ctypes.byref(c), _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                       _ptr(beta), _ptr(S0), _ptr(o), _ptr(S_T), _stream(stream)))


def la_decode_step(cfg: Config, q, k, v, g, beta, S, o, codes=None, scales=None, stream=None) -> None:
    lib = load_library()
    c = cfg.c()
    _check(lib.la_decode_step(ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                              _ptr(S), _ptr(o), _ptr(codes), _ptr(scales), _stream(stream)))


def la_decode_step_slots(cfg: Config, q, k, v, g, beta, S_pool, slots, n_slots: int, o, codes=None,
                         scales=None, stream=None) -> None:
    lib = load_library()
    c = cfg.c()
    _check(lib.la_decode_step_slots(ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                    _ptr(S_pool), _ptr(slots), int(n_slots), _ptr(o), _ptr(codes),
                                    _ptr(scales), _stream(stream)))


def la_bwd_workspace_bytes(cfg: Config) -> int:
    c = cfg.c()
    return int(load_library().la_bwd_workspace_bytes(ctypes.byref(c)))


def la_recurrent_bwd_ste(cfg: Config, q, k, v, g, beta, S0, ckpts, dout, dS_T, dq, dk, dv, dg,
                         dbeta, dS0, workspace, ws_bytes: int, stream=None) -> None:
    lib = load_library()
    c = cfg.c()
    _check(lib.la_recurrent_bwd_ste(ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                    _ptr(S0), _ptr(ckpts), _ptr(dout), _ptr(dS_T), _ptr(dq), _ptr(dk),
                                    _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(dS0), _ptr(workspace),
                                    int(ws_bytes), _stream(stream)))


def la_fwd_kernel_name(cfg: Config) -> str:
    """Which forward kernel serves cfg: "block", "wave", "fast" or "token" ("" if invalid)."""
    c = cfg.c()
    return load_library().la_fwd_kernel_name(ctypes.byref(c)).decode()


def la_bwd_kernel_name(cfg: Config) -> str:
    """Which backward serves cfg: "block" or "token" ("" if invalid)."""
    c = cfg.c()
    return load_library().la_bwd_kernel_name(ctypes.byref(c)).decode()


def la_status_string(status: int) -> str:
    return load_library().la_status_string(status).decode()


def la_last_error() -> str:
    return load_library().la_last_error().decode()
