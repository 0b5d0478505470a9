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
LA_KERNEL_AUTO, LA_KERNEL_BLOCK, LA_KERNEL_WAVE, LA_KERNEL_FAST, LA_KERNEL_TOKEN, LA_KERNEL_CHUNK = range(6)
LA_SOLVE_EXACT, LA_SOLVE_NEUMANN = 0, 1


class LaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"la status {status}: {detail}")
        self.status = status


class la_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "T", "H", "d_k", "d_v", "gate", "qdq", "group", "hadamard", "qdq_interval",
                 "ckpt_interval", "qkv_dtype", "gate_dtype", "out_dtype", "state_rotated", "kernel", "replay", "solve",
                 "degree")]


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
    kernel: int = LA_KERNEL_AUTO
    replay: int = 0
    solve: int = LA_SOLVE_EXACT
    degree: int = 0

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
        lib.la_recurrent_fwd_chunk.restype = ctypes.c_int
        lib.la_recurrent_fwd_chunk.argtypes = [cp] + [vp] * 10 + [ctypes.c_size_t, vp]
        lib.la_chunk_workspace_bytes.restype = ctypes.c_size_t
        lib.la_chunk_workspace_bytes.argtypes = [cp]
        lib.la_recurrent_fwd_entries.restype = ctypes.c_int
        lib.la_recurrent_fwd_entries.argtypes = [cp] + [vp] * 11
        lib.la_recurrent_fwd_varlen.restype = ctypes.c_int
        lib.la_recurrent_fwd_varlen.argtypes = [cp] + [vp] * 10
        lib.la_recurrent_fwd_split.restype = ctypes.c_int
        lib.la_recurrent_fwd_split.argtypes = [cp, cp] + [vp] * 12
        lib.la_recurrent_bwd_ste_varlen.restype = ctypes.c_int
        lib.la_recurrent_bwd_ste_varlen.argtypes = [cp] + [vp] * 16 + [ctypes.c_size_t, vp]
        lib.la_bwd_varlen_workspace_bytes.restype = ctypes.c_size_t
        lib.la_bwd_varlen_workspace_bytes.argtypes = [cp]
        lib.la_recurrent_bwd_ste_split.restype = ctypes.c_int
        lib.la_recurrent_bwd_ste_split.argtypes = [cp, cp] + [vp] * 18 + [ctypes.c_size_t, vp]
        lib.la_bwd_split_workspace_bytes.restype = ctypes.c_size_t
        lib.la_bwd_split_workspace_bytes.argtypes = [cp, cp]
        lib.la_decode_step_replay.restype = ctypes.c_int
        lib.la_decode_step_replay.argtypes = [cp] + [vp] * 14
        lib.la_decode_step_slots.restype = ctypes.c_int
        lib.la_decode_step_slots.argtypes = [cp] + [vp] * 7 + [ctypes.c_int32] + [vp] * 4
        if hasattr(lib, "la_recurrent_bwd_ste_noalloc"):
            lib.la_recurrent_bwd_ste_noalloc.restype = ctypes.c_int
            lib.la_recurrent_bwd_ste_noalloc.argtypes = [cp] + [vp] * 16
            lib.la_noalloc_workspace_limit.restype = ctypes.c_size_t
            lib.la_noalloc_workspace_limit.argtypes = []
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


def _torch_dtype(code: int):
    import torch
    return torch.bfloat16 if code == LA_BF16 else torch.float32


def _arg(t, name: str, numel: int, dtypes=None) -> Optional[int]:
    """Address of a device tensor argument after checking, on the host, that it lives on a
    GPU, has one of the expected dtypes and holds at least `numel` elements: a host tensor,
    a wrong dtype or a short buffer would otherwise reach the kernels.  Raw integer
    addresses are passed through unchecked."""
    if t is None or isinstance(t, int):
        return _ptr(t)
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (got device {t.device})")
    if dtypes is not None:
        dts = dtypes if isinstance(dtypes, (tuple, list)) else (dtypes,)
        if t.dtype not in dts:
            raise ValueError(f"{name} has dtype {t.dtype}, expected {' or '.join(str(d) for d in dts)}")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, the configuration needs {numel}")
    return _ptr(t)


def _f32():
    import torch
    return torch.float32


def _gate_numel(cfg: Config, tokens: int) -> int:
    return tokens * cfg.H * (cfg.d_k if cfg.gate == LA_GATE_KEY else 1)


def _state_numel(cfg: Config, units: int) -> int:
    return units * cfg.H * cfg.d_k * cfg.d_v


def _inputs(cfg: Config, tokens: int, q, k, v, g, beta):
    """Checked addresses of q, k, v, g, beta for `tokens` token positions per head."""
    qd, gd = _torch_dtype(cfg.qkv_dtype), _torch_dtype(cfg.gate_dtype)
    return (_arg(q, "q", tokens * cfg.H * cfg.d_k, qd), _arg(k, "k", tokens * cfg.H * cfg.d_k, qd),
            _arg(v, "v", tokens * cfg.H * cfg.d_v, qd), _arg(g, "g", _gate_numel(cfg, tokens), gd),
            _arg(beta, "beta", tokens * cfg.H, gd))


def _codes_scales(cfg: Config, codes, scales):
    import torch
    n = _state_numel(cfg, cfg.B)
    nsc = cfg.B * cfg.H * (cfg.d_k * (cfg.d_v // cfg.group) if cfg.qdq == LA_QDQ_INT8_GROUP else cfg.d_v // 64)
    return (_arg(codes, "codes", n, (torch.int8, torch.uint8)), _arg(scales, "scales", nsc, _f32()))


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
    tok = cfg.B * cfg.T
    nck = (cfg.T + cfg.ckpt_interval - 1) // cfg.ckpt_interval if cfg.ckpt_interval > 0 else 0
    args = _inputs(cfg, tok, q, k, v, g, beta)
    _check(lib.la_recurrent_fwd(ctypes.byref(c), *args, _arg(S0, "S0", _state_numel(cfg, cfg.B), _f32()),
                                _arg(o, "o", tok * cfg.H * cfg.d_v, _torch_dtype(cfg.out_dtype)),
                                _arg(S_T, "S_T", _state_numel(cfg, cfg.B), _f32()),
                                _arg(ckpts, "ckpts", _state_numel(cfg, cfg.B) * nck, _f32()), _stream(stream)))


def la_chunk_workspace_bytes(cfg: Config) -> int:
    c = cfg.c()
    return int(load_library().la_chunk_workspace_bytes(ctypes.byref(c)))


def la_recurrent_fwd_chunk(cfg: Config, q, k, v, g, beta, S0, o, S_T, ckpts, workspace, ws_bytes: int,
                           stream=None) -> None:
    """The 64-token chunk form (exact or Neumann solve); workspace of la_chunk_workspace_bytes."""
    lib = load_library()
    c = cfg.c()
    tok = cfg.B * cfg.T
    nck = (cfg.T + cfg.ckpt_interval - 1) // cfg.ckpt_interval if cfg.ckpt_interval > 0 else 0
    args = _inputs(cfg, tok, q, k, v, g, beta)
    _check(lib.la_recurrent_fwd_chunk(ctypes.byref(c), *args, _arg(S0, "S0", _state_numel(cfg, cfg.B), _f32()),
                                      _arg(o, "o", tok * cfg.H * cfg.d_v, _torch_dtype(cfg.out_dtype)),
                                      _arg(S_T, "S_T", _state_numel(cfg, cfg.B), _f32()),
                                      _arg(ckpts, "ckpts", _state_numel(cfg, cfg.B) * nck, _f32()),
                                      _workspace(workspace, ws_bytes), int(ws_bytes), _stream(stream)))


def la_recurrent_fwd_entries(cfg: Config, q, k, v, g, beta, S0, o, S_T, ckpts, entries, stream=None) -> None:
    """la_recurrent_fwd in replay mode, also writing each token's BF16 update entry
    (entries: bf16 [B, T, H, d_v])."""
    import torch
    lib = load_library()
    c = cfg.c()
    tok = cfg.B * cfg.T
    nck = (cfg.T + cfg.ckpt_interval - 1) // cfg.ckpt_interval if cfg.ckpt_interval > 0 else 0
    args = _inputs(cfg, tok, q, k, v, g, beta)
    _check(lib.la_recurrent_fwd_entries(ctypes.byref(c), *args, _arg(S0, "S0", _state_numel(cfg, cfg.B), _f32()),
                                        _arg(o, "o", tok * cfg.H * cfg.d_v, _torch_dtype(cfg.out_dtype)),
                                        _arg(S_T, "S_T", _state_numel(cfg, cfg.B), _f32()),
                                        _arg(ckpts, "ckpts", _state_numel(cfg, cfg.B) * nck, _f32()),
                                        _arg(entries, "entries", tok * cfg.H * cfg.d_v, (torch.bfloat16, torch.int16)),
                                        _stream(stream)))


def la_recurrent_fwd_varlen(cfg: Config, cu_seqlens, q, k, v, g, beta, S0, o, S_T=None, stream=None) -> None:
    import torch
    lib = load_library()
    c = cfg.c()
    args = _inputs(cfg, cfg.T, q, k, v, g, beta)
    _check(lib.la_recurrent_fwd_varlen(ctypes.byref(c), _arg(cu_seqlens, "cu_seqlens", cfg.B + 1, torch.int32),
                                       *args, _arg(S0, "S0", _state_numel(cfg, cfg.B), _f32()),
                                       _arg(o, "o", cfg.T * cfg.H * cfg.d_v, _torch_dtype(cfg.out_dtype)),
                                       _arg(S_T, "S_T", _state_numel(cfg, cfg.B), _f32()), _stream(stream)))


def la_decode_step(cfg: Config, q, k, v, g, beta, S, o, codes=None, scales=None, stream=None) -> None:
    lib = load_library()
    c = cfg.c()
    args = _inputs(cfg, cfg.B, q, k, v, g, beta)
    _check(lib.la_decode_step(ctypes.byref(c), *args, _arg(S, "S", _state_numel(cfg, cfg.B), _f32()),
                              _arg(o, "o", cfg.B * cfg.H * cfg.d_v, _torch_dtype(cfg.out_dtype)),
                              *_codes_scales(cfg, codes, scales), _stream(stream)))


def _packed_grads(cfg: Config, dq, dk, dv, dg, dbeta, dS0):
    f32 = _f32()
    tok = cfg.T
    return (_arg(dq, "dq", tok * cfg.H * cfg.d_k, f32), _arg(dk, "dk", tok * cfg.H * cfg.d_k, f32),
            _arg(dv, "dv", tok * cfg.H * cfg.d_v, f32), _arg(dg, "dg", _gate_numel(cfg, tok), f32),
            _arg(dbeta, "dbeta", tok * cfg.H, f32), _arg(dS0, "dS0", _state_numel(cfg, cfg.B), f32))


def _workspace(workspace, ws_bytes):
    if workspace is not None and not isinstance(workspace, int):
        if not workspace.is_cuda:
            raise ValueError("workspace must be a GPU tensor")
        if workspace.numel() * workspace.element_size() < int(ws_bytes):
            raise ValueError(f"workspace holds fewer than the {int(ws_bytes)} bytes passed as ws_bytes")
    return _ptr(workspace)


def la_recurrent_fwd_split(prefix_cfg: Config, suffix_cfg: Config, cu_seqlens, prefix_len, q, k, v, g, beta, S0, o,
                           S_mid, S_T=None, stream=None) -> None:
    """Packed sequences, each cut into a prefix (prefix_cfg) and a suffix (suffix_cfg) at
    prefix_len[b] tokens; S_mid receives the handoff states."""
    import torch
    lib = load_library()
    cp, cs = prefix_cfg.c(), suffix_cfg.c()
    cfg = prefix_cfg
    args = _inputs(cfg, cfg.T, q, k, v, g, beta)
    n = _state_numel(cfg, cfg.B)
    _check(lib.la_recurrent_fwd_split(ctypes.byref(cp), ctypes.byref(cs),
                                      _arg(cu_seqlens, "cu_seqlens", cfg.B + 1, torch.int32),
                                      _arg(prefix_len, "prefix_len", cfg.B, torch.int32), *args,
                                      _arg(S0, "S0", n, _f32()),
                                      _arg(o, "o", cfg.T * cfg.H * cfg.d_v, _torch_dtype(cfg.out_dtype)),
                                      _arg(S_mid, "S_mid", n, _f32()), _arg(S_T, "S_T", n, _f32()), _stream(stream)))


def la_bwd_varlen_workspace_bytes(cfg: Config) -> int:
    c = cfg.c()
    return int(load_library().la_bwd_varlen_workspace_bytes(ctypes.byref(c)))


def la_recurrent_bwd_ste_varlen(cfg: Config, cu_seqlens, q, k, v, g, beta, S0, dout, dS_T, dq, dk, dv, dg, dbeta,
                                dS0, workspace, ws_bytes: int, stream=None) -> None:
    import torch
    lib = load_library()
    c = cfg.c()
    n = _state_numel(cfg, cfg.B)
    args = _inputs(cfg, cfg.T, q, k, v, g, beta)
    _check(lib.la_recurrent_bwd_ste_varlen(ctypes.byref(c), _arg(cu_seqlens, "cu_seqlens", cfg.B + 1, torch.int32),
                                           *args, _arg(S0, "S0", n, _f32()),
                                           _arg(dout, "dout", cfg.T * cfg.H * cfg.d_v, _f32()),
                                           _arg(dS_T, "dS_T", n, _f32()),
                                           *_packed_grads(cfg, dq, dk, dv, dg, dbeta, dS0),
                                           _workspace(workspace, ws_bytes), int(ws_bytes), _stream(stream)))


def la_bwd_split_workspace_bytes(prefix_cfg: Config, suffix_cfg: Config) -> int:
    cp, cs = prefix_cfg.c(), suffix_cfg.c()
    return int(load_library().la_bwd_split_workspace_bytes(ctypes.byref(cp), ctypes.byref(cs)))


def la_recurrent_bwd_ste_split(prefix_cfg: Config, suffix_cfg: Config, cu_seqlens, prefix_len, q, k, v, g, beta, S0,
                               S_mid, dout, dS_T, dq, dk, dv, dg, dbeta, dS0, workspace, ws_bytes: int,
                               stream=None) -> None:
    import torch
    lib = load_library()
    cp, cs = prefix_cfg.c(), suffix_cfg.c()
    cfg = prefix_cfg
    n = _state_numel(cfg, cfg.B)
    args = _inputs(cfg, cfg.T, q, k, v, g, beta)
    _check(lib.la_recurrent_bwd_ste_split(ctypes.byref(cp), ctypes.byref(cs),
                                          _arg(cu_seqlens, "cu_seqlens", cfg.B + 1, torch.int32),
                                          _arg(prefix_len, "prefix_len", cfg.B, torch.int32), *args,
                                          _arg(S0, "S0", n, _f32()), _arg(S_mid, "S_mid", n, _f32()),
                                          _arg(dout, "dout", cfg.T * cfg.H * cfg.d_v, _f32()),
                                          _arg(dS_T, "dS_T", n, _f32()),
                                          *_packed_grads(cfg, dq, dk, dv, dg, dbeta, dS0),
                                          _workspace(workspace, ws_bytes), int(ws_bytes), _stream(stream)))


def la_decode_step_replay(cfg: Config, q, k, v, g, beta, S, log_k, log_d, log_g, pos, o, codes=None, scales=None,
                          stream=None) -> None:
    """One decode token in replay mode: S holds the window's checkpoint, log_k/log_d (bf16)
    and log_g (float32) the entries of its earlier tokens, pos (int32 [B]) how many."""
    import torch
    lib = load_library()
    c = cfg.c()
    W1 = max(cfg.qdq_interval - 1, 0)
    args = _inputs(cfg, cfg.B, q, k, v, g, beta)
    nl = cfg.B * cfg.H * W1
    _check(lib.la_decode_step_replay(ctypes.byref(c), *args, _arg(S, "S", _state_numel(cfg, cfg.B), _f32()),
                                     _arg(log_k, "log_k", nl * cfg.d_k, (torch.bfloat16, torch.int16)),
                                     _arg(log_d, "log_d", nl * cfg.d_v, (torch.bfloat16, torch.int16)),
                                     _arg(log_g, "log_g", nl * (cfg.d_k if cfg.gate == LA_GATE_KEY else 1), _f32()),
                                     _arg(pos, "pos", cfg.B, torch.int32),
                                     _arg(o, "o", cfg.B * cfg.H * cfg.d_v, _torch_dtype(cfg.out_dtype)),
                                     *_codes_scales(cfg, codes, scales), _stream(stream)))


def la_decode_step_slots(cfg: Config, q, k, v, g, beta, S_pool, slots, n_slots: int, o, codes=None,
                         scales=None, stream=None) -> None:
    import torch
    lib = load_library()
    c = cfg.c()
    args = _inputs(cfg, cfg.B, q, k, v, g, beta)
    _check(lib.la_decode_step_slots(ctypes.byref(c), *args,
                                    _arg(S_pool, "S_pool", _state_numel(cfg, max(int(n_slots), 0)), _f32()),
                                    _arg(slots, "slots", cfg.B, torch.int32), int(n_slots),
                                    _arg(o, "o", cfg.B * cfg.H * cfg.d_v, _torch_dtype(cfg.out_dtype)),
                                    *_codes_scales(cfg, codes, scales), _stream(stream)))


def la_bwd_workspace_bytes(cfg: Config) -> int:
    c = cfg.c()
    return int(load_library().la_bwd_workspace_bytes(ctypes.byref(c)))


def la_recurrent_bwd_ste(cfg: Config, q, k, v, g, beta, S0, ckpts, dout, dS_T, dq, dk, dv, dg,
                         dbeta, dS0, workspace, ws_bytes: int, stream=None) -> None:
    lib = load_library()
    c = cfg.c()
    f32 = _f32()
    tok = cfg.B * cfg.T
    nck = (cfg.T + cfg.ckpt_interval - 1) // cfg.ckpt_interval if cfg.ckpt_interval > 0 else 0
    nst = _state_numel(cfg, cfg.B)
    args = _inputs(cfg, tok, q, k, v, g, beta)
    if workspace is not None and not isinstance(workspace, int):
        if not workspace.is_cuda:
            raise ValueError("workspace must be a GPU tensor")
        if workspace.numel() * workspace.element_size() < int(ws_bytes):
            raise ValueError(f"workspace holds fewer than the {int(ws_bytes)} bytes passed as ws_bytes")
    _check(lib.la_recurrent_bwd_ste(ctypes.byref(c), *args, _arg(S0, "S0", nst, f32),
                                    _arg(ckpts, "ckpts", nst * nck, f32),
                                    _arg(dout, "dout", tok * cfg.H * cfg.d_v, f32), _arg(dS_T, "dS_T", nst, f32),
                                    _arg(dq, "dq", tok * cfg.H * cfg.d_k, f32),
                                    _arg(dk, "dk", tok * cfg.H * cfg.d_k, f32),
                                    _arg(dv, "dv", tok * cfg.H * cfg.d_v, f32),
                                    _arg(dg, "dg", _gate_numel(cfg, tok), f32), _arg(dbeta, "dbeta", tok * cfg.H, f32),
                                    _arg(dS0, "dS0", nst, f32), _ptr(workspace), int(ws_bytes), _stream(stream)))


def la_recurrent_bwd_ste_noalloc(cfg: Config, q, k, v, g, beta, S0, ckpts, dout, dS_T, dq, dk, dv, dg,
                                 dbeta, dS0, stream=None) -> None:
    """la_recurrent_bwd_ste with the library's fixed device array as its workspace (no
    allocation; the workspace must fit la_noalloc_workspace_limit() bytes)."""
    lib = load_library()
    c = cfg.c()
    f32 = _f32()
    tok = cfg.B * cfg.T
    nck = (cfg.T + cfg.ckpt_interval - 1) // cfg.ckpt_interval if cfg.ckpt_interval > 0 else 0
    nst = _state_numel(cfg, cfg.B)
    args = _inputs(cfg, tok, q, k, v, g, beta)
    _check(lib.la_recurrent_bwd_ste_noalloc(ctypes.byref(c), *args, _arg(S0, "S0", nst, f32),
                                            _arg(ckpts, "ckpts", nst * nck, f32),
                                            _arg(dout, "dout", tok * cfg.H * cfg.d_v, f32),
                                            _arg(dS_T, "dS_T", nst, f32),
                                            _arg(dq, "dq", tok * cfg.H * cfg.d_k, f32),
                                            _arg(dk, "dk", tok * cfg.H * cfg.d_k, f32),
                                            _arg(dv, "dv", tok * cfg.H * cfg.d_v, f32),
                                            _arg(dg, "dg", _gate_numel(cfg, tok), f32),
                                            _arg(dbeta, "dbeta", tok * cfg.H, f32), _arg(dS0, "dS0", nst, f32),
                                            _stream(stream)))


def la_noalloc_workspace_limit() -> int:
    return int(load_library().la_noalloc_workspace_limit())


def la_fwd_kernel_name(cfg: Config) -> str:
    """Which forward kernel serves cfg: "block", "wave", "fast", "token" or "chunk" ("" if invalid)."""
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
