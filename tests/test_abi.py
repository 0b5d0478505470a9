"""The C ABI library on the host (no GPU needed): it loads, exports every entry point that
include/la.h declares, and rejects invalid calls on the host before any HIP call."""
import ctypes
import os
import re

import pytest

import quantized_state_qat_amd as la

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # a 16-byte aligned address that is never dereferenced: every call below is
                # rejected (or has no work) before the library touches device memory


def header_functions():
    text = open(os.path.join(ROOT, "include", "la.h")).read()
    return sorted(set(re.findall(r"^\s*(?:la_status|size_t|const char\*)\s+(la_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_function():
    lib = la.load_library()
    names = header_functions()
    assert set(names) == {"la_recurrent_fwd", "la_recurrent_fwd_varlen", "la_decode_step", "la_decode_step_slots",
                          "la_recurrent_bwd_ste", "la_bwd_workspace_bytes", "la_fwd_kernel_name", "la_bwd_kernel_name",
                          "la_status_string", "la_last_error", "la_recurrent_bwd_ste_noalloc",
                          "la_noalloc_workspace_limit", "la_recurrent_fwd_entries", "la_decode_step_replay",
                          "la_recurrent_fwd_split", "la_recurrent_bwd_ste_varlen", "la_bwd_varlen_workspace_bytes",
                          "la_recurrent_bwd_ste_split", "la_bwd_split_workspace_bytes", "la_recurrent_fwd_chunk",
                          "la_chunk_workspace_bytes"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    assert la.la_status_string(la.LA_OK) == "ok"
    assert la.la_status_string(la.LA_ERR_UNSUPPORTED) == "unsupported configuration"
    assert la.la_status_string(99) == "unknown status"


def cfg(**kw):
    base = dict(B=2, T=8, H=2, d_k=128, d_v=128, qdq=la.LA_QDQ_INT8_GROUP, group=32, ckpt_interval=4)
    base.update(kw)
    return la.Config(**base)


def fwd(c, **ptrs):
    p = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, S0=None, o=FAKE, S_T=None, ckpts=None)
    p.update(ptrs)
    return la.la_recurrent_fwd(c, p["q"], p["k"], p["v"], p["g"], p["beta"], p["S0"], p["o"],
                               p["S_T"], p["ckpts"], stream=0)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(d_k=96), la.LA_ERR_UNSUPPORTED, "d_k"),
    (dict(d_k=256), la.LA_ERR_UNSUPPORTED, "d_k"),
    (dict(d_v=96), la.LA_ERR_UNSUPPORTED, "d_v"),
    (dict(group=8), la.LA_ERR_UNSUPPORTED, "group"),
    (dict(qdq=la.LA_QDQ_E4M3_TILE, group=32), la.LA_ERR_UNSUPPORTED, "E4M3"),
    (dict(hadamard=1, gate=la.LA_GATE_KEY, state_rotated=1), la.LA_ERR_UNSUPPORTED, "state_rotated"),
    (dict(hadamard=1, qdq=la.LA_QDQ_NONE), la.LA_ERR_INVALID_ARG, "hadamard"),
    (dict(qdq_interval=0), la.LA_ERR_INVALID_ARG, "qdq_interval"),
    (dict(qdq=7), la.LA_ERR_INVALID_ARG, "qdq"),
    (dict(gate=3), la.LA_ERR_INVALID_ARG, "gate"),
    (dict(qkv_dtype=5), la.LA_ERR_INVALID_ARG, "dtype"),
    (dict(T=-1), la.LA_ERR_INVALID_ARG, "size"),
    (dict(B=70000), la.LA_ERR_UNSUPPORTED, "65535"),
    (dict(state_rotated=1), la.LA_ERR_INVALID_ARG, "state_rotated"),
    (dict(state_rotated=2, hadamard=1), la.LA_ERR_INVALID_ARG, "state_rotated"),
])
def test_fwd_rejects_invalid_config(kw, status, msg):
    with pytest.raises(la.LaError) as e:
        fwd(cfg(**kw))
    assert e.value.status == status
    assert msg in str(e.value)


def test_fwd_rejects_null_and_misaligned_pointers():
    with pytest.raises(la.LaError) as e:
        fwd(cfg(), q=None)
    assert e.value.status == la.LA_ERR_INVALID_ARG and "q is NULL" in str(e.value)
    with pytest.raises(la.LaError) as e:
        fwd(cfg(), v=FAKE + 4)
    assert e.value.status == la.LA_ERR_ALIGNMENT and "v" in str(e.value)
    with pytest.raises(la.LaError) as e:
        fwd(cfg(ckpt_interval=0), ckpts=FAKE)
    assert e.value.status == la.LA_ERR_INVALID_ARG


def test_null_cfg():
    lib = la.load_library()
    assert lib.la_recurrent_fwd(None, *([None] * 10)) == la.LA_ERR_INVALID_ARG
    assert b"cfg is NULL" in lib.la_last_error()
    assert lib.la_bwd_workspace_bytes(None) == 0


def test_empty_batch_is_a_no_op():
    fwd(cfg(B=0), q=None, k=None, v=None, g=None, beta=None, o=None)
    la.la_decode_step(cfg(T=1, H=0), None, None, None, None, None, None, None, stream=0)
    assert la.la_last_error() == ""


def test_decode_checks():
    with pytest.raises(la.LaError) as e:
        la.la_decode_step(cfg(T=2), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert "T == 1" in str(e.value)
    with pytest.raises(la.LaError) as e:
        la.la_decode_step(cfg(T=1, qdq=la.LA_QDQ_NONE), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                          codes=FAKE, stream=0)
    assert e.value.status == la.LA_ERR_INVALID_ARG


def test_decode_slots_checks():
    c = cfg(T=1)
    with pytest.raises(la.LaError) as e:
        la.la_decode_step_slots(c, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, stream=0)
    assert "n_slots" in str(e.value)
    with pytest.raises(la.LaError) as e:
        la.la_decode_step_slots(c, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 4, FAKE, stream=0)
    assert "slots" in str(e.value)
    with pytest.raises(la.LaError) as e:
        la.la_decode_step_slots(cfg(T=2), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, stream=0)
    assert "T == 1" in str(e.value)
    la.la_decode_step_slots(cfg(T=1, B=0), None, None, None, None, None, None, None, 1, None, stream=0)
    assert la.la_last_error() == ""


def test_bwd_workspace_and_checks():
    c = cfg(T=256, ckpt_interval=64)
    n = la.la_bwd_workspace_bytes(c)
    # INT8 groups of 32 after every token: the backward's tiles are 32 value columns wide (4 per
    # head).  Per workgroup (B x H x tiles) and chunk token the rounded state as fp16 codes and
    # one scale per (row, group), for two chunks (the adjoint of one runs beside the recompute
    # of the next); per tile and token the partial sums (two d_k rows, eight GDN gate terms,
    # beta); room for recomputed checkpoints
    nwg = 2 * 2 * 4
    states = nwg * 2 * 64 * (128 * 32 * 2 + 128 * 4)
    part = 4 * 2 * 256 * 2 * (2 * 128 + 8 + 1) * 4
    ck = 2 * 2 * 4 * 128 * 128 * 4
    assert n >= states + part + ck and n < states + part + ck + 3 * 256
    # rounding every second token: the state entering every fourth token of a chunk
    c2 = cfg(T=256, ckpt_interval=64, qdq_interval=2)
    n2 = la.la_bwd_workspace_bytes(c2)
    states2 = nwg * (64 // 4) * 128 * 32 * 4
    assert n2 >= states2 + part + ck and n2 < states2 + part + ck + 3 * 256
    c64 = cfg(T=256, ckpt_interval=64, group=64)   # groups of 64: tiles of 64 columns
    n64 = la.la_bwd_workspace_bytes(c64)
    states64 = 2 * 2 * 2 * 64 * (128 * 64 * 2 + 128 * 4)
    part64 = 2 * 2 * 256 * 2 * (2 * 128 + 8 + 1) * 4
    assert n64 >= states64 + part64 + ck and n64 < states64 + part64 + ck + 3 * 256
    assert la.la_bwd_workspace_bytes(cfg(ckpt_interval=0)) == 0
    args = [FAKE] * 5 + [None, None, FAKE, None] + [FAKE] * 6
    with pytest.raises(la.LaError) as e:
        la.la_recurrent_bwd_ste(c, *args, FAKE, n - 1, stream=0)
    assert e.value.status == la.LA_ERR_WORKSPACE
    with pytest.raises(la.LaError) as e:
        la.la_recurrent_bwd_ste(cfg(ckpt_interval=0), *args, FAKE, n, stream=0)
    assert "ckpt_interval" in str(e.value)


@pytest.mark.parametrize("kw,name", [
    (dict(qdq=la.LA_QDQ_E4M3_TILE, group=64, qdq_interval=64, ckpt_interval=64), "block"),
    (dict(qdq=la.LA_QDQ_INT8_GROUP, group=16, qdq_interval=16, ckpt_interval=16), "block"),
    (dict(qdq=la.LA_QDQ_NONE, ckpt_interval=0), "block"),
    (dict(qdq=la.LA_QDQ_E4M3_TILE, group=64, qdq_interval=64, ckpt_interval=8), "wave"),
    (dict(qdq=la.LA_QDQ_E4M3_TILE, group=64, qdq_interval=64, ckpt_interval=64, d_k=64), "wave"),
    (dict(qdq=la.LA_QDQ_INT8_GROUP, group=64, qdq_interval=8, ckpt_interval=8), "wave"),
    (dict(qdq=la.LA_QDQ_INT8_GROUP, group=32, qdq_interval=64, ckpt_interval=64, qkv_dtype=la.LA_F32), "wave"),
    (dict(qdq=la.LA_QDQ_INT8_GROUP, group=16, qdq_interval=3, ckpt_interval=3), "fast"),
    (dict(qdq=la.LA_QDQ_INT8_GROUP, group=32, qdq_interval=12, ckpt_interval=0), "fast"),
    (dict(qdq=la.LA_QDQ_INT8_GROUP, group=32, qdq_interval=1, ckpt_interval=0), "token"),
    (dict(qdq=la.LA_QDQ_INT8_GROUP, group=32, qdq_interval=64, ckpt_interval=64, hadamard=1), "token"),
    (dict(qdq=la.LA_QDQ_INT8_GROUP, group=32, qdq_interval=64, ckpt_interval=64, hadamard=1,
          gate=la.LA_GATE_KEY), "token"),
    (dict(qdq=la.LA_QDQ_E4M3_TILE, group=64, qdq_interval=64, ckpt_interval=64, gate=la.LA_GATE_KEY), "block"),
    (dict(qdq=la.LA_QDQ_E4M3_TILE, group=64, qdq_interval=24, ckpt_interval=24, gate=la.LA_GATE_KEY), "wave"),
    (dict(qdq=la.LA_QDQ_NONE, ckpt_interval=8, gate=la.LA_GATE_KEY, qkv_dtype=la.LA_F32), "wave"),
    (dict(qdq=la.LA_QDQ_INT8_GROUP, group=64, qdq_interval=1, ckpt_interval=64, gate=la.LA_GATE_KEY), "token"),
    (dict(qdq=la.LA_QDQ_INT8_GROUP, group=64, qdq_interval=12, ckpt_interval=12, gate=la.LA_GATE_KEY), "token"),
    (dict(qdq=la.LA_QDQ_INT8_GROUP, group=64, qdq_interval=64, ckpt_interval=12, gate=la.LA_GATE_KEY), "token"),
    (dict(qdq=la.LA_QDQ_INT8_GROUP, group=32, qdq_interval=64, ckpt_interval=16), "block"),
    (dict(qdq=la.LA_QDQ_INT8_GROUP, group=32, qdq_interval=64, ckpt_interval=4), "fast"),
])
def test_fwd_kernel_selection(kw, name):
    """Which forward kernel serves a configuration (host-side selection, documented in la.h)."""
    base = dict(B=2, T=100, H=2, d_k=128, d_v=128)
    base.update(kw)
    assert la.la_fwd_kernel_name(la.Config(**base)) == name


@pytest.mark.parametrize("kw,name", [
    (dict(qdq=la.LA_QDQ_E4M3_TILE, group=64, qdq_interval=64, ckpt_interval=64), "block"),
    (dict(qdq=la.LA_QDQ_NONE, ckpt_interval=64, gate_dtype=la.LA_BF16), "block"),
    # the forward of this configuration runs the per-token kernel (a rounding point falls
    # inside a 5-token checkpoint chunk), so the backward recomputes with it as well
    (dict(qdq=la.LA_QDQ_INT8_GROUP, group=32, qdq_interval=16, ckpt_interval=5), "token"),
    # rounding every 32 tokens inside 64-token checkpoint chunks: the per-token forward
    (dict(qdq=la.LA_QDQ_INT8_GROUP, group=16, qdq_interval=32, ckpt_interval=64, d_v=192), "token"),
    (dict(qdq=la.LA_QDQ_INT8_GROUP, group=16, qdq_interval=64, ckpt_interval=32, d_v=192), "block"),
    (dict(qdq=la.LA_QDQ_INT8_GROUP, group=32, qdq_interval=1, ckpt_interval=64), "token"),
    (dict(qdq=la.LA_QDQ_INT8_GROUP, group=32, qdq_interval=24, ckpt_interval=24), "token"),
    (dict(qdq=la.LA_QDQ_INT8_GROUP, group=32, qdq_interval=64, ckpt_interval=64, hadamard=1), "token"),
    (dict(qdq=la.LA_QDQ_E4M3_TILE, group=64, qdq_interval=64, ckpt_interval=64, gate=la.LA_GATE_KEY), "chunk"),
    (dict(qdq=la.LA_QDQ_E4M3_TILE, group=64, qdq_interval=64, ckpt_interval=64, qkv_dtype=la.LA_F32), "chunk"),
    (dict(qdq=la.LA_QDQ_E4M3_TILE, group=64, qdq_interval=64, ckpt_interval=32, gate=la.LA_GATE_KEY), "token"),
    (dict(qdq=la.LA_QDQ_INT8_GROUP, group=64, qdq_interval=1, ckpt_interval=64, gate=la.LA_GATE_KEY), "token"),
    (dict(qdq=la.LA_QDQ_INT8_GROUP, group=64, qdq_interval=128, ckpt_interval=64, gate=la.LA_GATE_KEY), "chunk"),
    (dict(ckpt_interval=64, gate=la.LA_GATE_KEY), "chunk"),
    (dict(qdq=la.LA_QDQ_E4M3_TILE, group=64, qdq_interval=64, ckpt_interval=64, gate=la.LA_GATE_KEY,
          kernel=la.LA_KERNEL_TOKEN), "token"),
    (dict(qdq=la.LA_QDQ_E4M3_TILE, group=64, qdq_interval=64, ckpt_interval=64, d_k=64), "token"),
    (dict(qdq=la.LA_QDQ_INT8_GROUP, group=64, qdq_interval=48, ckpt_interval=16, d_v=64), "block"),
])
def test_bwd_kernel_selection(kw, name):
    """Which backward serves a configuration: the block form needs the block forward's
    configurations (the user's checkpoint spacing aside: it recomputes every block's state)
    and whole 64-column workgroups; the chunk form serves the rest whose rounding points and
    checkpoints all fall on 64-token chunk ends (d_k = 128, no rotation), unless the token
    kernel is asked for; the token backward serves everything else."""
    base = dict(B=2, T=100, H=2, d_k=128, d_v=128)
    base.update(kw)
    assert la.la_bwd_kernel_name(la.Config(**base)) == name


def test_bwd_block_workspace():
    """Block backward workspace, for one segment of the sequence (here the whole sequence,
    rounded up to the checkpoint spacing: 128 tokens, 8 blocks): the state entering every
    16-token block (fp32 d_k x d_v per unit and block), one partial record of 4672 floats per
    unit, block and 64-column slice (two 16 x 128 key/query sums, two 16 x 16 Gram-term
    matrices, three 16-token vectors, padded), dS carried between segments, and room for the
    forward's checkpoints."""
    c = la.Config(B=3, T=100, H=2, d_k=128, d_v=192, qdq=la.LA_QDQ_E4M3_TILE, group=64, qdq_interval=64,
                  ckpt_interval=64)
    assert la.la_bwd_kernel_name(c) == "block"
    nb = 8
    states = 3 * 2 * nb * 128 * 192 * 4
    part = 3 * 2 * nb * 3 * 4672 * 4
    carry = 3 * 2 * 128 * 192 * 4
    ckpts = 3 * 2 * 2 * 128 * 192 * 4
    n = la.la_bwd_workspace_bytes(c)
    assert n >= states + part + carry + ckpts and n < states + part + carry + ckpts + 4 * 256


def test_bwd_block_workspace_long_sequence_under_1gb():
    """The long-sequence workload's backward walks segments of 512 tokens: its workspace stays
    below 1 GB (with room for the forward's checkpoints)."""
    c = la.Config(B=8, T=4096, H=16, d_k=128, d_v=128, qdq=la.LA_QDQ_E4M3_TILE, group=64, qdq_interval=64,
                  ckpt_interval=64, gate_dtype=la.LA_F32)
    assert la.la_bwd_kernel_name(c) == "block"
    assert la.la_bwd_workspace_bytes(c) < 10 ** 9


def test_fwd_kernel_name_invalid():
    assert la.la_fwd_kernel_name(la.Config(B=1, T=4, H=1, d_k=100, d_v=128)) == ""


def test_one_hip_runtime_per_process():
    """Loading the library before anything imports torch must still leave one HIP runtime
    in the process (two runtimes cannot share devices, pointers or streams)."""
    import subprocess
    import sys
    prog = ("import quantized_state_qat_amd as la; la.load_library(); import torch; "
            "paths = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}; "
            "print(len(paths), sorted(paths))")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, "-c", prog], cwd=root, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.split()[0] == "1", out.stdout


@pytest.mark.parametrize("kernel,kw,name", [
    (la.LA_KERNEL_WAVE, dict(qdq=la.LA_QDQ_E4M3_TILE, group=64, qdq_interval=64, ckpt_interval=64), "wave"),
    (la.LA_KERNEL_FAST, dict(qdq=la.LA_QDQ_E4M3_TILE, group=64, qdq_interval=64, ckpt_interval=64), "fast"),
    (la.LA_KERNEL_TOKEN, dict(qdq=la.LA_QDQ_E4M3_TILE, group=64, qdq_interval=64, ckpt_interval=64), "token"),
    (la.LA_KERNEL_BLOCK, dict(qdq=la.LA_QDQ_E4M3_TILE, group=64, qdq_interval=64, ckpt_interval=64), "block"),
    (la.LA_KERNEL_TOKEN, dict(qdq=la.LA_QDQ_INT8_GROUP, group=32, qdq_interval=1, hadamard=1), "token"),
    (la.LA_KERNEL_BLOCK, dict(qdq=la.LA_QDQ_INT8_GROUP, group=32, qdq_interval=1), ""),
    (la.LA_KERNEL_WAVE, dict(qdq=la.LA_QDQ_INT8_GROUP, group=32, qdq_interval=12), ""),
    (la.LA_KERNEL_FAST, dict(gate=la.LA_GATE_KEY, qdq=la.LA_QDQ_INT8_GROUP, group=32, qdq_interval=16), ""),
])
def test_forced_kernel(kernel, kw, name):
    """A requested forward kernel serves the configuration or is reported unsupported."""
    base = dict(B=2, T=100, H=2, d_k=128, d_v=128, kernel=kernel)
    base.update(kw)
    c = la.Config(**base)
    assert la.la_fwd_kernel_name(c) == name
    if name == "":
        assert "cannot serve" in la.la_last_error()
        with pytest.raises(la.LaError) as ei:
            fwd(c)
        assert ei.value.status == la.LA_ERR_UNSUPPORTED
        assert la.la_bwd_workspace_bytes(c) == 0
    elif name == "token":
        assert la.la_bwd_kernel_name(c) == "token"
    elif name != "block":
        # the block backward needs the block forward's rounding decisions; with every rounding
        # point on a checkpoint the chunk backward needs none
        assert la.la_bwd_kernel_name(c) == "chunk"


def test_kernel_field_checks():
    with pytest.raises(la.LaError) as ei:
        fwd(cfg(kernel=9))
    assert ei.value.status == la.LA_ERR_INVALID_ARG
    with pytest.raises(la.LaError) as ei:
        la.la_decode_step(cfg(T=1, kernel=la.LA_KERNEL_TOKEN), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert ei.value.status == la.LA_ERR_INVALID_ARG
    with pytest.raises(la.LaError) as ei:
        la.la_recurrent_fwd_varlen(cfg(kernel=la.LA_KERNEL_BLOCK), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                   stream=0)
    assert ei.value.status == la.LA_ERR_UNSUPPORTED


class FakeDeviceTensor:
    """Stands in for a GPU tensor in the binding's host-side checks; its address is never
    dereferenced because every call below is rejected before the library is called."""

    def __init__(self, numel, dtype):
        self._n, self.dtype, self.is_cuda = numel, dtype, True

    def numel(self):
        return self._n

    def element_size(self):
        return 4

    def is_contiguous(self):
        return True

    def data_ptr(self):
        return FAKE


def test_binding_rejects_bad_tensors():
    import torch
    c = cfg(qkv_dtype=la.LA_BF16, gate_dtype=la.LA_BF16)
    n_qk = c.B * c.T * c.H * c.d_k
    good = dict(q=FakeDeviceTensor(n_qk, torch.bfloat16), k=FakeDeviceTensor(n_qk, torch.bfloat16),
                v=FakeDeviceTensor(n_qk, torch.bfloat16), g=FakeDeviceTensor(c.B * c.T * c.H, torch.bfloat16),
                beta=FakeDeviceTensor(c.B * c.T * c.H, torch.bfloat16), o=FakeDeviceTensor(n_qk, torch.float32))
    # a host tensor
    with pytest.raises(ValueError, match="GPU tensor"):
        fwd(c, **{**good, "q": torch.zeros(n_qk, dtype=torch.bfloat16)})
    # wrong dtype
    with pytest.raises(ValueError, match="dtype"):
        fwd(c, **{**good, "k": FakeDeviceTensor(n_qk, torch.float32)})
    # too few elements
    with pytest.raises(ValueError, match="elements"):
        fwd(c, **{**good, "v": FakeDeviceTensor(n_qk - 1, torch.bfloat16)})
    with pytest.raises(ValueError, match="elements"):
        fwd(c, **{**good, "S0": FakeDeviceTensor(c.B * c.H * c.d_k * c.d_v - 1, torch.float32)})
    with pytest.raises(ValueError, match="dtype"):
        la.la_decode_step(cfg(T=1), good["q"], good["k"], good["v"], good["g"], good["beta"],
                          FakeDeviceTensor(c.B * c.H * c.d_k * c.d_v, torch.bfloat16), good["o"], stream=0)
    with pytest.raises(ValueError, match="int32"):
        la.la_decode_step_slots(cfg(T=1), good["q"], good["k"], good["v"], good["g"], good["beta"],
                                FakeDeviceTensor(3 * c.H * c.d_k * c.d_v, torch.float32),
                                FakeDeviceTensor(c.B, torch.int64), 3, good["o"], stream=0)


CHUNK_OK = dict(qdq=la.LA_QDQ_E4M3_TILE, group=64, qdq_interval=64, ckpt_interval=64)


def chunk_fwd(c, ws=FAKE, ws_bytes=1 << 40):
    return la.la_recurrent_fwd_chunk(c, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None, ws, ws_bytes, stream=0)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(solve=1, degree=5), la.LA_ERR_INVALID_ARG, "Neumann degree"),
    (dict(solve=1, degree=63), la.LA_ERR_INVALID_ARG, "Neumann degree"),
    (dict(solve=0, degree=3), la.LA_ERR_INVALID_ARG, "degree"),
    (dict(solve=2), la.LA_ERR_INVALID_ARG, "solve"),
])
def test_solve_field_checks(kw, status, msg):
    base = dict(CHUNK_OK)
    base.update(kw)
    with pytest.raises(la.LaError) as e:
        chunk_fwd(cfg(**base))
    assert e.value.status == status and msg in str(e.value)


def test_chunk_kernel_selection_and_workspace():
    for solve, degree, kernel in ((la.LA_SOLVE_NEUMANN, 7, la.LA_KERNEL_AUTO), (la.LA_SOLVE_EXACT, 0, la.LA_KERNEL_CHUNK)):
        c = cfg(T=150, solve=solve, degree=degree, kernel=kernel, **CHUNK_OK)
        assert la.la_fwd_kernel_name(c) == "chunk"
        # one forward record per chunk: Kp, Qp [64][132]; P, M [64][68]; Kd^T [128][68]; E_L [128];
        # beta [64] (fp32)
        rec = 2 * 64 * 132 + 2 * 64 * 68 + 128 * 68 + 128 + 64
        assert la.la_chunk_workspace_bytes(c) == c.B * c.H * 3 * rec * 4
        # the plain forward has no workspace argument: the chunk kernel is refused there
        with pytest.raises(la.LaError) as e:
            fwd(c)
        assert e.value.status == la.LA_ERR_UNSUPPORTED and "la_recurrent_fwd_chunk" in str(e.value)
        with pytest.raises(la.LaError) as e:
            chunk_fwd(c, ws=None, ws_bytes=0)
        assert e.value.status == la.LA_ERR_WORKSPACE
        with pytest.raises(la.LaError) as e:
            chunk_fwd(c, ws_bytes=la.la_chunk_workspace_bytes(c) - 1)
        assert e.value.status == la.LA_ERR_WORKSPACE
    # the exact solve with automatic choice never picks the chunk kernel
    c = cfg(T=150, **CHUNK_OK)
    assert la.la_fwd_kernel_name(c) != "chunk" and la.la_chunk_workspace_bytes(c) == 0


@pytest.mark.parametrize("kw", [
    dict(d_k=64), dict(qdq_interval=32), dict(ckpt_interval=16), dict(qdq=la.LA_QDQ_INT8_GROUP, group=32, hadamard=1),
    dict(qdq=la.LA_QDQ_INT8_GROUP, group=32, replay=1),
])
def test_chunk_kernel_cannot_serve(kw):
    base = dict(CHUNK_OK)
    base.update(kw)
    c = cfg(T=150, solve=la.LA_SOLVE_NEUMANN, degree=3, **base)
    assert la.la_fwd_kernel_name(c) == ""
    assert la.la_chunk_workspace_bytes(c) == 0
    with pytest.raises(la.LaError) as e:
        chunk_fwd(c)
    assert e.value.status == la.LA_ERR_UNSUPPORTED


def test_token_only_entries_refuse_the_neumann_solve():
    c = cfg(T=1, solve=la.LA_SOLVE_NEUMANN, degree=3, **CHUNK_OK)
    with pytest.raises(la.LaError) as e:
        la.la_decode_step(c, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert e.value.status == la.LA_ERR_INVALID_ARG
    c = cfg(T=150, solve=la.LA_SOLVE_NEUMANN, degree=3, **CHUNK_OK)
    with pytest.raises(la.LaError) as e:
        la.la_recurrent_fwd_varlen(c, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, stream=0)
    assert e.value.status == la.LA_ERR_UNSUPPORTED
    assert la.la_bwd_varlen_workspace_bytes(c) == 0
