// Launch parameters shared by the scalar-gate long-sequence kernels (fwd_fast.hip,
// fwd_wave.hip, fwd_mfma.hip): one workgroup per (sequence, head, 64-column value tile).
#pragma once

#include "la_device.hpp"
#include "la_internal.hpp"

namespace la {

constexpr int kTileCols = 64;

struct Params {
    int B, T, H, dk, dv;
    int qkv_dt, gate_dt, out_dt;
    int qdq_interval, ckpt_interval, nck;
    int rot;  // state tensors hold the rotated state (Hadamard mode)
    // Block kernel (scalar gate) only: chunk-parallel recompute for the block backward.  With
    // chunk > 0 the grid's z runs over B x nch chunks of `chunk` tokens of the token range
    // [t_off, t_end) of every sequence (stride_T tokens long); each chunk starts from S0 read
    // as checkpoint t_start / chunk of [B][H][nck_in] (the forward's own checkpoints: no
    // rounding point lies inside a chunk), rounds nowhere, and writes the state entering each
    // of its 16-token blocks at block (t_start - t_off) / 16 of [B][H][nck] (lane-major).
    int chunk = 0, nch = 0, t_off = 0, t_end = 0, stride_T = 0, nck_in = 0;
};

}  // namespace la
