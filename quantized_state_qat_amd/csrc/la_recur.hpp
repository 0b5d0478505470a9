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
};

}  // namespace la
