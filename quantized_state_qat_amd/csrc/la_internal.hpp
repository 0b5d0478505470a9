// Internal launch interface between the C ABI (la_api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/la.h"

namespace la {

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* g;
    const void* beta;
    const float* S0;
    void* o;        // may be null (backward recompute)
    float* ST;      // may be null
    float* ckpts;   // may be null
    // packed sequences (token kernel only): sequence b is tokens cu_seqlens[b] .. [b + 1] of
    // a [T][H][...] layout; null = the batched [B][T][H][...] layout
    const int32_t* cu_seqlens = nullptr;
    // block kernel only: checkpoints in the kernels' register order (lane-major: each lane's
    // 32 state values contiguous, per 16-column wave slice) instead of [d_k][d_v]; set by the
    // block backward for its own recompute, never seen by a caller
    int ckpt_lane_major = 0;
};

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* g;
    const void* beta;
    float* S;
    void* o;
    void* codes;    // may be null
    float* scales;  // may be null
    const int32_t* slots = nullptr;  // null: entry b is state b; else the state slot of entry b
    int n_slots = 0;                 // slots outside [1, n_slots) are padding
};

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* g;
    const void* beta;
    const float* ckpts;  // checkpoints every cfg.ckpt_interval tokens
    const float* dout;
    const float* dST;    // may be null
    float* dq;
    float* dk;
    float* dv;
    float* dg;
    float* dbeta;
    float* dS0;
    float* ws_states;    // per workgroup: the state entering every 4th token of a chunk (d_k x tile columns)
    float* ws_part;      // per value tile and token: partial row sums
};

// Host-side layout helpers (shared by the ABI and the launchers).
inline int n_value_blocks(const la_config& c) { return c.d_v / 64; }
// Value columns per workgroup of the token forward and the backward: 32 when every rounding
// group fits in 32 columns (no quantizer, or INT8 groups of 16 or 32) and d_k >= 32, else 64.
constexpr int tok_tile_cols(int dk, int qdq, int group) {
    return (dk >= 32 && (qdq == LA_QDQ_NONE || (qdq == LA_QDQ_INT8_GROUP && group <= 32))) ? 32 : 64;
}
inline int tok_tiles(const la_config& c) { return c.d_v / tok_tile_cols(c.d_k, c.qdq, c.group); }
inline int n_ckpts(const la_config& c) {
    return c.ckpt_interval > 0 ? (c.T + c.ckpt_interval - 1) / c.ckpt_interval : 0;
}
// Backward partial sums per (value tile, token): two d_k rows, the gate term (KDA: one per
// key row; GDN: one per wave of the eight-wave token layout) and beta.
inline int part_width(const la_config& c) { return 2 * c.d_k + (c.gate == LA_GATE_KEY ? c.d_k : 8) + 1; }
// Backward states per workgroup: the state entering every fourth token of a chunk.
inline int n_sub_states(const la_config& c) { return (c.ckpt_interval + 3) / 4; }

hipError_t launch_decode(const la_config& c, const DecodeArgs& a, hipStream_t s);
hipError_t launch_fwd(const la_config& c, const FwdArgs& a, hipStream_t s);
const char* fwd_kernel_name(const la_config& c);
bool fwd_fast_eligible(const la_config& c);
hipError_t launch_fwd_fast(const la_config& c, const FwdArgs& a, hipStream_t s);
bool fwd_mfma_eligible(const la_config& c);
hipError_t launch_fwd_mfma(const la_config& c, const FwdArgs& a, hipStream_t s);
bool fwd_wave_eligible(const la_config& c);
hipError_t launch_fwd_wave(const la_config& c, const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_tok(const la_config& c, const FwdArgs& a, hipStream_t s);
hipError_t launch_copy_state(const la_config& c, const float* src, float* dst, hipStream_t s);
hipError_t launch_bwd(const la_config& c, const BwdArgs& a, hipStream_t s);
// Block backward (bwd_mfma.hip): the block forward with a checkpoint every 16 tokens into
// a.ws_states (fa.ckpts), the block kernel writing partial records to a.ws_part, then their
// reduction.  Workspace: bwd_mfma_state_bytes + bwd_mfma_part_bytes.
bool bwd_mfma_eligible(const la_config& c);
size_t bwd_mfma_state_bytes(const la_config& c);
size_t bwd_mfma_part_bytes(const la_config& c);
hipError_t launch_bwd_mfma(const la_config& c, const FwdArgs& fa, const BwdArgs& a, hipStream_t s);

}  // namespace la
