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
    // packed sequences cut in two (la_recurrent_fwd_split): split[b] is sequence b's prefix
    // length (clamped to the sequence); split_part 0 runs the prefixes, 1 the suffixes
    const int32_t* split = nullptr;
    int split_part = 0;
    // block kernel only: checkpoints in the kernels' register order (per 16-column wave slice,
    // register quad i of lane l at (i 64 + l) 16 bytes) instead of [d_k][d_v]; set by the
    // block backward for its own recompute, never seen by a caller
    int ckpt_lane_major = 0;
    // token kernel only (replay windows): bf16 bits [B][T][H][d_v] of every token's delta
    // rounded to BF16, the update entry the replay encoding uses; null = not written
    uint16_t* entries = nullptr;
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
    // replay windows of `window` tokens (la_decode_step_replay): S holds the window's
    // checkpoint; entries 0 .. pos[b] - 1 of the log are the window's earlier tokens
    const int32_t* pos = nullptr;    // [B]; null: no replay
    uint16_t* log_k = nullptr;       // [B][H][window - 1][d_k] bf16
    uint16_t* log_d = nullptr;       // [B][H][window - 1][d_v] bf16
    float* log_g = nullptr;          // [B][H][window - 1] (scalar gate) or [..][d_k] (per key)
    int window = 1;
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
    // packed sequences (la_recurrent_bwd_ste_varlen / _split), as in FwdArgs; the checkpoints
    // are then in the packed slot layout (varlen_ckpt_slots)
    const int32_t* cu_seqlens = nullptr;
    const int32_t* split = nullptr;
    int split_part = 0;
};

// Packed sequences with checkpoints: sequence b's chunks occupy slots b + begin_b / C + c
// (begin_b its first token, C the checkpoint spacing), disjoint across sequences; a head's
// slots are [H][slots][d_k][d_v].  slots = B + T / C + 1 bounds them for any packing of T.
inline int varlen_ckpt_slots(const la_config& c) {
    return c.ckpt_interval > 0 ? c.B + c.T / c.ckpt_interval + 1 : 0;
}

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
// Token backward with every token a rounding point of the INT8 codec (no replay windows, no
// rotation around the rounding points, checkpoints at most kCodedMaxChunk tokens apart, an
// even number of key rows per lane): each rounded state is its codes times its group scales,
// so the chunk's recompute keeps the codes (as fp16) and the scales of every token, and the
// adjoint decodes the states instead of recomputing the chunk a second time.
constexpr int kCodedMaxChunk = 64;
constexpr int tok_rows_per_lane(int dk, int tc) { return (dk / 8) / (64 / tc); }
inline bool bwd_tok_coded(const la_config& c) {
    const int tc = tok_tile_cols(c.d_k, c.qdq, c.group);
    return c.qdq == LA_QDQ_INT8_GROUP && c.qdq_interval == 1 && !c.replay && !(c.hadamard && c.gate == LA_GATE_KEY) &&
           c.ckpt_interval >= 1 && c.ckpt_interval <= kCodedMaxChunk && tok_rows_per_lane(c.d_k, tc) % 2 == 0;
}
// The coded walk with 32-column tiles and the scalar gate runs the adjoint of one chunk beside
// the recompute of the chunk before it, so it keeps the codes of two chunks.
inline bool bwd_tok_coded_pipe(const la_config& c) {
    return bwd_tok_coded(c) && tok_tile_cols(c.d_k, c.qdq, c.group) == 32 && c.gate != LA_GATE_KEY;
}
// Floats of one workgroup's backward states for chunks of C tokens: coded, per token the
// d_k x tc codes as fp16 and the d_k tc / g scales, for one chunk or (pipe) two; else the state
// entering every fourth token.
constexpr size_t bwd_tok_ws_floats(int C, int dk, int tc, int g, bool coded, bool pipe) {
    return coded ? (pipe ? 2 : 1) * static_cast<size_t>(C) *
                       (static_cast<size_t>(dk) * tc / 2 + static_cast<size_t>(dk) * tc / g)
                 : static_cast<size_t>((C + 3) / 4) * dk * tc;
}
inline size_t bwd_tok_ws_floats(const la_config& c) {
    return bwd_tok_ws_floats(c.ckpt_interval, c.d_k, tok_tile_cols(c.d_k, c.qdq, c.group), c.group, bwd_tok_coded(c),
                             bwd_tok_coded_pipe(c));
}

hipError_t launch_decode(const la_config& c, const DecodeArgs& a, hipStream_t s);
// The forward kernel that serves c: c.kernel if it is not LA_KERNEL_AUTO and that kernel
// serves c (else LA_KERNEL_AUTO: none), otherwise the first of block, wave, fast, token that
// does.
la_kernel fwd_kernel(const la_config& c);
hipError_t launch_fwd(const la_config& c, const FwdArgs& a, hipStream_t s);
const char* fwd_kernel_name(const la_config& c);
bool fwd_fast_eligible(const la_config& c);
hipError_t launch_fwd_fast(const la_config& c, const FwdArgs& a, hipStream_t s);
bool fwd_mfma_eligible(const la_config& c);
hipError_t launch_fwd_mfma(const la_config& c, const FwdArgs& a, hipStream_t s);
bool fwd_wave_eligible(const la_config& c);
hipError_t launch_fwd_wave(const la_config& c, const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_tok(const la_config& c, const FwdArgs& a, hipStream_t s);
// 64-token chunk path (chunk_fwd.hip): d_k = 128, no rotation, no replay, rounding points and
// checkpoints on chunk ends.  The forward prepares every chunk's matrices into `records`
// (chunk_fwd_workspace_bytes) and then runs the state pass.
constexpr int kChunkTokens = 64;
bool chunk_eligible(const la_config& c);
size_t chunk_fwd_workspace_bytes(const la_config& c);
hipError_t launch_chunk_fwd(const la_config& c, const FwdArgs& a, float* records, hipStream_t s);
// Backward of the chunk form (chunk_bwd.hip), from checkpoints every 64 tokens (ba.ckpts, or
// recomputed into the workspace's room when null).  Workspace regions, byte offsets:
struct ChunkBwdLayout {
    size_t rec, ckpts, U, D, dD, dSe, dbp, total;
};
ChunkBwdLayout chunk_bwd_layout(const la_config& c);
struct BwdArgs;
hipError_t launch_chunk_bwd(const la_config& c, const FwdArgs& fa, const BwdArgs& ba, char* ws, hipStream_t s);
hipError_t launch_copy_state(const la_config& c, const float* src, float* dst, hipStream_t s);
hipError_t launch_bwd(const la_config& c, const BwdArgs& a, hipStream_t s);
// Token range [begin, end) of packed sequence b (part of it when split is given), on the
// host side's terms: the device computes the same from cu_seqlens.
// Block forward in chunk mode (la_recur.hpp Params::chunk): from checkpoints a.S0 (spacing
// c.ckpt_interval), the state entering every 16-token block of tokens [t_off, t_end) into
// a.ckpts, lane-major, every checkpoint chunk in parallel.
hipError_t launch_fwd_mfma_chunks(const la_config& c, const FwdArgs& a, int t_off, int t_end, hipStream_t s);
// Block backward (bwd_mfma.hip), segment by segment: a segment's block-start states (chunk
// recompute from a.ckpts, or from the forward's checkpoints recomputed into ck_room) into
// a.ws_states, the block kernel writing partial records to a.ws_part, their reduction; dS is
// carried between segments in `carry` ([B][H][d_k][d_v]).  Workspace: bwd_mfma_state_bytes
// + bwd_mfma_part_bytes (one segment each) + carry + checkpoint room.
bool bwd_mfma_eligible(const la_config& c);
int bwd_mfma_segment(const la_config& c);
// The backward kernel that serves c: the chunk form when the forward runs it; else the block
// backward when eligible; else, unless c.kernel asks for the token kernel, the chunk backward
// when every rounding point and checkpoint is a chunk end (ckpt_interval = 64: the checkpoints
// then carry every rounding decision, and a missing set is recomputed by c's own forward
// kernel); else the token backward.
la_kernel bwd_kernel(const la_config& c);
size_t bwd_mfma_state_bytes(const la_config& c);
size_t bwd_mfma_part_bytes(const la_config& c);
hipError_t launch_bwd_mfma(const la_config& c, const FwdArgs& fa, const BwdArgs& a, float* carry, float* ck_room,
                           hipStream_t s);

// The straight-through backward behind both backward entry points: host checks, workspace
// layout, launches.  With provide == nullptr the caller's workspace (ws_bytes) is used; else,
// after every host check and the size check against ws_bytes, provide() supplies the
// workspace (the allocation-free entry point's device array).
// Prefix and suffix configurations of la_recurrent_fwd_split / la_recurrent_bwd_ste_split.
la_status check_split(const la_config* prefix, const la_config* suffix);
// The packed-sequence backward (all sequences, or one part of each with split): checkpoints
// recomputed into the workspace, then the token backward and the reduction.
la_status bwd_varlen(const la_config& c, const int32_t* cu_seqlens, const int32_t* split, int part, const void* q,
                     const void* k, const void* v, const void* g, const void* beta, const float* S0,
                     const float* dout, const float* dS_T, float* dq, float* dk, float* dv, float* dg,
                     float* dbeta, float* dS0, void* workspace, size_t ws_bytes, void* stream);
using WorkspaceProvider = hipError_t (*)(void** workspace);
la_status bwd_ste(const la_config* cfg, const void* q, const void* k, const void* v, const void* g,
                  const void* beta, const float* S0, const float* ckpts, const float* dout,
                  const float* dS_T, float* dq, float* dk, float* dv, float* dg, float* dbeta,
                  float* dS0, void* workspace, size_t ws_bytes, WorkspaceProvider provide, void* stream);

}  // namespace la
