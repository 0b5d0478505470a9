// Recurrence core shared by the forward kernel and the backward kernel's recompute.
//
// One workgroup owns a 64-column tile of one (sequence, head) state: 4 waves, lane j holds
// value column j of the tile, wave w holds key rows [w*R, (w+1)*R), R = d_k / 4, as R FP32
// registers per lane.  Per token the key/query vectors are staged in LDS and read as
// wave-uniform broadcasts; the key-axis reductions (u = S~^T k and S~^T q) are an in-lane
// chain over the wave's rows followed by a fixed-order sum of the four waves' partials.
// Both kernels instantiate exactly these functions, so a recompute reproduces the
// forward's carried states bit for bit, including every quantization decision.
//
// The token update is written in the general form
//     S~ = diag(a) S,   u = S~^T kp,   delta = beta (v - u),   S' = S~ + ku delta^T,
//     o  = S'^T qq = S~^T qq + delta (ku . qq)
// with kp = ku = k, qq = q for the plain recurrence.  With the Hadamard rotation the state
// is carried rotated, Y = Hu S (Hu = the unnormalized Sylvester matrix, Hu Hu = d_k I), and
// since Hu commutes with the scalar gate the same update holds for Y with ku = Hu k,
// kp = Hu k / d_k and qq = Hu q / d_k.  The INT8 codec then acts on Y directly (the codes of
// Hu S' equal those of the normalized rotation; only the scale differs by sqrt(d_k)), and
// the carried state is mapped back with S = Hu Y / d_k at checkpoints and at the end.
#pragma once

#include "la_device.hpp"
#include "la_internal.hpp"

namespace la {

constexpr int kTileCols = 64;
constexpr int kThreads = 256;

struct Params {
    int B, T, H, dk, dv;
    int qkv_dt, gate_dt, out_dt;
    int qdq_interval, ckpt_interval, nck;
    int rot;  // state tensors hold the rotated state (Hadamard mode)
};

template <int DK>
struct Smem {
    // staged per-token vectors (key axis)
    float kp[DK];    // a_i * kp_i   (projection key, gate folded in)
    float qa[DK];    // a_i * qq_i   (query, gate folded in)
    float ku[DK];    // update key
    float a[DK];     // gate factors
    float kraw[DK];  // projection key without the gate (backward)
    float qraw[DK];  // query without the gate (backward)
    float beta, kq;
    float2 red[4][kTileCols];   // per-wave partial column sums
    float amax[4];
    float scal[4];
    float tile[DK * kTileCols]; // state staging for rotations
};

__device__ __forceinline__ bool is_qdq_point(int t, int T, int interval) {
    return ((t + 1) % interval == 0) || (t == T - 1);
}

// In-LDS unnormalized Walsh-Hadamard transform along the key axis of a DK x 64 tile.
// All threads of the workgroup must call it.
template <int DK>
__device__ __forceinline__ void tile_wht(float* tile) {
#pragma unroll 1
    for (int h = 1; h < DK; h <<= 1) {
        __syncthreads();
        for (int idx = threadIdx.x; idx < DK * (kTileCols / 2); idx += kThreads) {
            int c = idx & (kTileCols - 1);
            int p = idx / kTileCols;
            int i = (p / h) * 2 * h + (p % h);
            float x = tile[i * kTileCols + c];
            float y = tile[(i + h) * kTileCols + c];
            tile[i * kTileCols + c] = x + y;
            tile[(i + h) * kTileCols + c] = x - y;
        }
    }
    __syncthreads();
}

// In-LDS unnormalized Walsh-Hadamard transform of a length-DK vector (all threads call).
template <int DK>
__device__ __forceinline__ void vec_wht2(float* x, float* y) {
#pragma unroll 1
    for (int h = 1; h < DK; h <<= 1) {
        __syncthreads();
        int tid = threadIdx.x;
        if (tid < DK) {  // first DK/2 threads transform x, the next DK/2 transform y
            float* v = (tid < DK / 2) ? x : y;
            int p = tid & (DK / 2 - 1);
            int i = (p / h) * 2 * h + (p % h);
            float s0 = v[i], s1 = v[i + h];
            v[i] = s0 + s1;
            v[i + h] = s0 - s1;
        }
    }
    __syncthreads();
}

// Rotate the register state through LDS: s <- Hu s * scale (rows), all threads call.
template <int DK>
__device__ __forceinline__ void rotate_state(Smem<DK>& sm, float (&s)[DK / 4], float scale) {
    constexpr int R = DK / 4;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    __syncthreads();
#pragma unroll
    for (int m = 0; m < R; m++) sm.tile[(w * R + m) * kTileCols + lane] = s[m];
    tile_wht<DK>(sm.tile);
#pragma unroll
    for (int m = 0; m < R; m++) s[m] = sm.tile[(w * R + m) * kTileCols + lane] * scale;
    __syncthreads();
}

// Stage token `tok` (flattened (b*T + t)*H + h) into LDS.  All threads call; ends with a
// barrier so the staged values are visible.
template <int DK, bool HAD, bool KDA>
__device__ __forceinline__ void stage_token(Smem<DK>& sm, const void* q, const void* k,
                                            const void* g, const void* beta, size_t tok,
                                            int qkv_dt, int gate_dt) {
    const int tid = threadIdx.x;
    __syncthreads();  // previous users of the staging buffers are done
    float ai = 0.0f;
    if (tid < DK) {
        float kk = load_elem(k, tok * DK + tid, qkv_dt);
        float qv = load_elem(q, tok * DK + tid, qkv_dt);
        float gv = KDA ? load_elem(g, tok * DK + tid, gate_dt) : load_elem(g, tok, gate_dt);
        ai = expf(gv);
        sm.kraw[tid] = kk;
        sm.qraw[tid] = qv;
        sm.a[tid] = ai;
    }
    if (tid == 0) sm.beta = load_elem(beta, tok, gate_dt);
    if (HAD) {
        // rotate copies of k and q held in ku / qa
        __syncthreads();
        if (tid < DK) {
            sm.ku[tid] = sm.kraw[tid];
            sm.qa[tid] = sm.qraw[tid];
        }
        vec_wht2<DK>(sm.ku, sm.qa);
    }
    __syncthreads();
    if (tid < 64) {
        // kq = k . q over the key axis, fixed butterfly order
        float acc = 0.0f;
        for (int i = tid; i < DK; i += 64) acc = __builtin_fmaf(sm.kraw[i], sm.qraw[i], acc);
        acc = wave_sum(acc);
        if (tid == 0) sm.kq = acc;
    }
    __syncthreads();  // kraw/qraw are rewritten below in the rotated case
    if (tid < DK) {
        constexpr float inv = 1.0f / DK;
        if (HAD) {
            float kr = sm.ku[tid];           // Hu k
            float qr = sm.qa[tid] * inv;     // Hu q / d_k
            float kpr = kr * inv;            // Hu k / d_k
            sm.kraw[tid] = kpr;
            sm.qraw[tid] = qr;
            sm.kp[tid] = ai * kpr;
            sm.qa[tid] = ai * qr;
        } else {
            sm.ku[tid] = sm.kraw[tid];
            sm.kp[tid] = ai * sm.kraw[tid];
            sm.qa[tid] = ai * sm.qraw[tid];
        }
    }
    __syncthreads();
}

// One token: reduce, update, optionally quantize.  Returns u and delta of this lane's
// column through the references; o_out receives S'^T q for the column.
template <int DK, int QMODE, int G>
__device__ __forceinline__ void token_step(Smem<DK>& sm, float (&s)[DK / 4], float vj,
                                           bool qdq_now, float& u_out, float& d_out,
                                           float& o_out) {
    constexpr int R = DK / 4;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    float p = 0.0f, r = 0.0f;
#pragma unroll
    for (int m = 0; m < R; m++) {
        p = __builtin_fmaf(s[m], sm.kp[w * R + m], p);
        r = __builtin_fmaf(s[m], sm.qa[w * R + m], r);
    }
    sm.red[w][lane] = make_float2(p, r);
    __syncthreads();
    float2 r0 = sm.red[0][lane], r1 = sm.red[1][lane], r2 = sm.red[2][lane], r3 = sm.red[3][lane];
    float P = ((r0.x + r1.x) + r2.x) + r3.x;
    float Rq = ((r0.y + r1.y) + r2.y) + r3.y;
    float delta = sm.beta * (vj - P);
    o_out = __builtin_fmaf(delta, sm.kq, Rq);
    u_out = P;
    d_out = delta;
#pragma unroll
    for (int m = 0; m < R; m++) s[m] = __builtin_fmaf(sm.ku[w * R + m], delta, sm.a[w * R + m] * s[m]);
    if (QMODE == LA_QDQ_INT8_GROUP) {
        if (qdq_now) {
#pragma unroll
            for (int m = 0; m < R; m++) {
                float amax = group_max<G>(fabsf(s[m]));
                float sc = int8_scale(amax);
                s[m] = int8_code(s[m], sc) * sc;
            }
        }
    } else if (QMODE == LA_QDQ_E4M3_TILE) {
        if (qdq_now) {
            float mx = 0.0f;
#pragma unroll
            for (int m = 0; m < R; m++) mx = fmaxf(mx, fabsf(s[m]));
            mx = group_max<64>(mx);
            if (lane == 0) sm.amax[w] = mx;
            __syncthreads();
            float amax = fmaxf(fmaxf(sm.amax[0], sm.amax[1]), fmaxf(sm.amax[2], sm.amax[3]));
            float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
#pragma unroll
            for (int m = 0; m < R; m++) s[m] = e4m3_round(s[m] / sc) * sc;
        }
    }
    // the red/amax buffers are reused by the next token only after its staging barrier
}

}  // namespace la
