// The 64-token chunk path ("GDN state/W QAT foundation", What does this PR do?: 64-token
// chunks with the state rounded at chunk boundaries; "Experimental GDN/KDA approximate-inverse
// QAT", What does this PR do?: the chunk's exact triangular solve or an explicit Neumann
// polynomial in its place).  For a chunk of L tokens entering with the state S, cumulative
// per-key log decays G_r (a scalar gate is the same value on every key):
//
//   A_ri = beta_r sum_k k_r[k] k_i[k] e^{G_r[k] - G_i[k]}  (i < r)      P = (I + A)^-1 or
//   M_ri = sum_k q_r[k] k_i[k] e^{G_r[k] - G_i[k]}         (i <= r)         sum_{n<=d} (-A)^n
//   Delta = P diag(beta) (V - Kp S),  O = Qp S + M Delta,  S_end = diag(E_L) S + Kd^T Delta
//
// with Kp = k e^{G_r}, Qp = q e^{G_r}, Kd = k e^{G_{L-1} - G_r}, E_L = e^{G_{L-1}}.  Everything
// but S is known before the state arrives: a chunk-parallel prep kernel forms A, M, P, Kp, Qp,
// Kd and E_L for every chunk into a record in device memory; the state pass then walks the
// chunks of one (sequence, head, 64 value columns) with the fp32 matrix cores.
//
// State pass layout.  Four waves, wave w owns value columns 16 w .. 16 w + 15; lane (g, c) =
// lane 16 g + c holds column c.  Its 32 state registers hold keys kmap(m, g) =
// 16 (m / 4) + 4 (m % 4) + g (m = 0 .. 31), so that register m is the B operand of k-step m of a
// 16x16x4 fp32 MFMA contracting over keys; token vectors (V, beta, Delta, ...) use the same map
// over tokens (register 4 rt + r = token 16 rt + 4 r + g).  A-operand rows are taken in the
// order cmap(blk, c) = 16 blk + 4 (c % 4) + c / 4, which makes every MFMA result land in those
// same maps (output row 4 g + r of tile blk is cmap(blk, 4 g + r) = kmap(4 blk + r, g)).
#pragma once

#include "la_device.hpp"
#include "la_internal.hpp"
#include "la_mfma.hpp"
#include "la_wave.hpp"

namespace la {

constexpr int kCh = 64;          // tokens per chunk
constexpr int kChThreads = 256;  // four waves
constexpr int kChDk = 128;       // keys (the chunk path's d_k)

struct ChunkParams {
    int B, T, H, dv, nch, ntile;  // nch chunks per sequence, ntile = dv / 64
    int qkv_dt, gate_dt, out_dt;
    int qdq_interval, ckpt_interval, nck;
    int degree;                   // Neumann degree (2^m - 1), 0 = exact solve
};

struct ChunkIn {
    const void* q;
    const void* k;
    const void* v;
    const void* g;
    const void* beta;
};

// Record of one (sequence, head, chunk), fp32, in the state pass's LDS layout.  Row pitches
// are chosen so that the A-operand reads of 16 rows x 4 k-indices hit 64 distinct banks.
// Forward: P, M [64][68]; Kp, Qp [token][132]; Kd transposed [key][68]; E_L [128].
struct RecF {
    static constexpr int PP = 68, PK = 132, PD = 68;
    static constexpr int P = 0, M = P + kCh * PP, KP = M + kCh * PP, QP = KP + kCh * PK, KDT = QP + kCh * PK;
    static constexpr int EL = KDT + kChDk * PD, SIZE = EL + kChDk;
};
// Backward: the state gradient pass reads P and M transposed and Kp, Qp, Kd by token rows:
// P, M [64][80]; Kp, Qp [token][144]; Kd [token][132]; E_L [128] (the pass's LDS prefix), then
// A [64][68] for the gradient kernel.
struct RecB {
    static constexpr int PP = 80, PK = 144, PKD = 132, PA = 68;
    static constexpr int P = 0, M = P + kCh * PP, KP = M + kCh * PP, QP = KP + kCh * PK, KD = QP + kCh * PK;
    static constexpr int EL = KD + kCh * PKD, LDS_SIZE = EL + kChDk, A = LDS_SIZE, SIZE = A + kCh * PA;
};
static_assert(RecF::SIZE % 64 == 0 && RecB::SIZE % 64 == 0 && RecB::LDS_SIZE % 4 == 0, "record alignment");

__device__ __forceinline__ int cmap(int blk, int x) { return 16 * blk + 4 * (x & 3) + (x >> 2); }
__device__ __forceinline__ int kmap(int m, int g) { return 16 * (m >> 2) + 4 * (m & 3) + g; }

// Compiler-only fence (no instruction): loads are not moved across it, which bounds how many
// LDS operands of an unrolled product loop the scheduler hoists (and keeps live) at once.
__device__ __forceinline__ void sched_fence() { asm volatile("" ::: "memory"); }

// The same value, opaque to the compiler: lane indices passed through it at the top of a loop
// body keep the addresses derived from them inside the body.  Otherwise every LDS address of
// the unrolled products, being loop-invariant, is hoisted out of the chunk loop and held in
// registers for its whole length.
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

__device__ __forceinline__ f4 mfma4(float a, float b, f4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

constexpr int kPW = 68;  // pitch of the 64 x 64 work matrices in LDS

// C = op(A) op(B) (+ Cadd) for 64 x 64 fp32 matrices in LDS (pitch kPW) on the matrix cores,
// op = transpose when TA / TB; wave w forms rows 16 w .. 16 w + 15.  The barrier between the
// products and the stores lets C alias A, B or Cadd.  Every thread of the workgroup must call it.
template <bool TA, bool TB>
__device__ void mm64(const float* A, const float* B, float* C, const float* Cadd) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
    f4 acc[4];
#pragma unroll
    for (int ct = 0; ct < 4; ct++)
#pragma unroll
        for (int r = 0; r < 4; r++) acc[ct][r] = Cadd ? Cadd[(16 * w + 4 * g + r) * kPW + 16 * ct + c] : 0.0f;
#pragma unroll 4
    for (int s = 0; s < 16; s++) {
        const float a = TA ? A[(4 * s + g) * kPW + 16 * w + c] : A[(16 * w + c) * kPW + 4 * s + g];
#pragma unroll
        for (int ct = 0; ct < 4; ct++) {
            const float b = TB ? B[(16 * ct + c) * kPW + 4 * s + g] : B[(4 * s + g) * kPW + 16 * ct + c];
            acc[ct] = mfma4(a, b, acc[ct]);
        }
    }
    __syncthreads();
#pragma unroll
    for (int ct = 0; ct < 4; ct++)
#pragma unroll
        for (int r = 0; r < 4; r++) C[(16 * w + 4 * g + r) * kPW + 16 * ct + c] = acc[ct][r];
    __syncthreads();
}

// Copy n floats (a multiple of four, 16-byte aligned) from global memory into LDS.
__device__ __forceinline__ void copy_to_lds(float* dst, const float* __restrict__ src, int n) {
    const float4* s4 = reinterpret_cast<const float4*>(src);
    float4* d4 = reinterpret_cast<float4*>(dst);
#pragma unroll 4
    for (int i = threadIdx.x; i < n / 4; i += kChThreads) d4[i] = s4[i];
}

// Workgroup -> (value tile, sequence-head): the tiles of one sequence-head get block ids that
// are equal modulo 8, so they run on one XCD and share its L2 copy of the chunk records.
__device__ __forceinline__ void chunk_tile_of(int id, int ntile, int& tile, int& bh) {
    const int grp = id / (8 * ntile), rem = id - grp * 8 * ntile;
    tile = rem >> 3;
    bh = grp * 8 + (rem & 7);
}
inline unsigned chunk_tile_blocks(int bh, int ntile) { return static_cast<unsigned>((bh + 7) / 8 * 8 * ntile); }

}  // namespace la
