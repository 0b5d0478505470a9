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
// are chosen so that the A-operand reads of 16 rows x 4 k-indices hit 64 distinct banks.  Each
// record is two parts in the order the pass consumes them (part 1 is free once its first
// products are done, part 2 at the chunk's end), so that the next chunk's parts can be loaded
// into LDS while the current one is still being used.
// Forward: part 1 Kp, Qp [token][132]; part 2 P, M [64][68], Kd transposed [key][68], E_L [128],
// beta [64] (widened to fp32; zero past the sequence's end).
struct RecF {
    static constexpr int PP = 68, PK = 132, PD = 68;
    static constexpr int KP = 0, QP = KP + kCh * PK, PART2 = QP + kCh * PK;
    static constexpr int P = PART2, M = P + kCh * PP, KDT = M + kCh * PP, EL = KDT + kChDk * PD, BT = EL + kChDk,
                         SIZE = BT + kCh;
};
// Backward: the state gradient pass reads P and M transposed and Kp, Qp, Kd by token rows:
// part 1 Kd [token][132], M [64][80]; part 2 P [64][80], Qp, Kp [token][144], E_L [128], beta
// [64]; then A [64][68] for the gradient kernel.
struct RecB {
    static constexpr int PP = 80, PK = 144, PKD = 132, PA = 68;
    static constexpr int KD = 0, M = KD + kCh * PKD, PART2 = M + kCh * PP;
    static constexpr int P = PART2, QP = P + kCh * PP, KP = QP + kCh * PK, EL = KP + kCh * PK, BT = EL + kChDk;
    static constexpr int LDS_SIZE = BT + kCh, A = LDS_SIZE, SIZE = A + kCh * PA;
};
static_assert(RecF::SIZE % 64 == 0 && RecB::SIZE % 64 == 0 && RecB::LDS_SIZE % 4 == 0, "record alignment");
static_assert(RecF::PART2 % 4 == 0 && RecB::PART2 % 4 == 0 && RecB::BT % 4 == 0,
              "record parts and the beta row start on 16-byte boundaries");

typedef __attribute__((address_space(3))) void lds_void_t;

// Start an asynchronous copy of n floats (a multiple of four, 16-byte aligned) from global
// memory into LDS with direct-to-LDS loads: 16 bytes per lane, one kilobyte per wave
// instruction, wave w taking kilobytes w, w + 4, ...  Complete after s_waitcnt vmcnt(0) in
// every wave and a barrier.
__device__ __forceinline__ void lds_dma(float* dst, const float* __restrict__ src, int n) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int full = n >> 8;
    for (int i = w; i < full; i += 4)
        __builtin_amdgcn_global_load_lds(src + (i << 8) + 4 * lane, (lds_void_t*)(dst + (i << 8)), 16,
                                         0, 0);
    const int rem = n & 255;
    if (rem && w == (full & 3) && 4 * lane < rem)
        __builtin_amdgcn_global_load_lds(src + (full << 8) + 4 * lane, (lds_void_t*)(dst + (full << 8)),
                                         16, 0, 0);
}

// lds_dma issued a piece at a time, so that the copy's instructions can sit between other work
// (a wave that issues the whole copy at once waits for the vector memory queue to take each
// instruction): piece j of wave w moves 256-float block w + 4 j, the partial block at the end
// with the piece that reaches it.  Pieces 0 .. lds_dma_pieces(n) - 1 together move what
// lds_dma(dst, src, n) moves.
constexpr int lds_dma_pieces(int n) { return (n >> 10) + 1; }
__device__ __forceinline__ void lds_dma_piece(float* dst, const float* __restrict__ src, int n, int j) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int full = n >> 8, i = w + 4 * j, rem = n & 255;
    if (i < full)
        __builtin_amdgcn_global_load_lds(src + (i << 8) + 4 * lane, (lds_void_t*)(dst + (i << 8)), 16, 0, 0);
    else if (i == full && rem && 4 * lane < rem)
        __builtin_amdgcn_global_load_lds(src + (full << 8) + 4 * lane, (lds_void_t*)(dst + (full << 8)), 16, 0, 0);
}

// Rows 0 .. 63 of a [token][128] bf16 or fp32 input (token r at element (tok0 + r H) 128) in
// 16-byte pieces: thread t of NT holds pieces t + NT u of the chunk (1024 pieces for bf16, 2048
// for fp32; piece pc is row pc / P, bytes 16 (pc % P) of it, P = 16 or 32 pieces per row).  rows_load
// only issues loads (a row past the end reads row 0), so the pieces of several arrays can all
// be in flight together; rows_store widens them into LDS dst[r * 132 + k], rows L .. 63 zero.
template <int NT = kChThreads>
struct Rows {
    uint4 x[2048 / NT];
};
template <int NT>
__device__ __forceinline__ void rows_load(Rows<NT>& R, const void* src, size_t tok0, int H, int L, int dtype) {
    constexpr int NU = 2048 / NT;  // pieces per thread for fp32 (half of them for bf16)
    const bool f32 = dtype == LA_F32;
    const int sh = f32 ? 5 : 4, nu = f32 ? NU : NU / 2;
    const size_t esz = f32 ? 4 : 2;
    const char* base = static_cast<const char*>(src) + tok0 * kChDk * esz;
    const size_t rstride = static_cast<size_t>(H) * kChDk * esz;
#pragma unroll
    for (int u = 0; u < NU; u++) {
        if (u < nu) {
            const int pc = threadIdx.x + NT * u, r = pc >> sh, o = pc & ((1 << sh) - 1);
            R.x[u] = *reinterpret_cast<const uint4*>(base + static_cast<size_t>(r < L ? r : 0) * rstride + 16 * o);
        }
    }
}
template <int NT>
__device__ __forceinline__ void rows_store(float* dst, const Rows<NT>& R, int L, int dtype) {
    constexpr int NU = 2048 / NT;
    if (dtype == LA_F32) {
#pragma unroll
        for (int u = 0; u < NU; u++) {
            const int pc = threadIdx.x + NT * u, r = pc >> 5, o = pc & 31;
            const uint32_t m = r < L ? 0xFFFFFFFFu : 0u;
            const uint4 x = R.x[u];
            *reinterpret_cast<float4*>(dst + r * 132 + 4 * o) = make_float4(
                __uint_as_float(x.x & m), __uint_as_float(x.y & m), __uint_as_float(x.z & m), __uint_as_float(x.w & m));
        }
    } else {
#pragma unroll
        for (int u = 0; u < NU / 2; u++) {
            const int pc = threadIdx.x + NT * u, r = pc >> 4, o = pc & 15;
            const uint32_t m = r < L ? 0xFFFFFFFFu : 0u;
            const uint32_t w[4] = {R.x[u].x & m, R.x[u].y & m, R.x[u].z & m, R.x[u].w & m};
            float4* d = reinterpret_cast<float4*>(dst + r * 132 + 8 * o);
            d[0] = make_float4(__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xFFFF0000u),
                               __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xFFFF0000u));
            d[1] = make_float4(__uint_as_float(w[2] << 16), __uint_as_float(w[2] & 0xFFFF0000u),
                               __uint_as_float(w[3] << 16), __uint_as_float(w[3] & 0xFFFF0000u));
        }
    }
}

// Inclusive prefix sum over the 64 lanes of a wave (lane l holds x), in six shift-and-add steps.
template <typename F>
__device__ __forceinline__ F wave_prefix_sum(F x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const F y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    return x;
}

// Cumulative log decays of a chunk, in float: per key G[r * 132 + key] in place (rows past the
// end hold zero gates), one thread per key; for a scalar gate the 64 lanes of one wave, lane r
// holding row r's gate.  Late in a chunk under steep decay these are large numbers whose
// differences keep an absolute error of about |G| 2^-24 per step (rounding once from a double
// sum does not help: the two rounded ends of a difference then err independently).
__device__ __forceinline__ void cumsum_cols(float* G, int key) {
    float run = 0.0f;
    for (int r = 0; r < kCh; r++) {
        run += G[r * 132 + key];
        G[r * 132 + key] = run;
    }
}
__device__ __forceinline__ float cumsum_lanes(float g) { return wave_prefix_sum(g); }

// Whether a chunk's per-key cumulative log decays G (LDS, [token][132], rows past the end
// repeating row L - 1) allow every decay e^{G_r - G_i} to be factored as e^{G_r - ref}
// e^{ref - G_i} with no factor overflowing or underflowing: off-diagonal 16-token blocks take
// ref = G at the end of the earlier block, so both factors are decays unless a gate is positive
// (then the chunk's range must stay within 80); a diagonal block takes ref = G at its eighth
// token, so every G of the block must lie within 80 of it.  Every thread of the workgroup
// calls it (it synchronises); one thread per key does the scan.
__device__ __forceinline__ bool chunk_factorable(const float* G, int L, int* flag) {
    if (threadIdx.x == 0) *flag = 0;
    __syncthreads();
    if (threadIdx.x < kChDk) {
        const int key = threadIdx.x;
        float gmin = 0.0f, gmax = 0.0f, prev = 0.0f, spread = 0.0f;
        bool pos = false;
        for (int r = 0; r < L; r++) {
            const float x = G[r * 132 + key];
            pos = pos || x > prev;
            prev = x;
            gmin = fminf(gmin, x);
            gmax = fmaxf(gmax, x);
            spread = fmaxf(spread, fabsf(x - G[((r & ~15) + 7) * 132 + key]));
        }
        if ((pos && gmax - gmin > 80.0f) || !(spread <= 80.0f)) atomicOr(flag, 1);
    }
    __syncthreads();
    return *flag == 0;
}

// Rows kmap(i, g) of a chunk of a row-major array, addressed by buffer instructions with 32-bit
// offsets: the lane part (g stride + col) esz bytes in a VGPR, the register part
// (16 (i / 4) + 4 (i % 4)) stride esz bytes in an SGPR, over a resource of `bytes` bytes from
// `base` (reads past it return zero, stores there are dropped).  The 64-bit products of general
// pointer arithmetic (several quarter-rate instructions per element) are left out.
struct ChunkRows {
    __amdgpu_buffer_rsrc_t rs;
    int voff, step;
    __device__ __forceinline__ int soff(int i) const { return (16 * (i >> 2) + 4 * (i & 3)) * step; }
    __device__ __forceinline__ uint32_t ld32(int i) const { return __builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff(i), 0); }
    __device__ __forceinline__ uint32_t ld16(int i) const { return __builtin_amdgcn_raw_buffer_load_b16(rs, voff, soff(i), 0); }
    __device__ __forceinline__ void st32(int i, uint32_t x) const { __builtin_amdgcn_raw_buffer_store_b32(x, rs, voff, soff(i), 0); }
    __device__ __forceinline__ void st16(int i, uint16_t x) const { __builtin_amdgcn_raw_buffer_store_b16(x, rs, voff, soff(i), 0); }
    __device__ __forceinline__ float ldf(int i) const { return __uint_as_float(ld32(i)); }
    __device__ __forceinline__ void stf(int i, float x) const { st32(i, __float_as_uint(x)); }
};
__device__ __forceinline__ ChunkRows chunk_rows(const void* base, size_t bytes, int stride, int g, int col, int esz) {
    return ChunkRows{make_rsrc(base, bytes), (g * stride + col) * esz, stride * esz};
}

// x, or zero when !ok, component by component (a select between whole vectors can leave
// them in private memory).
__device__ __forceinline__ float4 keep_if(bool ok, float4 x) {
    return make_float4(ok ? x.x : 0.0f, ok ? x.y : 0.0f, ok ? x.z : 0.0f, ok ? x.w : 0.0f);
}

// N elements idx(0) .. idx(N-1) of a bf16 or fp32 array as raw bits (bf16 zero-extended),
// the dtype switch outside the loads.  Nothing here reads a loaded value, so all N loads are
// in flight together; a conversion or a select on each value right after its load would make
// every load wait for those before it (and for any other memory operation still in flight).
// raw_f32 turns the bits into the float where the value is used.
template <int N, typename Idx>
__device__ __forceinline__ void load_raw(uint32_t (&r)[N], const void* p, int dtype, Idx idx) {
    if (dtype == LA_F32) {
        const uint32_t* s = static_cast<const uint32_t*>(p);
#pragma unroll
        for (int i = 0; i < N; i++) r[i] = s[idx(i)];
    } else {
        const uint16_t* s = static_cast<const uint16_t*>(p);
#pragma unroll
        for (int i = 0; i < N; i++) r[i] = s[idx(i)];
    }
}
__device__ __forceinline__ float raw_f32(uint32_t r, int dtype) { return __uint_as_float(dtype == LA_F32 ? r : r << 16); }

// Wait until every memory operation this wave issued has completed.
__device__ __forceinline__ void wait_all_mem() { __builtin_amdgcn_s_waitcnt(0); }

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
__device__ __forceinline__ float opaque_f(float x) {
    asm volatile("" : "+v"(x));
    return x;
}

// e^x to about two ulp for the chunk form's decays, in under ten instructions: x log2(e) as the
// rounded product t plus its rounding error (exact by an FMA, the TwoProduct of Ogita, Rump and
// Oishi) and that of the constant itself, then 2^t by the hardware (v_exp_f32) corrected to
// first order, 2^t (1 + e ln 2).  Below the normal range 2^t is taken as 2^(t + 64) 2^-64, so
// that subnormal results are rounded once (the hardware exponential flushes them); the
// arguments here stay below +88, where 2^t does not overflow.
__device__ __forceinline__ float exp_acc(float x) {
    constexpr float kL2E = 1.44269502162933349609375f;  // log2(e) rounded to float
    constexpr float kL2Elo = 1.925963033500011e-08f;    // log2(e) - kL2E
    constexpr float kLn2 = 0.693147180559945309f;
    const float t = x * kL2E;
    const float e = __builtin_fmaf(x, kL2Elo, __builtin_fmaf(x, kL2E, -t));
    const bool sub = t < -126.0f;
    const float r = __builtin_amdgcn_exp2f(sub ? t + 64.0f : t);
    const float y = __builtin_fmaf(r, e * kLn2, r);
    return sub ? y * 5.42101086242752217e-20f : y;  // 2^-64
}

__device__ __forceinline__ f4 mfma4(float a, float b, f4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

constexpr int kPW = 68;  // pitch of the 64 x 64 work matrices in LDS

// C = op(A) op(B) (+ Cadd) for 64 x 64 fp32 matrices in LDS (pitch kPW) on the matrix cores,
// op = transpose when TA / TB, by a workgroup of NW = 4 or 8 waves: wave w forms rows
// 16 (w % 4) .. + 15 and, of those, column tiles (w / 4) (4 / (NW / 4)) onwards.  The barrier
// between the products and the stores lets C alias A, B or Cadd.  Every thread of the workgroup
// must call it.
template <bool TA, bool TB, int NW = 4>
__device__ void mm64(const float* A, const float* B, float* C, const float* Cadd) {
    constexpr int NCT = 16 / NW;  // column tiles per wave
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
    const int rw = w & 3, ct0 = (w >> 2) * NCT;
    f4 acc[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ct++)
#pragma unroll
        for (int r = 0; r < 4; r++) acc[ct][r] = Cadd ? Cadd[(16 * rw + 4 * g + r) * kPW + 16 * (ct0 + ct) + c] : 0.0f;
#pragma unroll 4
    for (int s = 0; s < 16; s++) {
        const float a = TA ? A[(4 * s + g) * kPW + 16 * rw + c] : A[(16 * rw + c) * kPW + 4 * s + g];
#pragma unroll
        for (int ct = 0; ct < NCT; ct++) {
            const int col = 16 * (ct0 + ct);
            const float b = TB ? B[(col + c) * kPW + 4 * s + g] : B[(4 * s + g) * kPW + col + c];
            acc[ct] = mfma4(a, b, acc[ct]);
        }
    }
    __syncthreads();
#pragma unroll
    for (int ct = 0; ct < NCT; ct++)
#pragma unroll
        for (int r = 0; r < 4; r++) C[(16 * rw + 4 * g + r) * kPW + 16 * (ct0 + ct) + c] = acc[ct][r];
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
