// Straight-through backward on the matrix cores, for the configurations the block forward
// serves: scalar gate, no rotation, d_k = 128, bf16 keys, queries and values, every rounding
// point on a 16-token block end.
//
// Three launches.  (1) The block forward (fwd_mfma.hip) with a checkpoint every 16 tokens
// into the workspace: the state entering every block, rounding points included, written in
// the kernels' register order (each lane's 32 values contiguous).  (2) This
// file's block kernel walks the blocks last to first with dS = dL/dS carried in registers.
// (3) A reduction finishes the key, query and gate gradients.  The quantizer passes the
// gradient through unchanged, so a block's adjoint is that of the exact recurrence.
//
// Block algebra (16 tokens, local index j; G_j the inclusive sum of the log gates inside the
// block, gamma_j = exp(G_j), rho_j = exp(G_15 - G_j), r_ji = exp(G_j - G_i) for i <= j: every
// factor is the decay the recurrence itself applies between two tokens, so no range guard):
//   A_ji = r_ji k_j . k_i (i < j),  C_ji = r_ji q_j . k_i (i <= j),  N = (I + diag(beta) A)^-1
//   W = V - diag(gamma) K S_0,  Delta = N diag(beta) W          (Delta_j = the token's delta)
//   O = diag(gamma) Q S_0 + C Delta,  S_16 = gamma_15 S_0 + sum_i rho_i k_i delta_i^T.
// Adjoint, given dO and dS' = dL/dS_16:
//   dDelta = C^T dO + diag(rho) K dS',  lambda = N^T dDelta,  dv = beta lambda,  dU = -dv
//   dbeta_j = lambda_j . (W - A Delta)_j,  dA_ji = -beta_j lambda_j . delta_i,  dC_ji = dO_j . delta_i
//   dS_0 = gamma_15 dS' + Q^T diag(gamma) dO + K^T diag(gamma) dU
//   dk = diag(gamma) dU S_0^T + diag(rho) Delta dS'^T + (Ab + Ab^T) K + Cb^T Q,  Ab = dA o r, Cb = dC o r
//   dq = diag(gamma) dO S_0^T + Cb K
//   dG_j = (gamma U)_j . dU_j - rho_j (K dS')_j . delta_j + rowsum_j(E) - colsum_j(E) + q_j . (dq_j from S_0)
//          + [j = 15] (gamma_15 <dS', S_0> + sum_i rho_i (K dS')_i . delta_i),   E = dA o A + dC o C
//   dg_l = sum_{j >= l} dG_j  (G_j sums the gates of tokens <= j).
// Per wave (16 value columns; lane 16 g + c): the state slices in the forward's layout
// (state_row), 16 x 16 token matrices in the accumulator layout of the 16x16 MFMAs ("D": lane
// (g, c) holds rows 4 g .. 4 g + 3 of column c) or transposed ("T": lane (g, c) holds row c,
// columns 4 g .. 4 g + 3).  Products over the 128 key rows use bf16 MFMAs of the raw keys and
// queries (exact) with the other operand split exactly into three bf16 parts; products over 16
// tokens or 16 columns use fp32 MFMAs (16x16x4).  The key/query sums over value columns are
// formed per workgroup (each wave reads the other waves' rows from LDS and takes 32 key rows),
// the small per-token sums are added across the four waves in LDS; the reduction kernel adds
// the workgroups of a head in a fixed order and applies the Gram-matrix terms once per head.
#include "la_device.hpp"
#include "la_internal.hpp"
#include "la_mfma.hpp"
#include "la_wave.hpp"

namespace la {

namespace {

constexpr int kBwWaves = 4;                   // column waves: 64 value columns per workgroup
constexpr int kBwThreads = (kBwWaves + 1) * 64;  // and one producer wave
constexpr int kBwDK = 128;
constexpr int kDppRowShr = 0x110;  // row_shr:n = kDppRowShr + n

// Partial record of one (sequence, head, block, 64-column slice), in floats.
constexpr int kRecDk = 0;      // [16 tokens][128 rows]: diag(gamma) dU S_0^T + diag(rho) Delta dS'^T
constexpr int kRecDq = 2048;   // [16][128]: diag(gamma) dO S_0^T
constexpr int kRecA = 4096;    // [16][16]: Ab
constexpr int kRecC = 4352;    // [16][16]: Cb
constexpr int kRecGr = 4608;   // [16]: dG terms collected by token row
constexpr int kRecGc = 4624;   // [16]: dG terms collected by token column
constexpr int kRecB = 4640;    // [16]: dbeta
constexpr int kRec = 4672;     // record stride (256-byte multiple)

// One segment [t_off, t_off + T) of sequences stride_T tokens long; nb = its 16-token blocks.
struct BwParams {
    int T, H, dv, nb;
    int stride_T, t_off;
};

// Per column wave LDS (16-byte aligned for the 16-byte accesses).
struct alignas(16) BwShared {
    float SdS[2][kBwDK][16];     // S_0 and dS' by [row][column]
    float small[5][64][4];       // small partial sums for the cross-wave reduction
    float XD[kBlk][20];          // Delta by [token][column]
    float XL[kBlk][20];          // lambda by [token][column]
    float XO[kBlk][16];          // dO by [token][column]
};
// One block's state-independent data, written by the producer wave one block ahead.  The
// 16 x 16 token matrices are stored so that lane (g, c) reads its four values (rows 4 g .. 4 g + 3
// of column c) as one 16-byte word at [c][4 g].
struct alignas(16) BwSlot {
    uint16_t kN[kBlk][kKeyRow];  // keys [token][row] (projection operands, transposed update reads)
    uint16_t qN[kBlk][kKeyRow];  // queries
    float RR[kBlk][kBlk];        // [c][j] = r_{j c} (0 for c > j)
    float A4[kBlk][kBlk];        // [c][j] = A_{j c}
    float C4[kBlk][kBlk];        // [c][j] = C_{j c}
    float AT[kBlk][kBlk];        // [c][j] = A_{c j}
    float Ns[kBlk][20];          // [c][j] = N_{j c}
    float G[kBlk], beta[kBlk];   // G_j and beta_j (0 past the end)
    float GAM[kBlk], RHO[kBlk];  // exp(G_j), exp(G_15 - G_j)
};
// The producer's own staging for the solve.
struct alignas(16) BwProd {
    float AmT[kBlk][20];  // [i][j] = A_ji
    float dd[4][kBlk][4]; // stage values of tokens 4 g + r, [g][column][r]
};

// Inclusive prefix sum over each row of 16 lanes.
__device__ __forceinline__ float row_prefix_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kDppRowShr + 1, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kDppRowShr + 2, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kDppRowShr + 4, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kDppRowShr + 8, 0xF, 0xF, false));
    return x;
}

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
}

__device__ __forceinline__ f4 mfma4(float a, float b, f4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

// Slice st of a product over key rows: lane (g, c) register r += sum over rows
// state_row(8 st .. 8 st + 7, g') of key_{4g+r}[row] x[row][c], with the keys of token c as
// loaded (kv[st] = those rows) and x in the state layout, x in three exact bf16 parts.
__device__ __forceinline__ f4 project_slice(f4 acc, const float (&x)[32], const u4 (&kv)[4], int st) {
    uint32_t hh[4], ll[4], l2[4];
#pragma unroll
    for (int i = 0; i < 4; i++) split3_pair(x[8 * st + 2 * i], x[8 * st + 2 * i + 1], hh[i], ll[i], l2[i]);
    const bf8 ak = __builtin_bit_cast(bf8, kv[st]);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, __builtin_bit_cast(bf8, u4{l2[0], l2[1], l2[2], l2[3]}), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, __builtin_bit_cast(bf8, u4{ll[0], ll[1], ll[2], ll[3]}), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, __builtin_bit_cast(bf8, u4{hh[0], hh[1], hh[2], hh[3]}), acc, 0, 0, 0);
    return acc;
}

}  // namespace

template <bool GF32>
__global__ __launch_bounds__(kBwThreads) void bwd_mfma_kernel(BwParams p, BwdArgs a) {
    constexpr int DK = kBwDK, R = 32;
    constexpr int GB = GF32 ? 4 : 2;
    __shared__ BwShared shw[kBwWaves];
    __shared__ BwSlot slots[2];
    __shared__ BwProd prod;

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, c = lane & 15;
    const int h = blockIdx.y, b = blockIdx.z;
    const int T = p.T, H = p.H, DV = p.dv, nb = p.nb;
    const int nwg = gridDim.x;
    const size_t bh = static_cast<size_t>(b) * H + h;
    const size_t seq0 = (static_cast<size_t>(b) * p.stride_T + p.t_off) * H;  // the segment's first token
    const size_t seq_tok = static_cast<size_t>(T) * H;

    // buffer resources over exactly this sequence's tokens (offsets < 2^31, checked on the host):
    // reads past its last token return zero, stores there are dropped
    const auto rk = make_rsrc(static_cast<const char*>(a.k) + seq0 * DK * 2, seq_tok * DK * 2);
    const auto rq = make_rsrc(static_cast<const char*>(a.q) + seq0 * DK * 2, seq_tok * DK * 2);

    if (w == kBwWaves) {
        // ------------------------------------------------------------ producer
        // Block blk - 1 (the next in walking order) while the column waves run block blk, its
        // loads one block further ahead (block 0 again at the end: no branch in the loop).
        const auto rgt = make_rsrc(static_cast<const char*>(a.g) + seq0 * GB, seq_tok * GB);
        const auto rbt = make_rsrc(static_cast<const char*>(a.beta) + seq0 * GB, seq_tok * GB);
        const int voff_kq = (c * H * DK + 8 * g) * 2;  // token c, rows 32 i + 8 g .. + 7 (load i)
        const int voff_gate = c * H * GB;
        struct ProdIn {
            u4 k[4], q[4];
            uint32_t g, b;
        };
        auto pfetch = [&](ProdIn& in, int blk) __attribute__((always_inline)) {
            const int t0 = blk * kBlk;
            const int so_kq = (t0 * H + h) * DK * 2;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                in.k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, voff_kq + 64 * i, so_kq, 0);
                in.q[i] = __builtin_amdgcn_raw_buffer_load_b128(rq, voff_kq + 64 * i, so_kq, 0);
            }
            const int so_g = (t0 * H + h) * GB;
            if (GF32) {
                in.g = __builtin_amdgcn_raw_buffer_load_b32(rgt, voff_gate, so_g, 0);
                in.b = __builtin_amdgcn_raw_buffer_load_b32(rbt, voff_gate, so_g, 0);
            } else {
                in.g = __builtin_amdgcn_raw_buffer_load_b16(rgt, voff_gate, so_g, 0);
                in.b = __builtin_amdgcn_raw_buffer_load_b16(rbt, voff_gate, so_g, 0);
            }
        };
        auto produce = [&](const ProdIn& in, int blk, BwSlot& sl) __attribute__((always_inline)) {
            const int t0 = blk * kBlk;
            // gk (lane (g, c), register r) = k_{4g+r} . k_c, gqk = q_{4g+r} . k_c
            f4 gk = {0.0f, 0.0f, 0.0f, 0.0f}, gqk = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const bf8 ak = __builtin_bit_cast(bf8, in.k[i]), aq = __builtin_bit_cast(bf8, in.q[i]);
                gk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, ak, gk, 0, 0, 0);
                gqk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, ak, gqk, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; i++) {
                *reinterpret_cast<u4*>(&sl.kN[c][32 * i + 8 * g]) = in.k[i];
                *reinterpret_cast<u4*>(&sl.qN[c][32 * i + 8 * g]) = in.q[i];
            }
            // lane (g, c): token t0 + c; tokens past the end take gate 0 and beta 0
            const bool valid = t0 + c < T;
            const float gv = valid ? (GF32 ? __uint_as_float(in.g) : bf_lo(in.g)) : 0.0f;
            const float bv = valid ? (GF32 ? __uint_as_float(in.b) : bf_lo(in.b)) : 0.0f;
            const float Gc = row_prefix_sum(gv);  // G_c
            const float G15 = lane_of(Gc, kBlk - 1);
            if (g == 0) {
                sl.G[c] = Gc;
                sl.beta[c] = bv;
                sl.GAM[c] = expf(Gc);
                sl.RHO[c] = expf(G15 - Gc);
            }
            wave_lds_sync();
            const f4 G4 = *reinterpret_cast<const f4*>(&sl.G[4 * g]);
            const f4 b4 = *reinterpret_cast<const f4*>(&sl.beta[4 * g]);
            f4 Rr, a4, c4, aT4;
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int j = 4 * g + r;
                Rr[r] = c <= j ? expf(c <= j ? G4[r] - Gc : 0.0f) : 0.0f;     // r_{j c}
                const float rt = j < c ? expf(j < c ? Gc - G4[r] : 0.0f) : 0.0f;  // r_{c j}
                a4[r] = c < j ? Rr[r] * gk[r] : 0.0f;   // A_{j c}
                c4[r] = Rr[r] * gqk[r];                 // C_{j c}
                aT4[r] = rt * gk[r];                    // A_{c j}
            }
            *reinterpret_cast<f4*>(&sl.RR[c][4 * g]) = Rr;
            *reinterpret_cast<f4*>(&sl.A4[c][4 * g]) = a4;
            *reinterpret_cast<f4*>(&sl.C4[c][4 * g]) = c4;
            *reinterpret_cast<f4*>(&sl.AT[c][4 * g]) = aT4;
            // N = (I + diag(beta) A)^-1: lane (g, c) solves column c for tokens 4 g .. 4 g + 3 in
            // four stages; after stage st, lane group st's values are final and one MFMA adds
            // their contribution to later tokens
            *reinterpret_cast<f4*>(&prod.AmT[c][4 * g]) = a4;  // AmT[i][j] = A_ji
            wave_lds_sync();
            const float c10 = prod.AmT[4 * g][4 * g + 1], c20 = prod.AmT[4 * g][4 * g + 2];
            const float c21 = prod.AmT[4 * g + 1][4 * g + 2], c30 = prod.AmT[4 * g][4 * g + 3];
            const float c31 = prod.AmT[4 * g + 1][4 * g + 3], c32 = prod.AmT[4 * g + 2][4 * g + 3];
            f4 dm = {0.0f, 0.0f, 0.0f, 0.0f}, nsel = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int st = 0; st < 4; st++) {
                const float e0 = 4 * g == c ? 1.0f : 0.0f, e1 = 4 * g + 1 == c ? 1.0f : 0.0f;
                const float e2 = 4 * g + 2 == c ? 1.0f : 0.0f, e3 = 4 * g + 3 == c ? 1.0f : 0.0f;
                const float x0 = e0 - b4[0] * dm[0];
                const float x1 = e1 - b4[1] * (dm[1] + c10 * x0);
                const float x2 = e2 - b4[2] * (dm[2] + c20 * x0 + c21 * x1);
                const float x3 = e3 - b4[3] * (dm[3] + c30 * x0 + c31 * x1 + c32 * x2);
                if (g == st) nsel = f4{x0, x1, x2, x3};
                if (st < 3) {
                    *reinterpret_cast<f4*>(&prod.dd[g][c][0]) = f4{x0, x1, x2, x3};
                    wave_lds_sync();
                    // A: lane (kk, j) = A_{j, 4 st + kk} for tokens j of later groups; B: N_{4 st + kk, c}
                    const float ast = c >= 4 * st + 4 ? prod.AmT[4 * st + g][c] : 0.0f;
                    dm = mfma4(ast, prod.dd[st][c][g], dm);
                    wave_lds_sync();
                }
            }
            *reinterpret_cast<f4*>(&sl.Ns[c][4 * g]) = nsel;  // Ns[c][j] = N_jc
        };

        ProdIn cur, nxt;
        pfetch(cur, nb - 1);
        pfetch(nxt, nb > 1 ? nb - 2 : 0);
        produce(cur, nb - 1, slots[(nb - 1) & 1]);
        cur = nxt;
        __syncthreads();  // the last block's slot is ready
#pragma unroll 1
        for (int blk = nb - 1; blk >= 0; blk--) {
            pfetch(nxt, blk > 1 ? blk - 2 : 0);
            if (blk > 0) produce(cur, blk - 1, slots[(blk - 1) & 1]);
            __syncthreads();  // the column waves' first barrier of the block
            __syncthreads();  // and their second: the slots change hands
            cur = nxt;
        }
        return;
    }

    // ---------------------------------------------------------------- column waves
    const int cw0 = blockIdx.x * 64 + w * 16;  // this wave's first value column
    const int col = cw0 + c;
    BwShared& sh = shw[w];
    const auto rv = make_rsrc(static_cast<const char*>(a.v) + seq0 * DV * 2, seq_tok * DV * 2);
    const auto rdo = make_rsrc(a.dout + seq0 * DV, seq_tok * DV * 4);
    const auto rdv = make_rsrc(a.dv + seq0 * DV, seq_tok * DV * 4);
    // this unit's block-start states, lane-major per 16-column wave slice (the recompute's
    // order; the eligibility check keeps their offsets below 2^31)
    const auto rst = make_rsrc(a.ws_states + bh * static_cast<size_t>(nb) * DK * DV, static_cast<size_t>(nb) * DK * DV * 4);
    // block-start states per 16-column wave slice, register quad i of lane l at (i 64 + l) 16 bytes
    const int voff_st = ((col >> 4) * (R / 4) * 64 + lane) * 16;

    float dS[R];
#pragma unroll
    for (int m = 0; m < R; m++)
        dS[m] = a.dST ? a.dST[bh * DK * DV + static_cast<size_t>(state_row(m, g)) * DV + col] : 0.0f;

    const int voff_v = (4 * g * H * DV + col) * 2;  // token 4 g + r (soffset), column col
    const int voff_do = (4 * g * H * DV + col) * 4;
    const int voff_doT = (c * H * DV + cw0 + 4 * g) * 4;  // token c, columns cw0 + 4 g .. + 3

    // A block's own inputs (lane (g, c)): values and dO of tokens t0 + 4 g + r at column col;
    // dO of token t0 + c at columns cw0 + 4 g .. + 3; the state entering the block in the
    // state layout.  The next block (in walking order) is fetched while this one is processed,
    // in two parts.
    struct BlockIn {
        uint32_t v[4];
        f4 dO, dOT;
        float s[R];
    };
    auto fetch_part = [&](BlockIn& in, int blk, int part) __attribute__((always_inline)) {
        const int t0 = blk * kBlk;
        if (part == 0) {
#pragma unroll
            for (int r = 0; r < 4; r++) {
                in.v[r] = __builtin_amdgcn_raw_buffer_load_b16(rv, voff_v, ((t0 + r) * H + h) * DV * 2, 0);
                in.dO[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rdo, voff_do, ((t0 + r) * H + h) * DV * 4, 0));
            }
            in.dOT = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(rdo, voff_doT, (t0 * H + h) * DV * 4, 0));
        } else {
            // the recompute wrote the states in register order: this lane's 32 values as eight
            // 16-byte quads, each quad of the 64 lanes one contiguous kilobyte
            const int so = blk * DK * DV * 4;
#pragma unroll
            for (int i = 0; i < R / 4; i++) {
                const u4 x = __builtin_amdgcn_raw_buffer_load_b128(rst, voff_st + 1024 * i, so, 0);
#pragma unroll
                for (int e = 0; e < 4; e++) in.s[4 * i + e] = __uint_as_float(x[e]);
            }
        }
    };

    BlockIn cur, nxt;
    fetch_part(cur, nb - 1, 0);
    fetch_part(cur, nb - 1, 1);
    __syncthreads();  // the last block's slot is ready
#pragma unroll 1
    for (int blk = nb - 1; blk >= 0; blk--) {
        const int t0 = blk * kBlk;
        // the block walked next (block 0 again after the last: no branch, so the compiler's
        // waits for this block's loads do not also wait for the next block's)
        const int bn = blk > 0 ? blk - 1 : 0;
        const BwSlot& sl = slots[blk & 1];
        const float(&s)[R] = cur.s;
        const f4 dO4 = cur.dO;
        const f4 dOT = cur.dOT;
        float V4[4];
#pragma unroll
        for (int r = 0; r < 4; r++) V4[r] = bf_lo(cur.v[r]);
        fetch_part(nxt, bn, 0);

        // ------------------------------------------------------------ the block's slot
        const f4 b4 = *reinterpret_cast<const f4*>(&sl.beta[4 * g]);
        const f4 gam4 = *reinterpret_cast<const f4*>(&sl.GAM[4 * g]);
        const f4 rho4 = *reinterpret_cast<const f4*>(&sl.RHO[4 * g]);
        const float gam15 = sl.GAM[kBlk - 1];
        const float gam_c = sl.GAM[c], rho_c = sl.RHO[c], bv = sl.beta[c];
        const f4 Rr = *reinterpret_cast<const f4*>(&sl.RR[c][4 * g]);
        const f4 a4 = *reinterpret_cast<const f4*>(&sl.A4[c][4 * g]);
        const f4 c4 = *reinterpret_cast<const f4*>(&sl.C4[c][4 * g]);
        const f4 aT4 = *reinterpret_cast<const f4*>(&sl.AT[c][4 * g]);
        const f4 nsel = *reinterpret_cast<const f4*>(&sl.Ns[c][4 * g]);  // N_{4g+r, c}

        // ------------------------------------------------------------ forward quantities
        // P = K S_0, Z = K dS' (lane (g, c), register r: token 4 g + r, column c), the keys of
        // token c from the slot (the rows of slice st), the state and dS' in three bf16 parts
        f4 P4 = {0.0f, 0.0f, 0.0f, 0.0f}, Z4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int st = 0; st < 4; st++) {
            u4 kv[4];
            kv[st] = *reinterpret_cast<const u4*>(&sl.kN[c][32 * st + 8 * g]);
            P4 = project_slice(P4, s, kv, st);
            Z4 = project_slice(Z4, dS, kv, st);
        }
        f4 W4;
#pragma unroll
        for (int r = 0; r < 4; r++) W4[r] = V4[r] - gam4[r] * P4[r];
        // Delta = N diag(beta) W: slice s pairs token 4 g + s; A = N_{c, 4g+s}, B = beta W
        f4 D4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int sl_ = 0; sl_ < 4; sl_++) D4 = mfma4(sl.Ns[4 * g + sl_][c], b4[sl_] * W4[sl_], D4);

        // ------------------------------------------------------------ adjoint of the block
        f4 dD4;
#pragma unroll
        for (int r = 0; r < 4; r++) dD4[r] = rho4[r] * Z4[r];
#pragma unroll
        for (int sl = 0; sl < 4; sl++) dD4 = mfma4(c4[sl], dO4[sl], dD4);  // + C^T dO
        f4 L4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int sl = 0; sl < 4; sl++) L4 = mfma4(nsel[sl], dD4[sl], L4);  // lambda = N^T dDelta
        f4 AD4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int sl = 0; sl < 4; sl++) AD4 = mfma4(aT4[sl], D4[sl], AD4);  // A Delta
        f4 dV4, dU4;
        float e1[4], e2[4], db[4];
#pragma unroll
        for (int r = 0; r < 4; r++) {
            dV4[r] = b4[r] * L4[r];
            dU4[r] = -dV4[r];
            db[r] = group_sum<16>(L4[r] * (W4[r] - AD4[r]));
            e1[r] = group_sum<16>(gam4[r] * P4[r] * dU4[r]);
            e2[r] = group_sum<16>(rho4[r] * Z4[r] * D4[r]);
        }
#pragma unroll
        for (int r = 0; r < 4; r++)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dV4[r]), rdv, voff_do, ((t0 + r) * H + h) * DV * 4, 0);
        float sd = 0.0f;
#pragma unroll
        for (int m = 0; m < R; m++) sd += dS[m] * s[m];
        const float sdot = wave_sum(sd);                           // <dS', S_0> over this wave's columns
        const float e2tot = rows_sum(e2[0] + e2[1] + e2[2] + e2[3]);  // sum over the block's tokens

        // Delta and lambda to the T layout
#pragma unroll
        for (int r = 0; r < 4; r++) {
            sh.XD[4 * g + r][c] = D4[r];
            sh.XL[4 * g + r][c] = L4[r];
        }
        *reinterpret_cast<f4*>(&sh.XO[c][4 * g]) = dOT;  // for the other waves' key/query sums
        wave_lds_sync();
        const f4 DT = *reinterpret_cast<const f4*>(&sh.XD[c][4 * g]);
        const f4 LT = *reinterpret_cast<const f4*>(&sh.XL[c][4 * g]);
        // dC = dO Delta^T, lambda Delta^T: slice s pairs column 4 g + s
        f4 dC4 = {0.0f, 0.0f, 0.0f, 0.0f}, dAr4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int sl = 0; sl < 4; sl++) {
            dC4 = mfma4(dOT[sl], DT[sl], dC4);
            dAr4 = mfma4(LT[sl], DT[sl], dAr4);
        }
        f4 Ab4, Cb4, dgr4;
        float ecol = 0.0f;
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int j = 4 * g + r;
            const float dA = c < j ? -b4[r] * dAr4[r] : 0.0f;
            const float dC = c <= j ? dC4[r] : 0.0f;
            Ab4[r] = dA * Rr[r];
            Cb4[r] = dC * Rr[r];
            const float E = dA * a4[r] + dC * c4[r];
            ecol += E;
            dgr4[r] = e1[r] - e2[r] + group_sum<16>(E) + (j == kBlk - 1 ? gam15 * sdot + e2tot : 0.0f);
        }
        const float dgc = -rows_sum(ecol);

        // ------------------------------------------------------------ dS_0
        // gamma_15 dS' + K^T (gamma dU) + Q^T (gamma dO): tile tau = dS[4 tau .. 4 tau + 3]
        // (accumulator row 4 g' + r = key row state_row(4 tau + r, g')), A = keys or queries
        // read transposed from LDS, B = the token vectors in three bf16 parts.  S_0 and dS'
        // (before the update) go to LDS first, for the key/query sums below.
#pragma unroll
        for (int m = 0; m < R; m++) {
            sh.SdS[0][state_row(m, g)][c] = s[m];
            sh.SdS[1][state_row(m, g)][c] = dS[m];
        }
        *reinterpret_cast<f4*>(&sh.small[0][lane][0]) = Ab4;
        *reinterpret_cast<f4*>(&sh.small[1][lane][0]) = Cb4;
        *reinterpret_cast<f4*>(&sh.small[2][lane][0]) = dgr4;
        *reinterpret_cast<f4*>(&sh.small[3][lane][0]) = f4{db[0], db[1], db[2], db[3]};
        *reinterpret_cast<f4*>(&sh.small[4][lane][0]) = f4{dgc, 0.0f, 0.0f, 0.0f};
        {
            f4 x1, x3;
#pragma unroll
            for (int r = 0; r < 4; r++) {
                x1[r] = gam4[r] * dU4[r];
                x3[r] = gam4[r] * dO4[r];
            }
            bf4 h1, l1, m1, h3, l3, m3;
            split3<4>(x1, h1, l1, m1);
            split3<4>(x3, h3, l3, m3);
#pragma unroll
            for (int tau = 0; tau < 8; tau++) {
                const s4 kr = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(&sl.kN[0][0] + tr_offset(g, c, tau)));
                const s4 qr = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(&sl.qN[0][0] + tr_offset(g, c, tau)));
                f4 st = {gam15 * dS[4 * tau], gam15 * dS[4 * tau + 1], gam15 * dS[4 * tau + 2], gam15 * dS[4 * tau + 3]};
                st = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(kr, __builtin_bit_cast(s4, m1), st, 0, 0, 0);
                st = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(qr, __builtin_bit_cast(s4, m3), st, 0, 0, 0);
                st = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(kr, __builtin_bit_cast(s4, l1), st, 0, 0, 0);
                st = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(qr, __builtin_bit_cast(s4, l3), st, 0, 0, 0);
                st = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(kr, __builtin_bit_cast(s4, h1), st, 0, 0, 0);
                st = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(qr, __builtin_bit_cast(s4, h3), st, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 4; r++) dS[4 * tau + r] = st[r];
            }
        }
        // the next block's state: this block's is in LDS now, so the two are never both live
        fetch_part(nxt, bn, 1);
        __syncthreads();

        // ------------------------------------------------------------ key/query sums
        // over the workgroup's 64 columns, wave w taking key rows 32 w .. 32 w + 31 (tiles u = 0,
        // 1 of 16 rows): dk_S[i][row] = sum_col X1[i][col] S_0[row][col] + X2[i][col] dS'[row][col],
        // dq_S with X3; X1 = gamma dU = -gamma beta lambda, X2 = rho Delta, X3 = gamma dO, all
        // row-scaled per token i (lane (g, c): token c).  Source wave ww, slice s pairs column
        // 16 ww + 4 g + s: A from its lambda / Delta / dO rows (XL, XD, XO), B from its S_0 /
        // dS' rows.  The sums are over the workgroup's columns: no cross-wave step.
        {
            const float k1 = -gam_c * bv;
            f4 ak[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
            f4 aq[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
            // operands of source wave ww: lambda, Delta and dO rows of token c, then S_0 and dS'
            // at rows 32 w + 16 u + c
#pragma unroll
            for (int ww = 0; ww < kBwWaves; ww++) {
                const f4 x1 = k1 * *reinterpret_cast<const f4*>(&shw[ww].XL[c][4 * g]);
                const f4 x2 = rho_c * *reinterpret_cast<const f4*>(&shw[ww].XD[c][4 * g]);
                const f4 x3 = gam_c * *reinterpret_cast<const f4*>(&shw[ww].XO[c][4 * g]);
#pragma unroll
                for (int u = 0; u < 2; u++) {
                    const int row = 32 * w + 16 * u + c;
                    const f4 Sf = *reinterpret_cast<const f4*>(&shw[ww].SdS[0][row][4 * g]);
                    const f4 dSf = *reinterpret_cast<const f4*>(&shw[ww].SdS[1][row][4 * g]);
#pragma unroll
                    for (int sl_ = 0; sl_ < 4; sl_++) {
                        ak[u] = mfma4(x1[sl_], Sf[sl_], ak[u]);
                        aq[u] = mfma4(x3[sl_], Sf[sl_], aq[u]);
                        ak[u] = mfma4(x2[sl_], dSf[sl_], ak[u]);
                    }
                }
            }
            float* rec = a.ws_part + ((bh * nb + blk) * nwg + blockIdx.x) * static_cast<size_t>(kRec);
#pragma unroll
            for (int u = 0; u < 2; u++) {
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    rec[kRecDk + (4 * g + r) * DK + 32 * w + 16 * u + c] = ak[u][r];
                    rec[kRecDq + (4 * g + r) * DK + 32 * w + 16 * u + c] = aq[u][r];
                }
            }
            // the small sums: wave w adds slot w of the four waves (wave 0 also slot 4)
            f4 sm = *reinterpret_cast<const f4*>(&shw[0].small[w][lane][0]);
#pragma unroll
            for (int ww = 1; ww < kBwWaves; ww++) sm += *reinterpret_cast<const f4*>(&shw[ww].small[w][lane][0]);
            if (w < 2) {
#pragma unroll
                for (int r = 0; r < 4; r++) rec[(w == 0 ? kRecA : kRecC) + (4 * g + r) * kBlk + c] = sm[r];
            } else if (c == 0) {
#pragma unroll
                for (int r = 0; r < 4; r++) rec[(w == 2 ? kRecGr : kRecB) + 4 * g + r] = sm[r];
            }
            if (w == 0 && g == 0) {
                float x = shw[0].small[4][lane][0];
#pragma unroll
                for (int ww = 1; ww < kBwWaves; ww++) x += shw[ww].small[4][lane][0];
                rec[kRecGc + c] = x;
            }
        }
        __syncthreads();
        cur = nxt;
    }

#pragma unroll
    for (int m = 0; m < R; m++) a.dS0[bh * DK * DV + static_cast<size_t>(state_row(m, g)) * DV + col] = dS[m];
}

// Per (block, head, sequence): the workgroups' partial records summed in slice order, the
// Gram-matrix terms (Ab + Ab^T) K + Cb^T Q and Cb K, the query term of dG, and dg as the
// suffix sum of dG over the block's tokens.  Thread (i, rc) owns token i, rows 8 rc .. 8 rc + 7
// (16-byte loads and stores; the 16 threads of a token cover its 512-byte row).
__global__ __launch_bounds__(256) void bwd_mfma_reduce_kernel(BwParams p, BwdArgs a, int nwg) {
    constexpr int DK = kBwDK;
    __shared__ float Kf[kBlk][DK + 4], Qf[kBlk][DK + 4];
    __shared__ float Ab[kBlk][kBlk + 1], Cb[kBlk][kBlk + 1];
    __shared__ float dG[kBlk], qd[kBlk];
    const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const int T = p.T, H = p.H, nb = p.nb;
    const int t0 = blk * kBlk;
    const size_t bh = static_cast<size_t>(b) * H + h;
    const float* rec0 = a.ws_part + (bh * nb + blk) * nwg * static_cast<size_t>(kRec);
    const int i = tid >> 4, rc = tid & 15;
    const bool ok = t0 + i < T;
    const size_t tseq = static_cast<size_t>(b) * p.stride_T + p.t_off;  // the segment's first token
    const size_t o = ((tseq + t0 + i) * H + h) * DK + 8 * rc;
    // k and q of this thread's token and rows (a valid address for every thread; rows past the
    // sequence are zeroed), loaded before the records so that their latencies overlap
    const size_t oc = ok ? o : ((tseq + t0) * H + h) * DK + 8 * rc;
    u4 kw = *reinterpret_cast<const u4*>(static_cast<const uint16_t*>(a.k) + oc);
    u4 qw = *reinterpret_cast<const u4*>(static_cast<const uint16_t*>(a.q) + oc);
    const int tg = tid & (kBlk - 1);
    float sa = 0.0f, sc = 0.0f, sg = 0.0f, sb = 0.0f;
    // the slices' key/query sums for this thread's eight rows
    f4 dks[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
    f4 dqs[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
    // one slice's fields, loaded together, then added in slice order
    struct Slice {
        float a, c, gr, gc, b;
        f4 dk[2], dq[2];
    };
    auto load_slice = [&](int wg, Slice& x) __attribute__((always_inline)) {
        const float* r = rec0 + wg * static_cast<size_t>(kRec);
        x.a = r[kRecA + tid];
        x.c = r[kRecC + tid];
        x.gr = r[kRecGr + tg];
        x.gc = r[kRecGc + tg];
        x.b = r[kRecB + tg];
        const float* rr = r + i * DK + 8 * rc;
#pragma unroll
        for (int hh = 0; hh < 2; hh++) {
            x.dk[hh] = *reinterpret_cast<const f4*>(rr + kRecDk + 4 * hh);
            x.dq[hh] = *reinterpret_cast<const f4*>(rr + kRecDq + 4 * hh);
        }
    };
    auto add_slice = [&](const Slice& x) __attribute__((always_inline)) {
        sa += x.a;
        sc += x.c;
        sg += x.gr + x.gc;
        sb += x.b;
#pragma unroll
        for (int hh = 0; hh < 2; hh++) {
            dks[hh] += x.dk[hh];
            dqs[hh] += x.dq[hh];
        }
    };
    if (nwg == 2) {  // (d_v = 128) both slices' loads in flight together
        Slice x0, x1;
        load_slice(0, x0);
        load_slice(1, x1);
        add_slice(x0);
        add_slice(x1);
    } else {
        for (int wg = 0; wg < nwg; wg++) {
            Slice x;
            load_slice(wg, x);
            add_slice(x);
        }
    }
    if (!ok) {
        kw = u4{0u, 0u, 0u, 0u};
        qw = u4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int e = 0; e < 4; e++) {
        Kf[i][8 * rc + 2 * e] = __uint_as_float(kw[e] << 16);
        Kf[i][8 * rc + 2 * e + 1] = __uint_as_float(kw[e] & 0xFFFF0000u);
        Qf[i][8 * rc + 2 * e] = __uint_as_float(qw[e] << 16);
        Qf[i][8 * rc + 2 * e + 1] = __uint_as_float(qw[e] & 0xFFFF0000u);
    }
    Ab[tid / kBlk][tid % kBlk] = sa;
    Cb[tid / kBlk][tid % kBlk] = sc;
    if (tid < kBlk) {
        dG[tid] = sg;
        if (t0 + tid < T) a.dbeta[(tseq + t0 + tid) * H + h] = sb;
    }
    __syncthreads();
    float qdot = 0.0f;
    f4 dko[2] = {dks[0], dks[1]}, dqo[2] = {dqs[0], dqs[1]};
#pragma unroll
    for (int hh = 0; hh < 2; hh++) {
        const f4 qv = *reinterpret_cast<const f4*>(&Qf[i][8 * rc + 4 * hh]);
        qdot += qv[0] * dqs[hh][0] + qv[1] * dqs[hh][1] + qv[2] * dqs[hh][2] + qv[3] * dqs[hh][3];
    }
#pragma unroll 4
    for (int j = 0; j < kBlk; j++) {
        const float ca = Ab[i][j] + Ab[j][i], cq = Cb[j][i], cc = Cb[i][j];
#pragma unroll
        for (int hh = 0; hh < 2; hh++) {
            const f4 kv = *reinterpret_cast<const f4*>(&Kf[j][8 * rc + 4 * hh]);
            const f4 qv = *reinterpret_cast<const f4*>(&Qf[j][8 * rc + 4 * hh]);
            dko[hh] += ca * kv + cq * qv;
            dqo[hh] += cc * kv;
        }
    }
    if (ok) {
#pragma unroll
        for (int hh = 0; hh < 2; hh++) {
            *reinterpret_cast<f4*>(a.dk + o + 4 * hh) = dko[hh];
            *reinterpret_cast<f4*>(a.dq + o + 4 * hh) = dqo[hh];
        }
    }
    qdot = group_sum<16>(qdot);
    if (rc == 0) qd[i] = qdot;
    __syncthreads();
    if (tid < kBlk && t0 + tid < T) {
        float x = 0.0f;
        for (int j = kBlk - 1; j >= tid; j--) x += dG[j] + qd[j];
        a.dg[(tseq + t0 + tid) * H + h] = x;
    }
}

bool bwd_mfma_eligible(const la_config& c) {
    if (c.gate != LA_GATE_SCALAR || c.d_v % 64 != 0) return false;
    // the caller's forward must itself have run on the block kernel, so that the recompute
    // (the block kernel with 16-token checkpoints) meets the forward's rounding decisions
    if (fwd_kernel(c) != LA_KERNEL_BLOCK) return false;
    la_config c16 = c;
    c16.ckpt_interval = kBlk;
    c16.kernel = LA_KERNEL_AUTO;
    if (!fwd_mfma_eligible(c16)) return false;
    // 32-bit buffer offsets over one sequence's upstream gradient (its last block included)
    const size_t span = static_cast<size_t>(c.T + kBlk) * c.H * c.d_v * 4;
    return span < (static_cast<size_t>(1) << 31);
}

// Tokens per segment: a multiple of the checkpoint spacing, sized so that a segment's
// block-start states and partial records take about 256 MiB (at least one chunk, at most
// the sequence).
int bwd_mfma_segment(const la_config& c) {
    const size_t units = static_cast<size_t>(c.B) * c.H;
    const size_t per_tok = units * (static_cast<size_t>(c.d_k) * c.d_v * 4 + (c.d_v / 64) * kRec * 4) / kBlk;
    const int C = c.ckpt_interval;
    size_t L = (static_cast<size_t>(256) << 20) / (per_tok > 0 ? per_tok : 1);
    L = L / C * C;
    const size_t Tr = (static_cast<size_t>(c.T) + C - 1) / C * C;
    if (L < static_cast<size_t>(C)) L = C;
    if (L > Tr) L = Tr;
    return static_cast<int>(L);
}

size_t bwd_mfma_state_bytes(const la_config& c) {
    return static_cast<size_t>(c.B) * c.H * ((bwd_mfma_segment(c) + kBlk - 1) / kBlk) * c.d_k * c.d_v * sizeof(float);
}

size_t bwd_mfma_part_bytes(const la_config& c) {
    return static_cast<size_t>(c.B) * c.H * ((bwd_mfma_segment(c) + kBlk - 1) / kBlk) * (c.d_v / 64) * kRec *
           sizeof(float);
}

// Segments last to first: (1) the state entering every 16-token block of the segment,
// recomputed from the forward's checkpoints, every checkpoint chunk in parallel (the block
// forward in chunk mode; the caller's checkpoints, or when none are given, the block forward's
// own first written into ck_room); (2) the block adjoint over the segment, dS carried between
// segments in `carry` (in place: each workgroup reads and writes its own elements); (3) the
// reduction of the segment's records.
hipError_t launch_bwd_mfma(const la_config& c, const FwdArgs& fa, const BwdArgs& a, float* carry, float* ck_room,
                           hipStream_t s) {
    const float* ck = a.ckpts;
    if (!ck) {
        FwdArgs f = fa;
        f.o = nullptr;
        f.ST = nullptr;
        f.ckpts = ck_room;
        hipError_t e = launch_fwd_mfma(c, f, s);
        if (e != hipSuccess) return e;
        ck = ck_room;
    }
    const int L = bwd_mfma_segment(c);
    const int nseg = (c.T + L - 1) / L;
    for (int sg = nseg - 1; sg >= 0; sg--) {
        const int s0 = sg * L, s1 = min(c.T, s0 + L), n = s1 - s0;
        FwdArgs f = fa;
        f.S0 = ck;
        f.o = nullptr;
        f.ST = nullptr;
        f.ckpts = a.ws_states;
        f.ckpt_lane_major = 1;
        hipError_t e = launch_fwd_mfma_chunks(c, f, s0, s1, s);
        if (e != hipSuccess) return e;
        const BwParams p{n, c.H, c.d_v, (n + kBlk - 1) / kBlk, c.T, s0};
        BwdArgs b = a;
        b.dST = sg == nseg - 1 ? a.dST : carry;
        b.dS0 = sg == 0 ? a.dS0 : carry;
        dim3 grid(c.d_v / 64, c.H, c.B);
        if (c.gate_dtype == LA_F32)
            hipLaunchKernelGGL((bwd_mfma_kernel<true>), grid, dim3(kBwThreads), 0, s, p, b);
        else
            hipLaunchKernelGGL((bwd_mfma_kernel<false>), grid, dim3(kBwThreads), 0, s, p, b);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(bwd_mfma_reduce_kernel, dim3(p.nb, c.H, c.B), dim3(256), 0, s, p, b, c.d_v / 64);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace la
