// Long-sequence forward on the matrix cores: scalar gate, d_k = 128, bf16 keys, queries and
// values, state rounded at most once per block of 16 tokens (no quantizer, or INT8/E4M3 at an
// interval that is a multiple of 16).
//
// The recurrence is advanced a block of 16 tokens at a time.  With S_0 the (true) state
// entering the block, Gamma_j the product of the block's gates up to token j and
// dd_j = delta_j / Gamma_j, the state inside the block is
//     S_j = Gamma_j (S_0 + sum_{i<=j} k_i dd_i^T),
// so every token's key and query projections follow from one projection of S_0:
//     u_j = Gamma_j (P'_j + sum_{i<j} (k_i . k_j) dd_i),      P' = S_0^T K
//     o_j = Gamma_j (Q'_j + sum_{i<=j} (k_i . q_j) dd_i),     Q' = S_0^T Q
//     dd_j = beta_j (v_j / Gamma_j - P'_j - sum_{i<j} (k_i . k_j) dd_i)
// and the block ends with S_16 = Gamma_15 (S_0 + K^T DD).  This is the gated delta rule
// itself, regrouped; every product is formed in fp32.
//
// A workgroup is one (sequence, head, 64 value columns): four column waves (consumers) and one
// producer wave.  The producer does the block's state-independent work once for the four:
//  * loads the keys, queries, gates and beta of block b + 1 (b + 2 in flight);
//  * the Gram matrices K K^T and K Q^T: bf16 MFMAs on the raw keys and queries (exact
//    products, fp32 sums);
//  * the gate products Gamma and their range check;
//  * M = (I + diag(beta) L)^-1 diag(beta) (L the strictly lower part of K K^T), solved on the
//    identity in four stages: lane group g solves tokens 4 g .. 4 g + 3 of each column, and
//    after each stage one fp32 MFMA adds its values to the later tokens;
// and writes keys, queries, M, K Q^T and the gate values into one of two LDS slots.  Each
// consumer (128 key rows x 16 value columns, lane 16 g + c holding column c and key row
// 32 (m / 8) + 8 g + m % 8 in s[m]) runs block b from the other slot:
//  * P', Q' (16 tokens x 16 columns each): bf16 MFMAs (16x16x32) of the keys and queries with
//    the state split exactly into three bf16 parts, slice i of the state (s[8 i .. 8 i + 7])
//    against the same key rows of each token;
//  * dd = M (V / Gamma - P'): 4 fp32 MFMAs; o = Gamma (Q' + tril(K Q^T)^T DD): 4 more;
//  * S_0 + K^T DD: bf16 MFMAs (16x16x16) with s[4 tau .. 4 tau + 3] as the accumulator tile
//    tau, the keys read transposed from the slot and DD in three bf16 parts; then the fold by
//    Gamma_15.
// One barrier per block hands the slots over (the producer also takes part in the barriers of
// every rounding point, so all five waves execute the same barriers).
// A block whose gate products leave [2^-60, 2^60] is run token by token with the gates
// applied to the state (the DPP passes of the wave layout).  Tokens past the end read zero
// inputs and beta = 0 and leave the state unchanged; their outputs are dropped.
#include "la_device.hpp"
#include "la_internal.hpp"
#include "la_mfma.hpp"
#include "la_recur.hpp"
#include "la_wave.hpp"

namespace la {

Params make_params(const la_config& c);

namespace {

constexpr float kGammaLo = 0x1p-60f, kGammaHi = 0x1p60f;
constexpr int kDppRowShr = 0x110;              // row_shr:n = kDppRowShr + n
// Inclusive prefix sum over each row of 16 lanes (zero-filled shifts).
__device__ __forceinline__ float row_prefix_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kDppRowShr + 1, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kDppRowShr + 2, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kDppRowShr + 4, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kDppRowShr + 8, 0xF, 0xF, false));
    return x;
}

// Product with identity-filled lanes: x[lane - n] of the same row of 16, 1.0 below the row.
template <int N>
__device__ __forceinline__ float row_shr_or_one(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.0f), __float_as_int(x), kDppRowShr + N, 0xF, 0xF, false));
}

// One block's state-independent data, written by the producer wave one block ahead (16-byte
// aligned: the 16-byte LDS accesses of the second slot need it).
struct alignas(16) PcSlot {
    uint16_t kN[kBlk][kKeyRow];  // keys [token][row] (projection operands and transposed update reads)
    uint16_t qN[kBlk][kKeyRow];  // queries [token][row]
    float Ms[kBlk][20];          // [c][j] = M[j][c]
    float GQ[kBlk][kBlk];        // [c][4 g + r] = k_{4g+r} . q_c: lane (g, c) reads its four values
    float gam[kBlk], rgam[kBlk], beta[kBlk], eg[kBlk];
    int in_range;
};
// The producer's own staging for the solve.
struct alignas(16) PcProd {
    float Gk[kBlk][kBlk];  // [j][i] = k_i . k_j
    float dd[4][kBlk][4];  // stage values of tokens 4 g + r, [g][column][r]
};
constexpr int kPcThreads = (kWaveTileWaves + 1) * 64;  // four consumer waves + one producer

__device__ __forceinline__ void pc_wave_sync() {
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
}

}  // namespace

template <int QMODE, int G, bool GF32, bool OBF16>
__global__ __launch_bounds__(kPcThreads) void fwd_mfma_kernel(Params p, FwdArgs a) {
    constexpr int DK = 128, R = 32;
    constexpr int GB = GF32 ? 4 : 2, OB = OBF16 ? 2 : 4;
    // barriers inside one rounding point (the cross-wave maxima of wave_quantize)
    constexpr int kQBar = (QMODE == LA_QDQ_E4M3_TILE || (QMODE == LA_QDQ_INT8_GROUP && G > kWaveCols)) ? 1 : 0;

    __shared__ WaveQdqShared<DK, QMODE, G> qsh;
    __shared__ PcSlot slots[2];
    __shared__ PcProd prod;

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, c = lane & 15;
    const int h = blockIdx.y;
    const int H = p.H, DV = p.dv;
    const bool chunked = p.chunk > 0;
    int b = blockIdx.z, T = p.T;
    size_t seq0 = static_cast<size_t>(b) * T * H;
    size_t s0_off = 0, ck_off = 0;
    if (chunked) {
        // one checkpoint chunk of the block backward's recompute (Params: chunk)
        b = blockIdx.z / p.nch;
        const int t_start = p.t_off + (blockIdx.z - b * p.nch) * p.chunk;
        T = min(p.chunk, p.t_end - t_start);
        seq0 = (static_cast<size_t>(b) * p.stride_T + t_start) * H;
        s0_off = ((static_cast<size_t>(b) * H + h) * p.nck_in + t_start / p.chunk) * DK * DV;
        ck_off = ((static_cast<size_t>(b) * H + h) * p.nck + (t_start - p.t_off) / kBlk) * DK * DV;
    }
    const int nblk = (T + kBlk - 1) / kBlk;
    const size_t bh = static_cast<size_t>(b) * H + h;
    const size_t seq_tok = static_cast<size_t>(T) * H;
    const int qi = p.qdq_interval;
    // last token of the next rounding interval (T: none); the same schedule in every wave
    auto next_q = [&](int qn) { return qn + qi <= T - 1 ? qn + qi : (qn < T - 1 ? T - 1 : T); };

    // Buffer resources over exactly this sequence's tokens (offsets < 2^31, checked on the
    // host): reads past its last token return zero, stores there are dropped.
    const auto rk = make_rsrc(static_cast<const char*>(a.k) + seq0 * DK * 2, seq_tok * DK * 2);
    const auto rq = make_rsrc(static_cast<const char*>(a.q) + seq0 * DK * 2, seq_tok * DK * 2);

    if (w == kWaveTileWaves) {
        // ------------------------------------------------------------ producer
        const auto rgt = make_rsrc(static_cast<const char*>(a.g) + seq0 * GB, seq_tok * GB);
        const auto rbt = make_rsrc(static_cast<const char*>(a.beta) + seq0 * GB, seq_tok * GB);
        const int voff_kq = (c * H * DK + 8 * g) * 2;  // token c, rows 32 i + 8 g .. + 7 (load i)
        const int voff_gate = c * H * GB;
        struct ProdIn {
            u4 k[4], q[4];
            uint32_t g, b;
        };
        auto pfetch = [&](ProdIn& in, int t0) __attribute__((always_inline)) {
            const int so = (t0 * H + h) * DK * 2;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                in.k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, voff_kq + 64 * i, so, 0);
                in.q[i] = __builtin_amdgcn_raw_buffer_load_b128(rq, voff_kq + 64 * i, so, 0);
            }
            const int sg = (t0 * H + h) * GB;
            if (GF32) {
                in.g = __builtin_amdgcn_raw_buffer_load_b32(rgt, voff_gate, sg, 0);
                in.b = __builtin_amdgcn_raw_buffer_load_b32(rbt, voff_gate, sg, 0);
            } else {
                in.g = __builtin_amdgcn_raw_buffer_load_b16(rgt, voff_gate, sg, 0);
                in.b = __builtin_amdgcn_raw_buffer_load_b16(rbt, voff_gate, sg, 0);
            }
        };
        auto produce = [&](const ProdIn& in, int t0, PcSlot& sl) __attribute__((always_inline)) {
            // Gram matrices: gk (lane (g, n), register r) = k_{4g+r} . k_n, gq = k_{4g+r} . q_n
            f4 gk = {0.0f, 0.0f, 0.0f, 0.0f}, gq = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const bf8 ak = __builtin_bit_cast(bf8, in.k[i]), aq = __builtin_bit_cast(bf8, in.q[i]);
                gk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, ak, gk, 0, 0, 0);
                gq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, aq, gq, 0, 0, 0);
            }
            // gates: lane (g, c) holds token t0 + c; every row of 16 forms the same products
            const bool valid = t0 + c < T;
            const float gv = GF32 ? __uint_as_float(in.g) : bf_lo(in.g);
            const float bv = GF32 ? __uint_as_float(in.b) : bf_lo(in.b);
            const float eg = valid ? expf(gv) : 1.0f;
            float gam = eg;
            gam *= row_shr_or_one<1>(gam);
            gam *= row_shr_or_one<2>(gam);
            gam *= row_shr_or_one<4>(gam);
            gam *= row_shr_or_one<8>(gam);
            const bool in_range = __all(gam >= kGammaLo && gam <= kGammaHi);
            if (g == 0) {
                sl.gam[c] = gam;
                sl.rgam[c] = 1.0f / gam;
                sl.beta[c] = valid ? bv : 0.0f;
                sl.eg[c] = eg;
            }
            if (lane == 0) sl.in_range = in_range ? 1 : 0;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                *reinterpret_cast<u4*>(&sl.kN[c][32 * i + 8 * g]) = in.k[i];
                *reinterpret_cast<u4*>(&sl.qN[c][32 * i + 8 * g]) = in.q[i];
            }
            *reinterpret_cast<f4*>(&sl.GQ[c][4 * g]) = gq;
            *reinterpret_cast<f4*>(&prod.Gk[c][4 * g]) = gk;  // symmetric: [c][i] = k_i . k_c
            pc_wave_sync();
            if (!in_range) return;
            // M = (I + diag(beta) L)^{-1} diag(beta) on the identity in four stages (lane (g, c):
            // column c, tokens 4 g .. 4 g + 3), as in the one-wave kernel
            const f4 beta4 = *reinterpret_cast<const f4*>(&sl.beta[4 * g]);
            const float c01 = prod.Gk[4 * g + 1][4 * g], c02 = prod.Gk[4 * g + 2][4 * g];
            const float c12 = prod.Gk[4 * g + 2][4 * g + 1], c03 = prod.Gk[4 * g + 3][4 * g];
            const float c13 = prod.Gk[4 * g + 3][4 * g + 1], c23 = prod.Gk[4 * g + 3][4 * g + 2];
            f4 dm = {0.0f, 0.0f, 0.0f, 0.0f}, selm = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int st = 0; st < 4; st++) {
                const float e0 = 4 * g == c ? 1.0f : 0.0f, e1 = 4 * g + 1 == c ? 1.0f : 0.0f;
                const float e2 = 4 * g + 2 == c ? 1.0f : 0.0f, e3 = 4 * g + 3 == c ? 1.0f : 0.0f;
                const float x0 = beta4[0] * (e0 - dm[0]);
                const float x1 = beta4[1] * (e1 - __builtin_fmaf(c01, x0, dm[1]));
                const float x2 = beta4[2] * (e2 - __builtin_fmaf(c12, x1, __builtin_fmaf(c02, x0, dm[2])));
                const float x3 = beta4[3] * (e3 - __builtin_fmaf(c23, x2, __builtin_fmaf(c13, x1, __builtin_fmaf(c03, x0, dm[3]))));
                if (g == st) selm = f4{x0, x1, x2, x3};
                if (st < 3) {
                    *reinterpret_cast<f4*>(&prod.dd[g][c][0]) = f4{x0, x1, x2, x3};
                    pc_wave_sync();
                    // A: lane (kk, j) = k_{4 st + kk} . k_j for tokens j of later groups, else 0;
                    // B: lane (kk, n) = M[4 st + kk][n]
                    const float ast = c >= 4 * st + 4 ? prod.Gk[c][4 * st + g] : 0.0f;
                    dm = __builtin_amdgcn_mfma_f32_16x16x4f32(ast, prod.dd[st][c][g], dm, 0, 0, 0);
                    pc_wave_sync();
                }
            }
            *reinterpret_cast<f4*>(&sl.Ms[c][4 * g]) = selm;
        };

        int q_next = QMODE != LA_QDQ_NONE && !chunked ? min(qi, T) - 1 : T;
        ProdIn cur, nxt;
        pfetch(cur, 0);
        pfetch(nxt, kBlk);
        produce(cur, 0, slots[0]);
        cur = nxt;
        __syncthreads();  // block 0 ready
#pragma unroll 1
        for (int blk = 0; blk < nblk; blk++) {
            const int t0 = blk * kBlk;
            // the block after next (past the end: zero reads, never used)
            pfetch(nxt, t0 + 2 * kBlk);
            if (blk + 1 < nblk) produce(cur, t0 + kBlk, slots[(blk + 1) & 1]);
            if (min(t0 + kBlk, T) - 1 == q_next) {
#pragma unroll
                for (int i = 0; i < kQBar; i++) __syncthreads();
                q_next = next_q(q_next);
            }
            __syncthreads();  // slots handed over
            cur = nxt;
        }
        return;
    }

    // ---------------------------------------------------------------- consumers
    const int col = blockIdx.x * kTileCols + w * kWaveCols + c;
    const size_t state_off = bh * DK * DV;
    const auto rv = make_rsrc(static_cast<const char*>(a.v) + seq0 * DV * 2, seq_tok * DV * 2);
    const size_t ck_unit = static_cast<size_t>(chunked ? nblk : p.nck) * DK * DV;
    const auto rck = make_rsrc(a.ckpts ? a.ckpts + (chunked ? ck_off : bh * ck_unit) : nullptr, a.ckpts ? ck_unit * 4 : 0);
    const int voff_ck = (state_row(0, g) * DV + col) * 4;
    const bool has_o = a.o != nullptr;
    const auto ro = make_rsrc(has_o ? static_cast<const char*>(a.o) + seq0 * DV * OB : nullptr,
                              has_o ? seq_tok * DV * OB : 0);

    float s[R];
    const size_t s0_base = chunked ? s0_off : state_off;
#pragma unroll
    for (int m = 0; m < R; m++)
        s[m] = a.S0 ? a.S0[s0_base + static_cast<size_t>(state_row(m, g)) * DV + col] : 0.0f;
    __builtin_amdgcn_s_waitcnt(0);

    // values of tokens t0 + 4 g .. 4 g + 3 at this lane's column
    const int voff_v = (4 * g * H * DV + col) * 2;
    auto vfetch = [&](uint32_t (&v)[4], int t0) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 4; r++) v[r] = __builtin_amdgcn_raw_buffer_load_b16(rv, voff_v, ((t0 + r) * H + h) * DV * 2, 0);
    };
    const int voff_o = (4 * g * H * DV + col) * OB;  // register r: token t0 + 4 g + r
    auto store_o = [&](int t0, int r, float ov) __attribute__((always_inline)) {
        const int so = ((t0 + r) * H + h) * DV * OB;
        if (OBF16) __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(ov), ro, voff_o, so, 0);
        else __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ov), ro, voff_o, so, 0);
    };

    int qpar = 0;
    int q_next = QMODE != LA_QDQ_NONE && !chunked ? min(qi, T) - 1 : T;
    int ck_next = a.ckpts ? 0 : T;
    uint32_t vcur[4], vnxt[4];
    vfetch(vcur, 0);
    __syncthreads();  // block 0 ready
#pragma unroll 1
    for (int blk = 0; blk < nblk; blk++) {
        const int t0 = blk * kBlk;
        const PcSlot& sl = slots[blk & 1];
        vfetch(vnxt, t0 + kBlk);
        if (t0 == ck_next) {
            const int so = t0 / p.ckpt_interval * DK * DV * 4;
            if (a.ckpt_lane_major) {
                // per 16-column wave slice, register quad i of lane l at (i * 64 + l) * 16 bytes:
                // every store instruction writes one contiguous kilobyte
                const int vo = ((col >> 4) * (R / 4) * 64 + lane) * 16;
#pragma unroll
                for (int i = 0; i < R / 4; i++)
                    __builtin_amdgcn_raw_buffer_store_b128(
                        u4{__float_as_uint(s[4 * i]), __float_as_uint(s[4 * i + 1]), __float_as_uint(s[4 * i + 2]),
                           __float_as_uint(s[4 * i + 3])}, rck, vo + 1024 * i, so, 0);
            } else {
#pragma unroll
                for (int m = 0; m < R; m++)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s[m]), rck, voff_ck,
                                                          so + (32 * (m >> 3) + (m & 7)) * DV * 4, 0);
            }
            ck_next += p.ckpt_interval;
        }

        float fold = 1.0f;
        if (__builtin_expect(__builtin_amdgcn_readfirstlane(sl.in_range) != 0, 1)) {
            const f4 gam4 = *reinterpret_cast<const f4*>(&sl.gam[4 * g]);
            const f4 rgam4 = *reinterpret_cast<const f4*>(&sl.rgam[4 * g]);
            // projections dk = P', dq = Q' (lane (g, c), register r: token 4 g + r, column c):
            // the keys and queries of token c from the slot, the state in three bf16 parts
            f4 dk = {0.0f, 0.0f, 0.0f, 0.0f}, dq = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int st = 0; st < 4; st++) {
                const bf8 ak = __builtin_bit_cast(bf8, *reinterpret_cast<const u4*>(&sl.kN[c][32 * st + 8 * g]));
                const bf8 aq = __builtin_bit_cast(bf8, *reinterpret_cast<const u4*>(&sl.qN[c][32 * st + 8 * g]));
                uint32_t hh[4], ll[4], l2[4];
#pragma unroll
                for (int i = 0; i < 4; i++) split3_pair(s[8 * st + 2 * i], s[8 * st + 2 * i + 1], hh[i], ll[i], l2[i]);
                const bf8 bh_ = __builtin_bit_cast(bf8, u4{hh[0], hh[1], hh[2], hh[3]});
                const bf8 bl_ = __builtin_bit_cast(bf8, u4{ll[0], ll[1], ll[2], ll[3]});
                const bf8 bl2 = __builtin_bit_cast(bf8, u4{l2[0], l2[1], l2[2], l2[3]});
                dk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, bl2, dk, 0, 0, 0);
                dq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, bl2, dq, 0, 0, 0);
                dk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, bl_, dk, 0, 0, 0);
                dq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, bl_, dq, 0, 0, 0);
                dk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, bh_, dk, 0, 0, 0);
                dq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, bh_, dq, 0, 0, 0);
            }
            // dd = M R with R = V / Gamma - P': slice s pairs input token 4 g + s (lane group g)
            // with A = M[c][4 g + s] and B = R[4 g + s][c], this lane's register s of R
            f4 ddm = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int sl_ = 0; sl_ < 4; sl_++) {
                const float rr = __builtin_fmaf(bf_lo(vcur[sl_]), rgam4[sl_], -dk[sl_]);
                ddm = __builtin_amdgcn_mfma_f32_16x16x4f32(sl.Ms[4 * g + sl_][c], rr, ddm, 0, 0, 0);
            }
            // o_i = Gamma_i (Q'_i + sum_{j <= i} (k_j . q_i) dd_j)
            const f4 gq = *reinterpret_cast<const f4*>(&sl.GQ[c][4 * g]);
            f4 ov = dq;
#pragma unroll
            for (int kp = 0; kp < 4; kp++) {
                const float am = 4 * g + kp <= c ? gq[kp] : 0.0f;
                ov = __builtin_amdgcn_mfma_f32_16x16x4f32(am, ddm[kp], ov, 0, 0, 0);
            }
            // S_0 + K^T DD, the keys read transposed from the slot (tr_offset), DD in three parts
            bf4 dh, dl, dl2;
            split3<4>(ddm, dh, dl, dl2);
#pragma unroll
            for (int tau = 0; tau < 8; tau++) {
                const s4 kr = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(&sl.kN[0][0] + tr_offset(g, c, tau)));
                f4 st = {s[4 * tau], s[4 * tau + 1], s[4 * tau + 2], s[4 * tau + 3]};
                st = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(kr, __builtin_bit_cast(s4, dl2), st, 0, 0, 0);
                st = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(kr, __builtin_bit_cast(s4, dl), st, 0, 0, 0);
                st = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(kr, __builtin_bit_cast(s4, dh), st, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 4; r++) s[4 * tau + r] = st[r];
            }
            if (has_o) {
#pragma unroll
                for (int r = 0; r < 4; r++) store_o(t0, r, gam4[r] * ov[r]);
            }
            fold = sl.gam[kBlk - 1];
        } else {
            // steep gates: token by token, each gate applied to the state
#pragma unroll 1
            for (int j = 0; j < kBlk && t0 + j < T; j++) {
                const float aj = sl.eg[j];
                const float bj = sl.beta[j];
#pragma unroll
                for (int m = 0; m < R; m++) s[m] *= aj;
                const int so = ((t0 + j) * H + h) * DK * 2;
                const int eoff = state_row(2 * c, g) * 2;
                const uint32_t kwd = __builtin_amdgcn_raw_buffer_load_b32(rk, eoff, so, 0);
                const uint32_t qwd = __builtin_amdgcn_raw_buffer_load_b32(rq, eoff, so, 0);
                float k0, k1, q0, q1;
                widen_pairs(kwd, qwd, k0, k1, q0, q1);
                const float kq = wave_sum(__builtin_fmaf(k1, q1, k0 * q0));
                float pk, pq, P, Q;
                dot_pass<R>(s, k0, k1, q0, q1, pk, pq);
                rows_sum2(pk, pq, P, Q);
                const uint32_t vwd = __builtin_amdgcn_raw_buffer_load_b16(rv, col * 2, ((t0 + j) * H + h) * DV * 2, 0);
                const float delta = bj * (bf_lo(vwd) - P);
                const float o = __builtin_fmaf(delta, kq, Q);
                update_pass<R>(s, k0, k1, delta);
                if (has_o && g == 0) {
                    const int so_o = ((t0 + j) * H + h) * DV * OB;
                    if (OBF16) __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(o), ro, col * OB, so_o, 0);
                    else __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o), ro, col * OB, so_o, 0);
                }
            }
        }

#pragma unroll
        for (int m = 0; m < R; m++) s[m] *= fold;

        if (min(t0 + kBlk, T) - 1 == q_next) {
            wave_quantize<R, QMODE, G>(s, qsh, lane, w, qpar);
            q_next = next_q(q_next);
        }
        __syncthreads();  // slots handed over
#pragma unroll
        for (int r = 0; r < 4; r++) vcur[r] = vnxt[r];
    }
    if (a.ST) {
#pragma unroll
        for (int m = 0; m < R; m++) a.ST[state_off + static_cast<size_t>(state_row(m, g)) * DV + col] = s[m];
    }
}

// ============================================================================ KDA (per-key gates)
// The same blocks with a gate per key row.  With G_j the inclusive sum of the block's log gates
// (a d_k-vector per token), Kb = K o exp(G), Qb = Q o exp(G), Kh = K o exp(-G) and
// Kt = K o exp(G_15 - G) (rows are tokens, o the elementwise product):
//     A = tril(Kb Kh^T, -1),  C = tril(Qb Kh^T),  Delta = M (V - Kb S_0),  M = (I + diag(beta) A)^-1 diag(beta)
//     O = Qb S_0 + C Delta,   S_16 = diag(exp(G_15)) S_0 + Kt^T Delta
// (Delta holds the tokens' true deltas; every entry of A and C and every Kt factor is a decay
// the recurrence itself applies between two tokens).  None of the scaled operands is a bf16
// value, so each product takes the six significant pairs of the two three-part splits.  The
// exponentials and splits are most of a block's vector work, so two producer waves share them,
// each taking half of the key rows: it forms the scaled operands of its rows, their parts and
// its partial Gram products.  Each consumer adds the partial Grams (in a fixed order), solves
// M itself (no barrier between the producers is needed) and runs the projections, Delta, the
// outputs and the update.  Blocks whose gate sums leave [-60, 60] run token by token with the
// gates applied to the state.
namespace {

constexpr float kKdaGLim = 60.0f;

constexpr int kKdaProd = 2;                  // producer waves
constexpr int kKdaSlices = 4 / kKdaProd;     // 32-row key slices per producer
struct alignas(16) KdaSlot {
    uint16_t Kb[3][kBlk][kKeyRow];  // the three bf16 parts of Kb, [token][row]
    uint16_t Qb[3][kBlk][kKeyRow];  // of Qb
    uint16_t Kt[3][kBlk][kKeyRow];  // of Kt (transposed reads of the update)
    float GK[kKdaProd][kBlk][kBlk];  // per producer (its key rows): [c][4 g + r] = Kb_{4g+r} . Kh_c
    float GQ[kKdaProd][kBlk][kBlk];  // [c][4 g + r] = Kh_{4g+r} . Qb_c
    float eG15[128];                // exp(G_15) per key row
    float beta[kBlk];
    int ok[kKdaProd];               // per producer: its gate sums stay in range
};
// A column wave's staging for its solve of M.
struct alignas(16) KdaSolve {
    float AmT[kBlk][20];   // [i][j] = A_ji
    float dd[4][kBlk][4];  // stage values of tokens 4 g + r, [g][column][r]
    float Ms[kBlk][20];    // [c][j] = M[j][c]
};
constexpr int kKdaThreads = (kWaveTileWaves + kKdaProd) * 64;  // four column waves + the producers

// e^x for |x| <= 60 (the block's gate-sum range): e^x = 2^(x log2 e), with x log2 e carried as
// an fp32 sum hi + lo (the product's rounding error recovered by one FMA, plus the low part of
// log2 e), 2^hi from the hardware exponential and the factor 2^lo = 1 + lo ln 2 to first order
// (|lo| < 2^-17, so the dropped terms are below 2^-35).  A few vector instructions instead of
// the library's general-range routine: within one ulp of e^x over [-60, 60] with a correctly
// rounded 2^hi (checked on the host over 2M arguments), plus the hardware exponential's error.
__device__ __forceinline__ float exp_bounded(float x) {
    constexpr float kLog2eHi = 1.44269502162933349609375f;   // log2(e) rounded to fp32
    constexpr float kLog2eLo = 1.925963033500011079e-8f;     // log2(e) - kLog2eHi
    constexpr float kLn2 = 0.693147180559945309f;
    const float hi = x * kLog2eHi;
    const float lo = __builtin_fmaf(x, kLog2eHi, -hi) + x * kLog2eLo;
    const float r = __builtin_amdgcn_exp2f(hi);
    return __builtin_fmaf(r, lo * kLn2, r);
}

// bf16 word pair of parts p (0 = hi, 1 = lo, 2 = lo2) of slice values
__device__ __forceinline__ bf8 parts_bf8(const uint32_t (&x)[4]) {
    return __builtin_bit_cast(bf8, u4{x[0], x[1], x[2], x[3]});
}
// acc += a b over the six significant pairs of two three-part splits, smallest first
__device__ __forceinline__ f4 mfma6_32(const bf8 (&a)[3], const bf8 (&b)[3], f4 acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], b[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[2], b[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1], b[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], b[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1], b[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], b[0], acc, 0, 0, 0);
    return acc;
}

}  // namespace

template <int QMODE, int G, bool GF32, bool OBF16>
__global__ __launch_bounds__(kKdaThreads) void fwd_mfma_kda_kernel(Params p, FwdArgs a) {
    constexpr int DK = 128, R = 32;
    constexpr int GB = GF32 ? 4 : 2, OB = OBF16 ? 2 : 4;
    constexpr int kQBar = (QMODE == LA_QDQ_E4M3_TILE || (QMODE == LA_QDQ_INT8_GROUP && G > kWaveCols)) ? 1 : 0;
    constexpr int NGW = GF32 ? 8 : 4;  // 16-byte gate words per lane and token (32 key rows)

    __shared__ WaveQdqShared<DK, QMODE, G> qsh;
    __shared__ KdaSlot slots[2];
    __shared__ KdaSolve solve[kWaveTileWaves];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, c = lane & 15;
    const int h = blockIdx.y, b = blockIdx.z;
    const int T = p.T, H = p.H, DV = p.dv;
    const int nblk = (T + kBlk - 1) / kBlk;
    const size_t bh = static_cast<size_t>(b) * H + h;
    const size_t seq0 = static_cast<size_t>(b) * T * H;
    const size_t seq_tok = static_cast<size_t>(T) * H;
    const int qi = p.qdq_interval;
    auto next_q = [&](int qn) { return qn + qi <= T - 1 ? qn + qi : (qn < T - 1 ? T - 1 : T); };

    const auto rk = make_rsrc(static_cast<const char*>(a.k) + seq0 * DK * 2, seq_tok * DK * 2);
    const auto rq = make_rsrc(static_cast<const char*>(a.q) + seq0 * DK * 2, seq_tok * DK * 2);
    const auto rgk = make_rsrc(static_cast<const char*>(a.g) + seq0 * DK * GB, seq_tok * DK * GB);
    // this lane's gate words of one token: rows 32 i + 8 g .. + 7 of slice i (GF32: two words)
    auto gate_word_off = [&](int i, int half) { return (32 * i + 8 * g) * GB + 16 * half; };

    if (w >= kWaveTileWaves) {
        // ------------------------------------------------------------ producers
        // producer pw takes key slices kKdaSlices pw ..  kKdaSlices (pw + 1) - 1 (32 rows each);
        // producer 0 also writes beta
        const int pw = w - kWaveTileWaves;
        const auto rbt = make_rsrc(static_cast<const char*>(a.beta) + seq0 * GB, seq_tok * GB);
        const int voff_kq = (c * H * DK + 32 * kKdaSlices * pw + 8 * g) * 2;
        const int voff_g = c * H * DK * GB;
        const int voff_gate = c * H * GB;
        struct ProdIn {
            u4 k[kKdaSlices], q[kKdaSlices], gw[NGW / 4 * kKdaSlices];
            uint32_t b;
        };
        auto pfetch = [&](ProdIn& in, int t0) __attribute__((always_inline)) {
            const int so = (t0 * H + h) * DK * 2;
#pragma unroll
            for (int i = 0; i < kKdaSlices; i++) {
                in.k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, voff_kq + 64 * i, so, 0);
                in.q[i] = __builtin_amdgcn_raw_buffer_load_b128(rq, voff_kq + 64 * i, so, 0);
            }
            const int sg = (t0 * H + h) * DK * GB;
#pragma unroll
            for (int i = 0; i < kKdaSlices; i++)
#pragma unroll
                for (int hf = 0; hf < NGW / 4; hf++)
                    in.gw[i * (NGW / 4) + hf] = __builtin_amdgcn_raw_buffer_load_b128(rgk, voff_g + gate_word_off(kKdaSlices * pw + i, hf), sg, 0);
            const int sb = (t0 * H + h) * GB;
            in.b = GF32 ? __builtin_amdgcn_raw_buffer_load_b32(rbt, voff_gate, sb, 0)
                        : __builtin_amdgcn_raw_buffer_load_b16(rbt, voff_gate, sb, 0);
        };
        auto produce = [&](const ProdIn& in, int t0, KdaSlot& sl) __attribute__((always_inline)) {
            const bool valid = t0 + c < T;
            bool ok = true;
            f4 gk = {0.0f, 0.0f, 0.0f, 0.0f}, gq = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int i = 0; i < kKdaSlices; i++) {
                const int st = kKdaSlices * pw + i;
                // this lane's 8 key rows of slice st: token c's keys, queries and gates
                float kf[8], qf[8], gf[8];
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    kf[2 * e] = __uint_as_float(in.k[i][e] << 16);
                    kf[2 * e + 1] = __uint_as_float(in.k[i][e] & 0xFFFF0000u);
                    qf[2 * e] = __uint_as_float(in.q[i][e] << 16);
                    qf[2 * e + 1] = __uint_as_float(in.q[i][e] & 0xFFFF0000u);
                }
                if (GF32) {
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        gf[e] = __uint_as_float(in.gw[2 * i][e]);
                        gf[4 + e] = __uint_as_float(in.gw[2 * i + 1][e]);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        gf[2 * e] = __uint_as_float(in.gw[i][e] << 16);
                        gf[2 * e + 1] = __uint_as_float(in.gw[i][e] & 0xFFFF0000u);
                    }
                }
                float kb[8], qb[8], kh[8], kt[8], e15[8];
#pragma unroll
                for (int j = 0; j < 8; j++) {
                    // inclusive sum over the block's tokens (lanes c of the row), broadcast of token 15
                    const float Gj = row_prefix_sum(valid ? gf[j] : 0.0f);
                    ok = ok && Gj >= -kKdaGLim && Gj <= kKdaGLim;
                    // in range or not, |Gj| <= 60 is what the block path uses; other blocks run
                    // token by token and never read these
                    const float Gc = fminf(fmaxf(Gj, -kKdaGLim), kKdaGLim);
                    const float eg = exp_bounded(Gc), emg = exp_bounded(-Gc);
                    // exp(G_15) of the row: token 15's value (row_newbcast:15)
                    e15[j] = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(eg), 0x15F, 0xF, 0xF, false));
                    kb[j] = kf[j] * eg;
                    qb[j] = qf[j] * eg;
                    kh[j] = kf[j] * emg;
                    kt[j] = kf[j] * (e15[j] * emg);
                }
                uint32_t kbp[3][4], qbp[3][4], khp[3][4], ktp[3][4];
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    split3_pair(kb[2 * e], kb[2 * e + 1], kbp[0][e], kbp[1][e], kbp[2][e]);
                    split3_pair(qb[2 * e], qb[2 * e + 1], qbp[0][e], qbp[1][e], qbp[2][e]);
                    split3_pair(kh[2 * e], kh[2 * e + 1], khp[0][e], khp[1][e], khp[2][e]);
                    split3_pair(kt[2 * e], kt[2 * e + 1], ktp[0][e], ktp[1][e], ktp[2][e]);
                }
#pragma unroll
                for (int pp = 0; pp < 3; pp++) {
                    *reinterpret_cast<u4*>(&sl.Kb[pp][c][32 * st + 8 * g]) = u4{kbp[pp][0], kbp[pp][1], kbp[pp][2], kbp[pp][3]};
                    *reinterpret_cast<u4*>(&sl.Qb[pp][c][32 * st + 8 * g]) = u4{qbp[pp][0], qbp[pp][1], qbp[pp][2], qbp[pp][3]};
                    *reinterpret_cast<u4*>(&sl.Kt[pp][c][32 * st + 8 * g]) = u4{ktp[pp][0], ktp[pp][1], ktp[pp][2], ktp[pp][3]};
                }
                if (c == 0) {
                    *reinterpret_cast<f4*>(&sl.eG15[32 * st + 8 * g]) = f4{e15[0], e15[1], e15[2], e15[3]};
                    *reinterpret_cast<f4*>(&sl.eG15[32 * st + 8 * g + 4]) = f4{e15[4], e15[5], e15[6], e15[7]};
                }
                // lane (g, c) register r: Kb_{4g+r} . Kh_c (gk) and Kh_{4g+r} . Qb_c (gq) over
                // this producer's key rows
                const bf8 akb[3] = {parts_bf8(kbp[0]), parts_bf8(kbp[1]), parts_bf8(kbp[2])};
                const bf8 akh[3] = {parts_bf8(khp[0]), parts_bf8(khp[1]), parts_bf8(khp[2])};
                const bf8 aqb[3] = {parts_bf8(qbp[0]), parts_bf8(qbp[1]), parts_bf8(qbp[2])};
                gk = mfma6_32(akb, akh, gk);
                gq = mfma6_32(akh, aqb, gq);
            }
            const bool in_range = __all(ok);
            if (pw == 0 && g == 0) sl.beta[c] = valid ? (GF32 ? __uint_as_float(in.b) : bf_lo(in.b)) : 0.0f;
            if (lane == 0) sl.ok[pw] = in_range ? 1 : 0;
            *reinterpret_cast<f4*>(&sl.GK[pw][c][4 * g]) = gk;
            *reinterpret_cast<f4*>(&sl.GQ[pw][c][4 * g]) = gq;
        };

        int q_next = QMODE != LA_QDQ_NONE ? min(qi, T) - 1 : T;
        ProdIn cur, nxt;
        pfetch(cur, 0);
        pfetch(nxt, kBlk);
        produce(cur, 0, slots[0]);
        cur = nxt;
        __syncthreads();  // block 0 ready
#pragma unroll 1
        for (int blk = 0; blk < nblk; blk++) {
            const int t0 = blk * kBlk;
            pfetch(nxt, t0 + 2 * kBlk);
            if (blk + 1 < nblk) produce(cur, t0 + kBlk, slots[(blk + 1) & 1]);
            if (min(t0 + kBlk, T) - 1 == q_next) {
#pragma unroll
                for (int i = 0; i < kQBar; i++) __syncthreads();
                q_next = next_q(q_next);
            }
            __syncthreads();  // slots handed over
            cur = nxt;
        }
        return;
    }

    // ---------------------------------------------------------------- consumers
    const int col = blockIdx.x * kTileCols + w * kWaveCols + c;
    const size_t state_off = bh * DK * DV;
    const auto rv = make_rsrc(static_cast<const char*>(a.v) + seq0 * DV * 2, seq_tok * DV * 2);
    const size_t ck_unit = static_cast<size_t>(p.nck) * DK * DV;
    const auto rck = make_rsrc(a.ckpts ? a.ckpts + bh * ck_unit : nullptr, a.ckpts ? ck_unit * 4 : 0);
    const int voff_ck = (state_row(0, g) * DV + col) * 4;
    const bool has_o = a.o != nullptr;
    const auto ro = make_rsrc(has_o ? static_cast<const char*>(a.o) + seq0 * DV * OB : nullptr,
                              has_o ? seq_tok * DV * OB : 0);

    float s[R];
#pragma unroll
    for (int m = 0; m < R; m++)
        s[m] = a.S0 ? a.S0[state_off + static_cast<size_t>(state_row(m, g)) * DV + col] : 0.0f;
    __builtin_amdgcn_s_waitcnt(0);

    const int voff_v = (4 * g * H * DV + col) * 2;
    auto vfetch = [&](uint32_t (&v)[4], int t0) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 4; r++) v[r] = __builtin_amdgcn_raw_buffer_load_b16(rv, voff_v, ((t0 + r) * H + h) * DV * 2, 0);
    };
    const int voff_o = (4 * g * H * DV + col) * OB;
    auto store_o = [&](int t0, int r, float ov) __attribute__((always_inline)) {
        const int so = ((t0 + r) * H + h) * DV * OB;
        if (OBF16) __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(ov), ro, voff_o, so, 0);
        else __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ov), ro, voff_o, so, 0);
    };

    int qpar = 0;
    int q_next = QMODE != LA_QDQ_NONE ? min(qi, T) - 1 : T;
    int ck_next = a.ckpts ? 0 : T;
    uint32_t vcur[4], vnxt[4];
    vfetch(vcur, 0);
    __syncthreads();  // block 0 ready
#pragma unroll 1
    for (int blk = 0; blk < nblk; blk++) {
        const int t0 = blk * kBlk;
        const KdaSlot& sl = slots[blk & 1];
        vfetch(vnxt, t0 + kBlk);
        if (t0 == ck_next) {
            const int so = t0 / p.ckpt_interval * DK * DV * 4;
#pragma unroll
            for (int m = 0; m < R; m++)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s[m]), rck, voff_ck,
                                                      so + (32 * (m >> 3) + (m & 7)) * DV * 4, 0);
            ck_next += p.ckpt_interval;
        }

        int in_range = sl.ok[0];
#pragma unroll
        for (int pw = 1; pw < kKdaProd; pw++) in_range &= sl.ok[pw];
        if (__builtin_expect(__builtin_amdgcn_readfirstlane(in_range) != 0, 1)) {
            // P' = Kb S_0, Q' = Qb S_0 (lane (g, c), register r: token 4 g + r, column c)
            f4 dk = {0.0f, 0.0f, 0.0f, 0.0f}, dq = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int st = 0; st < 4; st++) {
                bf8 akb[3], aqb[3];
#pragma unroll
                for (int pp = 0; pp < 3; pp++) {
                    akb[pp] = __builtin_bit_cast(bf8, *reinterpret_cast<const u4*>(&sl.Kb[pp][c][32 * st + 8 * g]));
                    aqb[pp] = __builtin_bit_cast(bf8, *reinterpret_cast<const u4*>(&sl.Qb[pp][c][32 * st + 8 * g]));
                }
                uint32_t sp[3][4];
#pragma unroll
                for (int e = 0; e < 4; e++) split3_pair(s[8 * st + 2 * e], s[8 * st + 2 * e + 1], sp[0][e], sp[1][e], sp[2][e]);
                const bf8 bs[3] = {parts_bf8(sp[0]), parts_bf8(sp[1]), parts_bf8(sp[2])};
                dk = mfma6_32(akb, bs, dk);
                dq = mfma6_32(aqb, bs, dq);
            }
            // M = (I + diag(beta) A)^{-1} diag(beta), solved by each wave on the identity in four
            // stages (lane group g: tokens 4 g .. 4 g + 3 of column c; after each stage one fp32
            // MFMA adds its values to the later tokens).  A_{j i} is the sum of the producers'
            // partial products GK[.][i][j]; A is not symmetric here.
            KdaSolve& sv = solve[w];
            auto gkc = [&](int i, int j) __attribute__((always_inline)) {
                float x = sl.GK[0][i][j];
#pragma unroll
                for (int pw = 1; pw < kKdaProd; pw++) x += sl.GK[pw][i][j];
                return x;
            };
            const f4 beta4 = *reinterpret_cast<const f4*>(&sl.beta[4 * g]);
            const float c01 = gkc(4 * g, 4 * g + 1), c02 = gkc(4 * g, 4 * g + 2);
            const float c12 = gkc(4 * g + 1, 4 * g + 2), c03 = gkc(4 * g, 4 * g + 3);
            const float c13 = gkc(4 * g + 1, 4 * g + 3), c23 = gkc(4 * g + 2, 4 * g + 3);
            f4 dm = {0.0f, 0.0f, 0.0f, 0.0f}, selm = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int st = 0; st < 4; st++) {
                const float e0 = 4 * g == c ? 1.0f : 0.0f, e1 = 4 * g + 1 == c ? 1.0f : 0.0f;
                const float e2 = 4 * g + 2 == c ? 1.0f : 0.0f, e3 = 4 * g + 3 == c ? 1.0f : 0.0f;
                const float x0 = beta4[0] * (e0 - dm[0]);
                const float x1 = beta4[1] * (e1 - __builtin_fmaf(c01, x0, dm[1]));
                const float x2 = beta4[2] * (e2 - __builtin_fmaf(c12, x1, __builtin_fmaf(c02, x0, dm[2])));
                const float x3 = beta4[3] * (e3 - __builtin_fmaf(c23, x2, __builtin_fmaf(c13, x1, __builtin_fmaf(c03, x0, dm[3]))));
                if (g == st) selm = f4{x0, x1, x2, x3};
                if (st < 3) {
                    *reinterpret_cast<f4*>(&sv.dd[g][c][0]) = f4{x0, x1, x2, x3};
                    pc_wave_sync();
                    // A: lane (kk, j) = A_{j, 4 st + kk} for tokens j of later groups
                    const float ast = c >= 4 * st + 4 ? gkc(4 * st + g, c) : 0.0f;
                    dm = __builtin_amdgcn_mfma_f32_16x16x4f32(ast, sv.dd[st][c][g], dm, 0, 0, 0);
                    pc_wave_sync();
                }
            }
            *reinterpret_cast<f4*>(&sv.Ms[c][4 * g]) = selm;
            pc_wave_sync();
            // Delta = M (V - P'): slice s pairs token 4 g + s
            f4 ddm = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int sl_ = 0; sl_ < 4; sl_++)
                ddm = __builtin_amdgcn_mfma_f32_16x16x4f32(sv.Ms[4 * g + sl_][c], bf_lo(vcur[sl_]) - dk[sl_], ddm, 0, 0, 0);
            // o_i = Q'_i + sum_{j <= i} (Kh_j . Qb_i) delta_j
            f4 gq = *reinterpret_cast<const f4*>(&sl.GQ[0][c][4 * g]);
#pragma unroll
            for (int pw = 1; pw < kKdaProd; pw++) gq += *reinterpret_cast<const f4*>(&sl.GQ[pw][c][4 * g]);
            f4 ov = dq;
#pragma unroll
            for (int kp = 0; kp < 4; kp++) {
                const float am = 4 * g + kp <= c ? gq[kp] : 0.0f;
                ov = __builtin_amdgcn_mfma_f32_16x16x4f32(am, ddm[kp], ov, 0, 0, 0);
            }
            // S_16 = diag(exp(G_15)) S_0 + Kt^T Delta: the row decay, then tiles of the update with
            // the three parts of Kt read transposed and Delta in three parts
#pragma unroll
            for (int st = 0; st < 4; st++) {
                const f4 e0 = *reinterpret_cast<const f4*>(&sl.eG15[32 * st + 8 * g]);
                const f4 e1 = *reinterpret_cast<const f4*>(&sl.eG15[32 * st + 8 * g + 4]);
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    s[8 * st + j] *= e0[j];
                    s[8 * st + 4 + j] *= e1[j];
                }
            }
            bf4 dp[3];
            split3<4>(ddm, dp[0], dp[1], dp[2]);
#pragma unroll
            for (int tau = 0; tau < 8; tau++) {
                s4 kr[3];
#pragma unroll
                for (int pp = 0; pp < 3; pp++)
                    kr[pp] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(&sl.Kt[pp][0][0] + tr_offset(g, c, tau)));
                f4 st = {s[4 * tau], s[4 * tau + 1], s[4 * tau + 2], s[4 * tau + 3]};
                st = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(kr[0], __builtin_bit_cast(s4, dp[2]), st, 0, 0, 0);
                st = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(kr[2], __builtin_bit_cast(s4, dp[0]), st, 0, 0, 0);
                st = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(kr[1], __builtin_bit_cast(s4, dp[1]), st, 0, 0, 0);
                st = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(kr[0], __builtin_bit_cast(s4, dp[1]), st, 0, 0, 0);
                st = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(kr[1], __builtin_bit_cast(s4, dp[0]), st, 0, 0, 0);
                st = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(kr[0], __builtin_bit_cast(s4, dp[0]), st, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 4; r++) s[4 * tau + r] = st[r];
            }
            if (has_o) {
#pragma unroll
                for (int r = 0; r < 4; r++) store_o(t0, r, ov[r]);
            }
        } else {
            // steep gates: token by token, each token's per-key gates applied to the state rows
            const int voff_g = 0;
#pragma unroll 1
            for (int j = 0; j < kBlk && t0 + j < T; j++) {
                const float bj = sl.beta[j];
                const int sg = ((t0 + j) * H + h) * DK * GB;
#pragma unroll
                for (int st = 0; st < 4; st++) {
                    float gv[8];
                    if (GF32) {
                        const u4 w0 = __builtin_amdgcn_raw_buffer_load_b128(rgk, voff_g + gate_word_off(st, 0), sg, 0);
                        const u4 w1 = __builtin_amdgcn_raw_buffer_load_b128(rgk, voff_g + gate_word_off(st, 1), sg, 0);
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            gv[e] = __uint_as_float(w0[e]);
                            gv[4 + e] = __uint_as_float(w1[e]);
                        }
                    } else {
                        const u4 w0 = __builtin_amdgcn_raw_buffer_load_b128(rgk, voff_g + gate_word_off(st, 0), sg, 0);
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            gv[2 * e] = __uint_as_float(w0[e] << 16);
                            gv[2 * e + 1] = __uint_as_float(w0[e] & 0xFFFF0000u);
                        }
                    }
#pragma unroll
                    for (int e = 0; e < 8; e++) s[8 * st + e] *= expf(gv[e]);
                }
                const int so = ((t0 + j) * H + h) * DK * 2;
                const int eoff = state_row(2 * c, g) * 2;
                const uint32_t kwd = __builtin_amdgcn_raw_buffer_load_b32(rk, eoff, so, 0);
                const uint32_t qwd = __builtin_amdgcn_raw_buffer_load_b32(rq, eoff, so, 0);
                float k0, k1, q0, q1;
                widen_pairs(kwd, qwd, k0, k1, q0, q1);
                const float kq = wave_sum(__builtin_fmaf(k1, q1, k0 * q0));
                float pk, pq, P, Q;
                dot_pass<R>(s, k0, k1, q0, q1, pk, pq);
                rows_sum2(pk, pq, P, Q);
                const uint32_t vwd = __builtin_amdgcn_raw_buffer_load_b16(rv, col * 2, ((t0 + j) * H + h) * DV * 2, 0);
                const float delta = bj * (bf_lo(vwd) - P);
                const float o = __builtin_fmaf(delta, kq, Q);
                update_pass<R>(s, k0, k1, delta);
                if (has_o && g == 0) {
                    const int so_o = ((t0 + j) * H + h) * DV * OB;
                    if (OBF16) __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(o), ro, col * OB, so_o, 0);
                    else __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o), ro, col * OB, so_o, 0);
                }
            }
        }

        if (min(t0 + kBlk, T) - 1 == q_next) {
            wave_quantize<R, QMODE, G>(s, qsh, lane, w, qpar);
            q_next = next_q(q_next);
        }
        __syncthreads();  // slots handed over
#pragma unroll
        for (int r = 0; r < 4; r++) vcur[r] = vnxt[r];
    }
    if (a.ST) {
#pragma unroll
        for (int m = 0; m < R; m++) a.ST[state_off + static_cast<size_t>(state_row(m, g)) * DV + col] = s[m];
    }
}

namespace {

template <int QMODE, int G, bool GF32>
hipError_t launch_mfma_o(const la_config& c, const FwdArgs& a, hipStream_t s) {
    dim3 grid(c.d_v / kTileCols, c.H, c.B);
    if (c.gate == LA_GATE_KEY) {
        if (c.out_dtype == LA_BF16)
            hipLaunchKernelGGL((fwd_mfma_kda_kernel<QMODE, G, GF32, true>), grid, dim3(kKdaThreads), 0, s, make_params(c), a);
        else
            hipLaunchKernelGGL((fwd_mfma_kda_kernel<QMODE, G, GF32, false>), grid, dim3(kKdaThreads), 0, s, make_params(c), a);
    } else if (c.out_dtype == LA_BF16) {
        hipLaunchKernelGGL((fwd_mfma_kernel<QMODE, G, GF32, true>), grid, dim3(kPcThreads), 0, s, make_params(c), a);
    } else {
        hipLaunchKernelGGL((fwd_mfma_kernel<QMODE, G, GF32, false>), grid, dim3(kPcThreads), 0, s, make_params(c), a);
    }
    return hipGetLastError();
}

template <int QMODE, int G>
hipError_t launch_mfma_t(const la_config& c, const FwdArgs& a, hipStream_t s) {
    if (c.gate_dtype == LA_F32) return launch_mfma_o<QMODE, G, true>(c, a, s);
    return launch_mfma_o<QMODE, G, false>(c, a, s);
}

template <int QMODE, int G>
hipError_t launch_chunks_t(const la_config& c, const FwdArgs& a, const Params& p, hipStream_t s) {
    dim3 grid(c.d_v / kTileCols, c.H, c.B * p.nch);
    if (c.gate_dtype == LA_F32)
        hipLaunchKernelGGL((fwd_mfma_kernel<QMODE, G, true, false>), grid, dim3(kPcThreads), 0, s, p, a);
    else
        hipLaunchKernelGGL((fwd_mfma_kernel<QMODE, G, false, false>), grid, dim3(kPcThreads), 0, s, p, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_mfma_chunks(const la_config& c, const FwdArgs& a, int t_off, int t_end, hipStream_t s) {
    la_config cc = c;
    cc.ckpt_interval = kBlk;
    Params p = make_params(cc);
    p.chunk = c.ckpt_interval;
    p.nch = (t_end - t_off + p.chunk - 1) / p.chunk;
    p.t_off = t_off;
    p.t_end = t_end;
    p.stride_T = c.T;
    p.nck_in = n_ckpts(c);
    p.nck = (t_end - t_off + kBlk - 1) / kBlk;
    if (c.qdq == LA_QDQ_NONE) return launch_chunks_t<LA_QDQ_NONE, 1>(c, a, p, s);
    if (c.qdq == LA_QDQ_E4M3_TILE) return launch_chunks_t<LA_QDQ_E4M3_TILE, 64>(c, a, p, s);
    switch (c.group) {
        case 16: return launch_chunks_t<LA_QDQ_INT8_GROUP, 16>(c, a, p, s);
        case 32: return launch_chunks_t<LA_QDQ_INT8_GROUP, 32>(c, a, p, s);
        default: return launch_chunks_t<LA_QDQ_INT8_GROUP, 64>(c, a, p, s);
    }
}

bool fwd_mfma_eligible(const la_config& c) {
    if (c.replay && c.qdq_interval > 1) return false;  // encoded updates: token by token
    if (c.gate == LA_GATE_KEY) {
        // per-key gates: the scalar-gate kernels' rounding conditions, without their rescale
        if (c.hadamard) return false;
        if (c.qdq != LA_QDQ_NONE &&
            (c.qdq_interval < 2 || (c.ckpt_interval > 0 && c.qdq_interval % c.ckpt_interval != 0)))
            return false;
    } else if (!fwd_fast_eligible(c)) {
        return false;
    }
    if (c.d_k != 128 || c.qkv_dtype != LA_BF16) return false;
    if (c.qdq != LA_QDQ_NONE && c.qdq_interval % kBlk != 0) return false;
    if (c.ckpt_interval > 0 && c.ckpt_interval % kBlk != 0) return false;
    // 32-bit buffer offsets within one sequence, the prefetched block included
    const size_t span = static_cast<size_t>(c.T + 2 * kBlk) * c.H * (c.d_k > c.d_v ? c.d_k : c.d_v) * 4;
    // and within one unit's checkpoints
    const size_t ck_span = static_cast<size_t>(n_ckpts(c)) * c.d_k * c.d_v * 4;
    return span < (static_cast<size_t>(1) << 31) && ck_span < (static_cast<size_t>(1) << 31);
}

hipError_t launch_fwd_mfma(const la_config& c, const FwdArgs& a, hipStream_t s) {
    if (c.qdq == LA_QDQ_NONE) return launch_mfma_t<LA_QDQ_NONE, 1>(c, a, s);
    if (c.qdq == LA_QDQ_E4M3_TILE) return launch_mfma_t<LA_QDQ_E4M3_TILE, 64>(c, a, s);
    switch (c.group) {
        case 16: return launch_mfma_t<LA_QDQ_INT8_GROUP, 16>(c, a, s);
        case 32: return launch_mfma_t<LA_QDQ_INT8_GROUP, 32>(c, a, s);
        default: return launch_mfma_t<LA_QDQ_INT8_GROUP, 64>(c, a, s);
    }
}

}  // namespace la
