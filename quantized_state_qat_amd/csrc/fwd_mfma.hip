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
// itself, regrouped; every product is formed in fp32.  Per wave (128 key rows x 16 value
// columns, lane 16 g + c holding column c and rows 32 g + m in s[m]):
//  * P', Q' (16 tokens x 16 columns each): bf16 MFMAs (16x16x32) of the raw keys and queries
//    (exact in bf16) with the state split exactly into three bf16 parts, 3 x 4 K-slices each;
//    slice i uses s[8 i .. 8 i + 7], and the key rows are assigned so that the same slice of
//    a token's keys is the lane's 16-byte load i (the four lane groups together reading one
//    coalesced 64-byte line): s[m] of lane group g is key row 32 (m / 8) + 8 g + m % 8;
//  * the Gram matrices K K^T and K Q^T: bf16 MFMAs on the raw keys and queries (exact
//    products, fp32 sums);
//  * the triangular recurrence for dd in four stages: lane group g solves tokens 4 g .. 4 g + 3
//    of its column from its own coefficients, and after each stage one fp32 MFMA adds the
//    stage's dd to the projections of all later tokens;
//  * o = Gamma (Q' + tril(K Q^T)^T DD): 4 fp32 MFMAs on the Gram output registers;
//  * S_0 + K^T DD: bf16 MFMAs (16x16x16) with s[4 tau .. 4 tau + 3] as the accumulator tile
//    tau, the keys read transposed from LDS and DD split exactly into three bf16 parts; then
//    the fold by Gamma_15.
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

constexpr int kMThreads = kWaveTileWaves * 64;  // 4 waves = 64 value columns
constexpr float kGammaLo = 0x1p-60f, kGammaHi = 0x1p60f;
constexpr int kDppRowShr = 0x110;              // row_shr:n = kDppRowShr + n
// Per-wave LDS of one block.
struct BlockShared {
    float Gk[kBlk][kBlk];    // [j][i] = k_i . k_j
    float dd[4][kBlk][4];    // [lane group][column][r]: stage values of tokens 4 g + r, for the stage MFMAs
    float Ms[kBlk][20];      // [c][j] = M[j][c] (rows padded to 20 floats: no bank conflicts)
    float gam[kBlk], rgam[kBlk], beta[kBlk];
};

// Product with identity-filled lanes: x[lane - n] of the same row of 16, 1.0 below the row.
template <int N>
__device__ __forceinline__ float row_shr_or_one(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.0f), __float_as_int(x), kDppRowShr + N, 0xF, 0xF, false));
}

}  // namespace

template <int QMODE, int G, bool GF32, bool OBF16>
__global__ __launch_bounds__(kMThreads) void fwd_mfma_kernel(Params p, FwdArgs a) {
    constexpr int DK = 128, R = 32;
    constexpr int GB = GF32 ? 4 : 2, OB = OBF16 ? 2 : 4;

    __shared__ WaveQdqShared<DK, QMODE, G> qsh;
    __shared__ uint16_t kN[kWaveTileWaves][kBlk][kKeyRow];  // per wave: the block's keys, [token][row]
    __shared__ BlockShared bsh[kWaveTileWaves];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, c = lane & 15;
    const int h = blockIdx.y, b = blockIdx.z;
    const int col = blockIdx.x * kTileCols + w * kWaveCols + c;
    const int T = p.T, H = p.H, DV = p.dv;
    const size_t bh = static_cast<size_t>(b) * H + h;
    const size_t state_off = bh * DK * DV;
    const size_t seq0 = static_cast<size_t>(b) * T * H;
    const size_t seq_tok = static_cast<size_t>(T) * H;
    BlockShared& sh = bsh[w];

    // Buffer resources over exactly this sequence's tokens (offsets < 2^31, checked on the
    // host): reads past its last token return zero, stores there are dropped.
    const auto rk = make_rsrc(static_cast<const char*>(a.k) + seq0 * DK * 2, seq_tok * DK * 2);
    const auto rq = make_rsrc(static_cast<const char*>(a.q) + seq0 * DK * 2, seq_tok * DK * 2);
    const auto rv = make_rsrc(static_cast<const char*>(a.v) + seq0 * DV * 2, seq_tok * DV * 2);
    const auto rgt = make_rsrc(static_cast<const char*>(a.g) + seq0 * GB, seq_tok * GB);
    const auto rbt = make_rsrc(static_cast<const char*>(a.beta) + seq0 * GB, seq_tok * GB);
    // this unit's checkpoints (the eligibility check keeps their offsets below 2^31)
    const size_t ck_unit = static_cast<size_t>(p.nck) * DK * DV;
    const auto rck = make_rsrc(a.ckpts ? a.ckpts + bh * ck_unit : nullptr, a.ckpts ? ck_unit * 4 : 0);
    const int voff_ck = (state_row(0, g) * DV + col) * 4;
    const bool has_o = a.o != nullptr;
    const auto ro = make_rsrc(has_o ? static_cast<const char*>(a.o) + seq0 * DV * OB : nullptr,
                              has_o ? seq_tok * DV * OB : 0);

    // ---------------------------------------------------------------- state
    float s[R];
#pragma unroll
    for (int m = 0; m < R; m++)
        s[m] = a.S0 ? a.S0[state_off + static_cast<size_t>(state_row(m, g)) * DV + col] : 0.0f;
    __builtin_amdgcn_s_waitcnt(0);

    // ---------------------------------------------------------------- block inputs
    // Lane (g, c): the keys and queries of token t0 + c at rows state_row(0..31, g) (load i
    // brings rows 32 i + 8 g .. + 7, the four lane groups together one 64-byte line); the
    // values of tokens t0 + 4 g .. 4 g + 3 at its column; gate and beta of token t0 + c.
    struct BlockIn {
        u4 k[4], q[4];
        uint32_t v[4];
        uint32_t g, b;
    };
    const int voff_kq = (c * H * DK + 8 * g) * 2;
    const int voff_v = (4 * g * H * DV + col) * 2;
    const int voff_gate = c * H * GB;
    // The loads of a block in three parts (keys; queries; values, gates and beta).  The four
    // waves of a workgroup load the same keys and queries, so a burst of all of them fills the
    // CU's address queue and stalls the issuing wave for about a thousand cycles; the block
    // loop spreads the parts of the next block's loads over its first steps instead.
    auto fetch_part = [&](BlockIn& in, int t0, int part) __attribute__((always_inline)) {
        const int so = (t0 * H + h) * DK * 2;
        if (part == 0) {
#pragma unroll
            for (int i = 0; i < 4; i++) in.k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, voff_kq + 64 * i, so, 0);
            return;
        }
        if (part == 1) {
#pragma unroll
            for (int i = 0; i < 4; i++) in.q[i] = __builtin_amdgcn_raw_buffer_load_b128(rq, voff_kq + 64 * i, so, 0);
            return;
        }
#pragma unroll
        for (int r = 0; r < 4; r++)
            in.v[r] = __builtin_amdgcn_raw_buffer_load_b16(rv, voff_v, ((t0 + r) * H + h) * DV * 2, 0);
        const int sg = (t0 * H + h) * GB;
        if (GF32) {
            in.g = __builtin_amdgcn_raw_buffer_load_b32(rgt, voff_gate, sg, 0);
            in.b = __builtin_amdgcn_raw_buffer_load_b32(rbt, voff_gate, sg, 0);
        } else {
            in.g = __builtin_amdgcn_raw_buffer_load_b16(rgt, voff_gate, sg, 0);
            in.b = __builtin_amdgcn_raw_buffer_load_b16(rbt, voff_gate, sg, 0);
        }
    };
    auto fetch = [&](BlockIn& in, int t0) __attribute__((always_inline)) {
        fetch_part(in, t0, 0);
        fetch_part(in, t0, 1);
        fetch_part(in, t0, 2);
    };

    // ---------------------------------------------------------------- outputs
    const int voff_o = (4 * g * H * DV + col) * OB;  // register r: token t0 + 4 g + r
    auto store_o = [&](int t0, int r, float ov) __attribute__((always_inline)) {
        const int so = ((t0 + r) * H + h) * DV * OB;
        if (OBF16) __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(ov), ro, voff_o, so, 0);
        else __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ov), ro, voff_o, so, 0);
    };

    // ---------------------------------------------------------------- block loop
    // Order of issue within a block: the Gram MFMAs, with the next block's loads spread over the
    // gates and the transposed keys; the solve for M interleaved with the projection MFMAs;
    // dd = M R; the output and update MFMAs; the fold.
    int qpar = 0;
    const int qi = p.qdq_interval;
    int q_next = QMODE != LA_QDQ_NONE ? min(qi, T) - 1 : T;
    int ck_next = a.ckpts ? 0 : T;

    BlockIn cur, nxt;
    fetch(cur, 0);
#pragma unroll 1
    for (int t0 = 0; t0 < T; t0 += kBlk) {
        if (t0 == ck_next) {
            const int so = t0 / p.ckpt_interval * DK * DV * 4;
            if (a.ckpt_lane_major) {
                // lane-major: s[0..31] of lane L of wave slice col / 16 at float (slice 64 + L) 32
                const int vo = ((col >> 4) * 64 + lane) * R * 4;
#pragma unroll
                for (int i = 0; i < R / 4; i++)
                    __builtin_amdgcn_raw_buffer_store_b128(
                        u4{__float_as_uint(s[4 * i]), __float_as_uint(s[4 * i + 1]), __float_as_uint(s[4 * i + 2]),
                           __float_as_uint(s[4 * i + 3])}, rck, vo + 16 * i, so, 0);
            } else {
                // rows state_row(m, g) = state_row(0, g) + 32 (m / 8) + m % 8: the row step is uniform
#pragma unroll
                for (int m = 0; m < R; m++)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s[m]), rck, voff_ck,
                                                          so + (32 * (m >> 3) + (m & 7)) * DV * 4, 0);
            }
            ck_next += p.ckpt_interval;
        }

        // Gram matrices: gk (lane (g, n), register r) = k_{4g+r} . k_n, gq = k_{4g+r} . q_n
        f4 gk = {0.0f, 0.0f, 0.0f, 0.0f}, gq = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const bf8 ak = __builtin_bit_cast(bf8, cur.k[i]), aq = __builtin_bit_cast(bf8, cur.q[i]);
            gk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, ak, gk, 0, 0, 0);
            gq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, aq, gq, 0, 0, 0);
        }
        fetch_part(nxt, t0 + kBlk, 0);  // the next block's keys

        // gates of the block: lane (g, c) holds token t0 + c; every row of 16 computes the
        // same inclusive product
        const bool valid = t0 + c < T;
        const float gv = GF32 ? __uint_as_float(cur.g) : bf_lo(cur.g);
        const float bv = GF32 ? __uint_as_float(cur.b) : bf_lo(cur.b);
        const float eg = valid ? expf(gv) : 1.0f;
        float gam = eg;
        gam *= row_shr_or_one<1>(gam);
        gam *= row_shr_or_one<2>(gam);
        gam *= row_shr_or_one<4>(gam);
        gam *= row_shr_or_one<8>(gam);
        const bool in_range = __all(gam >= kGammaLo && gam <= kGammaHi);
        if (g == 0) {
            sh.gam[c] = gam;
            sh.rgam[c] = 1.0f / gam;
            sh.beta[c] = valid ? bv : 0.0f;
        }
        fetch_part(nxt, t0 + kBlk, 1);  // ... its queries
        // the block's keys into this wave's own LDS copy for the update, as loaded (token c,
        // rows 32 i + 8 g .. + 7 from load i), so that the update waits for no other wave
        uint16_t (*kNw)[kKeyRow] = kN[w];
#pragma unroll
        for (int i = 0; i < 4; i++) *reinterpret_cast<u4*>(&kNw[c][32 * i + 8 * g]) = cur.k[i];
        fetch_part(nxt, t0 + kBlk, 2);  // ... its values, gates and beta
        *reinterpret_cast<f4*>(&sh.Gk[c][4 * g]) = gk;  // symmetric: [c][i] = k_i . k_c
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_sched_barrier(0);

        // Gamma_15, applied to the state after either path (1 after the token-by-token one): the
        // loop-carried state leaves both paths through the same multiply, so no register copies
        float fold = 1.0f;
        if (__builtin_expect(in_range, 1)) {
            // per-lane constants of the recurrence: this lane group's tokens 4 g + r ...
            const f4 gam4 = *reinterpret_cast<const f4*>(&sh.gam[4 * g]);
            const f4 rgam4 = *reinterpret_cast<const f4*>(&sh.rgam[4 * g]);
            const f4 beta4 = *reinterpret_cast<const f4*>(&sh.beta[4 * g]);
            // ... k_{4g+i} . k_{4g+j} within the group (i < j) ...
            const float c01 = sh.Gk[4 * g + 1][4 * g], c02 = sh.Gk[4 * g + 2][4 * g];
            const float c12 = sh.Gk[4 * g + 2][4 * g + 1], c03 = sh.Gk[4 * g + 3][4 * g];
            const float c13 = sh.Gk[4 * g + 3][4 * g + 1], c23 = sh.Gk[4 * g + 3][4 * g + 2];
            // ... and the stage MFMAs' A operands: lane (kk, j) = k_{4s+kk} . k_j for tokens j
            // of later groups (j >= 4 s + 4), else 0
            float ast[3];
#pragma unroll
            for (int st = 0; st < 3; st++) ast[st] = c >= 4 * st + 4 ? sh.Gk[c][4 * st + g] : 0.0f;

            // M = (I + diag(beta) L)^{-1} diag(beta), L the strictly lower part of K K^T, so that
            // dd = M (V / Gamma - P'): the four-stage solve on the identity (lane (g, c) solves
            // column c for tokens 4 g .. 4 g + 3; after stage st, lane group st's values are final
            // and the stage MFMA adds their contribution to the later tokens).  It needs only the
            // keys and beta, so its stages are interleaved with the slices of the projections of
            // the entering state, whose MFMAs run while a stage waits on its own results.
            // Projections: dk (lane (g, c), register r) = P'_{4g+r}[c], dq = Q'.
            f4 dk = {0.0f, 0.0f, 0.0f, 0.0f}, dq = {0.0f, 0.0f, 0.0f, 0.0f}, dm = {0.0f, 0.0f, 0.0f, 0.0f};
            f4 selm = {0.0f, 0.0f, 0.0f, 0.0f};
            // The exact bf16 parts of the state slices (slice st: s[8 st .. 8 st + 7], key rows
            // 32 st .. 32 st + 31 of this lane's list), one slice ahead: slice st + 1 is split while
            // slice st's MFMAs run, one MFMA between every seven vector instructions.
            uint32_t ph[2][4], pl[2][4], pl2[2][4];
            auto split_pairs = [&](int st, int b, int i0) __attribute__((always_inline)) {
#pragma unroll
                for (int i = i0; i < i0 + 2; i++)
                    split3_pair(s[8 * st + 2 * i], s[8 * st + 2 * i + 1], ph[b][i], pl[b][i], pl2[b][i]);
            };
            auto bf8_of = [](const uint32_t (&x)[4]) __attribute__((always_inline)) {
                return __builtin_bit_cast(bf8, u4{x[0], x[1], x[2], x[3]});
            };
            split_pairs(0, 0, 0);
            split_pairs(0, 0, 2);
#pragma unroll
            for (int st = 0; st < 4; st++) {
                const int b = st & 1;
                const float e0 = 4 * g == c ? 1.0f : 0.0f, e1 = 4 * g + 1 == c ? 1.0f : 0.0f;
                const float e2 = 4 * g + 2 == c ? 1.0f : 0.0f, e3 = 4 * g + 3 == c ? 1.0f : 0.0f;
                const float x0 = beta4[0] * (e0 - dm[0]);
                const float x1 = beta4[1] * (e1 - __builtin_fmaf(c01, x0, dm[1]));
                const float x2 = beta4[2] * (e2 - __builtin_fmaf(c12, x1, __builtin_fmaf(c02, x0, dm[2])));
                const float x3 = beta4[3] * (e3 - __builtin_fmaf(c23, x2, __builtin_fmaf(c13, x1, __builtin_fmaf(c03, x0, dm[3]))));
                if (g == st) selm = f4{x0, x1, x2, x3};
                if (st < 3) {
                    const f4 xv = {x0, x1, x2, x3};
                    *reinterpret_cast<f4*>(&sh.dd[g][c][0]) = xv;
                }
                __builtin_amdgcn_sched_barrier(0);
                const bf8 ak = __builtin_bit_cast(bf8, cur.k[st]), aq = __builtin_bit_cast(bf8, cur.q[st]);
                const bf8 h = bf8_of(ph[b]), l = bf8_of(pl[b]), l2 = bf8_of(pl2[b]);
                dk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, l2, dk, 0, 0, 0);
                dq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, l2, dq, 0, 0, 0);
                dk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, l, dk, 0, 0, 0);
                if (st < 3) split_pairs(st + 1, b ^ 1, 0);
#pragma unroll
                for (int r = 0; r < 3; r++) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
                if (st < 3) {
                    __builtin_amdgcn_wave_barrier();
                    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
                    const float bst = sh.dd[st][c][g];  // B: lane (kk, n) = M[4 st + kk][n]
                    dm = __builtin_amdgcn_mfma_f32_16x16x4f32(ast[st], bst, dm, 0, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
                dq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, l, dq, 0, 0, 0);
                dk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, h, dk, 0, 0, 0);
                dq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, h, dq, 0, 0, 0);
                if (st < 3) split_pairs(st + 1, b ^ 1, 2);
#pragma unroll
                for (int r = 0; r < 3; r++) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            // M transposed through LDS: lane (g, c) needs M[c][4 g + s], the A operand of slice s
            *reinterpret_cast<f4*>(&sh.Ms[c][4 * g]) = selm;
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            // dd = M R with R = V / Gamma - P': slice s pairs input token 4 g + s (lane group g)
            // with A = M[c][4 g + s] and B = R[4 g + s][c], this lane's register s of R
            f4 ddm = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int sl = 0; sl < 4; sl++) {
                const float rr = __builtin_fmaf(bf_lo(cur.v[sl]), rgam4[sl], -dk[sl]);
                ddm = __builtin_amdgcn_mfma_f32_16x16x4f32(sh.Ms[4 * g + sl][c], rr, ddm, 0, 0, 0);
            }
            const float sel[4] = {ddm[0], ddm[1], ddm[2], ddm[3]};

            // o_i = Gamma_i (Q'_i + sum_{j <= i} (k_j . q_i) dd_j)
            f4 ov = dq;
#pragma unroll
            for (int kp = 0; kp < 4; kp++) {
                const float am = 4 * g + kp <= c ? gq[kp] : 0.0f;
                ov = __builtin_amdgcn_mfma_f32_16x16x4f32(am, sel[kp], ov, 0, 0, 0);
            }

            // S_0 + K^T DD, tile tau = s[4 tau .. 4 tau + 3]: accumulator row i = 4 g' + r is
            // key row state_row(4 tau + r, g'); A (row i = c, tokens 4 g .. 4 g + 3) = the keys
            // of those tokens there; B (tokens 4 g + j, column c) = dd, in three bf16 parts.
            // A comes from the gfx950 transposed LDS read (tr_offset).
            const f4 ddv = {sel[0], sel[1], sel[2], sel[3]};
            bf4 dh, dl, dl2;
            split3<4>(ddv, dh, dl, dl2);
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
            for (int tau = 0; tau < 8; tau++) {
                const s4 kr = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(&kN[w][0][0] + tr_offset(g, c, tau)));
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
            fold = lane_of(gam, kBlk - 1);
        } else {
            // steep gates: token by token, each gate applied to the state
#pragma unroll 1
            for (int j = 0; j < kBlk && t0 + j < T; j++) {
                const float aj = lane_of(eg, j);
                const float bj = sh.beta[j];
#pragma unroll
                for (int m = 0; m < R; m++) s[m] *= aj;
                // keys and queries of token t0 + j in the DPP layout: lane L of row group g holds
                // rows 2 L, 2 L + 1 of the group's list, state_row(2 L, g) and the next
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
            q_next = q_next + qi <= T - 1 ? q_next + qi : (q_next < T - 1 ? T - 1 : T);
        }
        cur = nxt;
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
    if (c.out_dtype == LA_BF16)
        hipLaunchKernelGGL((fwd_mfma_kernel<QMODE, G, GF32, true>), grid, dim3(kMThreads), 0, s, make_params(c), a);
    else
        hipLaunchKernelGGL((fwd_mfma_kernel<QMODE, G, GF32, false>), grid, dim3(kMThreads), 0, s, make_params(c), a);
    return hipGetLastError();
}

template <int QMODE, int G>
hipError_t launch_mfma_t(const la_config& c, const FwdArgs& a, hipStream_t s) {
    if (c.gate_dtype == LA_F32) return launch_mfma_o<QMODE, G, true>(c, a, s);
    return launch_mfma_o<QMODE, G, false>(c, a, s);
}

}  // namespace

bool fwd_mfma_eligible(const la_config& c) {
    if (!fwd_fast_eligible(c)) return false;
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
