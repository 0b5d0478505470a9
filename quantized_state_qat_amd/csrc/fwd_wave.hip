// Long-sequence forward for the scalar gate when the state is rounded at most once per block
// of 8 tokens (no quantizer, or INT8/E4M3 at an interval that is a multiple of 8): the
// FP32-VALU-bound path, with no barrier and no LDS traffic per token.
//
// One wave owns 16 value columns of one (sequence, head); four waves (64 columns, one E4M3
// tile) form a workgroup and meet only at quantization points.  Lane 16 r + c holds column c
// and key rows [r R, (r+1) R), R = d_k / 4, in registers.  Per token:
//  * the row group's keys and queries arrive spread over its 16 lanes (one word per lane)
//    and reach the FMAs through DPP row broadcasts (row_newbcast), so the pass
//    P = Shat^T k, Q = Shat^T q costs two FMAs per state element and nothing else;
//  * the four row groups' partial sums meet through two permlane swaps;
//  * the state is carried rescaled, S = F Shat, with F the product of the gates since the
//    last fold, so the update S' = a S + k delta^T is one FMA per element:
//    Shat += k (delta / F');
//  * gates come in windows of 64 tokens: lane i of the window registers holds exp(g),
//    beta and the running gate product of token w0 + i, and a token reads its three
//    scalars with readlane.  The product is range-checked once per block of 8 tokens and
//    folded into Shat before it leaves [2^-30, 2^30]; a block whose own gates span more
//    than that range is run with the gate applied to the state token by token;
//  * k, q and v of the next 8 tokens are in flight in a register ring (buffer loads; reads
//    past the end of the tensor return zero and are never used).
// Rounding points and checkpoints fall on block boundaries, where the state is folded
// (F = 1) before it is rounded or stored.
#include <type_traits>
#include <utility>

#include "la_device.hpp"
#include "la_internal.hpp"
#include "la_recur.hpp"

namespace la {

Params make_params(const la_config& c);

namespace {

constexpr int kWaveCols = 16;
constexpr int kWaveTileWaves = kTileCols / kWaveCols;  // 4 waves = 64 columns
constexpr int kWaveThreads = kWaveTileWaves * 64;
constexpr int kRing = 8;   // tokens per block and depth of the input ring
constexpr int kWin = 64;   // tokens per gate window
constexpr float kFoldLo = 0x1p-30f, kFoldHi = 0x1p30f;

// The two FMA passes are written as blocks of DPP instructions: acc (+)= x[lane L of this
// lane's row of 16] * y (row_newbcast:L).  A DPP instruction must not read a VGPR that a
// VALU instruction wrote in the two preceding wait states; inside the blocks the four
// accumulator chains are interleaved so that each accumulator is rewritten every fourth
// instruction, the state rows read by the dot pass were written one pass earlier, and the
// update blocks start with s_nop 1 because the scale they read has just been computed.
#define LA_DPP(op, d, x, y, L) #op " %" #d ", %" #x ", %" #y " row_newbcast:" #L " row_mask:0xf bank_mask:0xf\n\t"

// d_k = 128: lane L holds key rows 2L (k0) and 2L+1 (k1) of its row group.  Operands:
// %0..%3 = pk0, pq0, pk1, pq1; %4..%7 = k0, k1, q0, q1; %8..%39 = the 32 state rows.
#define LA_DOT2(L, E, O) \
    LA_DPP(v_fmac_f32_dpp, 0, 4, E, L) LA_DPP(v_fmac_f32_dpp, 1, 6, E, L) \
    LA_DPP(v_fmac_f32_dpp, 2, 5, O, L) LA_DPP(v_fmac_f32_dpp, 3, 7, O, L)
#define LA_DOT2_FIRST(L, E, O) \
    LA_DPP(v_mul_f32_dpp, 0, 4, E, L) LA_DPP(v_mul_f32_dpp, 1, 6, E, L) \
    LA_DPP(v_mul_f32_dpp, 2, 5, O, L) LA_DPP(v_mul_f32_dpp, 3, 7, O, L)
// update: %0..%31 = the 32 state rows (in/out); %32, %33 = k0, k1; %34 = scale
#define LA_UPD2(L, E, O) LA_DPP(v_fmac_f32_dpp, E, 32, 34, L) LA_DPP(v_fmac_f32_dpp, O, 33, 34, L)

// d_k = 64: lane L holds key row L.  Even rows accumulate into pk0/pq0, odd rows into
// pk1/pq1.  Operands: %0..%3 = pk0, pq0, pk1, pq1; %4, %5 = k, q; %6..%21 = 16 state rows.
#define LA_DOT1(L0, L1, S0, S1) \
    LA_DPP(v_fmac_f32_dpp, 0, 4, S0, L0) LA_DPP(v_fmac_f32_dpp, 1, 5, S0, L0) \
    LA_DPP(v_fmac_f32_dpp, 2, 4, S1, L1) LA_DPP(v_fmac_f32_dpp, 3, 5, S1, L1)
// update: %0..%15 = state rows; %16 = k; %17 = scale
#define LA_UPD1(L, S) LA_DPP(v_fmac_f32_dpp, S, 16, 17, L)

#define LA_S16(a) "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]), \
    "+v"(a[7]), "+v"(a[8]), "+v"(a[9]), "+v"(a[10]), "+v"(a[11]), "+v"(a[12]), "+v"(a[13]), "+v"(a[14]), "+v"(a[15])
#define LA_I16(a) "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), \
    "v"(a[8]), "v"(a[9]), "v"(a[10]), "v"(a[11]), "v"(a[12]), "v"(a[13]), "v"(a[14]), "v"(a[15])
#define LA_S32(a) LA_S16(a), LA_S16((a + 16))
#define LA_I32(a) LA_I16(a), LA_I16((a + 16))

// Single DPP FMAs for the small key sizes (d_k = 16, 32), where the pass is short; each
// waits out the hazard itself, whatever the compiler placed before it.
template <int L>
__device__ __forceinline__ void fmac_bcast(float& acc, float x, float y) {
    asm("s_nop 1\n\tv_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
        : "+v"(acc) : "v"(x), "v"(y), "n"(L));
}

// P, Q = partial sums over this lane's R rows of Shat^T k and Shat^T q.
template <int R>
__device__ __forceinline__ void dot_pass(const float* s, float k0, float k1, float q0, float q1, float& P, float& Q) {
    float pk0, pq0, pk1, pq1;
    if constexpr (R == 32) {
        asm("s_nop 1\n\t"
            LA_DOT2_FIRST(0, 8, 9) LA_DOT2(1, 10, 11) LA_DOT2(2, 12, 13) LA_DOT2(3, 14, 15)
            LA_DOT2(4, 16, 17) LA_DOT2(5, 18, 19) LA_DOT2(6, 20, 21) LA_DOT2(7, 22, 23)
            LA_DOT2(8, 24, 25) LA_DOT2(9, 26, 27) LA_DOT2(10, 28, 29) LA_DOT2(11, 30, 31)
            LA_DOT2(12, 32, 33) LA_DOT2(13, 34, 35) LA_DOT2(14, 36, 37) LA_DOT2(15, 38, 39)
            : "=&v"(pk0), "=&v"(pq0), "=&v"(pk1), "=&v"(pq1)
            : "v"(k0), "v"(k1), "v"(q0), "v"(q1), LA_I32(s));
    } else if constexpr (R == 16) {
        asm("s_nop 1\n\t"
            LA_DPP(v_mul_f32_dpp, 0, 4, 6, 0) LA_DPP(v_mul_f32_dpp, 1, 5, 6, 0)
            LA_DPP(v_mul_f32_dpp, 2, 4, 7, 1) LA_DPP(v_mul_f32_dpp, 3, 5, 7, 1)
            LA_DOT1(2, 3, 8, 9) LA_DOT1(4, 5, 10, 11) LA_DOT1(6, 7, 12, 13) LA_DOT1(8, 9, 14, 15)
            LA_DOT1(10, 11, 16, 17) LA_DOT1(12, 13, 18, 19) LA_DOT1(14, 15, 20, 21)
            : "=&v"(pk0), "=&v"(pq0), "=&v"(pk1), "=&v"(pq1)
            : "v"(k0), "v"(q0), LA_I16(s));
    } else {
        pk0 = pq0 = pk1 = pq1 = 0.0f;
        [&]<int... M>(std::integer_sequence<int, M...>) {
            ((fmac_bcast<M>(M & 1 ? pk1 : pk0, k0, s[M]), fmac_bcast<M>(M & 1 ? pq1 : pq0, q0, s[M])), ...);
        }(std::make_integer_sequence<int, R>{});
    }
    P = pk0 + pk1;
    Q = pq0 + pq1;
}

// Shat[row] += k[row] * dd over this lane's R rows.
template <int R>
__device__ __forceinline__ void update_pass(float* s, float k0, float k1, float dd) {
    if constexpr (R == 32) {
        asm("s_nop 1\n\t"
            LA_UPD2(0, 0, 1) LA_UPD2(1, 2, 3) LA_UPD2(2, 4, 5) LA_UPD2(3, 6, 7) LA_UPD2(4, 8, 9)
            LA_UPD2(5, 10, 11) LA_UPD2(6, 12, 13) LA_UPD2(7, 14, 15) LA_UPD2(8, 16, 17) LA_UPD2(9, 18, 19)
            LA_UPD2(10, 20, 21) LA_UPD2(11, 22, 23) LA_UPD2(12, 24, 25) LA_UPD2(13, 26, 27)
            LA_UPD2(14, 28, 29) LA_UPD2(15, 30, 31)
            : LA_S32(s) : "v"(k0), "v"(k1), "v"(dd));
    } else if constexpr (R == 16) {
        asm("s_nop 1\n\t"
            LA_UPD1(0, 0) LA_UPD1(1, 1) LA_UPD1(2, 2) LA_UPD1(3, 3) LA_UPD1(4, 4) LA_UPD1(5, 5) LA_UPD1(6, 6)
            LA_UPD1(7, 7) LA_UPD1(8, 8) LA_UPD1(9, 9) LA_UPD1(10, 10) LA_UPD1(11, 11) LA_UPD1(12, 12)
            LA_UPD1(13, 13) LA_UPD1(14, 14) LA_UPD1(15, 15)
            : LA_S16(s) : "v"(k0), "v"(dd));
    } else {
        [&]<int... M>(std::integer_sequence<int, M...>) { (fmac_bcast<M>(s[M], k0, dd), ...); }(
            std::make_integer_sequence<int, R>{});
    }
}

// Sums of p and of q over the four lanes {i, i^16, i^32, i^48}, both in every lane, with
// three permlane swaps: swap rows 1,3 of p with rows 0,2 of q and add (row pairs of p in
// rows 0,2, of q in rows 1,3), swap halves and add ([P, Q, P, Q] by rows), then one more row
// swap separates P and Q.  Every lane adds the same operands in the same order.
__device__ __forceinline__ void rows_sum2(float p, float q, float& P, float& Q) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(p), __float_as_uint(q), false, false);
    const float x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = __uint_as_float(b[0]) + __uint_as_float(b[1]);
    auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    P = __uint_as_float(c[0]);
    Q = __uint_as_float(c[1]);
}

// Sums over all 64 lanes of four per-lane values a, b, c, d; row r of the result holds the
// sum of the r-th of them.  Row swaps pair a with b and c with d, a half swap pairs the
// two results (rows now hold the four-row sums of a, b, c, d), then four DPP steps sum
// within each row.  Every lane of a row adds the same operands in the same order.
__device__ __forceinline__ float sum4_by_rows(float a, float b, float c, float d) {
    auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(c), __float_as_uint(d), false, false);
    const float ab = __uint_as_float(x[0]) + __uint_as_float(x[1]);  // [a01, b01, a23, b23]
    const float cd = __uint_as_float(y[0]) + __uint_as_float(y[1]);  // [c01, d01, c23, d23]
    auto z = __builtin_amdgcn_permlane32_swap(__float_as_uint(ab), __float_as_uint(cd), false, false);
    float r = __uint_as_float(z[0]) + __uint_as_float(z[1]);         // [a, b, c, d] per lane position
    r = r + dpp<kDppXor1>(r);
    r = r + dpp<kDppXor2>(r);
    r = r + dpp<kDppHalfMirror>(r);
    r = r + dpp<kDppMirror>(r);
    return r;
}

// Two bf16 pairs (key word, query word), or two single bf16 values, to floats.
__device__ __forceinline__ void widen_pairs(uint32_t kw, uint32_t qw, float& k0, float& k1, float& q0, float& q1) {
    k0 = __uint_as_float(kw << 16);
    k1 = __uint_as_float(kw & 0xFFFF0000u);
    q0 = __uint_as_float(qw << 16);
    q1 = __uint_as_float(qw & 0xFFFF0000u);
}

__device__ __forceinline__ float lane_of(float x, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, size_t bytes) {
    const uint32_t n = bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : static_cast<uint32_t>(bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(n), 0x00020000);
}

}  // namespace

template <int DK, int QMODE, int G, bool BF16, bool GF32, bool OBF16>
__global__ __launch_bounds__(kWaveThreads) void fwd_wave_kernel(Params p, FwdArgs a) {
    constexpr int R = DK / 4;                       // state rows per lane
    constexpr int KPL = R >= 32 ? 2 : 1;            // key (query) values per lane
    constexpr int NW = (KPL == 2 && !BF16) ? 2 : 1; // raw words per lane per key row
    constexpr int IB = BF16 ? 2 : 4;                // input element bytes
    constexpr int OB = OBF16 ? 2 : 4;
    constexpr int GB = GF32 ? 4 : 2;

    __shared__ float amax_s[2][kWaveTileWaves];
    __shared__ float gmax_s[(QMODE == LA_QDQ_INT8_GROUP && G > kWaveCols) ? 2 : 1][kWaveTileWaves][DK];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rg = lane >> 4, c = lane & 15;
    const int h = blockIdx.y, b = blockIdx.z;
    const int col = blockIdx.x * kTileCols + w * kWaveCols + c;
    const int T = p.T, H = p.H, DV = p.dv;
    const size_t bh = static_cast<size_t>(b) * H + h;
    const size_t state_off = bh * DK * DV;
    const size_t seq0 = static_cast<size_t>(b) * T * H;  // token (b, 0, head 0)
    const size_t seq_tok = static_cast<size_t>(T) * H;   // token-heads of one sequence

    // Buffer resources over exactly this sequence's tokens (offsets < 2^31, checked on the
    // host): reads of tokens >= T return zero and stores to them are dropped, so the last
    // block runs as a full one (zero keys, values and beta leave the state unchanged).
    const auto rk = make_rsrc(static_cast<const char*>(a.k) + seq0 * DK * IB, seq_tok * DK * IB);
    const auto rq = make_rsrc(static_cast<const char*>(a.q) + seq0 * DK * IB, seq_tok * DK * IB);
    const auto rv = make_rsrc(static_cast<const char*>(a.v) + seq0 * DV * IB, seq_tok * DV * IB);
    const auto rgt = make_rsrc(static_cast<const char*>(a.g) + seq0 * GB, seq_tok * GB);
    const auto rbt = make_rsrc(static_cast<const char*>(a.beta) + seq0 * GB, seq_tok * GB);
    const bool has_o = a.o != nullptr;
    const auto ro = make_rsrc(has_o ? static_cast<const char*>(a.o) + seq0 * DV * OB : nullptr,
                              has_o ? seq_tok * DV * OB : 0);
    // this lane's key element(s) within a token's row, its value column, its output slot
    const int voff_k = (KPL == 2 ? 2 * lane : rg * R + (c % R)) * IB;
    const int voff_v = col * IB;
    const int voff_o = (rg * H * DV + col) * OB;  // row group r stores token t4 + r

    // ---------------------------------------------------------------- state
    float s[R];
#pragma unroll
    for (int m = 0; m < R; m++)
        s[m] = a.S0 ? a.S0[state_off + static_cast<size_t>(rg * R + m) * DV + col] : 0.0f;
    // Settle the conditional state loads before the loop's loads start, so that the wait
    // analysis does not carry them around the token loop.
    __builtin_amdgcn_s_waitcnt(0);

    // ---------------------------------------------------------------- inputs
    struct Raw {
        uint32_t k[NW], q[NW], v;
    };
    auto fetch = [&](Raw& r, int tt) {
        const int so_k = (tt * H + h) * (DK * IB);
        const int so_v = (tt * H + h) * (DV * IB);
        if (KPL == 2 && !BF16) {
            r.k[0] = __builtin_amdgcn_raw_buffer_load_b32(rk, voff_k, so_k, 0);
            r.k[NW - 1] = __builtin_amdgcn_raw_buffer_load_b32(rk, voff_k + 4, so_k, 0);
            r.q[0] = __builtin_amdgcn_raw_buffer_load_b32(rq, voff_k, so_k, 0);
            r.q[NW - 1] = __builtin_amdgcn_raw_buffer_load_b32(rq, voff_k + 4, so_k, 0);
        } else if (KPL == 2 || !BF16) {
            r.k[0] = __builtin_amdgcn_raw_buffer_load_b32(rk, voff_k, so_k, 0);
            r.q[0] = __builtin_amdgcn_raw_buffer_load_b32(rq, voff_k, so_k, 0);
        } else {
            r.k[0] = __builtin_amdgcn_raw_buffer_load_b16(rk, voff_k, so_k, 0);
            r.q[0] = __builtin_amdgcn_raw_buffer_load_b16(rq, voff_k, so_k, 0);
        }
        if (BF16) r.v = __builtin_amdgcn_raw_buffer_load_b16(rv, voff_v, so_v, 0);
        else r.v = __builtin_amdgcn_raw_buffer_load_b32(rv, voff_v, so_v, 0);
    };

    // ---------------------------------------------------------------- gate windows
    float eg_w = 1.0f, beta_w = 0.0f, cum_w = 1.0f, rcum_w = 1.0f, bmin_w = 1.0f, bmax_w = 1.0f;
    uint32_t graw = 0, braw = 0;  // raw gates of the next window, in flight
    auto fetch_window = [&](int w0n) {
        const int so = (w0n * H + h) * GB;  // wave-uniform part
        const int vo = lane * H * GB;       // lane i: token w0n + i
        if (GF32) {
            graw = __builtin_amdgcn_raw_buffer_load_b32(rgt, vo, so, 0);
            braw = __builtin_amdgcn_raw_buffer_load_b32(rbt, vo, so, 0);
        } else {
            graw = __builtin_amdgcn_raw_buffer_load_b16(rgt, vo, so, 0);
            braw = __builtin_amdgcn_raw_buffer_load_b16(rbt, vo, so, 0);
        }
    };
    auto open_window = [&](int w0) {
        const bool valid = w0 + lane < T;
        const float g = GF32 ? __uint_as_float(graw) : __uint_as_float(graw << 16);
        const float bt = GF32 ? __uint_as_float(braw) : __uint_as_float(braw << 16);
        eg_w = valid ? expf(g) : 1.0f;
        beta_w = valid ? bt : 0.0f;
    };
    // Running gate product from window lane L on (1 before it), its reciprocal, and the
    // extremes of the product over each block of 8 lanes.
    auto rescan = [&](int L) {
        float x = lane >= L ? eg_w : 1.0f;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const float y = __shfl_up(x, d, 64);
            if (lane >= d) x *= y;
        }
        cum_w = x;
        rcum_w = __builtin_amdgcn_rcpf(x);
        float lo = x, hi = x;
        lo = fminf(lo, dpp<kDppXor1>(lo)); hi = fmaxf(hi, dpp<kDppXor1>(hi));
        lo = fminf(lo, dpp<kDppXor2>(lo)); hi = fmaxf(hi, dpp<kDppXor2>(hi));
        lo = fminf(lo, dpp<kDppHalfMirror>(lo)); hi = fmaxf(hi, dpp<kDppHalfMirror>(hi));
        bmin_w = lo;
        bmax_w = hi;
    };
    auto fold = [&](float f) {
#pragma unroll
        for (int m = 0; m < R; m++) s[m] *= f;
    };

    // ---------------------------------------------------------------- one token
    struct Keys {
        float k0, k1, q0, q1;
    };
    auto widen = [&](const Raw& r) {
        Keys x;
        x.k1 = x.q1 = 0.0f;
        if (BF16) {
            if (KPL == 2) widen_pairs(r.k[0], r.q[0], x.k0, x.k1, x.q0, x.q1);
            else { x.k0 = __uint_as_float(r.k[0] << 16); x.q0 = __uint_as_float(r.q[0] << 16); }
        } else {
            x.k0 = __uint_as_float(r.k[0]); x.q0 = __uint_as_float(r.q[0]);
            x.k1 = __uint_as_float(r.k[NW - 1]); x.q1 = __uint_as_float(r.q[NW - 1]);
        }
        return x;
    };
    // this lane's share of k . q (lanes past the row group's keys hold copies and add 0)
    auto kq_part = [&](const Keys& x) {
        float v = x.k0 * x.q0;
        if (KPL == 2) v = __builtin_fmaf(x.k1, x.q1, v);
        if (R < 16) v = c < R ? v : 0.0f;
        return v;
    };
    // With Ap the gate product since the last fold (S = Ap Shat before the update) and kq =
    // k . q, returns o (the state before rounding read by q).
    auto token = [&](const Keys& x, uint32_t vraw, float kq, float Ap, float rAp, float bt) {
        const float vj = BF16 ? __uint_as_float(vraw << 16) : __uint_as_float(vraw);
        float pk, pq, P, Q;
        dot_pass<R>(s, x.k0, x.k1, x.q0, x.q1, pk, pq);
        rows_sum2(pk, pq, P, Q);
        const float delta = bt * (vj - Ap * P);
        const float o = __builtin_fmaf(delta, kq, Ap * Q);
        update_pass<R>(s, x.k0, x.k1, delta * rAp);
        return o;
    };
    // o of tokens t4 .. t4+3 (row group r holds token t4 + r); dropped past the last token
    auto store_o = [&](int t4, float ov) {
        const int so = (t4 * H + h) * DV * OB;
        if (OBF16) __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(ov), ro, voff_o, so, 0);
        else __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ov), ro, voff_o, so, 0);
    };

    // ---------------------------------------------------------------- quantization
    int qpar = 0;
    auto quantize = [&]() {
        if (QMODE == LA_QDQ_E4M3_TILE) {
            float mx = 0.0f;
#pragma unroll
            for (int m = 0; m < R; m++) mx = fmaxf(mx, fabsf(s[m]));
            mx = group_max<64>(mx);
            if (lane == 0) amax_s[qpar][w] = mx;
            __syncthreads();
            float amax = amax_s[qpar][0];
#pragma unroll
            for (int ww = 1; ww < kWaveTileWaves; ww++) amax = fmaxf(amax, amax_s[qpar][ww]);
            const float sce = amax > 0.0f ? amax / 448.0f : 1.0f;
            if (sce >= kFastQuotMinScaleE4M3) {
                const float y = 1.0f / sce;
#pragma unroll
                for (int m = 0; m < R; m++) s[m] = e4m3_round(quot_rn(s[m], sce, y)) * sce;
            } else {
#pragma unroll
                for (int m = 0; m < R; m++) s[m] = e4m3_round(s[m] / sce) * sce;
            }
        } else if (QMODE == LA_QDQ_INT8_GROUP) {
            float gm[R];
#pragma unroll
            for (int m = 0; m < R; m++) gm[m] = group_max<(G < kWaveCols ? G : kWaveCols)>(fabsf(s[m]));
            if (G > kWaveCols) {
                // groups span G / 16 waves: exchange the per-row maxima through LDS
                constexpr int NG = G / kWaveCols;
                const int gpar = (QMODE == LA_QDQ_INT8_GROUP && G > kWaveCols) ? qpar : 0;
                if (c == 0) {
#pragma unroll
                    for (int m = 0; m < R; m++) gmax_s[gpar][w][rg * R + m] = gm[m];
                }
                __syncthreads();
                const int w_first = (w / NG) * NG;
#pragma unroll
                for (int i = 0; i < NG; i++) {
                    const int ww = w_first + i;
                    if (ww == w) continue;
#pragma unroll
                    for (int m = 0; m < R; m++) gm[m] = fmaxf(gm[m], gmax_s[gpar][ww][rg * R + m]);
                }
            }
#pragma unroll
            for (int m = 0; m < R; m++) {
                const float sc8 = int8_scale(gm[m]);
                const float cde = sc8 >= kFastQuotMinScale ? int8_code_y(s[m], sc8, 1.0f / sc8) : int8_code(s[m], sc8);
                s[m] = cde * sc8;
            }
        }
        qpar ^= 1;  // the LDS slots of this point are rewritten two points later, after a barrier
    };

    // ---------------------------------------------------------------- token loop
    Raw ring[kRing];
    fetch_window(0);
#pragma unroll
    for (int j = 0; j < kRing; j++) fetch(ring[j], j);

    const int qi = p.qdq_interval;
    int q_next = QMODE != LA_QDQ_NONE ? min(qi, T) - 1 : T;  // last token of the rounding interval
    int ck_next = a.ckpts ? 0 : T;
    int w0 = 0, w_next = 0;
    float F = 1.0f;  // S = F * Shat
    bool rescan_due = false;

    // after the block starting at t: round the state if the block ends a rounding interval
    auto block_end = [&](int t) {
        if (min(t + kRing, T) - 1 == q_next) {
            fold(F);
            F = 1.0f;
            quantize();
            q_next = q_next + qi <= T - 1 ? q_next + qi : (q_next < T - 1 ? T - 1 : T);
            rescan_due = true;
        }
    };

    int t = 0;
#pragma unroll 1
    while (t < T) {
        // Blocks whose gate product stays within range; leaves the loop at a block that
        // needs the gates applied token by token.
        bool careful = false;
#pragma unroll 1
        for (; t < T; t += kRing) {
            if (t == w_next) {
                fold(F);
                F = 1.0f;
                w0 = t;
                w_next = t + kWin;
                open_window(w0);
                fetch_window(w_next);
                rescan(0);
                rescan_due = false;
            } else if (rescan_due) {
                rescan(t - w0);
                rescan_due = false;
            }
            if (t == ck_next) {
                float* dst = a.ckpts + (bh * p.nck + t / p.ckpt_interval) * DK * DV;
#pragma unroll
                for (int m = 0; m < R; m++) dst[static_cast<size_t>(rg * R + m) * DV + col] = F * s[m];
                ck_next += p.ckpt_interval;
            }
            const int tw = t - w0;
            if (!(lane_of(bmin_w, tw) >= kFoldLo && lane_of(bmax_w, tw) <= kFoldHi)) {
                fold(F);
                F = 1.0f;
                rescan(tw);
                if (!(lane_of(bmin_w, tw) >= kFoldLo && lane_of(bmax_w, tw) <= kFoldHi)) {
                    careful = true;
                    break;
                }
            }
            // Eight tokens from the ring.  Tokens past the end read zero inputs and beta = 0
            // and leave the state unchanged.
            float o_acc = 0.0f;
#pragma unroll
            for (int j0 = 0; j0 < kRing; j0 += 4) {
                // each group of 4 tokens waits only for its own inputs
                __builtin_amdgcn_sched_barrier(0);
                // take the group's inputs out of the ring and refill it with the tokens one
                // block ahead, so that every load has a block of tokens to arrive
                Keys x[4];
                uint32_t vr[4];
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    x[i] = widen(ring[j0 + i]);
                    vr[i] = ring[j0 + i].v;
                    fetch(ring[j0 + i], t + j0 + i + kRing);
                }
                const float kq4 = sum4_by_rows(kq_part(x[0]), kq_part(x[1]), kq_part(x[2]), kq_part(x[3]));
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int j = j0 + i;
                    // row group i holds this token's k . q: its o is the one kept
                    const float o = token(x[i], vr[i], kq4, lane_of(cum_w, tw + j), lane_of(rcum_w, tw + j),
                                          lane_of(beta_w, tw + j));
                    o_acc = rg == i ? o : o_acc;
                }
                store_o(t + j0, o_acc);
            }
            F = lane_of(cum_w, tw + kRing - 1);
            block_end(t);
        }
        if (!careful) break;
        // Gates too steep for one rescale per block: apply each token's gate to the state
        // (F = 1 here) and read the block's inputs again, then refill the ring.
        const int tw = t - w0;
#pragma unroll 1
        for (int j = 0; j < kRing && t + j < T; j++) {
            fold(lane_of(eg_w, tw + j));
            Raw r;
            fetch(r, t + j);
            const Keys x = widen(r);
            const float o = token(x, r.v, wave_sum(kq_part(x)), 1.0f, 1.0f, lane_of(beta_w, tw + j));
            if (rg == 0) store_o(t + j, o);
        }
#pragma unroll
        for (int j = 0; j < kRing; j++) fetch(ring[j], t + j + kRing);
        rescan_due = true;
        block_end(t);
        t += kRing;
    }
    fold(F);
    if (a.ST) {
#pragma unroll
        for (int m = 0; m < R; m++) a.ST[state_off + static_cast<size_t>(rg * R + m) * DV + col] = s[m];
    }
}

namespace {

template <int DK, int QMODE, int G, bool BF16, bool GF32>
hipError_t launch_wave_o(const la_config& c, const FwdArgs& a, hipStream_t s) {
    dim3 grid(c.d_v / kTileCols, c.H, c.B);
    if (c.out_dtype == LA_BF16)
        hipLaunchKernelGGL((fwd_wave_kernel<DK, QMODE, G, BF16, GF32, true>), grid, dim3(kWaveThreads), 0, s,
                           make_params(c), a);
    else
        hipLaunchKernelGGL((fwd_wave_kernel<DK, QMODE, G, BF16, GF32, false>), grid, dim3(kWaveThreads), 0, s,
                           make_params(c), a);
    return hipGetLastError();
}

template <int DK, int QMODE, int G>
hipError_t launch_wave_t(const la_config& c, const FwdArgs& a, hipStream_t s) {
    const bool bf = c.qkv_dtype == LA_BF16, gf = c.gate_dtype == LA_F32;
    if (bf && gf) return launch_wave_o<DK, QMODE, G, true, true>(c, a, s);
    if (bf) return launch_wave_o<DK, QMODE, G, true, false>(c, a, s);
    if (gf) return launch_wave_o<DK, QMODE, G, false, true>(c, a, s);
    return launch_wave_o<DK, QMODE, G, false, false>(c, a, s);
}

template <int DK>
hipError_t launch_wave_dk(const la_config& c, const FwdArgs& a, hipStream_t s) {
    if (c.qdq == LA_QDQ_NONE) return launch_wave_t<DK, LA_QDQ_NONE, 1>(c, a, s);
    if (c.qdq == LA_QDQ_E4M3_TILE) return launch_wave_t<DK, LA_QDQ_E4M3_TILE, 64>(c, a, s);
    switch (c.group) {
        case 16: return launch_wave_t<DK, LA_QDQ_INT8_GROUP, 16>(c, a, s);
        case 32: return launch_wave_t<DK, LA_QDQ_INT8_GROUP, 32>(c, a, s);
        default: return launch_wave_t<DK, LA_QDQ_INT8_GROUP, 64>(c, a, s);
    }
}

}  // namespace

bool fwd_wave_eligible(const la_config& c) {
    if (!fwd_fast_eligible(c)) return false;
    if (c.qdq != LA_QDQ_NONE && c.qdq_interval % kRing != 0) return false;
    if (c.ckpt_interval > 0 && c.ckpt_interval % kRing != 0) return false;
    // 32-bit buffer offsets within one sequence, ring prefetch included
    const size_t span = static_cast<size_t>(c.T + 2 * kRing + kWin) * c.H * (c.d_k > c.d_v ? c.d_k : c.d_v) * 4;
    return span < (static_cast<size_t>(1) << 31);
}

hipError_t launch_fwd_wave(const la_config& c, const FwdArgs& a, hipStream_t s) {
    switch (c.d_k) {
        case 16: return launch_wave_dk<16>(c, a, s);
        case 32: return launch_wave_dk<32>(c, a, s);
        case 64: return launch_wave_dk<64>(c, a, s);
        default: return launch_wave_dk<128>(c, a, s);
    }
}

}  // namespace la
