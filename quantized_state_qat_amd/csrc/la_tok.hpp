// Per-token layout shared by the token forward kernel (fwd_tok.hip) and the backward's
// recompute (bwd.hip): the two run exactly these functions, so a recompute meets the
// forward's carried states and rounding decisions bit for bit.
//
// One workgroup per (sequence, head, tile of 64 or 32 value columns), eight waves: each lane
// holds one value column of the tile and R key rows of it in registers (TokShape).
// Per token:
//  * one wave has published the token's operands in an LDS ring (keys and queries, rotated
//    by the Walsh-Hadamard transform in Hadamard mode; the gate, exp(g), per key row or
//    scalar; beta; k . q; the tile's values), a block of eight tokens ahead of use;
//  * the decayed state's projections onto the key and the query are in-lane chains over the
//    wave's rows, and the eight waves' partial sums meet in LDS behind one barrier, summed in
//    a fixed order;
//  * the update is one FMA per element;
//  * at a rounding point the INT8 group maxima are taken by a reduce-scatter across the
//    lanes (each lane ends with the maximum of one (row, group)), the lane computes that
//    group's scale and reciprocal once, and the wave reads all of them back through LDS.
// In Hadamard mode the state is carried rotated, Y = Hu S (Hu the unnormalized Sylvester
// matrix): the update is the same map with Hu k in place of k, projections scaled by 1/d_k
// (an exact power of two), and the INT8 codec acts on Y directly.
#pragma once

#include "la_device.hpp"
#include "la_internal.hpp"

#include <type_traits>

namespace la {

constexpr int kTokWaves = 8;                  // waves per workgroup = tokens per block
constexpr int kTokThreads = kTokWaves * 64;
constexpr int kTokRing = 2 * kTokWaves;       // token records in the LDS ring

struct TokParams {
    int B, T, H, dk, dv;
    int qkv_dt, gate_dt, out_dt;
    int qdq_interval, ckpt_interval, nck;
    int rot;     // state tensors hold the rotated state (Hadamard mode)
    int replay;  // replay windows: updates between rounding points from BF16-encoded deltas
    long ntok;   // token-heads of the call: B T H, or T H for packed sequences
};

// Token range [begin, end) of packed sequence b: cu_seqlens[b] .. cu_seqlens[b + 1], clamped
// to [0, T_total] (an inverted pair is empty), then, with split, the prefix of split[b]
// tokens (part 0) or the rest (part 1).
__device__ __forceinline__ void packed_range(const int32_t* cu, const int32_t* split, int part, int b, int T_total,
                                             int& begin, int& end) {
    begin = min(max(cu[b], 0), T_total);
    end = min(max(cu[b + 1], begin), T_total);
    if (split) {
        const int mid = min(max(begin + split[b], begin), end);
        if (part == 0) end = mid;
        else begin = mid;
    }
}


// ------------------------------------------------------------------ lane reduce-scatter
// Reduce N values per lane (x[0..N-1], value i belonging to row i) over aligned groups of
// G lanes so that each lane ends with the reduction of one row over its group.  Each level
// halves the values a lane carries: the lane keeps one half and combines it with its
// partner's copy of that half.  Levels, in order: lanes 32 apart (permlane32 swap, G = 64),
// 16 apart (permlane16 swap, G >= 32), then within each row of 16 lanes the DPP mirror
// (lane i <-> 15 - i), half mirror (i <-> 7 - i within 8), and the quad exchanges i ^ 2 and
// i ^ 1.  Once a lane carries a single value the remaining levels reduce it in place.
// The row a lane ends with is reduce_scatter_row<N, G>(lane).
// Op::T is the value type moved between lanes.  OpMaxAbs reduces absolute values as their
// bit patterns (sign cleared): for non-negative floats the unsigned integer order is the float
// order, and the integer max needs none of the canonicalizing moves a float max takes after a
// cross-lane move.
struct OpMaxAbs {
    using T = uint32_t;
    static __device__ __forceinline__ T f(T a, T b) { return a > b ? a : b; }
};
struct OpAdd {
    using T = float;
    static __device__ __forceinline__ T f(T a, T b) { return a + b; }
};

template <class T>
__device__ __forceinline__ uint32_t as_u32(T x) { return __builtin_bit_cast(uint32_t, x); }
template <class T>
__device__ __forceinline__ T from_u32(uint32_t x) { return __builtin_bit_cast(T, x); }

// DPP move with every lane in range (bound_ctrl set, all rows and banks): the move folds into
// the instruction that consumes it.
template <int CTRL, class T>
__device__ __forceinline__ T dpp_mov(T x) {
    return from_u32<T>(static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(as_u32(x)), CTRL, 0xF, 0xF, true)));
}

// One swap level over lanes 32 (SW = 32) or 16 (SW = 16) apart.  After a permlane swap of
// (A, B), A's register holds in the lower half of each lane pair the lane's own A and in the
// upper half the partner's B, and B's register the partner's A and the lane's own B.
template <class Op, int SW, int N>
__device__ __forceinline__ void rs_swap_level(typename Op::T* x) {
    using T = typename Op::T;
    auto swap = [](T a, T b) __attribute__((always_inline)) {
        return SW == 32 ? __builtin_amdgcn_permlane32_swap(as_u32(a), as_u32(b), false, false)
                        : __builtin_amdgcn_permlane16_swap(as_u32(a), as_u32(b), false, false);
    };
    if constexpr (N == 1) {
        const auto r = swap(x[0], x[0]);
        x[0] = Op::f(from_u32<T>(r[0]), from_u32<T>(r[1]));
    } else {
#pragma unroll
        for (int i = 0; i < N / 2; i++) {
            const auto r = swap(x[i], x[i + N / 2]);
            x[i] = Op::f(from_u32<T>(r[0]), from_u32<T>(r[1]));
        }
    }
}

// One DPP level: the partner differs from the lane in bit BIT of the lane index (and the
// pattern keeps every bit above BIT within the row of 16).
template <class Op, int CTRL, int BIT, int N>
__device__ __forceinline__ void rs_dpp_level(typename Op::T* x, int lane) {
    using T = typename Op::T;
    if constexpr (N == 1) {
        x[0] = Op::f(x[0], dpp_mov<CTRL>(x[0]));
    } else {
        const bool hi = (lane >> BIT) & 1;
#pragma unroll
        for (int i = 0; i < N / 2; i++) {
            const T send = hi ? x[i] : x[i + N / 2];
            const T keep = hi ? x[i + N / 2] : x[i];
            x[i] = Op::f(keep, dpp_mov<CTRL>(send));
        }
    }
}

constexpr int kCtrlMirror = 0x140, kCtrlHalfMirror = 0x141, kCtrlXor2 = 0x4E, kCtrlXor1 = 0xB1;

template <class Op, int N, int G>
__device__ __forceinline__ typename Op::T reduce_scatter(typename Op::T* x, int lane) {
    static_assert(G == 16 || G == 32 || G == 64, "groups of 16, 32 or 64 lanes");
    constexpr int N1 = G == 64 ? (N > 1 ? N / 2 : 1) : N;
    constexpr int N2 = G >= 32 ? (N1 > 1 ? N1 / 2 : 1) : N1;
    constexpr int N3 = N2 > 1 ? N2 / 2 : 1;
    constexpr int N4 = N3 > 1 ? N3 / 2 : 1;
    constexpr int N5 = N4 > 1 ? N4 / 2 : 1;
    if constexpr (G == 64) rs_swap_level<Op, 32, N>(x);
    if constexpr (G >= 32) rs_swap_level<Op, 16, N1>(x);
    rs_dpp_level<Op, kCtrlMirror, 3, N2>(x, lane);
    rs_dpp_level<Op, kCtrlHalfMirror, 2, N3>(x, lane);
    rs_dpp_level<Op, kCtrlXor2, 1, N4>(x, lane);
    rs_dpp_level<Op, kCtrlXor1, 0, N5>(x, lane);
    return x[0];
}

// Row whose reduction lane `lane` holds after reduce_scatter<Op, N, G>: every level that
// splits n > 1 values sends the lane to the upper half (offset n/2) when its bit is set.
template <int N, int G>
__device__ __forceinline__ int reduce_scatter_row(int lane) {
    int row = 0, n = N;
    if (G == 64) {
        if (n > 1) { row += ((lane >> 5) & 1) * (n / 2); n /= 2; }
    }
    if (G >= 32) {
        if (n > 1) { row += ((lane >> 4) & 1) * (n / 2); n /= 2; }
    }
    if (n > 1) { row += ((lane >> 3) & 1) * (n / 2); n /= 2; }
    if (n > 1) { row += ((lane >> 2) & 1) * (n / 2); n /= 2; }
    if (n > 1) { row += ((lane >> 1) & 1) * (n / 2); n /= 2; }
    if (n > 1) { row += (lane & 1) * (n / 2); n /= 2; }
    return row;
}

// ------------------------------------------------------------------ tile shape
// A workgroup covers TC value columns of one (sequence, head): 64, or 32 when every rounding
// group fits in 32 columns (tok_tile_cols), which doubles the workgroups of a small batch.  The
// 64 lanes of a wave are TC columns x RH = 64 / TC row groups; wave w holds key rows
// [w RW, (w+1) RW), RW = d_k / 8, and lane (rh, c) rows w RW + rh R .. + R - 1 of column c.
template <int DK_, int QMODE_, int G_>
struct TokShape {
    static constexpr int DK = DK_, QMODE = QMODE_, G = G_;
    static constexpr int TC = tok_tile_cols(DK, QMODE, G);
    static constexpr int RH = 64 / TC;
    static constexpr int RW = DK / kTokWaves;
    static constexpr int R = RW / RH;
    static_assert(R >= 1 && (QMODE != LA_QDQ_E4M3_TILE || (TC == 64 && R % 2 == 0)), "token tile shape");
    static_assert(QMODE != LA_QDQ_INT8_GROUP || G <= TC, "INT8 groups within a tile");
};

// ------------------------------------------------------------------ token records
// One token's operands in the LDS ring, written by one wave and read by all eight.
template <class S, bool KDA, bool BWD>
struct TokRing {
    float ku[kTokRing][S::DK];                 // k, or Hu k
    float qu[kTokRing][S::DK];                 // q, or Hu q
    float ga[kTokRing][KDA ? S::DK : 1];       // exp(g) per key row (KDA)
    float v[kTokRing][S::TC];                  // the tile's values
    float dout[kTokRing][BWD ? S::TC : 1];
    float4 sc[kTokRing];                       // (exp(g) (scalar gate; 1 for KDA), beta, k . q, 0)
};

struct TokInputs {
    const void *q, *k, *v, *g, *beta;
    const float* dout;
};

// Element layout of a length-DK vector over the lanes of one wave: bf16 rows arrive as one
// word (two elements) per lane, element 2 lane + e; fp32 rows as element lane + 64 e.
__device__ __forceinline__ int tok_elem(bool bf16, int lane, int e) { return bf16 ? 2 * lane + e : lane + 64 * e; }

// Value of lane ^ M (M a power of two below 64), by DPP within rows of 16 lanes and the
// permlane swaps across rows.
template <int M>
__device__ __forceinline__ float lane_xor(float x, int lane) {
    if constexpr (M == 1) return dpp_mov<kCtrlXor1>(x);
    else if constexpr (M == 2) return dpp_mov<kCtrlXor2>(x);
    else if constexpr (M == 4) {
        const float up = dpp_mov<0x104>(x), dn = dpp_mov<0x114>(x);  // row_shl:4, row_shr:4
        return (lane & 4) ? dn : up;
    } else if constexpr (M == 8) return dpp_mov<0x128>(x);       // row_ror:8
    else {
        const Pair p = M == 16 ? swap16(x) : swap32(x);
        return (lane & M) ? p.a : p.b;
    }
}

// Unnormalized Sylvester Walsh-Hadamard transform of a length-DK vector held in that layout:
// the in-lane element bit is one butterfly stage, every lane bit one more (partner lane ^ m,
// new value partner + x or partner - x by the lane's side).
template <int DK>
__device__ __forceinline__ void lane_wht(float& x0, float& x1, int lane, bool bf16) {
    auto stage = [&](auto mc) __attribute__((always_inline)) {
        constexpr int M = decltype(mc)::value;
        const float sg = (lane & M) ? -1.0f : 1.0f;
        const float p0 = lane_xor<M>(x0, lane), p1 = lane_xor<M>(x1, lane);
        x0 = __builtin_fmaf(sg, x0, p0);
        x1 = __builtin_fmaf(sg, x1, p1);
    };
    auto lane_stages = [&](auto first) __attribute__((always_inline)) {  // lane bits m = 1 .. < bound
        constexpr int B = decltype(first)::value;                        // number of lane bits
        if constexpr (B > 0) stage(std::integral_constant<int, 1>{});
        if constexpr (B > 1) stage(std::integral_constant<int, 2>{});
        if constexpr (B > 2) stage(std::integral_constant<int, 4>{});
        if constexpr (B > 3) stage(std::integral_constant<int, 8>{});
        if constexpr (B > 4) stage(std::integral_constant<int, 16>{});
        if constexpr (B > 5) stage(std::integral_constant<int, 32>{});
    };
    constexpr int LOG = DK == 128 ? 7 : DK == 64 ? 6 : DK == 32 ? 5 : 4;
    if (bf16) {
        const float a = x0 + x1, b = x0 - x1;
        x0 = a;
        x1 = b;
        lane_stages(std::integral_constant<int, LOG - 1>{});
    } else {
        lane_stages(std::integral_constant<int, (LOG < 6 ? LOG : 6)>{});
        if (DK > 64) {
            const float a = x0 + x1, b = x0 - x1;
            x0 = a;
            x1 = b;
        }
    }
}

// Raw words of one token for the wave that publishes it (widened only when published, so
// that the loads are not waited on early).  col: this lane's value column (lanes < TC).
template <class S, bool KDA, bool BWD>
struct TokFetch {
    static constexpr int DK = S::DK;
    uint32_t k0 = 0, k1 = 0, q0 = 0, q1 = 0, g0 = 0, g1 = 0, gh = 0, b = 0, bh = 0, v = 0;
    float d = 0.0f;

    // Every load is issued by every lane with no branch around it, from an address inside the
    // tensor (lanes past a field's width read a word of the same row; the dtype only changes the
    // address), so that the compiler keeps the loads in flight until publish instead of waiting
    // for them where branches join.  publish selects what each lane uses.
    __device__ __forceinline__ void fetch(const TokInputs& in, const TokParams& p, size_t tok, int col, int lane) {
        const bool bf = p.qkv_dt == LA_BF16, gf = p.gate_dt == LA_F32;
        // k and q: a row holds DK / 2 words (bf16 pairs) or DK words (fp32: lane and lane + 64)
        const int w0 = min(lane, bf ? DK / 2 - 1 : DK - 1);
        const int w1 = bf ? w0 : min(lane + 64, DK - 1);
        const size_t rb = tok * DK * (bf ? 2 : 4);
        const uint32_t* kp = reinterpret_cast<const uint32_t*>(static_cast<const char*>(in.k) + rb);
        const uint32_t* qp = reinterpret_cast<const uint32_t*>(static_cast<const char*>(in.q) + rb);
        k0 = kp[w0];
        k1 = kp[w1];
        q0 = qp[w0];
        q1 = qp[w1];
        // v: the word holding this column's element (bf16: the pair of columns 2i, 2i + 1; d_v is
        // even, so the pair lies in the row)
        const size_t ve = tok * p.dv + col;
        v = *(bf ? reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(in.v) + (ve & ~static_cast<size_t>(1)))
                 : static_cast<const uint32_t*>(in.v) + ve);
        if (KDA) {
            const int u0 = min(lane, gf ? DK - 1 : DK / 2 - 1);
            const int u1 = gf ? min(lane + 64, DK - 1) : u0;
            const uint32_t* gp = reinterpret_cast<const uint32_t*>(static_cast<const char*>(in.g) + tok * DK * (gf ? 4 : 2));
            g0 = gp[u0];
            g1 = gp[u1];
        } else {
            // one element: two 16-bit loads (the fp32 value's halves, or the bf16 value twice)
            const uint16_t* gp = static_cast<const uint16_t*>(in.g) + (gf ? 2 * tok : tok);
            g0 = gp[0];
            gh = gp[gf ? 1 : 0];
        }
        const uint16_t* bp = static_cast<const uint16_t*>(in.beta) + (gf ? 2 * tok : tok);
        b = bp[0];
        bh = bp[gf ? 1 : 0];
        if (BWD) d = in.dout[ve];
    }

    template <bool HAD>
    __device__ __forceinline__ void publish(TokRing<S, KDA, BWD>& ring, int slot, const TokParams& p, int lane) const {
        const bool bf = p.qkv_dt == LA_BF16, gf = p.gate_dt == LA_F32;
        auto wid = [](uint32_t x, bool b16) { return b16 ? __uint_as_float(x << 16) : __uint_as_float(x); };
        // the words past the row's width are zero (they enter k . q)
        const bool ok0 = lane < (bf ? DK / 2 : DK), ok1 = !bf && lane + 64 < DK;
        const uint32_t k0 = ok0 ? this->k0 : 0u, q0 = ok0 ? this->q0 : 0u;
        const uint32_t k1 = ok1 ? this->k1 : 0u, q1 = ok1 ? this->q1 : 0u;
        const uint32_t g0w = gf ? (gh << 16) | g0 : g0, bw = gf ? (bh << 16) | b : b;
        const uint32_t vw = bf ? ((lane & 1) ? v >> 16 : v & 0xFFFFu) : v;  // the column's parity is the lane's
        float kx0, kx1, qx0, qx1;
        if (bf) {
            kx0 = __uint_as_float(k0 << 16);
            kx1 = __uint_as_float(k0 & 0xFFFF0000u);
            qx0 = __uint_as_float(q0 << 16);
            qx1 = __uint_as_float(q0 & 0xFFFF0000u);
        } else {
            kx0 = __uint_as_float(k0);
            kx1 = __uint_as_float(k1);
            qx0 = __uint_as_float(q0);
            qx1 = __uint_as_float(q1);
        }
        const float kq = wave_sum(__builtin_fmaf(kx1, qx1, kx0 * qx0));
        if (HAD) {
            lane_wht<DK>(kx0, kx1, lane, bf);
            lane_wht<DK>(qx0, qx1, lane, bf);
        }
#pragma unroll
        for (int e = 0; e < 2; e++) {
            const int i = tok_elem(bf, lane, e);
            if (i < DK && (bf || lane < 64)) {
                ring.ku[slot][i] = e ? kx1 : kx0;
                ring.qu[slot][i] = e ? qx1 : qx0;
            }
        }
        float a = 1.0f;
        if (KDA) {
            float gx0, gx1;
            if (!gf) {
                gx0 = __uint_as_float(g0 << 16);
                gx1 = __uint_as_float(g0 & 0xFFFF0000u);
            } else {
                gx0 = __uint_as_float(g0);
                gx1 = __uint_as_float(g1);
            }
#pragma unroll
            for (int e = 0; e < 2; e++) {
                const int i = tok_elem(!gf, lane, e);
                if (i < DK) ring.ga[slot][i] = expf(e ? gx1 : gx0);
            }
        } else {
            a = expf(wid(g0w, !gf));
        }
        if (lane < S::TC) {
            ring.v[slot][lane] = wid(vw, bf);
            if (BWD) ring.dout[slot][lane] = d;
        }
        if (lane == 0) ring.sc[slot] = make_float4(a, wid(bw, !gf), kq, 0.0f);
    }
};

// A wave's view of one token: its rows of the key, query (and KDA gate) vectors, the scalars
// and its column's value (and upstream output gradient).
template <class S, bool KDA>
struct TokOps {
    float kr[S::R], qr[S::R], ar[KDA ? S::R : 1];
    float a, beta, kq, vj, dj;
};

// First key row of this lane (rows row0 .. row0 + R - 1).
template <class S>
__device__ __forceinline__ int tok_row0(int w, int lane) { return w * S::RW + (lane / S::TC) * S::R; }

template <class S, bool KDA, bool BWD>
__device__ __forceinline__ void tok_read(TokOps<S, KDA>& op, const TokRing<S, KDA, BWD>& ring, int slot, int w, int lane) {
    const int r0 = tok_row0<S>(w, lane);
#pragma unroll
    for (int m = 0; m < S::R; m++) {
        op.kr[m] = ring.ku[slot][r0 + m];
        op.qr[m] = ring.qu[slot][r0 + m];
        if (KDA) op.ar[m] = ring.ga[slot][r0 + m];
    }
    const float4 sc = ring.sc[slot];
    op.a = sc.x;
    op.beta = sc.y;
    op.kq = sc.z;
    const int c = lane % S::TC;
    op.vj = ring.v[slot][c];
    op.dj = BWD ? ring.dout[slot][c] : 0.0f;
}

// Sum of a value over the RH row groups of a wave (lanes 32 apart hold the same column when
// RH = 2); every lane of the column ends with the same bits.
template <class S>
__device__ __forceinline__ float tok_rows_combine(float x) {
    if constexpr (S::RH == 2) {
        const Pair p = swap32(x);
        return p.a + p.b;
    } else {
        return x;
    }
}

// ------------------------------------------------------------------ one token
// The two halves of a token step around its barrier (tok_step runs both): the decay and the
// partial projections into red, then the sums, delta and the update.
template <class S, bool KDA>
__device__ __forceinline__ void tok_step_pre(float (&s)[S::R], const TokOps<S, KDA>& op, float2 (*red)[S::TC], int w,
                                             int lane) {
    float pk = 0.0f, pq = 0.0f;
#pragma unroll
    for (int m = 0; m < S::R; m++) {
        s[m] = (KDA ? op.ar[m] : op.a) * s[m];
        pk = __builtin_fmaf(s[m], op.kr[m], pk);
        pq = __builtin_fmaf(s[m], op.qr[m], pq);
    }
    pk = tok_rows_combine<S>(pk);
    pq = tok_rows_combine<S>(pq);
    if (lane < S::TC) red[w][lane] = make_float2(pk, pq);
}

template <class S, bool KDA, bool HAD>
__device__ __forceinline__ void tok_step_post(float (&s)[S::R], const TokOps<S, KDA>& op, const float2 (*red)[S::TC],
                                              int lane, float& u, float& delta, float& o, bool enc = false) {
    const int c = lane % S::TC;
    float2 x[kTokWaves];
#pragma unroll
    for (int i = 0; i < kTokWaves; i++) x[i] = red[i][c];
    float P = x[0].x, Q = x[0].y;
#pragma unroll
    for (int i = 1; i < kTokWaves; i++) {
        P += x[i].x;
        Q += x[i].y;
    }
    if (HAD) {
        P *= 1.0f / S::DK;
        Q *= 1.0f / S::DK;
    }
    delta = op.beta * (op.vj - P);
    o = __builtin_fmaf(delta, op.kq, Q);
    u = P;
    const float du = enc ? bf16_rne(delta) : delta;
#pragma unroll
    for (int m = 0; m < S::R; m++) s[m] = __builtin_fmaf(op.kr[m], du, s[m]);
}

// s: the state entering the token (this lane's rows of its column), advanced in place to
// S' = a S + ku delta^T (before rounding), or, with enc (a replay-window token that is not a
// rounding point), to a S + ku bf16(delta)^T.  red: this token's reduction buffer (kTokWaves
// x TC float2).  Returns u = S~^T k, delta and o = S'^T q for the column (from the unencoded
// delta).
template <class S, bool KDA, bool HAD>
__device__ __forceinline__ void tok_step(float (&s)[S::R], const TokOps<S, KDA>& op, float2 (*red)[S::TC],
                                         int w, int lane, float& u, float& delta, float& o, bool enc = false) {
    tok_step_pre<S, KDA>(s, op, red, w, lane);
    __syncthreads();
    tok_step_post<S, KDA, HAD>(s, op, red, lane, u, delta, o, enc);
}

// ------------------------------------------------------------------ codecs
// INT8 groups of G columns: each lane takes the maximum of one (row, group) by a
// reduce-scatter, computes s = amax / 127 (1 when amax = 0) and y = RN(1 / s) once
// (int8_scale_recip), and the wave reads every (s, y) of its groups back from LDS (scr: 64 / G
// x R float2 per wave); each element is then coded by int8_code_fast.  A group whose scale is
// below 2^-100 takes the IEEE division and the clamp instead (the whole wave, when any lane
// has one).
// With KEEP the codes are also returned (hc: pairs of rows as fp16, which holds every code and
// the sign of a zero code exactly, so that float(code) * scale gives back the rounded state bit
// for bit) with the scale of this lane's (row, group) (sc_out).
template <int R, int G, bool KEEP = false>
__device__ __forceinline__ void tok_int8(float (&s)[R], float2* scr, int lane, uint32_t* hc = nullptr,
                                         float* sc_out = nullptr) {
    uint32_t x[R];
#pragma unroll
    for (int m = 0; m < R; m++) x[m] = __float_as_uint(s[m]) & 0x7FFFFFFFu;
    const float mx = __uint_as_float(reduce_scatter<OpMaxAbs, R, G>(x, lane));
    const int row = reduce_scatter_row<R, G>(lane), grp = lane / G;
    float sc, y;
    const bool tiny_l = !int8_scale_recip(mx, sc, y);
    if constexpr (KEEP) *sc_out = sc;
    scr[grp * R + row] = make_float2(sc, y);
    const bool tiny = __any(tiny_l);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    float2 sy[R];
#pragma unroll
    for (int m = 0; m < R; m++) sy[m] = scr[grp * R + m];
    float cd[R];
    if (!tiny) {
#pragma unroll
        for (int m = 0; m < R; m++) cd[m] = int8_code_fast(s[m], sy[m].x, sy[m].y);
    } else {
#pragma unroll
        for (int m = 0; m < R; m++) cd[m] = int8_code(s[m], sy[m].x);
    }
#pragma unroll
    for (int m = 0; m < R; m++) s[m] = cd[m] * sy[m].x;
    if constexpr (KEEP) {
        static_assert(R % 2 == 0, "codes kept in row pairs");
#pragma unroll
        for (int m = 0; m < R; m += 2) hc[m / 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(cd[m], cd[m + 1]));
    }
    __builtin_amdgcn_wave_barrier();  // scr is rewritten only after every lane has read it
}

// E4M3 with one scale per 64-column tile (all key rows: the eight waves meet through LDS).
template <int R>
__device__ __forceinline__ void tok_e4m3(float (&s)[R], float* amax_sh, int w, int lane) {
    float mx = 0.0f;
#pragma unroll
    for (int m = 0; m < R; m++) mx = fmaxf(mx, fabsf(s[m]));
    mx = wave_max_abs(mx);
    if (lane == 0) amax_sh[w] = mx;
    __syncthreads();
    float amax = amax_sh[0];
#pragma unroll
    for (int i = 1; i < kTokWaves; i++) amax = fmaxf(amax, amax_sh[i]);
    float sce, y;
    float yv[R];
    if (e4m3_scale_recip(amax, sce, y)) {
#pragma unroll
        for (int m = 0; m < R; m++) yv[m] = quot_rn_fast(s[m], sce, y);
    } else {
#pragma unroll
        for (int m = 0; m < R; m++) yv[m] = s[m] / sce;
    }
#pragma unroll
    for (int m = 0; m < R; m += 2) {
        e4m3_round2(yv[m], yv[m + 1]);
        s[m] = yv[m] * sce;
        s[m + 1] = yv[m + 1] * sce;
    }
}

template <class S>
struct TokQdqShared {
    static constexpr bool I8 = S::QMODE == LA_QDQ_INT8_GROUP;
    float2 scr[I8 ? kTokWaves : 1][I8 ? (64 / S::G) * S::R : 1];
    float amax[kTokWaves];
};

template <class S>
__device__ __forceinline__ void tok_qdq(float (&s)[S::R], TokQdqShared<S>& sh, int w, int lane) {
    if constexpr (S::QMODE == LA_QDQ_INT8_GROUP) tok_int8<S::R, S::G>(s, sh.scr[w], lane);
    else if constexpr (S::QMODE == LA_QDQ_E4M3_TILE) tok_e4m3<S::R>(s, sh.amax, w, lane);
}

// ------------------------------------------------------------------ state rotation
// s <- (Hu s) * scale along the key axis (Sylvester butterflies over row bits 1, 2, 4, ...
// in that order).  A lane's R rows are consecutive and R-aligned, so the stages over row bits
// below R stay in registers; each higher stage exchanges rows with the lane or wave that holds
// the partner rows through one of two LDS tiles of DK x TC floats, used in turn: a stage
// writes the tile whose reads ended before the previous stage's barrier, so one barrier per
// stage (and one on entry) suffices.  Every thread of the workgroup calls it (uniformly).
template <class S>
__device__ __forceinline__ void tok_rotate(float (&s)[S::R], float* tile, int w, int lane, float scale) {
    constexpr int DK = S::DK, TC = S::TC, R = S::R;
    const int r0 = tok_row0<S>(w, lane), c = lane % TC;
#pragma unroll
    for (int h = 1; h < R; h <<= 1) {
#pragma unroll
        for (int m = 0; m < R; m++) {
            if ((m & h) == 0) {
                const float x = s[m], y = s[m + h];
                s[m] = x + y;
                s[m + h] = x - y;
            }
        }
    }
    __syncthreads();  // the tiles' previous readers are done
    int buf = 0;
#pragma unroll
    for (int h = R; h < DK; h <<= 1) {
        float* tb = tile + buf * DK * TC;
        buf ^= 1;
#pragma unroll
        for (int m = 0; m < R; m++) tb[(r0 + m) * TC + c] = s[m];
        __syncthreads();
        // every row of this lane has the same bit h (h >= R): the lower rows add the partner,
        // the upper rows subtract themselves from it
        const bool upper = (r0 & h) != 0;
#pragma unroll
        for (int m = 0; m < R; m++) {
            const float p = tb[((r0 + m) ^ h) * TC + c];
            s[m] = upper ? p - s[m] : s[m] + p;
        }
    }
#pragma unroll
    for (int m = 0; m < R; m++) s[m] *= scale;
}

// A rounding point.  ROT (Hadamard mode with per-key gates, whose state is carried unrotated:
// a per-row decay does not commute with the key-axis rotation): the codes are those of Hu S'
// and the state carried on is Hu Q(Hu S') / d_k, which is Hn Q(Hn S') because the codecs
// commute with a common scale of their group up to the rounding of that scale (the same
// reading as the rotated carry of the scalar gate).  Every thread of the workgroup calls it.
template <class S, bool ROT>
__device__ __forceinline__ void tok_qdq_at(float (&s)[S::R], TokQdqShared<S>& sh, float* tile, int w, int lane) {
    if constexpr (ROT) tok_rotate<S>(s, tile, w, lane, 1.0f);
    tok_qdq<S>(s, sh, w, lane);
    if constexpr (ROT) tok_rotate<S>(s, tile, w, lane, 1.0f / S::DK);
}

}  // namespace la
