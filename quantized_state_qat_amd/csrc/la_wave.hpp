// Device code shared by the wave-layout forward kernels (one wave per (sequence, head,
// 16 value columns); lane 16 g + c holds column c and key rows [g R, (g+1) R), R = d_k / 4,
// in registers): DPP row-broadcast FMA passes over the state, cross-row reductions, input
// widening and buffer resources.
#pragma once

#include <type_traits>
#include <utility>

#include "la_device.hpp"
#include "../../include/la.h"

namespace la {

constexpr int kWaveCols = 16;
constexpr int kWaveTileWaves = 64 / kWaveCols;  // waves per 64-column tile (one E4M3 tile)

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

// Single DPP multiply for the small key sizes: x = a[lane L of this lane's row of 16] * x.
template <int L>
__device__ __forceinline__ void mul_bcast(float& x, float a) {
    asm("s_nop 1\n\tv_mul_f32_dpp %0, %1, %0 row_newbcast:%2 row_mask:0xf bank_mask:0xf" : "+v"(x) : "v"(a), "n"(L));
}

// d_k = 128: S[row] *= a[row] with lane L holding the gates of rows 2L (a0) and 2L+1 (a1).
// Operands: %0..%31 = the 32 state rows (in/out); %32, %33 = a0, a1.
#define LA_DEC2(L, E, O) LA_DPP(v_mul_f32_dpp, E, 32, E, L) LA_DPP(v_mul_f32_dpp, O, 33, O, L)
// d_k = 64: lane L holds the gate of row L.  %0..%15 = state rows; %16 = a.
#define LA_DEC1(L) LA_DPP(v_mul_f32_dpp, L, 16, L, L)

// Per-key gate (KDA): S[row] *= a[row] over this lane's R rows, the gates spread over the row
// group's lanes like the keys.
template <int R>
__device__ __forceinline__ void decay_pass(float* s, float a0, float a1) {
    if constexpr (R == 32) {
        asm("s_nop 1\n\t"
            LA_DEC2(0, 0, 1) LA_DEC2(1, 2, 3) LA_DEC2(2, 4, 5) LA_DEC2(3, 6, 7) LA_DEC2(4, 8, 9)
            LA_DEC2(5, 10, 11) LA_DEC2(6, 12, 13) LA_DEC2(7, 14, 15) LA_DEC2(8, 16, 17) LA_DEC2(9, 18, 19)
            LA_DEC2(10, 20, 21) LA_DEC2(11, 22, 23) LA_DEC2(12, 24, 25) LA_DEC2(13, 26, 27)
            LA_DEC2(14, 28, 29) LA_DEC2(15, 30, 31)
            : LA_S32(s) : "v"(a0), "v"(a1));
    } else if constexpr (R == 16) {
        asm("s_nop 1\n\t"
            LA_DEC1(0) LA_DEC1(1) LA_DEC1(2) LA_DEC1(3) LA_DEC1(4) LA_DEC1(5) LA_DEC1(6) LA_DEC1(7)
            LA_DEC1(8) LA_DEC1(9) LA_DEC1(10) LA_DEC1(11) LA_DEC1(12) LA_DEC1(13) LA_DEC1(14) LA_DEC1(15)
            : LA_S16(s) : "v"(a0));
    } else {
        (void)a1;
        [&]<int... M>(std::integer_sequence<int, M...>) { (mul_bcast<M>(s[M], a0), ...); }(
            std::make_integer_sequence<int, R>{});
    }
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


// ------------------------------------------------------------------ rounding the state
// LDS for the cross-wave maxima of one workgroup (four waves, 64 columns).  Each rounding
// point uses slot qpar and flips it; a slot is rewritten two points later, after a barrier.
template <int DK, int QMODE, int G>
struct WaveQdqShared {
    float amax[2][kWaveTileWaves];
    float gmax[(QMODE == LA_QDQ_INT8_GROUP && G > kWaveCols) ? 2 : 1][kWaveTileWaves][DK];
};

// Round the state (true scale, this lane's R rows of its column) with the configured codec:
// INT8 groups of G columns along the value axis (groups wider than the wave's 16 columns
// meet through LDS) or one E4M3 scale per 64-column tile (the workgroup).  Every wave of the
// workgroup must call it at the same points: it contains barriers.
template <int R, int QMODE, int G, int DK>
__device__ __forceinline__ void wave_quantize(float* s, WaveQdqShared<DK, QMODE, G>& sh, int lane, int w, int& qpar) {
    const int rg = lane >> 4, c = lane & 15;
    if (QMODE == LA_QDQ_E4M3_TILE) {
        float mx = 0.0f;
#pragma unroll
        for (int m = 0; m < R; m++) mx = fmaxf(mx, fabsf(s[m]));
        mx = wave_max_abs(mx);
        if (lane == 0) sh.amax[qpar][w] = mx;
        __syncthreads();
        float amax = sh.amax[qpar][0];
#pragma unroll
        for (int ww = 1; ww < kWaveTileWaves; ww++) amax = fmaxf(amax, sh.amax[qpar][ww]);
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
    } else if (QMODE == LA_QDQ_INT8_GROUP) {
        float gm[R];
#pragma unroll
        for (int m = 0; m < R; m++) gm[m] = group_max_abs<(G < kWaveCols ? G : kWaveCols)>(s[m]);
        if constexpr (G > kWaveCols) {
            constexpr int NG = G / kWaveCols;
            if (c == 0) {
#pragma unroll
                for (int m = 0; m < R; m++) sh.gmax[qpar][w][rg * R + m] = gm[m];
            }
            __syncthreads();
            const int w_first = (w / NG) * NG;
#pragma unroll
            for (int i = 0; i < NG; i++) {
                const int ww = w_first + i;
                if (ww == w) continue;
#pragma unroll
                for (int m = 0; m < R; m++) gm[m] = fmaxf(gm[m], sh.gmax[qpar][ww][rg * R + m]);
            }
        }
#pragma unroll
        for (int m = 0; m < R; m++) {
            float sc8, y;
            const float cde = int8_scale_recip(gm[m], sc8, y) ? int8_code_fast(s[m], sc8, y) : int8_code(s[m], sc8);
            s[m] = cde * sc8;
        }
    }
    qpar ^= 1;
}

}  // namespace la
