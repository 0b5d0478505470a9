// Straight-through backward of the recurrence.
//
// One workgroup per (sequence, head, 64-column value tile), the same lane/row layout as
// the forward.  Chunks of C = ckpt_interval tokens are processed last to first:
//   phase A  recompute the chunk from its checkpoint with the forward's own device code
//            (la_recur.hpp), spilling the state entering each token and (u, delta) of each
//            token to a per-workgroup workspace;
//   phase B  walk the chunk backwards with the adjoint lambda = dL/dS in VGPRs.
// Per token (general form of la_recur.hpp: S~ = diag(a) S, u = S~^T kp, S' = S~ + ku delta^T,
// o = S'^T qq, identity straight-through gradient through the quantizer):
//   dS'    = lambda + qq do^T
//   dqq    = S' do                        (row sums over value columns)
//   ddelta = dS'^T ku,  dv = beta ddelta, du = -beta ddelta, dbeta = ddelta . (v - u)
//   dku    = dS' delta,  dkp = S~ du      (row sums)
//   dS~    = dS' + kp du^T
//   da_i   = sum_j S_ij dS~_ij,  dg = a da (KDA per row; GDN summed over the state)
//   lambda = diag(a) dS~
// Row sums are partial over the tile's 64 columns; they are written per value tile and
// summed in a fixed order by bwd_reduce_kernel, which also maps the rotated-domain key and
// query gradients back (dk = Hu (dku + dkp / d_k), dq = Hu dqq / d_k) in Hadamard mode.
#include "la_recur.hpp"

namespace la {

Params make_params(const la_config& c);

// Sum over the 64 lanes of x[i] for every i < R, delivered transposed: afterwards lane L
// holds the total of row rowsum_row<R>(L).  A reduce-scatter butterfly: at each step a lane
// keeps one half of its vector and adds the partner's copy of that half.
template <int R>
__device__ __forceinline__ float rowsum(float (&x)[R], int lane) {
#pragma unroll
    for (int st = 0; (R >> st) > 1; st++) {
        const int len = R >> st, half = len / 2, mask = 32 >> st;
        const bool up = (lane & mask) != 0;
#pragma unroll
        for (int i = 0; i < half; i++) {
            float send = up ? x[i] : x[i + half];
            float keep = up ? x[i + half] : x[i];
            x[i] = keep + xor_shfl(send, mask);
        }
    }
    float y = x[0];
#pragma unroll
    for (int m = (64 / R) / 2; m >= 1; m >>= 1) y += xor_shfl(y, m);
    return y;
}

template <int R>
__device__ __forceinline__ int rowsum_row(int lane) {
    int row = 0;
#pragma unroll
    for (int st = 0; (R >> st) > 1; st++) row += ((lane >> (5 - st)) & 1) * (R >> (st + 1));
    return row;
}

template <int DK, int QMODE, int G, bool HAD, bool KDA>
__global__ __launch_bounds__(kThreads) void bwd_kernel(Params p, BwdArgs a) {
    constexpr int R = DK / 4;
    constexpr int GW = KDA ? DK : 1;
    constexpr int PW = 2 * DK + GW + 1;
    constexpr float c1 = HAD ? 1.0f / DK : 1.0f;
    __shared__ Smem<DK> sm;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int T = p.T, H = p.H, DV = p.dv, C = p.ckpt_interval;
    const int NB = DV / kTileCols;
    const int col = blk * kTileCols + lane;
    const size_t bh = static_cast<size_t>(b) * H + h;
    const size_t state_off = bh * DK * DV;
    const size_t wg = bh * NB + blk;
    const size_t ntok = static_cast<size_t>(p.B) * T * H;
    float* wsS = a.ws_states + wg * static_cast<size_t>(C) * DK * kTileCols;
    float* wsV = a.ws_vecs + wg * static_cast<size_t>(C) * 4 * 2 * kTileCols;
    const int my_row = w * R + rowsum_row<R>(lane);
    const bool row_writer = (lane & (64 / R - 1)) == 0;

    float lam[R];
#pragma unroll
    for (int m = 0; m < R; m++)
        lam[m] = a.dST ? a.dST[state_off + static_cast<size_t>(w * R + m) * DV + col] : 0.0f;
    if (HAD && !p.rot) rotate_state<DK>(sm, lam, 1.0f / DK);  // dL/dY = Hu dL/dS / d_k

#pragma unroll 1
    for (int c = p.nck - 1; c >= 0; c--) {
        const int t0 = c * C;
        const int t1 = min(T, t0 + C);
        // ---------------- phase A: recompute the chunk's carried states
        float s[R];
        const float* ck = a.ckpts + (bh * p.nck + c) * DK * DV;
#pragma unroll
        for (int m = 0; m < R; m++) s[m] = ck[static_cast<size_t>(w * R + m) * DV + col];
#pragma unroll 1
        for (int t = t0; t < t1; t++) {
            float* dst = wsS + static_cast<size_t>(t - t0) * DK * kTileCols;
#pragma unroll
            for (int m = 0; m < R; m++) dst[(w * R + m) * kTileCols + lane] = s[m];
            const size_t tok = (static_cast<size_t>(b) * T + t) * H + h;
            float vj = load_elem(a.v, tok * DV + col, p.qkv_dt);
            stage_token<DK, HAD, KDA>(sm, a.q, a.k, a.g, a.beta, tok, p.qkv_dt, p.gate_dt);
            float u, d, o;
            bool qnow = (QMODE != LA_QDQ_NONE) && is_qdq_point(t, T, p.qdq_interval);
            token_step<DK, QMODE, G>(sm, s, vj, qnow, u, d, o);
            float* vec = wsV + (static_cast<size_t>(t - t0) * 4 + w) * 2 * kTileCols;
            vec[lane] = u;
            vec[kTileCols + lane] = d;
        }
        // ---------------- phase B: reverse adjoint over the chunk
#pragma unroll 1
        for (int t = t1 - 1; t >= t0; t--) {
            const size_t tok = (static_cast<size_t>(b) * T + t) * H + h;
            stage_token<DK, HAD, KDA>(sm, a.q, a.k, a.g, a.beta, tok, p.qkv_dt, p.gate_dt);
            const float* src = wsS + static_cast<size_t>(t - t0) * DK * kTileCols;
            float sp[R];
#pragma unroll
            for (int m = 0; m < R; m++) sp[m] = src[(w * R + m) * kTileCols + lane];
            const float* vec = wsV + (static_cast<size_t>(t - t0) * 4 + w) * 2 * kTileCols;
            const float u = vec[lane], d = vec[kTileCols + lane];
            const float vj = load_elem(a.v, tok * DV + col, p.qkv_dt);
            const float doj = a.dout[tok * DV + col];
            const float beta = sm.beta;
            float x[R];
            // dS' = lambda + qq do^T ;  dqq = S' do  (S' recomputed exactly as the forward does)
#pragma unroll
            for (int m = 0; m < R; m++) {
                const int row = w * R + m;
                lam[m] = __builtin_fmaf(sm.qraw[row], doj, lam[m]);
                float spr = __builtin_fmaf(sm.ku[row], d, sm.a[row] * sp[m]);
                x[m] = spr * doj;
            }
            float X1 = rowsum<R>(x, lane);
            // ddelta = dS'^T ku (column sums over the key axis)
            float pd = 0.0f;
#pragma unroll
            for (int m = 0; m < R; m++) pd = __builtin_fmaf(lam[m], sm.ku[w * R + m], pd);
            sm.red[w][lane] = make_float2(pd, 0.0f);
            __syncthreads();
            const float ddel = ((sm.red[0][lane].x + sm.red[1][lane].x) + sm.red[2][lane].x) + sm.red[3][lane].x;
            const float du = -beta * ddel;
            // dku + c1 dkp = dS' delta + c1 S~ du
#pragma unroll
            for (int m = 0; m < R; m++) {
                const int row = w * R + m;
                x[m] = __builtin_fmaf(lam[m], d, c1 * ((sm.a[row] * sp[m]) * du));
            }
            float X2 = rowsum<R>(x, lane);
            // dS~ = dS' + kp du^T
#pragma unroll
            for (int m = 0; m < R; m++) lam[m] = __builtin_fmaf(sm.kraw[w * R + m], du, lam[m]);
            float X3 = 0.0f;
            if (KDA) {
#pragma unroll
                for (int m = 0; m < R; m++) x[m] = sp[m] * lam[m];
                X3 = rowsum<R>(x, lane);
            } else {
                float gp = 0.0f;
#pragma unroll
                for (int m = 0; m < R; m++) gp = __builtin_fmaf(sp[m], lam[m], gp);
                gp = wave_sum(gp);
                if (lane == 0) sm.scal[w] = gp;
                __syncthreads();
            }
            float* part = a.ws_part + (static_cast<size_t>(blk) * ntok + tok) * PW;
            if (row_writer) {
                part[my_row] = X1;
                part[DK + my_row] = X2;
                if (KDA) part[2 * DK + my_row] = sm.a[my_row] * X3;
            }
            if (w == 0) {
                a.dv[tok * DV + col] = beta * ddel;
                float db = wave_sum(ddel * (vj - u));
                if (lane == 0) {
                    part[2 * DK + GW] = db;
                    if (!KDA) part[2 * DK] = sm.a[0] * (((sm.scal[0] + sm.scal[1]) + sm.scal[2]) + sm.scal[3]);
                }
            }
            // lambda = diag(a) dS~  (= dL/dS_{t-1})
#pragma unroll
            for (int m = 0; m < R; m++) lam[m] = sm.a[w * R + m] * lam[m];
        }
    }
    if (HAD && !p.rot) rotate_state<DK>(sm, lam, 1.0f);  // dL/dS = Hu dL/dY
#pragma unroll
    for (int m = 0; m < R; m++) a.dS0[state_off + static_cast<size_t>(w * R + m) * DV + col] = lam[m];
}

// Sum the per-tile partials in tile order and write dq, dk, dg, dbeta.  One wave per token.
template <int DK, bool HAD, bool KDA>
__global__ __launch_bounds__(64) void bwd_reduce_kernel(Params p, BwdArgs a, int NB) {
    constexpr int GW = KDA ? DK : 1;
    constexpr int PW = 2 * DK + GW + 1;
    constexpr int NV = (DK + 63) / 64;
    const int lane = threadIdx.x;
    const size_t tok = blockIdx.x;
    const size_t ntok = static_cast<size_t>(p.B) * p.T * p.H;
    float x1[NV], x2[NV];
#pragma unroll
    for (int j = 0; j < NV; j++) {
        x1[j] = 0.0f;
        x2[j] = 0.0f;
        const int i = lane + 64 * j;
        if (i < DK) {
            for (int nb = 0; nb < NB; nb++) {
                const float* part = a.ws_part + (static_cast<size_t>(nb) * ntok + tok) * PW;
                x1[j] += part[i];
                x2[j] += part[DK + i];
            }
        }
    }
    if (HAD) {
        if (NV == 2) {
            float s0 = x1[0] + x1[NV - 1], s1 = x1[0] - x1[NV - 1];
            x1[0] = s0; x1[NV - 1] = s1;
            s0 = x2[0] + x2[NV - 1]; s1 = x2[0] - x2[NV - 1];
            x2[0] = s0; x2[NV - 1] = s1;
        }
#pragma unroll
        for (int hs = 1; hs < 64 && hs < DK; hs <<= 1) {
            const bool hi = (lane & hs) != 0;
#pragma unroll
            for (int j = 0; j < NV; j++) {
                float o1 = xor_shfl(x1[j], hs), o2 = xor_shfl(x2[j], hs);
                x1[j] = hi ? (o1 - x1[j]) : (x1[j] + o1);
                x2[j] = hi ? (o2 - x2[j]) : (x2[j] + o2);
            }
        }
    }
    constexpr float inv = 1.0f / DK;
#pragma unroll
    for (int j = 0; j < NV; j++) {
        const int i = lane + 64 * j;
        if (i < DK) {
            a.dq[tok * DK + i] = HAD ? x1[j] * inv : x1[j];
            a.dk[tok * DK + i] = x2[j];
        }
    }
    if (KDA) {
#pragma unroll
        for (int j = 0; j < NV; j++) {
            const int i = lane + 64 * j;
            if (i < DK) {
                float acc = 0.0f;
                for (int nb = 0; nb < NB; nb++) acc += a.ws_part[(static_cast<size_t>(nb) * ntok + tok) * PW + 2 * DK + i];
                a.dg[tok * DK + i] = acc;
            }
        }
    } else if (lane == 0) {
        float acc = 0.0f;
        for (int nb = 0; nb < NB; nb++) acc += a.ws_part[(static_cast<size_t>(nb) * ntok + tok) * PW + 2 * DK];
        a.dg[tok] = acc;
    }
    if (lane == 0) {
        float acc = 0.0f;
        for (int nb = 0; nb < NB; nb++) acc += a.ws_part[(static_cast<size_t>(nb) * ntok + tok) * PW + 2 * DK + GW];
        a.dbeta[tok] = acc;
    }
}

template <int DK, int QMODE, int G, bool HAD, bool KDA>
static hipError_t launch_bwd_t(const la_config& c, const BwdArgs& a, hipStream_t s) {
    Params p = make_params(c);
    dim3 grid(c.d_v / kTileCols, c.H, c.B);
    hipLaunchKernelGGL((bwd_kernel<DK, QMODE, G, HAD, KDA>), grid, dim3(kThreads), 0, s, p, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    size_t ntok = static_cast<size_t>(c.B) * c.T * c.H;
    if (ntok == 0) return hipSuccess;
    hipLaunchKernelGGL((bwd_reduce_kernel<DK, HAD, KDA>), dim3(static_cast<unsigned>(ntok)), dim3(64), 0, s, p,
                       a, c.d_v / kTileCols);
    return hipGetLastError();
}

template <int DK>
static hipError_t launch_bwd_dk(const la_config& c, const BwdArgs& a, hipStream_t s) {
    const bool kda = c.gate == LA_GATE_KEY;
    if (c.qdq == LA_QDQ_NONE)
        return kda ? launch_bwd_t<DK, LA_QDQ_NONE, 1, false, true>(c, a, s)
                   : launch_bwd_t<DK, LA_QDQ_NONE, 1, false, false>(c, a, s);
    if (c.qdq == LA_QDQ_E4M3_TILE)
        return kda ? launch_bwd_t<DK, LA_QDQ_E4M3_TILE, 64, false, true>(c, a, s)
                   : launch_bwd_t<DK, LA_QDQ_E4M3_TILE, 64, false, false>(c, a, s);
    if (c.hadamard) {
        switch (c.group) {
            case 16: return launch_bwd_t<DK, LA_QDQ_INT8_GROUP, 16, true, false>(c, a, s);
            case 32: return launch_bwd_t<DK, LA_QDQ_INT8_GROUP, 32, true, false>(c, a, s);
            default: return launch_bwd_t<DK, LA_QDQ_INT8_GROUP, 64, true, false>(c, a, s);
        }
    }
    switch (c.group) {
        case 16: return kda ? launch_bwd_t<DK, LA_QDQ_INT8_GROUP, 16, false, true>(c, a, s)
                            : launch_bwd_t<DK, LA_QDQ_INT8_GROUP, 16, false, false>(c, a, s);
        case 32: return kda ? launch_bwd_t<DK, LA_QDQ_INT8_GROUP, 32, false, true>(c, a, s)
                            : launch_bwd_t<DK, LA_QDQ_INT8_GROUP, 32, false, false>(c, a, s);
        default: return kda ? launch_bwd_t<DK, LA_QDQ_INT8_GROUP, 64, false, true>(c, a, s)
                            : launch_bwd_t<DK, LA_QDQ_INT8_GROUP, 64, false, false>(c, a, s);
    }
}

hipError_t launch_bwd(const la_config& c, const BwdArgs& a, hipStream_t s) {
    switch (c.d_k) {
        case 16: return launch_bwd_dk<16>(c, a, s);
        case 32: return launch_bwd_dk<32>(c, a, s);
        case 64: return launch_bwd_dk<64>(c, a, s);
        default: return launch_bwd_dk<128>(c, a, s);
    }
}

}  // namespace la
