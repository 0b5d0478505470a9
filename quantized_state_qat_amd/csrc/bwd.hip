// Straight-through backward of the recurrence.
//
// One workgroup per (sequence, head, value tile) in the token layout of la_tok.hpp (eight
// waves; each lane one value column of the tile and R key rows of it).  Chunks of
// C = ckpt_interval tokens are processed last to first, each in blocks of eight tokens:
//   phase A  recompute the chunk from its checkpoint with the forward's own token step,
//            storing the state entering every fourth token in the workspace;
//   phase B  for each group of four tokens, last to first: recompute it from the stored
//            state, keeping the state entering every token in registers, then walk it
//            backwards with the adjoint lambda = dL/dS in registers.
// A block's token records (la_tok.hpp) are published once per pass by its eight waves (wave w:
// token w of the block), and the next block's inputs are fetched while a block is processed.
// Per token (S~ = diag(a) S, u = S~^T k, S' = S~ + ku delta^T, o = S'^T qq; the quantizer
// passes the gradient through unchanged):
//   dS'    = lambda + qq do^T
//   dqq    = S' do                        (row sums over the value columns)
//   ddelta = dS'^T ku,  dv = beta ddelta, du = -beta ddelta, dbeta = ddelta . (v - u)
//   dku    = dS' delta,  dkp = S~ du      (row sums)
//   dS~    = dS' + kp du^T
//   da_i   = sum_j S_ij dS~_ij,  dg = a da (KDA per row; GDN summed over the state)
//   lambda = diag(a) dS~
// In Hadamard mode the state is carried rotated, Y = Hu S: ku = Hu k, kp = Hu k / d_k,
// qq = Hu q / d_k, and lambda is dL/dY.  Row sums are partial over the tile's columns; they are written per value tile and summed in a fixed order by
// bwd_reduce_kernel, which also maps the rotated-domain key and query gradients back
// (dk = Hu (dku + dkp / d_k), dq = Hu dqq / d_k).
#include "la_tok.hpp"

namespace la {

TokParams make_tok_params(const la_config& c);

constexpr int kBlkTok = kTokWaves;  // tokens per block (one record per wave)
constexpr int kSubTok = 4;          // tokens per stored state: phase B keeps kSubTok states live

// Partial-sum record of one token and value tile: dqq rows, dku + c1 dkp rows, the gate term
// (KDA: a_i da_i per row; GDN: a times one partial sum per wave) and dbeta.
template <int DK, bool KDA>
struct PartLayout {
    static constexpr int GW = KDA ? DK : kTokWaves;
    static constexpr int PW = 2 * DK + GW + 1;
};

// One token of the adjoint.  st: the state entering the token; u, dl: its u and delta;
// lam: dL/dS_t on entry, dL/dS_{t-1} on return.  Row sums run over the tile's TC columns.
template <class S, bool KDA, bool HAD>
__device__ __forceinline__ void tok_adjoint(const float (&st)[S::R], float u, float dl, const TokOps<S, KDA>& op,
                                            const float* ga_row, float (&lam)[S::R], float2 (*red)[S::TC], int w,
                                            int lane, float* part, float* dv_out, bool writer) {
    constexpr int R = S::R, TC = S::TC, DK = S::DK;
    constexpr float c1 = HAD ? 1.0f / DK : 1.0f;
    constexpr int GW = PartLayout<DK, KDA>::GW;
    const int row = tok_row0<S>(w, lane) + reduce_scatter_row<R, TC>(lane);
    // c1 is a power of two: (q c1) do and q (c1 do) round to the same value
    const float c1do = c1 * op.dj;
    float sa[R], x[R];
    float pd = 0.0f;
#pragma unroll
    for (int m = 0; m < R; m++) {
        sa[m] = (KDA ? op.ar[m] : op.a) * st[m];                     // S~
        const float spm = __builtin_fmaf(op.kr[m], dl, sa[m]);       // S' (before rounding)
        lam[m] = __builtin_fmaf(op.qr[m], c1do, lam[m]);             // dS' = lambda + qq do^T
        x[m] = spm * op.dj;
        pd = __builtin_fmaf(lam[m], op.kr[m], pd);
    }
    pd = tok_rows_combine<S>(pd);
    if (lane < TC) red[w][lane] = make_float2(pd, 0.0f);
    __syncthreads();
    const int c = lane % TC;
    float r[kTokWaves];
#pragma unroll
    for (int i = 0; i < kTokWaves; i++) r[i] = red[i][c].x;
    float ddel = r[0];
#pragma unroll
    for (int i = 1; i < kTokWaves; i++) ddel += r[i];
    const float x1 = reduce_scatter<OpAdd, R, TC>(x, lane);
    const float du = -op.beta * ddel;
    const float c1du = c1 * du;
#pragma unroll
    for (int m = 0; m < R; m++) {
        x[m] = __builtin_fmaf(lam[m], dl, sa[m] * c1du);            // dku + c1 dkp
        lam[m] = __builtin_fmaf(op.kr[m], c1du, lam[m]);             // dS~ = dS' + kp du^T
    }
    const float x2 = reduce_scatter<OpAdd, R, TC>(x, lane);
    part[row] = x1;
    part[DK + row] = x2;
    if (KDA) {
#pragma unroll
        for (int m = 0; m < R; m++) x[m] = st[m] * lam[m];
        const float x3 = reduce_scatter<OpAdd, R, TC>(x, lane);
        part[2 * DK + row] = ga_row[row] * x3;
    } else {
        float gp = 0.0f;
#pragma unroll
        for (int m = 0; m < R; m++) gp = __builtin_fmaf(st[m], lam[m], gp);
        gp = wave_sum(gp);
        if (lane == 0) part[2 * DK + w] = op.a * gp;
    }
#pragma unroll
    for (int m = 0; m < R; m++) lam[m] = (KDA ? op.ar[m] : op.a) * lam[m];
    if (writer) {
        if (lane < TC) *dv_out = op.beta * ddel;
        const float db = group_sum<TC>(ddel * (op.vj - u));
        if (lane == 0) part[2 * DK + GW] = db;
    }
}

template <int DK, int QMODE, int G, bool HAD, bool KDA>
__global__ __launch_bounds__(kTokThreads) void bwd_tok_kernel(TokParams p, BwdArgs a) {
    using S = TokShape<DK, QMODE, G>;
    constexpr int R = S::R, TC = S::TC;
    constexpr int PW = PartLayout<DK, KDA>::PW;
    // Hadamard mode: rotated carry for the scalar gate (RC), rotation around each rounding
    // point of the recompute for per-key gates (RQ; the adjoint is then the plain one)
    constexpr bool RC = HAD && !KDA, RQ = HAD && KDA;
    __shared__ TokRing<S, KDA, true> ring;
    __shared__ float2 red[2][kTokWaves][TC];
    __shared__ TokQdqShared<S> qsh;
    __shared__ float tile[HAD ? 2 * DK * TC : 1];  // tok_rotate's two tiles

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int T = p.T, H = p.H, DV = p.dv, C = p.ckpt_interval;
    const int NB = DV / TC;
    const int col = blk * TC + lane % TC;
    const int r0 = tok_row0<S>(w, lane);
    const size_t bh = static_cast<size_t>(b) * H + h;
    const size_t state_off = bh * DK * DV;
    const size_t wg = bh * NB + blk;
    const size_t ntok = static_cast<size_t>(p.B) * T * H;
    const size_t tok0 = static_cast<size_t>(b) * T * H + h;
    const int nsub = (C + kSubTok - 1) / kSubTok;
    float* wsS = a.ws_states + wg * static_cast<size_t>(nsub) * DK * TC;
    const TokInputs in{a.q, a.k, a.v, a.g, a.beta, a.dout};

    float lam[R];
#pragma unroll
    for (int m = 0; m < R; m++)
        lam[m] = a.dST ? a.dST[state_off + static_cast<size_t>(r0 + m) * DV + col] : 0.0f;
    if (RC && !p.rot) tok_rotate<S>(lam, tile, w, lane, 1.0f / DK);  // dL/dY = Hu dL/dS / d_k

    // Blocks in processing order: chunk c from last to first; in each, phase A over blocks
    // j = 0 .. nb-1, then phase B over j = nb-1 .. 0.  The inputs of the next block in this
    // order are fetched while a block is processed.
    auto nblocks = [&](int c) { return (min(T, (c + 1) * C) - c * C + kBlkTok - 1) / kBlkTok; };
    TokFetch<S, KDA, true> f;
    auto fetch = [&](int c, int j) __attribute__((always_inline)) {
        if (c < 0) return;
        const int t = c * C + kBlkTok * j + w;
        if (t < min(T, (c + 1) * C)) f.fetch(in, p, tok0 + static_cast<size_t>(t) * H, col, lane);
    };
    // publish block (c, j) from the fetched words, fetch (nc, nj), make the records visible
    auto publish = [&](int nt, int nc, int nj) __attribute__((always_inline)) {
        __syncthreads();  // the previous block's records are no longer read
        if (w < nt) f.template publish<RC>(ring, w, p, lane);
        fetch(nc, nj);
        __syncthreads();
    };

    fetch(p.nck - 1, 0);
    __builtin_amdgcn_s_waitcnt(0);
    int rp = 0;
#pragma unroll 1
    for (int c = p.nck - 1; c >= 0; c--) {
        const int t0 = c * C, t1 = min(T, t0 + C);
        const int nb = nblocks(c);
        const int last_sub = ((t1 - t0 - 1) / kSubTok) * kSubTok;  // chunk offset of the last stored state

        // ---------------- phase A: advance through the chunk, storing the state entering
        // every fourth token (the chunk's first state is its checkpoint)
        {
            float s[R];
            const float* ck = a.ckpts + (bh * p.nck + c) * DK * DV;
#pragma unroll
            for (int m = 0; m < R; m++) s[m] = ck[static_cast<size_t>(r0 + m) * DV + col];
#pragma unroll 1
            for (int j = 0; j < nb; j++) {
                const int tb = t0 + kBlkTok * j;
                const int nt = min(kBlkTok, t1 - tb);
                if (j + 1 < nb) publish(nt, c, j + 1);
                else publish(nt, c, j);  // phase B starts with the same block
#pragma unroll 1
                for (int i = 0; i < nt; i++) {
                    const int off = kBlkTok * j + i;  // token offset in the chunk
                    if ((off % kSubTok) == 0 && off > 0) {
                        float* dst = wsS + static_cast<size_t>(off / kSubTok) * DK * TC;
#pragma unroll
                        for (int m = 0; m < R; m++) dst[(r0 + m) * TC + lane % TC] = s[m];
                    }
                    // the last group of the chunk is recomputed in phase B from its stored state
                    if (off >= last_sub) break;
                    TokOps<S, KDA> op;
                    tok_read<S, KDA, true>(op, ring, i, w, lane);
                    float u, dl, o;
                    tok_step<S, KDA, RC>(s, op, red[rp], w, lane, u, dl, o);
                    rp ^= 1;
                    const int t = tb + i;
                    if (QMODE != LA_QDQ_NONE && (((t + 1) % p.qdq_interval) == 0 || t == T - 1))
                        tok_qdq_at<S, RQ>(s, qsh, tile, w, lane);
                }
            }
        }
        // ---------------- phase B: per group of four tokens, last first: recompute it keeping
        // every entering state, then the adjoint
#pragma unroll 1
        for (int j = nb - 1; j >= 0; j--) {
            const int tb = t0 + kBlkTok * j;
            const int nt = min(kBlkTok, t1 - tb);
            if (j > 0) publish(nt, c, j - 1);
            else publish(nt, c - 1, 0);
#pragma unroll 1
            for (int hh = (nt - 1) / kSubTok; hh >= 0; hh--) {
                const int i0 = kSubTok * hh, n = min(kSubTok, nt - i0);
                float s[R];
                if (j == 0 && hh == 0) {
                    const float* ck = a.ckpts + (bh * p.nck + c) * DK * DV;
#pragma unroll
                    for (int m = 0; m < R; m++) s[m] = ck[static_cast<size_t>(r0 + m) * DV + col];
                } else {
                    const float* src = wsS + static_cast<size_t>(kBlkTok / kSubTok * j + hh) * DK * TC;
#pragma unroll
                    for (int m = 0; m < R; m++) s[m] = src[(r0 + m) * TC + lane % TC];
                }
                float st[kSubTok][R];
                float uu[kSubTok], dd[kSubTok];
#pragma unroll
                for (int i = 0; i < kSubTok; i++) {
                    if (i < n) {
#pragma unroll
                        for (int m = 0; m < R; m++) st[i][m] = s[m];
                        TokOps<S, KDA> op;
                        tok_read<S, KDA, true>(op, ring, i0 + i, w, lane);
                        float o;
                        tok_step<S, KDA, RC>(s, op, red[rp], w, lane, uu[i], dd[i], o);
                        rp ^= 1;
                        const int t = tb + i0 + i;
                        if (QMODE != LA_QDQ_NONE && i + 1 < n && (((t + 1) % p.qdq_interval) == 0 || t == T - 1))
                            tok_qdq_at<S, RQ>(s, qsh, tile, w, lane);
                    }
                }
#pragma unroll
                for (int i = kSubTok - 1; i >= 0; i--) {
                    if (i < n) {
                        TokOps<S, KDA> op;
                        tok_read<S, KDA, true>(op, ring, i0 + i, w, lane);
                        const size_t tok = tok0 + static_cast<size_t>(tb + i0 + i) * H;
                        float* part = a.ws_part + (static_cast<size_t>(blk) * ntok + tok) * PW;
                        tok_adjoint<S, KDA, RC>(st[i], uu[i], dd[i], op, ring.ga[i0 + i], lam, red[rp], w, lane,
                                                  part, a.dv + tok * DV + col, w == i0 + i);
                        rp ^= 1;
                    }
                }
            }
        }
    }
    if (RC && !p.rot) tok_rotate<S>(lam, tile, w, lane, 1.0f);  // dL/dS = Hu dL/dY
#pragma unroll
    for (int m = 0; m < R; m++) a.dS0[state_off + static_cast<size_t>(r0 + m) * DV + col] = lam[m];
}

// Sum the per-tile partials in tile order and write dq, dk, dg, dbeta.  One wave per token.
template <int DK, bool HAD, bool KDA>
__global__ __launch_bounds__(64) void bwd_reduce_kernel(TokParams p, BwdArgs a, int NB) {
    constexpr int GW = PartLayout<DK, KDA>::GW;
    constexpr int PW = PartLayout<DK, KDA>::PW;
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
        for (int nb = 0; nb < NB; nb++)
            for (int i = 0; i < GW; i++) acc += a.ws_part[(static_cast<size_t>(nb) * ntok + tok) * PW + 2 * DK + i];
        a.dg[tok] = acc;
    }
    if (lane == 0) {
        float acc = 0.0f;
        for (int nb = 0; nb < NB; nb++) acc += a.ws_part[(static_cast<size_t>(nb) * ntok + tok) * PW + 2 * DK + GW];
        a.dbeta[tok] = acc;
    }
}

namespace {

template <int DK, int QMODE, int G, bool HAD, bool KDA>
hipError_t launch_bwd_t(const la_config& c, const BwdArgs& a, hipStream_t s) {
    const TokParams p = make_tok_params(c);
    constexpr int TC = tok_tile_cols(DK, QMODE, G);
    dim3 grid(c.d_v / TC, c.H, c.B);
    hipLaunchKernelGGL((bwd_tok_kernel<DK, QMODE, G, HAD, KDA>), grid, dim3(kTokThreads), 0, s, p, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t ntok = static_cast<size_t>(c.B) * c.T * c.H;
    if (ntok == 0) return hipSuccess;
    hipLaunchKernelGGL((bwd_reduce_kernel<DK, HAD && !KDA, KDA>), dim3(static_cast<unsigned>(ntok)), dim3(64), 0, s, p, a,
                       c.d_v / TC);
    return hipGetLastError();
}

template <int DK, bool HAD, bool KDA>
hipError_t launch_bwd_q(const la_config& c, const BwdArgs& a, hipStream_t s) {
    if (!HAD) {
        if (c.qdq == LA_QDQ_NONE) return launch_bwd_t<DK, LA_QDQ_NONE, 16, HAD, KDA>(c, a, s);
        if (c.qdq == LA_QDQ_E4M3_TILE) return launch_bwd_t<DK, LA_QDQ_E4M3_TILE, 64, HAD, KDA>(c, a, s);
    }
    switch (c.group) {
        case 16: return launch_bwd_t<DK, LA_QDQ_INT8_GROUP, 16, HAD, KDA>(c, a, s);
        case 32: return launch_bwd_t<DK, LA_QDQ_INT8_GROUP, 32, HAD, KDA>(c, a, s);
        default: return launch_bwd_t<DK, LA_QDQ_INT8_GROUP, 64, HAD, KDA>(c, a, s);
    }
}

template <int DK>
hipError_t launch_bwd_dk(const la_config& c, const BwdArgs& a, hipStream_t s) {
    if (c.hadamard)
        return c.gate == LA_GATE_KEY ? launch_bwd_q<DK, true, true>(c, a, s) : launch_bwd_q<DK, true, false>(c, a, s);
    if (c.gate == LA_GATE_KEY) return launch_bwd_q<DK, false, true>(c, a, s);
    return launch_bwd_q<DK, false, false>(c, a, s);
}

}  // namespace

hipError_t launch_bwd(const la_config& c, const BwdArgs& a, hipStream_t s) {
    switch (c.d_k) {
        case 16: return launch_bwd_dk<16>(c, a, s);
        case 32: return launch_bwd_dk<32>(c, a, s);
        case 64: return launch_bwd_dk<64>(c, a, s);
        default: return launch_bwd_dk<128>(c, a, s);
    }
}

}  // namespace la
