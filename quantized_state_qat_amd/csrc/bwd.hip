// Straight-through backward of the recurrence.
//
// One workgroup per (sequence, head, value tile) in the token layout of la_tok.hpp (eight
// waves; each lane one value column of the tile and R key rows of it).  Chunks of
// C = ckpt_interval tokens are processed last to first, each in blocks of eight tokens:
//   phase A  recompute the chunk from its checkpoint with the forward's own token step,
//            storing the state entering every fourth token in the workspace;
//   phase B  for each group of four tokens, last to first: recompute it from the stored
//            state, keeping the state entering every token in registers, then walk it
//            backwards with the adjoint lambda = dL/dS in registers.  For chunks of at most 64
//            tokens phase A keeps every token's u and delta in LDS and the recompute is the
//            decay and the update with the kept delta alone.
// When every token is a rounding point of the INT8 codec (bwd_tok_coded), each carried state
// is its codes times its group scales: phase A runs the whole chunk and keeps every token's
// codes (fp16, exact) and scales in the workspace and its u and delta in LDS, and phase B
// walks the chunk's tokens last to first decoding the state entering each (the codes of the
// token before, loaded one token ahead) with no recompute.
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

// One token of the adjoint, in two halves around its barrier.  st: the state entering the
// token; u, dl: its u and delta; lam: dL/dS_t on entry, dL/dS_{t-1} on return.  Row sums run
// over the tile's TC columns.  adj_pre forms dS' = lambda + qq do^T and the partial sums of
// ddelta = dS'^T ku into red; adj_post takes ddelta, forms S~ and S' again (the same
// operations, so the same values, and no registers held over the barrier), the row sums, du,
// dS~ and the gate term (ga: exp(g) of this lane's reduce-scatter row, per-key gates only), and
// returns lambda = diag(a) dS~.
template <class S, bool KDA, bool HAD>
__device__ __forceinline__ void adj_pre(const TokOps<S, KDA>& op, float (&lam)[S::R], float2 (*red)[S::TC], int w,
                                        int lane) {
    constexpr float c1 = HAD ? 1.0f / S::DK : 1.0f;
    // c1 is a power of two: (q c1) do and q (c1 do) round to the same value
    const float c1do = c1 * op.dj;
    float pd = 0.0f;
#pragma unroll
    for (int m = 0; m < S::R; m++) {
        lam[m] = __builtin_fmaf(op.qr[m], c1do, lam[m]);             // dS' = lambda + qq do^T
        pd = __builtin_fmaf(lam[m], op.kr[m], pd);
    }
    pd = tok_rows_combine<S>(pd);
    if (lane < S::TC) red[w][lane] = make_float2(pd, 0.0f);
}

template <class S, bool KDA, bool HAD>
__device__ __forceinline__ void adj_post(const float (&st)[S::R], float u, float dl, const TokOps<S, KDA>& op, float ga,
                                         float (&lam)[S::R], const float2 (*red)[S::TC], int w, int lane, float* part,
                                         float* dv_out, bool writer) {
    constexpr int R = S::R, TC = S::TC, DK = S::DK;
    constexpr float c1 = HAD ? 1.0f / DK : 1.0f;
    constexpr int GW = PartLayout<DK, KDA>::GW;
    const int row = tok_row0<S>(w, lane) + reduce_scatter_row<R, TC>(lane);
    const int c = lane % TC;
    float sa[R], x[R];
#pragma unroll
    for (int m = 0; m < R; m++) {
        sa[m] = (KDA ? op.ar[m] : op.a) * st[m];                     // S~
        const float spm = __builtin_fmaf(op.kr[m], dl, sa[m]);       // S' (before rounding)
        x[m] = spm * op.dj;
    }
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
        part[2 * DK + row] = ga * x3;
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

template <class S, bool KDA, bool HAD>
__device__ __forceinline__ void tok_adjoint(const float (&st)[S::R], float u, float dl, const TokOps<S, KDA>& op,
                                            const float* ga_row, float (&lam)[S::R], float2 (*red)[S::TC], int w,
                                            int lane, float* part, float* dv_out, bool writer) {
    adj_pre<S, KDA, HAD>(op, lam, red, w, lane);
    __syncthreads();
    const float ga = KDA ? ga_row[tok_row0<S>(w, lane) + reduce_scatter_row<S::R, S::TC>(lane)] : 0.0f;
    adj_post<S, KDA, HAD>(st, u, dl, op, ga, lam, red, w, lane, part, dv_out, writer);
}

template <int DK, int QMODE, int G, bool HAD, bool KDA, bool CODED>
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
    // u and delta of the chunk's tokens (both walks, for chunks of at most kCodedMaxChunk
    // tokens).  With 32-column tiles and the scalar gate (PIPE) the adjoint of one chunk runs beside the
    // recompute of the chunk before it: a second token ring and reduction buffers for the
    // adjoint, and u and delta of two chunks.
    static_assert(!CODED || (QMODE == LA_QDQ_INT8_GROUP && !RQ && R % 2 == 0), "coded walk");
    constexpr bool PIPE = CODED && TC == 32 && !KDA;
    __shared__ float2 ud[PIPE ? 2 : 1][kCodedMaxChunk][TC];
    __shared__ std::conditional_t<PIPE, TokRing<S, KDA, true>, char> ringB;
    __shared__ float2 redB[PIPE ? 2 : 1][kTokWaves][TC];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int H = p.H, DV = p.dv, C = p.ckpt_interval;
    const int NB = DV / TC;
    const int col = blk * TC + lane % TC;
    const int r0 = tok_row0<S>(w, lane);
    const size_t bh = static_cast<size_t>(b) * H + h;
    const size_t state_off = bh * DK * DV;
    const size_t wg = bh * NB + blk;
    const size_t ntok = static_cast<size_t>(p.ntok);
    int T = p.T;
    size_t tok0 = static_cast<size_t>(b) * T * H + h;
    size_t ck0 = bh * p.nck;  // this unit's first checkpoint
    if (a.cu_seqlens) {
        // packed sequences: this one's token range (or one part of it) and checkpoint slots
        int t_begin, t_end;
        packed_range(a.cu_seqlens, a.split, a.split_part, b, p.T, t_begin, t_end);
        T = t_end - t_begin;
        tok0 = static_cast<size_t>(t_begin) * H + h;
        ck0 = static_cast<size_t>(h) * p.nck + b + t_begin / C;
        if (T == 0) {
            // nothing to walk: dS0 = dS_T (uniform over the workgroup)
#pragma unroll
            for (int m = 0; m < R; m++) {
                const size_t e = state_off + static_cast<size_t>(r0 + m) * DV + col;
                a.dS0[e] = a.dST ? a.dST[e] : 0.0f;
            }
            return;
        }
    }
    const int nck = (T + C - 1) / C;
    float* wsS = a.ws_states + wg * bwd_tok_ws_floats(C, DK, TC, G, CODED, PIPE);
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
        // (tokens past the chunk or the sequence, or of no chunk, fetch a valid token that is
        // never published: the loads stay unconditional)
        const int t = min(max(c, 0) * C + kBlkTok * j + w, T - 1);
        f.fetch(in, p, tok0 + static_cast<size_t>(t) * H, col, lane);
    };
    // publish block (c, j) from the fetched words, fetch (nc, nj), make the records visible
    auto publish = [&](int nt, int nc, int nj) __attribute__((always_inline)) {
        __syncthreads();  // the previous block's records are no longer read
        if (w < nt) f.template publish<RC>(ring, w, p, lane);
        fetch(nc, nj);
        __syncthreads();
    };

    fetch(nck - 1, 0);
    __builtin_amdgcn_s_waitcnt(0);
    int rp = 0;
    if constexpr (CODED) {
        constexpr int NH = R / 2;            // fp16 code pairs per lane and token
        constexpr int NSC = (64 / G) * R;    // scales per wave and token
        const int tid = threadIdx.x;
        // per chunk parity: codes [C][kTokThreads][NH], then scales [C][kTokWaves][NSC]
        const size_t region = static_cast<size_t>(C) * (kTokThreads * NH + kTokWaves * NSC);
        auto code_ptr = [&](int c, int off) {
            return reinterpret_cast<uint32_t*>(wsS + (PIPE ? (c & 1) : 0) * region) +
                   (static_cast<size_t>(off) * kTokThreads + tid) * NH;
        };
        auto scale_row = [&](int c, int off) {  // this wave's scales after chunk token off
            return wsS + (PIPE ? (c & 1) : 0) * region + static_cast<size_t>(C) * kTokThreads * NH +
                   (static_cast<size_t>(off) * kTokWaves + w) * NSC;
        };
        auto udp = [&](int c) { return ud[PIPE ? (c & 1) : 0]; };
        const int wrow = (lane / G) * R + reduce_scatter_row<R, G>(lane);
        const bool wsc = (lane & (G / R - 1)) == 0;  // one lane of each (row, group) stores its scale
        auto load_ck = [&](int c, float (&x)[R]) __attribute__((always_inline)) {
            const float* ck = a.ckpts + (ck0 + c) * DK * DV;
#pragma unroll
            for (int m = 0; m < R; m++) x[m] = ck[static_cast<size_t>(r0 + m) * DV + col];
        };
        auto chunk_len = [&](int c) { return min(T, (c + 1) * C) - c * C; };
        // after the recompute's token off of chunk c (of L tokens): keep u and delta and, but for
        // the chunk's last token, round the state keeping its codes and scales
        auto keep = [&](int c, int off, int L, float (&st)[R], float u, float dl) __attribute__((always_inline)) {
            if (w == 0 && lane < TC) udp(c)[off][lane] = make_float2(u, dl);
            if (off + 1 < L) {
                uint32_t hc[NH];
                float scl;
                tok_int8<R, G, true>(st, qsh.scr[w], lane, hc, &scl);
                uint32_t* dst = code_ptr(c, off);
#pragma unroll
                for (int q = 0; q < NH; q++) dst[q] = hc[q];
                if (wsc) scale_row(c, off)[wrow] = scl;
            }
        };
        // the state entering a token, loaded one token ahead into the other of two register sets
        // (the sets alternate by token and every loop takes two tokens per pass, so that no
        // loaded value is copied between iterations and the loads stay in flight over the
        // adjoint)
        struct Entering {
            uint32_t hc[NH];  // codes
            float sc[R];      // their scales
        };
        // the codes and scales of the state after token k of chunk c
        auto load_codes = [&](int c, int k, Entering& e) __attribute__((always_inline)) {
            const uint32_t* src = code_ptr(c, k);
#pragma unroll
            for (int q = 0; q < NH; q++) e.hc[q] = src[q];
            const float* sp = scale_row(c, k) + (lane / G) * R;
            if constexpr (R % 4 == 0) {
#pragma unroll
                for (int m = 0; m < R / 4; m++) {
                    const float4 x = reinterpret_cast<const float4*>(sp)[m];
                    e.sc[4 * m] = x.x;
                    e.sc[4 * m + 1] = x.y;
                    e.sc[4 * m + 2] = x.z;
                    e.sc[4 * m + 3] = x.w;
                }
            } else {
#pragma unroll
                for (int m = 0; m < R / 2; m++) {
                    const float2 x = reinterpret_cast<const float2*>(sp)[m];
                    e.sc[2 * m] = x.x;
                    e.sc[2 * m + 1] = x.y;
                }
            }
        };
        // the state entering token k of chunk c: for k > 0 the codes and scales of token k - 1;
        // for k = 0 the checkpoint's values as scales of unit codes (1 x value is exact)
        auto load_entering = [&](int c, int k, Entering& e) __attribute__((always_inline)) {
            if (k > 0) {
                load_codes(c, k - 1, e);
                return;
            }
            float x[R];
            load_ck(c, x);
#pragma unroll
            for (int q = 0; q < NH; q++) e.hc[q] = 0x3C003C00u;  // fp16 (1, 1)
#pragma unroll
            for (int m = 0; m < R; m++) e.sc[m] = x[m];
        };
        auto decode = [&](const Entering& cur, float (&st)[R]) __attribute__((always_inline)) {
#pragma unroll
            for (int q = 0; q < NH; q++) {
                const auto hv = __builtin_bit_cast(_Float16 __attribute__((ext_vector_type(2))), cur.hc[q]);
                st[2 * q] = static_cast<float>(hv[0]) * cur.sc[2 * q];
                st[2 * q + 1] = static_cast<float>(hv[1]) * cur.sc[2 * q + 1];
            }
        };
        // the recompute of chunk c alone (the block protocol of the recompute-per-group walk)
        auto run_a = [&](int c) {
            const int L = chunk_len(c), nb = nblocks(c), t0 = c * C, t1 = t0 + L;
            float st[R];
            load_ck(c, st);
#pragma unroll 1
            for (int j = 0; j < nb; j++) {
                const int nt = min(kBlkTok, t1 - (t0 + kBlkTok * j));
                if (j + 1 < nb) publish(nt, c, j + 1);
                else publish(nt, c, j);  // the adjoint starts with the same block
#pragma unroll 1
                for (int i = 0; i < nt; i++) {
                    TokOps<S, KDA> op;
                    tok_read<S, KDA, true>(op, ring, i, w, lane);
                    float u, dl, o;
                    tok_step<S, KDA, RC>(st, op, red[rp], w, lane, u, dl, o);
                    rp ^= 1;
                    keep(c, kBlkTok * j + i, L, st, u, dl);
                }
            }
        };
        // the adjoint of chunk c alone, tokens last to first
        auto run_b = [&](int c) {
            __builtin_amdgcn_s_waitcnt(0);  // every kept code is stored before any lane reads it
            __syncthreads();
            const int L = chunk_len(c), nb = nblocks(c), t0 = c * C, t1 = t0 + L;
            // The pipelined kernel keeps registers free: the checkpoint arrives as the entering
            // set of the chunk's first token.  The others hold it in registers and load codes
            // unconditionally (a clamped index reads codes that are not used), which keeps
            // their token free of branches.
            float ckr[PIPE ? 1 : R];
            if constexpr (!PIPE) load_ck(c, ckr);
            auto token = [&](int j, int i, const Entering& cur, Entering& nxt) __attribute__((always_inline)) {
                const int off = kBlkTok * j + i;
                float st[R];
                if constexpr (PIPE) {
                    if (off > 0) load_entering(c, off - 1, nxt);
                    decode(cur, st);
                } else {
                    load_codes(c, max(off - 2, 0), nxt);
                    decode(cur, st);
#pragma unroll
                    for (int m = 0; m < R; m++) st[m] = off == 0 ? ckr[m] : st[m];
                }
                TokOps<S, KDA> op;
                tok_read<S, KDA, true>(op, ring, i, w, lane);
                const float2 x = udp(c)[off][lane % TC];
                const size_t tok = tok0 + static_cast<size_t>(t0 + off) * H;
                float* part = a.ws_part + (static_cast<size_t>(blk) * ntok + tok) * PW;
                tok_adjoint<S, KDA, RC>(st, x.x, x.y, op, ring.ga[i], lam, red[rp], w, lane, part,
                                        a.dv + tok * DV + col, w == i);
                rp ^= 1;
            };
            Entering e0, e1;
            if constexpr (PIPE) load_entering(c, L - 1, e0);
            else load_codes(c, max(L - 2, 0), e0);
#pragma unroll 1
            for (int j = nb - 1; j >= 0; j--) {
                const int nt = min(kBlkTok, t1 - (t0 + kBlkTok * j));
                if (j > 0) publish(nt, c, j - 1);
                else publish(nt, c - 1, 0);
                int i = nt - 1;
                if (nt & 1) {  // (only the chunk's last block can hold an odd number of tokens)
                    token(j, i, e0, e1);
                    e0 = e1;
                    i--;
                }
#pragma unroll 1
                for (; i >= 1; i -= 2) {
                    token(j, i, e0, e1);
                    token(j, i - 1, e1, e0);
                }
            }
        };
        if constexpr (!PIPE) {
#pragma unroll 1
            for (int c = nck - 1; c >= 0; c--) {
                run_a(c);
                run_b(c);
            }
        } else {
            // The adjoint of full chunk c beside the recompute of chunk c - 1: per step one token
            // of each, their partial sums meeting behind one barrier (double-buffered by token
            // parity), so that the two independent chains fill each other's latencies.
            TokFetch<S, KDA, true> fa;  // the recompute's next block (f holds the adjoint's)
            auto fetch_a = [&](int c, int j) __attribute__((always_inline)) {
                const int t = min(max(c, 0) * C + kBlkTok * j + w, T - 1);
                fa.fetch(in, p, tok0 + static_cast<size_t>(t) * H, col, lane);
            };
            auto run_ab = [&](int c, bool first) {
                __builtin_amdgcn_s_waitcnt(0);  // the kept codes of chunk c are stored
                __syncthreads();
                if (first) fetch_a(c - 1, 0);
                const int nbk = C / kBlkTok, t0 = c * C;
                float sa_[R];
                load_ck(c - 1, sa_);
                auto step = [&](int m, int i, const Entering& cur, Entering& nxt) __attribute__((always_inline)) {
                    // recompute: token 8m + i of chunk c - 1; adjoint: token C - 1 - (8m + i) of
                    // chunk c, which is slot 7 - i of the adjoint's ring
                    const int offa = kBlkTok * m + i, offb = C - 1 - offa, ib = kBlkTok - 1 - i;
                    TokOps<S, KDA> opa, opb;
                    tok_read<S, KDA, true>(opa, ring, i, w, lane);
                    tok_read<S, KDA, true>(opb, ringB, ib, w, lane);
                    const float2 x = udp(c)[offb][lane % TC];
                    const float ga = KDA ? ringB.ga[ib][r0 + reduce_scatter_row<R, TC>(lane)] : 0.0f;
                    if (offb > 0) load_entering(c, offb - 1, nxt);
                    float st[R];
                    decode(cur, st);
                    tok_step_pre<S, KDA>(sa_, opa, red[i & 1], w, lane);
                    adj_pre<S, KDA, RC>(opb, lam, redB[i & 1], w, lane);
                    __syncthreads();
                    float u, dl, o;
                    tok_step_post<S, KDA, RC>(sa_, opa, red[i & 1], lane, u, dl, o);
                    keep(c - 1, offa, C, sa_, u, dl);
                    const size_t tok = tok0 + static_cast<size_t>(t0 + offb) * H;
                    float* part = a.ws_part + (static_cast<size_t>(blk) * ntok + tok) * PW;
                    adj_post<S, KDA, RC>(st, x.x, x.y, opb, ga, lam, redB[i & 1], w, lane, part,
                                         a.dv + tok * DV + col, w == ib);
                };
                Entering e0, e1;
                load_entering(c, C - 1, e0);
#pragma unroll 1
                for (int m = 0; m < nbk; m++) {
                    // publish block nbk-1-m of the adjoint and block m of the recompute; fetch the next two
                    __syncthreads();
                    f.template publish<RC>(ringB, w, p, lane);
                    fa.template publish<RC>(ring, w, p, lane);
                    if (m + 1 < nbk) {
                        fetch(c, nbk - 2 - m);
                        fetch_a(c - 1, m + 1);
                    } else {
                        fetch(c - 1, nbk - 1);
                        fetch_a(c - 2, 0);
                    }
                    __syncthreads();
#pragma unroll 1
                    for (int i = 0; i < kBlkTok; i += 2) {
                        step(m, i, e0, e1);
                        step(m, i + 1, e1, e0);
                    }
                }
            };
            int c = nck - 1;
            if (C % kBlkTok != 0) {
#pragma unroll 1
                for (; c >= 0; c--) {
                    run_a(c);
                    run_b(c);
                }
            } else {
                if (chunk_len(c) != C) {  // a ragged last chunk runs alone
                    run_a(c);
                    run_b(c);
                    c--;
                }
                if (c >= 0) {
                    run_a(c);
                    bool first = true;
#pragma unroll 1
                    for (; c >= 1; c--) {
                        run_ab(c, first);
                        first = false;
                    }
                    run_b(0);
                }
            }
        }
    } else {
#pragma unroll 1
    for (int c = nck - 1; c >= 0; c--) {
        const int t0 = c * C, t1 = min(T, t0 + C);
        const int nb = nblocks(c);
        {
            const int last_sub = ((t1 - t0 - 1) / kSubTok) * kSubTok;  // chunk offset of the last stored state
            // chunks of at most kCodedMaxChunk tokens keep every token's u and delta in LDS, and
            // phase B then re-forms each group's states from the kept values alone (the decay and
            // the update with the same delta: the same operations as the token step, without its
            // projections and barrier)
            const bool kept = C <= kCodedMaxChunk;

            // ---------------- phase A: advance through the chunk, storing the state entering
            // every fourth token (the chunk's first state is its checkpoint)
            {
                float s[R];
                const float* ck = a.ckpts + (ck0 + c) * DK * DV;
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
                        // without kept values the last group of the chunk is recomputed in phase B
                        // from its stored state
                        if (!kept && off >= last_sub) break;
                        TokOps<S, KDA> op;
                        tok_read<S, KDA, true>(op, ring, i, w, lane);
                        float u, dl, o;
                        const int t = tb + i;
                        const bool qpt = QMODE != LA_QDQ_NONE && (((t + 1) % p.qdq_interval) == 0 || t == T - 1);
                        tok_step<S, KDA, RC>(s, op, red[rp], w, lane, u, dl, o, p.replay && !qpt);
                        rp ^= 1;
                        if (kept && w == 0 && lane < TC) ud[0][off][lane] = make_float2(u, dl);
                        if (qpt && t + 1 < t1) tok_qdq_at<S, RQ>(s, qsh, tile, w, lane);
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
                        const float* ck = a.ckpts + (ck0 + c) * DK * DV;
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
                            const int t = tb + i0 + i;
                            const bool qpt = QMODE != LA_QDQ_NONE && (((t + 1) % p.qdq_interval) == 0 || t == T - 1);
                            if (kept) {
                                const float2 x = ud[0][kBlkTok * j + i0 + i][lane % TC];
                                uu[i] = x.x;
                                dd[i] = x.y;
                                const float du = p.replay && !qpt ? bf16_rne(x.y) : x.y;
#pragma unroll
                                for (int m = 0; m < R; m++) {
                                    s[m] = (KDA ? op.ar[m] : op.a) * s[m];
                                    s[m] = __builtin_fmaf(op.kr[m], du, s[m]);
                                }
                            } else {
                                float o;
                                tok_step<S, KDA, RC>(s, op, red[rp], w, lane, uu[i], dd[i], o, p.replay && !qpt);
                                rp ^= 1;
                            }
                            if (qpt && i + 1 < n) tok_qdq_at<S, RQ>(s, qsh, tile, w, lane);
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
    const size_t ntok = static_cast<size_t>(p.ntok);
    if (a.cu_seqlens) {
        // packed sequences: the sequence holding this token (the first, should ranges overlap);
        // a token of no sequence gets zero gradients (from the prefix pass of a split call), a
        // token outside this call's part is left to the other part's pass
        const int t = static_cast<int>(tok / p.H);
        int owner = -1;
        bool in_part = false;
        for (int b0 = 0; b0 < p.B; b0 += 64) {
            const int bb = b0 + lane;
            bool hit = false, hitp = false;
            if (bb < p.B) {
                int beg, end;
                packed_range(a.cu_seqlens, nullptr, 0, bb, p.T, beg, end);
                hit = t >= beg && t < end;
                if (hit && a.split) {
                    packed_range(a.cu_seqlens, a.split, a.split_part, bb, p.T, beg, end);
                    hitp = t >= beg && t < end;
                } else {
                    hitp = hit;
                }
            }
            const uint64_t m = __ballot(hit);
            if (m) {
                const int first = __builtin_ctzll(m);
                owner = b0 + first;
                in_part = __shfl(static_cast<int>(hitp), first) != 0;
                break;
            }
        }
        if (owner < 0) {
            if (a.split && a.split_part != 0) return;
            for (int i = lane; i < DK; i += 64) {
                a.dq[tok * DK + i] = 0.0f;
                a.dk[tok * DK + i] = 0.0f;
                if (KDA) a.dg[tok * DK + i] = 0.0f;
            }
            for (int i = lane; i < p.dv; i += 64) a.dv[tok * p.dv + i] = 0.0f;
            if (lane == 0) {
                if (!KDA) a.dg[tok] = 0.0f;
                a.dbeta[tok] = 0.0f;
            }
            return;
        }
        if (!in_part) return;
    }
    // One loop over the tiles for every field, so that the loads of several tiles are in
    // flight together; each sum keeps its tile order.
    float x1[NV], x2[NV], x3[NV];
    float gacc = 0.0f, bacc = 0.0f;
#pragma unroll
    for (int j = 0; j < NV; j++) {
        x1[j] = 0.0f;
        x2[j] = 0.0f;
        x3[j] = 0.0f;
    }
#pragma unroll 4
    for (int nb = 0; nb < NB; nb++) {
        // loads with no branch around them where every lane owns rows (d_k a multiple of 64;
        // every lane also forms the per-token sums), so that the compiler issues them together
        const float* part = a.ws_part + (static_cast<size_t>(nb) * ntok + tok) * PW;
#pragma unroll
        for (int j = 0; j < NV; j++) {
            const int i = lane + 64 * j;
            if (DK % 64 == 0 || i < DK) {
                x1[j] += part[i];
                x2[j] += part[DK + i];
                if (KDA) x3[j] += part[2 * DK + i];
            }
        }
        if (!KDA) {
#pragma unroll
            for (int i = 0; i < GW; i++) gacc += part[2 * DK + i];
        }
        bacc += part[2 * DK + GW];
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
            if (i < DK) a.dg[tok * DK + i] = x3[j];
        }
    } else if (lane == 0) {
        a.dg[tok] = gacc;
    }
    if (lane == 0) a.dbeta[tok] = bacc;
}

namespace {

template <int DK, int QMODE, int G, bool HAD, bool KDA>
hipError_t launch_bwd_t(const la_config& c, const BwdArgs& a, hipStream_t s) {
    TokParams p = make_tok_params(c);
    if (a.cu_seqlens) {
        p.nck = varlen_ckpt_slots(c);
        p.ntok = static_cast<long>(c.T) * c.H;
    }
    constexpr int TC = tok_tile_cols(DK, QMODE, G);
    dim3 grid(c.d_v / TC, c.H, c.B);
    constexpr bool CODED_OK = QMODE == LA_QDQ_INT8_GROUP && !(HAD && KDA) && tok_rows_per_lane(DK, TC) % 2 == 0;
    if (CODED_OK && bwd_tok_coded(c))
        hipLaunchKernelGGL((bwd_tok_kernel<DK, QMODE, G, HAD, KDA, CODED_OK>), grid, dim3(kTokThreads), 0, s, p, a);
    else
        hipLaunchKernelGGL((bwd_tok_kernel<DK, QMODE, G, HAD, KDA, false>), grid, dim3(kTokThreads), 0, s, p, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t ntok = static_cast<size_t>(p.ntok);
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
