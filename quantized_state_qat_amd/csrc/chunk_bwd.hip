// 64-token chunk path, straight-through backward (the chain rule through each chunk's terms of
// la_chunk.hpp, identity through every rounding; "Experimental GDN/KDA approximate-inverse QAT",
// What does this PR do?: the backward differentiates the polynomial actually used).  From the
// forward's checkpoints (one per chunk), four launches:
//   prep      the chunk records in the backward layout (chunk_fwd.hip's prep kernel);
//   recompute U = V - Kp S and Delta = P diag(beta) U of every chunk, all chunks in parallel;
//   dstate    per (sequence, head, 64 value columns), chunks last to first: dS carried in
//             registers, dDelta = Kd dS_end + M^T dO, dR = P^T dDelta, dv = beta dR, the partial
//             beta gradient, dS <- E_L dS + Qp^T dO - Kp^T dv; dS0 at the end;
//   grad      per (sequence, head, chunk): the products over value columns (dP = dDelta R^T,
//             dM = dO Delta^T, dQp = dO S^T, dKp = -dv S^T, dKd = Delta dS_end^T, dE_L), the
//             backward of the solve, the decays and the pair sums, and the gate gradient as a
//             suffix sum of the cumulative-decay gradient.
#include "la_chunk.hpp"

namespace la {

ChunkParams make_chunk_params(const la_config& c);
hipError_t launch_chunk_prep(const la_config& c, const ChunkIn& in, float* rec, bool bwd, hipStream_t s);

namespace {

constexpr int kSP = 20;             // pitch of the gradient kernel's 16-column slabs
constexpr int kTK = kCh * 132;      // one token-by-key array (pitch 132)
constexpr int kWM = kCh * kPW;      // one 64 x 64 work matrix
constexpr int kBig = 6 * kWM;       // the gradient kernel's phase-shared LDS (floats)
constexpr int kGW = 8;              // the gradient kernel's waves (two per SIMD: its phases wait on
constexpr int kGT = 64 * kGW;       // memory and LDS, and the second wave fills those gaps)
static_assert(5 * kCh * kSP + 2 * kChDk * kSP <= 3 * kWM, "slabs overlap the dP buffer");
static_assert(3 * kTK <= kBig && 2 * kTK + kWM <= kBig, "phase buffers exceed the shared array");

struct ChunkBwdPtrs {
    const float* ckpts;   // [B][H][nch][128][d_v], the state entering every chunk
    const float* dout;
    const float* dST;
    float* dq;
    float* dk;
    float* dv;
    float* dg;
    float* dbeta;
    float* dS0;
    float* rec;           // [B H nch] backward records
    float* U;             // [B H nch][64][d_v]
    float* D;             // Delta, same layout
    float* dD;            // dDelta, same layout
    float* dSe;           // [B H nch][128][d_v]: dL/d(state after the chunk)
    float* dbp;           // [ntile][B H nch][64]: beta-gradient partial per value tile
};

// U and Delta of one (sequence, head, chunk, 64 columns) from the chunk's checkpoint.
__global__ __launch_bounds__(kChThreads) void chunk_recompute_kernel(ChunkParams p, ChunkIn in, ChunkBwdPtrs a) {
    __shared__ __align__(16) float Kp_s[kCh * RecB::PK];
    __shared__ __align__(16) float P_s[kCh * RecB::PP];
    __shared__ __align__(16) float b_s[kCh];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
    // the value tiles of a chunk 8 workgroups apart: one XCD, so the second reads the chunk's
    // record from that XCD's L2
    int tile, rest;
    chunk_tile_of(blockIdx.x, p.ntile, tile, rest);
    if (rest >= p.B * p.H * p.nch) return;
    const int cc = rest % p.nch, bh = rest / p.nch;
    const int b = bh / p.H, h = bh - b * p.H;
    const int dv = p.dv, col = tile * 64 + 16 * w + c;
    const size_t ch = static_cast<size_t>(bh) * p.nch + cc;
    const float* R = a.rec + ch * RecB::SIZE;
    const int t0 = cc * kCh, L = min(kCh, p.T - t0);
    const size_t tok0 = (static_cast<size_t>(b) * p.T + t0) * p.H + h;
    // v first, while nothing else is in flight (rows past the end are zeroed below)
    const size_t ntok = static_cast<size_t>(p.B) * p.T * p.H;
    uint32_t vr[16];
    {
        const int ve = p.qkv_dt == LA_F32 ? 4 : 2;
        const ChunkRows rv = chunk_rows(static_cast<const char*>(in.v) + tok0 * dv * ve, (ntok - tok0) * dv * ve,
                                        p.H * dv, g, col, ve);
        if (ve == 4) {
#pragma unroll
            for (int i = 0; i < 16; i++) vr[i] = rv.ld32(i);
        } else {
#pragma unroll
            for (int i = 0; i < 16; i++) vr[i] = rv.ld16(i);
        }
    }
    const size_t slab = static_cast<size_t>(kChDk) * dv * 4, rows = static_cast<size_t>(kCh) * dv * 4;
    const ChunkRows rs = chunk_rows(a.ckpts + ch * kChDk * dv, slab, dv, g, col, 4);
    float s[32];
#pragma unroll
    for (int m = 0; m < 32; m++) s[m] = rs.ldf(m);
    lds_dma(Kp_s, R + RecB::KP, kCh * RecB::PK);
    wait_all_mem();
    __syncthreads();
    // P and beta a piece per k-step of X = Kp S
    constexpr int nP = kCh * RecB::PP, nPc = lds_dma_pieces(nP);
    static_assert(nPc + lds_dma_pieces(kCh) <= 32, "P and beta pieces exceed the k-steps");
    f4 X[4];
#pragma unroll
    for (int rt = 0; rt < 4; rt++) X[rt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int m = 0; m < 32; m++) {
        if (m < nPc) lds_dma_piece(P_s, R + RecB::P, nP, m);
        else if (m < nPc + lds_dma_pieces(kCh)) lds_dma_piece(b_s, R + RecB::BT, kCh, m - nPc);
        const int key = kmap(m, g);
#pragma unroll
        for (int rt = 0; rt < 4; rt++) X[rt] = mfma4(Kp_s[cmap(rt, c) * RecB::PK + key], s[m], X[rt]);
        if ((m & 3) == 3) sched_fence();
    }
    wait_all_mem();
    __syncthreads();
    float vv[16], bb[16];
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const int tk = kmap(i, g);
        vv[i] = tk < L ? raw_f32(vr[i], p.qkv_dt) : 0.0f;
        bb[i] = b_s[tk];
    }
    float u[16], rv[16];
#pragma unroll
    for (int i = 0; i < 16; i++) {
        u[i] = vv[i] - X[i >> 2][i & 3];
        rv[i] = bb[i] * u[i];
    }
    f4 D[4];
#pragma unroll
    for (int rt = 0; rt < 4; rt++) D[rt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int m = 0; m < 16; m++) {
        const int tk = kmap(m, g);
#pragma unroll
        for (int rt = 0; rt < 4; rt++) D[rt] = mfma4(P_s[cmap(rt, c) * RecB::PP + tk], rv[m], D[rt]);
        if ((m & 3) == 3) sched_fence();
    }
    const ChunkRows ru = chunk_rows(a.U + ch * kCh * dv, rows, dv, g, col, 4);
    const ChunkRows rd = chunk_rows(a.D + ch * kCh * dv, rows, dv, g, col, 4);
#pragma unroll
    for (int i = 0; i < 16; i++) {
        ru.stf(i, u[i]);
        rd.stf(i, D[i >> 2][i & 3]);
    }
}

// dS carried through the chunks, last to first, for 64 value columns (la_chunk.hpp map).
__global__ __launch_bounds__(kChThreads, 1) void chunk_dstate_kernel(ChunkParams p, ChunkIn in, ChunkBwdPtrs a) {
    __shared__ __align__(16) float RA[RecB::PART2];                    // Kd, M
    __shared__ __align__(16) float RB[RecB::LDS_SIZE - RecB::PART2];   // P, Qp, Kp, E_L
    __shared__ float red[4][kCh];
    constexpr int bP = RecB::P - RecB::PART2, bQP = RecB::QP - RecB::PART2, bKP = RecB::KP - RecB::PART2,
                  bEL = RecB::EL - RecB::PART2, bBT = RecB::BT - RecB::PART2;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g0 = lane >> 4, c0 = lane & 15;
    int tile, bh;
    chunk_tile_of(blockIdx.x, p.ntile, tile, bh);
    const int BH = p.B * p.H;
    if (bh >= BH) return;
    const int b = bh / p.H, h = bh - b * p.H;
    const int dv = p.dv, col = tile * 64 + 16 * w + c0;
    const size_t soff = static_cast<size_t>(bh) * kChDk * dv + col;
    float ds[32];
#pragma unroll
    for (int m = 0; m < 32; m++) ds[m] = a.dST ? a.dST[soff + static_cast<size_t>(kmap(m, g0)) * dv] : 0.0f;
    const float* recu = a.rec + static_cast<size_t>(bh) * p.nch * RecB::SIZE;
    lds_dma(RA, recu + static_cast<size_t>(p.nch - 1) * RecB::SIZE, RecB::PART2);
    for (int cc = p.nch - 1; cc >= 0; cc--) {
        const int g = opaque(g0), c = opaque(c0);
        const int t0 = cc * kCh, L = min(kCh, p.T - t0);
        const size_t ch = static_cast<size_t>(bh) * p.nch + cc;
        const size_t tok0 = (static_cast<size_t>(b) * p.T + t0) * p.H + h;
        const ChunkRows rse = chunk_rows(a.dSe + ch * kChDk * dv, static_cast<size_t>(kChDk) * dv * 4, dv, g, col, 4);
#pragma unroll
        for (int m = 0; m < 32; m++) rse.stf(m, ds[m]);
        // part 1 of this chunk's record is here, part 2 of the later chunk free: load part 2
        wait_all_mem();
        __syncthreads();
        const float* part2 = recu + static_cast<size_t>(cc) * RecB::SIZE + RecB::PART2;
        constexpr int n2 = RecB::LDS_SIZE - RecB::PART2;
        static_assert(lds_dma_pieces(n2) <= 32, "part 2 pieces exceed the k-steps");
        // upstream gradient (rows past the end are zeroed where used) and U
        const size_t ntok = static_cast<size_t>(p.B) * p.T * p.H;
        const ChunkRows rdo = chunk_rows(a.dout + tok0 * dv, (ntok - tok0) * dv * 4, p.H * dv, g, col, 4);
        const ChunkRows rdv = chunk_rows(a.dv + tok0 * dv, (ntok - tok0) * dv * 4, p.H * dv, g, col, 4);
        const ChunkRows ru = chunk_rows(a.U + ch * kCh * dv, static_cast<size_t>(kCh) * dv * 4, dv, g, col, 4);
        const ChunkRows rdd = chunk_rows(a.dD + ch * kCh * dv, static_cast<size_t>(kCh) * dv * 4, dv, g, col, 4);
        float dOr[16], uu[16];
#pragma unroll
        for (int i = 0; i < 16; i++) {
            dOr[i] = rdo.ldf(i);
            uu[i] = ru.ldf(i);
        }
        // dDelta = Kd dS_end + M^T dO
        f4 DD[4];
#pragma unroll
        for (int rt = 0; rt < 4; rt++) DD[rt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int m = 0; m < 32; m++) {
            if (m < lds_dma_pieces(n2)) lds_dma_piece(RB, part2, n2, m);  // part 2, a piece per k-step
            const int key = kmap(m, g);
#pragma unroll
            for (int rt = 0; rt < 4; rt++) DD[rt] = mfma4(RA[RecB::KD + cmap(rt, c) * RecB::PKD + key], ds[m], DD[rt]);
            if ((m & 3) == 3) sched_fence();
        }
        // (the loaded values pass an empty asm here so that their first use, and the wait for
        // them, stay after the products above)
        float dO[16];
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const float x = opaque_f(dOr[i]);
            dO[i] = kmap(i, g) < L ? x : 0.0f;
        }
#pragma unroll
        for (int m = 0; m < 16; m++) {
            const int tk = kmap(m, g);
#pragma unroll
            for (int rt = 0; rt < 4; rt++) DD[rt] = mfma4(RA[RecB::M + tk * RecB::PP + cmap(rt, c)], dO[m], DD[rt]);
            if ((m & 3) == 3) sched_fence();
        }
        // part 2 is here and part 1 free: load the previous chunk's part 1
        wait_all_mem();
        __syncthreads();
        if (cc > 0) lds_dma(RA, recu + static_cast<size_t>(cc - 1) * RecB::SIZE, RecB::PART2);
        // dR = P^T dDelta
        f4 dR[4];
#pragma unroll
        for (int rt = 0; rt < 4; rt++) dR[rt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int m = 0; m < 16; m++) {
            const int tk = kmap(m, g);
            const float dm = DD[m >> 2][m & 3];
#pragma unroll
            for (int rt = 0; rt < 4; rt++) dR[rt] = mfma4(RB[bP + tk * RecB::PP + cmap(rt, c)], dm, dR[rt]);
            if ((m & 3) == 3) sched_fence();
        }
        float du[16];
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const int tk = kmap(i, g);
            rdd.stf(i, DD[i >> 2][i & 3]);
            du[i] = RB[bBT + tk] * dR[i >> 2][i & 3];
            if (tk < L) rdv.stf(i, du[i]);
        }
        // beta gradient of R = beta U, summed over this tile's columns
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const float v = group_sum<16>(dR[i >> 2][i & 3] * uu[i]);
            if (c == i) red[w][kmap(i, g)] = v;
        }
        __syncthreads();
        if (threadIdx.x < kCh) {
            const int t = threadIdx.x;
            a.dbp[(static_cast<size_t>(tile) * BH * p.nch + ch) * kCh + t] = (red[0][t] + red[1][t]) + (red[2][t] + red[3][t]);
        }
        // dS <- E_L dS + Qp^T dO - Kp^T dv
#pragma unroll
        for (int kt = 0; kt < 8; kt++) {
            f4 acc;
#pragma unroll
            for (int r = 0; r < 4; r++) acc[r] = RB[bEL + 16 * kt + 4 * r + g] * ds[4 * kt + r];
#pragma unroll
            for (int m = 0; m < 16; m++) {
                const int tk = kmap(m, g);
                acc = mfma4(RB[bQP + tk * RecB::PK + cmap(kt, c)], dO[m], acc);
                acc = mfma4(RB[bKP + tk * RecB::PK + cmap(kt, c)], -du[m], acc);
                if ((m & 3) == 3) sched_fence();
            }
#pragma unroll
            for (int r = 0; r < 4; r++) ds[4 * kt + r] = acc[r];
        }
    }
#pragma unroll
    for (int m = 0; m < 32; m++) a.dS0[soff + static_cast<size_t>(kmap(m, g0)) * dv] = ds[m];
}

// The ten 16 x 16 tiles of a 64 x 64 lower-triangular matrix.
__device__ __forceinline__ void low_tile(int i, int& rt, int& ct) {
    rt = i < 1 ? 0 : i < 3 ? 1 : i < 6 ? 2 : 3;
    ct = i - (rt * (rt + 1)) / 2;
}

// Gradients of one (sequence, head, chunk), eight waves.
template <bool KDA>
__global__ __launch_bounds__(kGT, 1) void chunk_grad_kernel(ChunkParams p, ChunkIn in, ChunkBwdPtrs a) {
    __shared__ __align__(16) float big[kBig];
    __shared__ float dAs[kWM], dMs[kWM];
    __shared__ float bS[kCh], gS[kCh], elS[kChDk];
    __shared__ float bpart[kGW][kCh];  // beta's pair term per wave and token
    const int t = threadIdx.x, lane = t & 63, w = t >> 6, g0 = lane >> 4, c0 = lane & 15;
    const int g = g0, c = c0;
    const int cc = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int bh = b * p.H + h, BH = p.B * p.H;
    const int dv = p.dv, t0 = cc * kCh, L = min(kCh, p.T - t0);
    const size_t ch = static_cast<size_t>(bh) * p.nch + cc;
    const size_t tok0 = (static_cast<size_t>(b) * p.T + t0) * p.H + h;
    const float* R = a.rec + ch * RecB::SIZE;
    float* dPs = big + 3 * kWM;
    for (int i = t; i < kWM; i += kGT) dPs[i] = dMs[i] = 0.0f;
    bpart[w][lane] = 0.0f;
    if (t < kCh) bS[t] = R[RecB::BT + t];

    // ---- products over the value columns, 16 at a time
    float* dDs = big;
    float* Rs = dDs + kCh * kSP;
    float* dOs = Rs + kCh * kSP;
    float* Ds = dOs + kCh * kSP;
    float* dUs = Ds + kCh * kSP;
    float* S0s = dUs + kCh * kSP;
    float* dSes = S0s + kChDk * kSP;
    // wave w: tiles (rt, w) of dQp, dKp, dKd (rows of block rt, keys 16 w + c) and tiles
    // w, w + 8, w + 16 (those below 20) of dP (0..9) and dM (10..19)
    f4 accQ[4], accK[4], accD[4], accPM[3];
#pragma unroll
    for (int j = 0; j < 4; j++) accQ[j] = accK[j] = accD[j] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int u = 0; u < 3; u++) accPM[u] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    float el = 0.0f;
    const float* Sck = a.ckpts + ch * kChDk * dv;
    const float* dSe = a.dSe + ch * kChDk * dv;
    // slab sb: the 16-byte pieces of S and dS_end of key t / 4 and, in waves 0-3, of U,
    // dDelta, Delta, dO, dv of token t / 4; slab sb + 1 is loaded while slab sb is multiplied (a
    // row past the end reads row 0 and is stored as zero)
    const bool tokw = t < 4 * kCh;  // uniform over a wave
    struct Slab {
        float4 u, dd, d, o, w, s0, se;
    };
    auto slab_load = [&](int sb, Slab& x) __attribute__((always_inline)) {
        const int tk = (t >> 2) & 63, cb = 16 * sb + ((t & 3) << 2);
        if (tokw) {
            const size_t wrow = (ch * kCh + tk) * dv + cb;
            const size_t grow = (tok0 + static_cast<size_t>(tk < L ? tk : 0) * p.H) * dv + cb;
            x.u = *reinterpret_cast<const float4*>(a.U + wrow);
            x.dd = *reinterpret_cast<const float4*>(a.dD + wrow);
            x.d = *reinterpret_cast<const float4*>(a.D + wrow);
            x.o = *reinterpret_cast<const float4*>(a.dout + grow);
            x.w = *reinterpret_cast<const float4*>(a.dv + grow);
        }
        const size_t kr = static_cast<size_t>(t >> 2) * dv + cb;
        x.s0 = *reinterpret_cast<const float4*>(Sck + kr);
        x.se = *reinterpret_cast<const float4*>(dSe + kr);
    };
    Slab nx;
    slab_load(0, nx);
    for (int sb = 0; sb < dv / 16; sb++) {
        const int g = opaque(g0), c = opaque(c0);
        __syncthreads();
        {
            const int tk = (t >> 2) & 63, j4 = (t & 3) << 2;
            if (tokw) {
                const bool ok = tk < L;
                const float bt = bS[tk];
                *reinterpret_cast<float4*>(Rs + tk * kSP + j4) = make_float4(nx.u.x * bt, nx.u.y * bt, nx.u.z * bt, nx.u.w * bt);
                *reinterpret_cast<float4*>(dDs + tk * kSP + j4) = nx.dd;
                *reinterpret_cast<float4*>(Ds + tk * kSP + j4) = nx.d;
                *reinterpret_cast<float4*>(dOs + tk * kSP + j4) = keep_if(ok, nx.o);
                *reinterpret_cast<float4*>(dUs + tk * kSP + j4) = keep_if(ok, nx.w);
            }
            *reinterpret_cast<float4*>(S0s + (t >> 2) * kSP + j4) = nx.s0;
            *reinterpret_cast<float4*>(dSes + (t >> 2) * kSP + j4) = nx.se;
        }
        __syncthreads();
        slab_load(sb + 1 < dv / 16 ? sb + 1 : sb, nx);  // the last slab reloads itself
#pragma unroll
        for (int s = 0; s < 4; s++) {
            const int kc = 4 * s + g;
            const int br = (16 * w + c) * kSP + kc;
            const float bs = S0s[br], be = dSes[br];
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int ar = (16 * j + c) * kSP + kc;
                accQ[j] = mfma4(dOs[ar], bs, accQ[j]);
                accK[j] = mfma4(dUs[ar], bs, accK[j]);
                accD[j] = mfma4(Ds[ar], be, accD[j]);
                if ((j & 1) == 1) sched_fence();
            }
#pragma unroll
            for (int u = 0; u < 3; u++) {
                // tiles w + 8 u below 20: the choice is uniform over the wave
                const int idx = w + 8 * u;
                if (idx < 20) {
                    int rt, ct;
                    low_tile(idx % 10, rt, ct);
                    const float* Ao = idx < 10 ? dDs : dOs;
                    const float* Bo = idx < 10 ? Rs : Ds;
                    accPM[u] = mfma4(Ao[(16 * rt + c) * kSP + kc], Bo[(16 * ct + c) * kSP + kc], accPM[u]);
                }
            }
        }
        if (t < kChDk) {
#pragma unroll
            for (int j = 0; j < 16; j++) el = __builtin_fmaf(dSes[t * kSP + j], S0s[t * kSP + j], el);
        }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 3; u++) {
        const int idx = w + 8 * u;
        if (idx < 20) {
            int rt, ct;
            low_tile(idx % 10, rt, ct);
            float* dst = idx < 10 ? dPs : dMs;
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int row = 16 * rt + 4 * g + r, cl = 16 * ct + c;
                if (cl <= row) dst[row * kPW + cl] = accPM[u][r];
            }
        }
    }
    if (t < kChDk) elS[t] = el;
    // accQ, accK and accD stay in registers: the pair sums below take the same tiles (rows of
    // block j, keys 16 w + c) in the same lanes
    __syncthreads();
    // k, q and the gates of the chunk, loaded now and stored to LDS after the solve's backward
    Rows<kGT> rk, rq, rg;
    uint32_t gr[1];
    rows_load(rk, in.k, tok0, p.H, L, p.qkv_dt);
    rows_load(rq, in.q, tok0, p.H, L, p.qkv_dt);
    if (KDA) rows_load(rg, in.g, tok0, p.H, L, p.gate_dt);
    else load_raw<1>(gr, in.g, p.gate_dt, [&](int) { return tok0 + static_cast<size_t>(t < L ? t & 63 : 0) * p.H; });

    // ---- backward of the solve: dA (strictly lower) from dP
    {
        float* Xb = big;
        float* Zb = big + kWM;
        float* Pb = big + 2 * kWM;
        float* Gb = dPs;
        float* dZn = big + 4 * kWM;
        float* dZb = big + 5 * kWM;
        if (p.degree == 0) {
            // P = (I + A)^-1: dA = -P^T dP P^T
#pragma unroll
            for (int i = t; i < kCh * kCh; i += kGT) Xb[(i >> 6) * kPW + (i & 63)] = R[RecB::P + (i >> 6) * RecB::PP + (i & 63)];
            __syncthreads();
            mm64<true, false, kGW>(Xb, Gb, Zb, nullptr);
            mm64<false, true, kGW>(Zb, Xb, Zb, nullptr);
            dZn = Zb;
        } else {
            // P = (I + Z_0)(I + Z_1) ... (I + Z_{m-1}), Z_j = X^(2^j), X = -A.  Reverse sweep
            // over the factors with G the gradient of the running product: dZ_j = P_{j-1}^T G
            // plus the squaring's dZ_{j+1} Z_j^T + Z_j^T dZ_{j+1}, then G <- G (I + Z_j)^T;
            // Z_j and the prefix P_{j-1} are recomputed from X at every step.
            int m = 0;
            while ((1 << m) - 1 < p.degree) m++;
#pragma unroll
            for (int i = t; i < kCh * kCh; i += kGT) Xb[(i >> 6) * kPW + (i & 63)] = -R[RecB::A + (i >> 6) * RecB::PA + (i & 63)];
            for (int j = m - 1; j >= 0; j--) {
                __syncthreads();
                for (int i = t; i < kCh * kCh; i += kGT) {
                    const int r = i >> 6, q = i & 63;
                    Zb[r * kPW + q] = Xb[r * kPW + q];
                    Pb[r * kPW + q] = r == q ? 1.0f : 0.0f;
                }
                __syncthreads();
                for (int i = 0; i < j; i++) {
                    mm64<false, false, kGW>(Pb, Zb, Pb, Pb);
                    mm64<false, false, kGW>(Zb, Zb, Zb, nullptr);
                }
                mm64<true, false, kGW>(Pb, Gb, dZb, nullptr);
                if (j < m - 1) {
                    mm64<false, true, kGW>(dZn, Zb, dZb, dZb);
                    mm64<true, false, kGW>(Zb, dZn, dZb, dZb);
                }
                if (j > 0) mm64<false, true, kGW>(Gb, Zb, Gb, Gb);
                float* tmp = dZn;
                dZn = dZb;
                dZb = tmp;
            }
        }
        // exact: dA = -(P^T dP P^T); Neumann: dA = -dX (X = -A)
        __syncthreads();
        for (int i = t; i < kCh * kCh; i += kGT) {
            const int r = i >> 6, q = i & 63;
            dAs[r * kPW + q] = q < r ? -dZn[r * kPW + q] : 0.0f;
        }
    }

    // ---- k, q and the cumulative log decays in LDS (rows past the end are zero; G repeats G_{L-1})
    float* kS = big;
    float* qS = big + kTK;
    float* Gs = big + 2 * kTK;
    __syncthreads();
    rows_store(kS, rk, L, p.qkv_dt);
    rows_store(qS, rq, L, p.qkv_dt);
    if (KDA) rows_store(Gs, rg, L, p.gate_dt);
    else if (t < kCh) gS[t] = t < L ? raw_f32(gr[0], p.gate_dt) : 0.0f;
    __syncthreads();
    if (KDA) {
        if (t < kChDk) cumsum_cols(Gs, t);
    } else if (t < kCh) {
        gS[t] = cumsum_lanes(gS[t]);  // zero past the end: those rows repeat G_{L-1}
    }
    __syncthreads();
    auto Gof = [&](int r, int kk) __attribute__((always_inline)) { return KDA ? Gs[r * 132 + kk] : gS[r]; };
    float* dABG = big + 2 * kTK;  // scalar gate only (no per-key decays in LDS then)
    if (!KDA) {
        // one decay per pair: dA o Gamma, dM o Gamma and beta dA o Gamma
        for (int i = t; i < kCh * kCh; i += kGT) {
            const int r = i >> 6, q = i & 63;
            const float gam = q <= r ? exp_acc(gS[r] - gS[q]) : 0.0f;
            const float da = dAs[r * kPW + q] * gam;
            dAs[r * kPW + q] = da;
            dMs[r * kPW + q] *= gam;
            dABG[r * kPW + q] = bS[r] * da;
        }
        __syncthreads();
    }

    // ---- the pair sums through A and M (D: the decays)
    //   T1 = sum_{i<r} dA_ri k_i D_ri,  T2 = sum_{i<=r} dM_ri k_i D_ri,
    //   T3 = sum_{s>r} beta_s dA_sr k_s D_sr + sum_{s>=r} dM_sr q_s D_sr,
    // with the elementwise terms of Kp = k E, Qp = q E, Kd = k F: the outputs dq, dk, the
    // cumulative-decay gradient dG and the Kd terms of the gate gradient (both held in registers
    // until the key and query arrays are no longer read), and beta's pair term k_r T1
    const size_t ntok = static_cast<size_t>(p.B) * p.T * p.H;
    const auto rdq = make_rsrc(a.dq + tok0 * kChDk, (ntok - tok0) * kChDk * 4);
    const auto rdk = make_rsrc(a.dk + tok0 * kChDk, (ntok - tok0) * kChDk * 4);
    auto finish = [&](int row, int key, float t1, float t2, float t3, float dQp, float dKp, float dKd, float& dG,
                      float& kdt) __attribute__((always_inline)) {
        const float G = Gof(row, key), GL = Gof(L - 1, key);
        const float E = exp_acc(G), F = exp_acc(GL - G);
        const float kv = kS[row * 132 + key], qv = qS[row * 132 + key], bt = bS[row];
        const float Kp = kv * E, Qp = qv * E, Kd = kv * F;
        if (row < L) {
            // row = 16 rt + 4 g + r: the lane part 4 g in the offset register, the rest scalar
            const int voff = (4 * g * p.H * kChDk + key) * 4, soff = (row - 4 * g) * p.H * kChDk * 4;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(__builtin_fmaf(E, dQp, t2)), rdq, voff, soff, 0);
            __builtin_amdgcn_raw_buffer_store_b32(
                __float_as_uint(__builtin_fmaf(E, dKp, __builtin_fmaf(F, dKd, __builtin_fmaf(bt, t1, t3)))), rdk, voff, soff, 0);
        }
        dG = __builtin_fmaf(dKp, Kp, dQp * Qp) + __builtin_fmaf(bt * kv, t1, __builtin_fmaf(qv, t2, -kv * t3));
        // Kd = k F, F = e^{G_{L-1} - G}: its term reaches the gates of the tokens after this row
        // only, summed below as a prefix (as the total at row L - 1 less a suffix it would
        // cancel badly under steep decay, where the later rows dominate the total)
        kdt = dKd * Kd;
    };
    // KDA: every decay factored on 16-token blocks (chunk_factorable), else per-key sums
    __shared__ int flag;
    const bool fact = !KDA || chunk_factorable(Gs, L, &flag);
    // tiles (rt, w) of this wave: rows of block rt, keys 16 w + c
    float bc[4][4], dGr[4][4], kdr[4][4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int rt = j, key = 16 * w + c;
        f4 T1 = {0.0f, 0.0f, 0.0f, 0.0f}, T2 = T1, T3 = T1;
        if (!KDA) {
            // one decay per pair, folded into dA and dM above
#pragma unroll 4
            for (int s = 0; s < 16; s++) {
                const int tk = 4 * s + g;
                const float bk = kS[tk * 132 + key], bq = qS[tk * 132 + key];
                T1 = mfma4(dAs[(16 * rt + c) * kPW + tk], bk, T1);
                T2 = mfma4(dMs[(16 * rt + c) * kPW + tk], bk, T2);
                T3 = mfma4(dABG[tk * kPW + 16 * rt + c], bk, T3);
                T3 = mfma4(dMs[tk * kPW + 16 * rt + c], bq, T3);
            }
        } else {
            if (fact) {
                // blocks I <= rt: e^{G_r - G_i} = e^{G_r - ref} e^{ref - G_i}, ref = G at the end
                // of block I (at the eighth token of block rt for I = rt, where dA and dM vanish
                // on the pairs with i past r); the products over block I's tokens on the matrix
                // cores
#pragma unroll
                for (int I = 0; I <= rt; I++) {
                    const float rf = Gs[(I < rt ? 16 * I + 15 : 16 * rt + 7) * 132 + key];
                    f4 P1 = {0.0f, 0.0f, 0.0f, 0.0f}, P2 = P1;
#pragma unroll
                    for (int s = 0; s < 4; s++) {
                        const int tk = 16 * I + 4 * s + g;
                        const float bl = kS[tk * 132 + key] * exp_acc(rf - Gs[tk * 132 + key]);
                        P1 = mfma4(dAs[(16 * rt + c) * kPW + tk], bl, P1);
                        P2 = mfma4(dMs[(16 * rt + c) * kPW + tk], bl, P2);
                    }
#pragma unroll
                    for (int r = 0; r < 4; r++) {
                        const float e = exp_acc(Gs[(16 * rt + 4 * g + r) * 132 + key] - rf);
                        T1[r] = __builtin_fmaf(e, P1[r], T1[r]);
                        T2[r] = __builtin_fmaf(e, P2[r], T2[r]);
                    }
                }
                // blocks R >= rt: e^{G_s - G_i} = e^{G_s - ref} e^{ref - G_i}, ref = G at the end of
                // block rt (at its eighth token for R = rt); products over block R's tokens
#pragma unroll
                for (int R2 = rt; R2 < 4; R2++) {
                    const float rf = Gs[(16 * rt + (R2 > rt ? 15 : 7)) * 132 + key];
                    f4 P3 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int s = 0; s < 4; s++) {
                        const int tk = 16 * R2 + 4 * s + g;
                        const float er = exp_acc(Gs[tk * 132 + key] - rf);
                        P3 = mfma4(bS[tk] * dAs[tk * kPW + 16 * rt + c], kS[tk * 132 + key] * er, P3);
                        P3 = mfma4(dMs[tk * kPW + 16 * rt + c], qS[tk * 132 + key] * er, P3);
                    }
#pragma unroll
                    for (int r = 0; r < 4; r++)
                        T3[r] = __builtin_fmaf(exp_acc(rf - Gs[(16 * rt + 4 * g + r) * 132 + key]), P3[r], T3[r]);
                }
            }
            // per-key sums over every token when the factors are not safe; dA is zero on and
            // above the diagonal and dM above it, and each term's decay is between the earlier
            // and the later token
            const int i_hi = fact ? 0 : kCh;
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int row = 16 * rt + 4 * g + r;
                const float Gr = Gs[row * 132 + key];
                float t1 = 0.0f, t2 = 0.0f, t3 = 0.0f;
                for (int i = 0; i < i_hi; i++) {
                    const float Gi = Gs[i * 132 + key], ki = kS[i * 132 + key];
                    const float d = exp_acc(i <= row ? Gr - Gi : Gi - Gr);
                    const float dl = i <= row ? d : 0.0f, du = i >= row ? d : 0.0f;  // no 0 * inf
                    t1 = __builtin_fmaf(dAs[row * kPW + i] * ki, dl, t1);
                    t2 = __builtin_fmaf(dMs[row * kPW + i] * ki, dl, t2);
                    t3 = __builtin_fmaf(__builtin_fmaf(bS[i] * dAs[i * kPW + row], ki, dMs[i * kPW + row] * qS[i * 132 + key]), du, t3);
                }
                T1[r] += t1;
                T2[r] += t2;
                T3[r] += t3;
            }
        }
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int row = 16 * rt + 4 * g + r;
            finish(row, key, T1[r], T2[r], T3[r], accQ[j][r], -accK[j][r], accD[j][r], dGr[rt][r], kdr[rt][r]);
            bc[rt][r] = kS[row * 132 + key] * T1[r];
        }
        sched_fence();
    }
#pragma unroll
    for (int rt = 0; rt < 4; rt++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const float v = group_sum<16>(bc[rt][r]);
            if (c == 0) bpart[w][16 * rt + 4 * g + r] = v;
        }

    // ---- gate and beta gradients: dG and the Kd terms into LDS over the key and query arrays
    // (no longer read once every wave is past the barrier)
    float* dGs = big;
    float* cS = big + kTK;
    __syncthreads();
#pragma unroll
    for (int rt = 0; rt < 4; rt++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int row = 16 * rt + 4 * g + r, kk = 16 * w + c;
            float v = dGr[rt][r];
            // E_L = exp(G_{L-1}) feeds dG_{L-1} as well
            if (row == L - 1) v += elS[kk] * exp_acc(Gof(L - 1, kk));
            dGs[row * 132 + kk] = row < L ? v : 0.0f;
            cS[row * 132 + kk] = row < L ? kdr[rt][r] : 0.0f;
        }
    __syncthreads();
    if (KDA) {
        // dg_r = sum_{r' >= r} dG_r' + sum_{r' < r} dKd_r' Kd_r' per key (G is the running sum of
        // g); thread (part, key) takes rows 16 part .. 16 part + 15 after the sums of the other
        // quarters (rows past the end hold zeros)
        const int key = t & (kChDk - 1), part = t >> 7;
        float* qC = big + 2 * kTK;  // [4][128] quarter sums of the Kd terms, then of dG
        float* qG = qC + 4 * kChDk;  // (over the cumulative gates, no longer read)
        float sc = 0.0f, sg = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; i++) {
            sc += cS[(16 * part + i) * 132 + key];
            sg += dGs[(16 * part + i) * 132 + key];
        }
        qC[part * kChDk + key] = sc;
        qG[part * kChDk + key] = sg;
        __syncthreads();
        float pre = 0.0f, acc = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; q++) {
            pre += q < part ? qC[q * kChDk + key] : 0.0f;
            acc += q > part ? qG[q * kChDk + key] : 0.0f;
        }
        float cp[16];
#pragma unroll
        for (int i = 0; i < 16; i++) {
            cp[i] = pre;
            pre += cS[(16 * part + i) * 132 + key];
        }
#pragma unroll
        for (int i = 15; i >= 0; i--) {
            const int r = 16 * part + i;
            acc += dGs[r * 132 + key];
            if (r < L) a.dg[(tok0 + static_cast<size_t>(r) * p.H) * kChDk + key] = acc + cp[i];
        }
    } else {
        // row sums over the keys by eight threads per row (16 keys each), then across the 64
        // rows a suffix of dG and an exclusive prefix of the Kd terms in one wave
        {
            const int row = t >> 3, part = t & 7;
            float rs = 0.0f, cs = 0.0f;
#pragma unroll
            for (int j = 0; j < 16; j++) {
                rs += dGs[row * 132 + 16 * part + j];
                cs += cS[row * 132 + 16 * part + j];
            }
#pragma unroll
            for (int o = 1; o < 8; o <<= 1) {
                rs += __shfl_xor(rs, o, 64);
                cs += __shfl_xor(cs, o, 64);
            }
            if (part == 0) {
                elS[row] = rs;
                gS[row] = cs;  // the cumulative gates are no longer read
            }
        }
        __syncthreads();
        if (t < kCh) {
            const float suf = wave_prefix_sum(elS[kCh - 1 - t]);  // lane i: rows 63 - i .. 63
            const float exc = __shfl_up(wave_prefix_sum(gS[t]), 1, 64);
            const float dgs = __shfl(suf, kCh - 1 - t, 64);
            if (t < L) a.dg[tok0 + static_cast<size_t>(t) * p.H] = dgs + (t > 0 ? exc : 0.0f);
        }
    }
    if (t < L) {
        float sbt = ((bpart[0][t] + bpart[1][t]) + (bpart[2][t] + bpart[3][t])) +
                    ((bpart[4][t] + bpart[5][t]) + (bpart[6][t] + bpart[7][t]));
        for (int tl = 0; tl < p.ntile; tl++) sbt += a.dbp[(static_cast<size_t>(tl) * BH * p.nch + ch) * kCh + t];
        a.dbeta[tok0 + static_cast<size_t>(t) * p.H] = sbt;
    }
}

}  // namespace

ChunkBwdLayout chunk_bwd_layout(const la_config& c) {
    auto up = [](size_t n) { return (n + 255) / 256 * 256; };
    const size_t nch = (static_cast<size_t>(c.T) + kCh - 1) / kCh;
    const size_t units = static_cast<size_t>(c.B) * c.H * nch;
    ChunkBwdLayout L;
    L.rec = 0;
    L.ckpts = L.rec + up(units * RecB::SIZE * sizeof(float));
    L.U = L.ckpts + up(units * kChDk * c.d_v * sizeof(float));
    L.D = L.U + up(units * kCh * c.d_v * sizeof(float));
    L.dD = L.D + up(units * kCh * c.d_v * sizeof(float));
    L.dSe = L.dD + up(units * kCh * c.d_v * sizeof(float));
    L.dbp = L.dSe + up(units * kChDk * c.d_v * sizeof(float));
    L.total = L.dbp + up(static_cast<size_t>(c.d_v / 64) * units * kCh * sizeof(float));
    return L;
}

hipError_t launch_chunk_bwd(const la_config& c, const FwdArgs& fa, const BwdArgs& ba, char* ws, hipStream_t s) {
    const ChunkParams p = make_chunk_params(c);
    const ChunkIn in{fa.q, fa.k, fa.v, fa.g, fa.beta};
    const ChunkBwdLayout L = chunk_bwd_layout(c);
    float* rec = reinterpret_cast<float*>(ws + L.rec);
    const float* ck = ba.ckpts;
    hipError_t e;
    if (!ck) {
        // checkpoints from the forward kernel that serves c: the chunk forward (its records in
        // the backward records' room), or the kernel the caller's forward ran, whose rounding
        // decisions the checkpoints must repeat
        float* room = reinterpret_cast<float*>(ws + L.ckpts);
        FwdArgs f = fa;
        f.o = nullptr;
        f.ST = nullptr;
        f.ckpts = room;
        e = fwd_kernel(c) == LA_KERNEL_CHUNK ? launch_chunk_fwd(c, f, rec, s) : launch_fwd(c, f, s);
        if (e != hipSuccess) return e;
        ck = room;
    }
    e = launch_chunk_prep(c, in, rec, true, s);
    if (e != hipSuccess) return e;
    ChunkBwdPtrs a{ck, ba.dout, ba.dST, ba.dq, ba.dk, ba.dv, ba.dg, ba.dbeta, ba.dS0, rec,
                   reinterpret_cast<float*>(ws + L.U), reinterpret_cast<float*>(ws + L.D),
                   reinterpret_cast<float*>(ws + L.dD), reinterpret_cast<float*>(ws + L.dSe),
                   reinterpret_cast<float*>(ws + L.dbp)};
    const unsigned units = static_cast<unsigned>(c.B) * c.H * p.nch;
    hipLaunchKernelGGL(chunk_recompute_kernel, dim3(chunk_tile_blocks(units, p.ntile)), dim3(kChThreads), 0, s, p, in, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(chunk_dstate_kernel, dim3(chunk_tile_blocks(c.B * c.H, p.ntile)), dim3(kChThreads), 0, s, p,
                       in, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 grid(p.nch, c.H, c.B);
    if (c.gate == LA_GATE_KEY) hipLaunchKernelGGL(chunk_grad_kernel<true>, grid, dim3(kGT), 0, s, p, in, a);
    else hipLaunchKernelGGL(chunk_grad_kernel<false>, grid, dim3(kGT), 0, s, p, in, a);
    return hipGetLastError();
}

}  // namespace la
