// 64-token chunk path, forward: the chunk-parallel prep kernel (one workgroup per sequence,
// head and chunk) and the state pass (one workgroup per sequence, head and 64 value columns).
// The formulas and the state pass's register layout are those of la_chunk.hpp.
#include "la_chunk.hpp"

namespace la {

ChunkParams make_chunk_params(const la_config& c) {
    ChunkParams p;
    p.B = c.B; p.T = c.T; p.H = c.H; p.dv = c.d_v;
    p.nch = (c.T + kCh - 1) / kCh;
    p.ntile = c.d_v / 64;
    p.qkv_dt = c.qkv_dtype; p.gate_dt = c.gate_dtype; p.out_dt = c.out_dtype;
    p.qdq_interval = c.qdq == LA_QDQ_NONE ? 1 : c.qdq_interval;
    p.ckpt_interval = c.ckpt_interval > 0 ? c.ckpt_interval : 1;
    p.nck = n_ckpts(c);
    p.degree = c.solve == LA_SOLVE_NEUMANN ? c.degree : 0;
    return p;
}

bool chunk_eligible(const la_config& c) {
    if (c.d_k != kChDk || c.hadamard || c.replay || c.state_rotated) return false;
    if (c.qdq != LA_QDQ_NONE && c.qdq_interval % kCh != 0) return false;
    if (c.ckpt_interval > 0 && c.ckpt_interval % kCh != 0) return false;
    return true;
}

size_t chunk_fwd_workspace_bytes(const la_config& c) {
    const size_t nch = (static_cast<size_t>(c.T) + kCh - 1) / kCh;
    return static_cast<size_t>(c.B) * c.H * nch * RecF::SIZE * sizeof(float);
}

namespace {

constexpr int kPT = 132;  // pitch of the prep kernel's token-by-key arrays
constexpr int kPrepW = 8;  // the prep kernel's waves (two per SIMD: its phases mostly wait on
constexpr int kPrepT = 64 * kPrepW;  // memory and LDS, and the second wave fills those gaps)

// Prep: A, M, the solve P, Kp, Qp, Kd, E_L of one chunk into its record (forward or backward
// layout).  Tokens past the sequence's end are zero rows (their beta, k and q are zero).
template <bool KDA, bool BWD>
__global__ __launch_bounds__(kPrepT, 1) void chunk_prep_kernel(ChunkParams p, ChunkIn in, float* __restrict__ rec) {
    __shared__ __align__(16) float big[3 * kCh * kPT];
    __shared__ float Am[kCh * kPW], Mm[kCh * kPW];
    __shared__ float bS[kCh], gS[kCh];
    float* kS = big;
    float* qS = big + kCh * kPT;
    float* GS = big + 2 * kCh * kPT;
    const int t = threadIdx.x;
    const int cc = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int H = p.H, T = p.T;
    const int t0 = cc * kCh, L = min(kCh, T - t0);
    const size_t tok0 = (static_cast<size_t>(b) * T + t0) * H + h;
    float* R = rec + ((static_cast<size_t>(b) * H + h) * p.nch + cc) * (BWD ? RecB::SIZE : RecF::SIZE);

    {
        // every load of the chunk's inputs in flight before any is used
        Rows<kPrepT> rk, rq, rg;
        rows_load(rk, in.k, tok0, H, L, p.qkv_dt);
        rows_load(rq, in.q, tok0, H, L, p.qkv_dt);
        if (KDA) rows_load(rg, in.g, tok0, H, L, p.gate_dt);
        uint32_t br[1], gr[1];
        const size_t te = tok0 + static_cast<size_t>(t < L ? t & 63 : 0) * H;
        load_raw<1>(br, in.beta, p.gate_dt, [&](int) { return te; });
        if (!KDA) load_raw<1>(gr, in.g, p.gate_dt, [&](int) { return te; });
        rows_store(kS, rk, L, p.qkv_dt);
        rows_store(qS, rq, L, p.qkv_dt);
        if (KDA) rows_store(GS, rg, L, p.gate_dt);
        if (t < kCh) {
            bS[t] = t < L ? raw_f32(br[0], p.gate_dt) : 0.0f;
            if (!KDA) gS[t] = t < L ? raw_f32(gr[0], p.gate_dt) : 0.0f;
        }
    }
    if (KDA) {
        // cumulative log decays per key (rows past the end repeat G_{L-1}): one thread per key
        // sums down its column of the gates loaded above
        __syncthreads();
        if (t < kChDk) cumsum_cols(GS, t);
    } else {
        // zero past the end, so those rows repeat G_{L-1}
        if (t < kCh) gS[t] = cumsum_lanes(gS[t]);
    }
    __syncthreads();
    auto Gof = [&](int r, int kk) __attribute__((always_inline)) { return KDA ? GS[r * kPT + kk] : gS[r]; };

    // decayed keys and queries
    for (int idx = t; idx < kCh * kChDk; idx += kPrepT) {
        const int r = idx >> 7, kk = idx & 127;
        const float G = Gof(r, kk);
        const float E = exp_acc(G);
        const float kv = kS[r * kPT + kk], qv = qS[r * kPT + kk];
        if (BWD) {
            const float F = exp_acc(Gof(L - 1, kk) - G);
            R[RecB::KP + r * RecB::PK + kk] = kv * E;
            R[RecB::QP + r * RecB::PK + kk] = qv * E;
            R[RecB::KD + r * RecB::PKD + kk] = kv * F;
        } else {
            R[RecF::KP + r * RecF::PK + kk] = kv * E;
            R[RecF::QP + r * RecF::PK + kk] = qv * E;
        }
    }
    if (!BWD) {
        for (int idx = t; idx < kCh * kChDk; idx += kPrepT) {
            const int kk = idx >> 6, r = idx & 63;
            R[RecF::KDT + kk * RecF::PD + r] = kS[r * kPT + kk] * exp_acc(Gof(L - 1, kk) - Gof(r, kk));
        }
    }
    if (t < kChDk) R[(BWD ? RecB::EL : RecF::EL) + t] = exp_acc(Gof(L - 1, t));
    if (t < kCh) R[(BWD ? RecB::BT : RecF::BT) + t] = bS[t];

    // A (strictly lower) and M (lower with the diagonal)
    if (KDA) {
        // The ten lower 16 x 16 tiles (rt >= ct) on the matrix cores: with ref a cumulative gate
        // (G at the end of block ct off the diagonal, at the eighth token of the block on it),
        // e^{G_r - G_i} = e^{G_r - ref} e^{ref - G_i}, so A and M of the tile are
        // (K o e^{G - ref}) (K o e^{ref - G})^T and (Q o e^{G - ref}) (K o e^{ref - G})^T.
        // chunk_factorable checks that no factor overflows; a chunk that fails takes the per-key
        // sums for every tile instead, one thread per four (row, column) pairs.
        const int lane = t & 63, w = t >> 6, g = lane >> 4, c = lane & 15;
        __shared__ int flag;
        const bool fact = chunk_factorable(GS, L, &flag);
        if (fact) {
            constexpr int PR[10] = {1, 2, 2, 3, 3, 3, 0, 1, 2, 3}, PC[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};
            for (int pi = w; pi < 10; pi += kPrepW) {
                const int rt = PR[pi], ct = PC[pi], ref = rt == ct ? 16 * ct + 7 : 16 * ct + 15;
                f4 aA = {0.0f, 0.0f, 0.0f, 0.0f}, aM = aA;
#pragma unroll 4
                for (int s2 = 0; s2 < 32; s2++) {
                    const int key = 4 * s2 + g;
                    const float rf = GS[ref * kPT + key];
                    const int ra = (16 * rt + c) * kPT + key, rb = (16 * ct + c) * kPT + key;
                    const float er = exp_acc(GS[ra] - rf);
                    const float bl = kS[rb] * exp_acc(rf - GS[rb]);
                    aA = mfma4(kS[ra] * er, bl, aA);
                    aM = mfma4(qS[ra] * er, bl, aM);
                }
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const int row = 16 * rt + 4 * g + r, col = 16 * ct + c;
                    Am[row * kPW + col] = col < row ? bS[row] * aA[r] : 0.0f;
                    Mm[row * kPW + col] = col <= row ? aM[r] : 0.0f;
                }
            }
            // the tiles above the diagonal
            for (int i = t; i < kCh * kCh; i += kPrepT) {
                const int r = i >> 6, q = i & 63;
                if ((q >> 4) > (r >> 4)) Am[r * kPW + q] = Mm[r * kPW + q] = 0.0f;
            }
        } else {
            for (int i = t; i < kCh * kPW; i += kPrepT) Am[i] = Mm[i] = 0.0f;
            __syncthreads();
            // lane: row 4 (lane / 16) + rr of the tile, column lane % 16
            for (int tl = w; tl < 10; tl += kPrepW) {
                const int rt = tl < 1 ? 0 : tl < 3 ? 1 : tl < 6 ? 2 : 3;
                const int ct = tl - (rt * (rt + 1)) / 2;
                const int col = 16 * ct + c;
                float aa[4] = {0.0f, 0.0f, 0.0f, 0.0f}, mm[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 2
                for (int kk = 0; kk < kChDk; kk++) {
                    const float kc = kS[col * kPT + kk], Gc = GS[col * kPT + kk];
#pragma unroll
                    for (int rr = 0; rr < 4; rr++) {
                        const int row = 16 * rt + 4 * g + rr;
                        const float kd = kc * exp_acc(col <= row ? GS[row * kPT + kk] - Gc : 0.0f);
                        aa[rr] = __builtin_fmaf(kS[row * kPT + kk], kd, aa[rr]);
                        mm[rr] = __builtin_fmaf(qS[row * kPT + kk], kd, mm[rr]);
                    }
                }
#pragma unroll
                for (int rr = 0; rr < 4; rr++) {
                    const int row = 16 * rt + 4 * g + rr;
                    Am[row * kPW + col] = col < row ? bS[row] * aa[rr] : 0.0f;
                    Mm[row * kPW + col] = col <= row ? mm[rr] : 0.0f;
                }
            }
        }
    } else {
        // one decay per token pair: K K^T and Q K^T on the matrix cores, then the decay
        const int lane = t & 63, w = t >> 6, g = lane >> 4, c = lane & 15;
        for (int tl = w; tl < 16; tl += kPrepW) {
            const int rt = tl >> 2, ct = tl & 3;
            f4 ak = {0.0f, 0.0f, 0.0f, 0.0f}, aq = ak;
            if (rt >= ct) {
#pragma unroll 4
                for (int s = 0; s < 32; s++) {
                    const float bk = kS[(16 * ct + c) * kPT + 4 * s + g];
                    ak = mfma4(kS[(16 * rt + c) * kPT + 4 * s + g], bk, ak);
                    aq = mfma4(qS[(16 * rt + c) * kPT + 4 * s + g], bk, aq);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int row = 16 * rt + 4 * g + r, i = 16 * ct + c;
                const float gam = i <= row ? exp_acc(gS[row] - gS[i]) : 0.0f;
                Am[row * kPW + i] = i < row ? bS[row] * (gam * ak[r]) : 0.0f;
                Mm[row * kPW + i] = gam * aq[r];
            }
        }
    }
    __syncthreads();

    // the solve, in the token arrays' space
    float* W0 = big;
    float* W1 = big + kCh * kPW;
    float* Ys = big + 2 * kCh * kPW;  // four 16 x 16 wave-private tiles
    const float* Pm;
    if (p.degree == 0) {
        // (I + A)^-1 in 16 x 16 blocks.  Diagonal blocks by forward substitution, wave w
        // inverting block w (lane (g, c) holds column c and sums rows i = g mod 4; a row's
        // values are read back by the same wave, whose LDS accesses are in order).  Then block
        // rows k = 1..3: T_kj = -T_kk sum_{l=j}^{k-1} A_kl T_lj, tile (k, j) on wave j.
        for (int idx = t; idx < kCh * kCh; idx += kPrepT) W0[(idx >> 6) * kPW + (idx & 63)] = 0.0f;
        __syncthreads();
        const int lane = t & 63, w = t >> 6, g = lane >> 4, c = lane & 15, o = 16 * w;
        if (w < 4) {
            for (int r = 0; r < 16; r++) {
                float part = 0.0f;
                for (int i = g; i < r; i += 4)
                    part = __builtin_fmaf(Am[(o + r) * kPW + o + i], W0[(o + i) * kPW + o + c], part);
                const float sum = rows_sum(part);
                if (g == 0) W0[(o + r) * kPW + o + c] = (r == c ? 1.0f : 0.0f) - sum;
            }
        }
        __syncthreads();
        float* Y = Ys + 256 * w;
        for (int k = 1; k < 4; k++) {
            if (w < k) {
                f4 y = {0.0f, 0.0f, 0.0f, 0.0f};
                for (int l = w; l < k; l++) {
#pragma unroll
                    for (int s2 = 0; s2 < 4; s2++)
                        y = mfma4(Am[(16 * k + c) * kPW + 16 * l + 4 * s2 + g], W0[(16 * l + 4 * s2 + g) * kPW + o + c], y);
                }
#pragma unroll
                for (int r = 0; r < 4; r++) Y[(4 * g + r) * 16 + c] = y[r];
                f4 z = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int s2 = 0; s2 < 4; s2++)
                    z = mfma4(W0[(16 * k + c) * kPW + 16 * k + 4 * s2 + g], Y[(4 * s2 + g) * 16 + c], z);
#pragma unroll
                for (int r = 0; r < 4; r++) W0[(16 * k + 4 * g + r) * kPW + o + c] = -z[r];
            }
            __syncthreads();
        }
        Pm = W0;
    } else {
        // sum_{n <= d} X^n, X = -A, d = 2^m - 1, as (I + X)(I + X^2)(I + X^4) ...: Z holds X^(2^j),
        // P the product so far
        for (int idx = t; idx < kCh * kCh; idx += kPrepT) {
            const int r = idx >> 6, i = idx & 63;
            const float x = -Am[r * kPW + i];
            W0[r * kPW + i] = x;
            W1[r * kPW + i] = r == i ? 1.0f + x : x;
        }
        __syncthreads();
        for (int done = 1; done < p.degree; done = 2 * done + 1) {
            mm64<false, false, kPrepW>(W0, W0, W0, nullptr);  // Z <- Z Z
            mm64<false, false, kPrepW>(W1, W0, W1, W1);       // P <- P + P Z
        }
        Pm = W1;
    }

    for (int idx = t; idx < kCh * kCh; idx += kPrepT) {
        const int r = idx >> 6, i = idx & 63;
        if (BWD) {
            R[RecB::P + r * RecB::PP + i] = Pm[r * kPW + i];
            R[RecB::M + r * RecB::PP + i] = Mm[r * kPW + i];
            R[RecB::A + r * RecB::PA + i] = Am[r * kPW + i];
        } else {
            R[RecF::P + r * RecF::PP + i] = Pm[r * kPW + i];
            R[RecF::M + r * RecF::PP + i] = Mm[r * kPW + i];
        }
    }
}

// State pass: chunks in order, the state of 64 value columns in registers (la_chunk.hpp map);
// outputs, checkpoints every ckpt_interval tokens, rounding at the chunk ends that are
// rounding points, the final state.
template <int QMODE, int G>
__global__ __launch_bounds__(kChThreads, 1) void chunk_fwd_kernel(ChunkParams p, ChunkIn in, const float* __restrict__ S0,
                                                                  void* o, float* ST, float* ckpts,
                                                                  const float* __restrict__ rec) {
    __shared__ __align__(16) float RA[RecF::PART2];               // Kp, Qp
    __shared__ __align__(16) float RB[RecF::SIZE - RecF::PART2];  // P, M, Kd^T, E_L
    __shared__ WaveQdqShared<kChDk, QMODE, G> qsh;
    constexpr int bP = RecF::P - RecF::PART2, bM = RecF::M - RecF::PART2, bKDT = RecF::KDT - RecF::PART2,
                  bEL = RecF::EL - RecF::PART2, bBT = RecF::BT - RecF::PART2;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g0 = lane >> 4, c0 = lane & 15;
    int tile, bh;
    chunk_tile_of(blockIdx.x, p.ntile, tile, bh);
    if (bh >= p.B * p.H) return;
    const int b = bh / p.H, h = bh - b * p.H;
    const int dv = p.dv, col = tile * 64 + 16 * w + c0;
    const size_t soff = static_cast<size_t>(bh) * kChDk * dv + col;
    float s[32];
#pragma unroll
    for (int m = 0; m < 32; m++) s[m] = S0 ? S0[soff + static_cast<size_t>(kmap(m, g0)) * dv] : 0.0f;
    int qpar = 0;
    const float* recu = rec + static_cast<size_t>(bh) * p.nch * RecF::SIZE;
    lds_dma(RA, recu, RecF::PART2);
    for (int cc = 0; cc < p.nch; cc++) {
        const int g = opaque(g0), c = opaque(c0);
        const int t0 = cc * kCh, L = min(kCh, p.T - t0);
        if (ckpts && t0 % p.ckpt_interval == 0) {
            const ChunkRows ck = chunk_rows(ckpts + (static_cast<size_t>(bh) * p.nck + t0 / p.ckpt_interval) * kChDk * dv,
                                            static_cast<size_t>(kChDk) * dv * 4, dv, g, col, 4);
#pragma unroll
            for (int m = 0; m < 32; m++) ck.stf(m, s[m]);
        }
        // part 1 of this chunk's record has arrived and every wave is done with part 2 of the
        // previous one
        wait_all_mem();
        __syncthreads();
        // v of this lane's tokens (a row past the end reads row 0 and is zeroed where it is
        // used), issued while nothing else is in flight: the dtype switch then costs no wait
        const size_t tok0 = (static_cast<size_t>(b) * p.T + t0) * p.H + h;
        const size_t ntok = static_cast<size_t>(p.B) * p.T * p.H;  // tokens x heads in the inputs
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
        // X = Kp S, Y = Qp S, with part 2 of the record loaded a piece per k-step meanwhile
        const float* part2 = recu + static_cast<size_t>(cc) * RecF::SIZE + RecF::PART2;
        constexpr int n2 = RecF::SIZE - RecF::PART2;
        static_assert(lds_dma_pieces(n2) <= 32, "part 2 pieces exceed the k-steps");
        f4 X[4], Y[4];
#pragma unroll
        for (int rt = 0; rt < 4; rt++) X[rt] = Y[rt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int m = 0; m < 32; m++) {
            if (m < lds_dma_pieces(n2)) lds_dma_piece(RB, part2, n2, m);
            const int key = kmap(m, g);
#pragma unroll
            for (int rt = 0; rt < 4; rt++) {
                const int row = cmap(rt, c) * RecF::PK + key;
                X[rt] = mfma4(RA[RecF::KP + row], s[m], X[rt]);
                Y[rt] = mfma4(RA[RecF::QP + row], s[m], Y[rt]);
            }
            if ((m & 3) == 3) sched_fence();
        }
        // part 2 has arrived and part 1 is free: load the next chunk's part 1
        wait_all_mem();
        __syncthreads();
        if (cc + 1 < p.nch) lds_dma(RA, recu + static_cast<size_t>(cc + 1) * RecF::SIZE, RecF::PART2);
        // beta (V - X), then Delta = P (beta (V - X))
        float rv[16];
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const int tk = kmap(i, g);
            const float vt = tk < L ? raw_f32(vr[i], p.qkv_dt) : 0.0f;
            rv[i] = RB[bBT + tk] * (vt - X[i >> 2][i & 3]);
        }
        f4 D[4];
#pragma unroll
        for (int rt = 0; rt < 4; rt++) D[rt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int m = 0; m < 16; m++) {
            const int tk = kmap(m, g);
#pragma unroll
            for (int rt = 0; rt < 4; rt++) D[rt] = mfma4(RB[bP + cmap(rt, c) * RecF::PP + tk], rv[m], D[rt]);
            if ((m & 3) == 3) sched_fence();
        }
        // O = Y + M Delta
#pragma unroll
        for (int m = 0; m < 16; m++) {
            const int tk = kmap(m, g);
            const float dm = D[m >> 2][m & 3];
#pragma unroll
            for (int rt = 0; rt < 4; rt++) Y[rt] = mfma4(RB[bM + cmap(rt, c) * RecF::PP + tk], dm, Y[rt]);
            if ((m & 3) == 3) sched_fence();
        }
        if (o) {
            const int oe = p.out_dt == LA_F32 ? 4 : 2;
            const ChunkRows ro = chunk_rows(static_cast<char*>(o) + tok0 * dv * oe, (ntok - tok0) * dv * oe, p.H * dv, g,
                                            col, oe);
#pragma unroll
            for (int i = 0; i < 16; i++) {
                if (kmap(i, g) < L) {
                    if (oe == 4) ro.stf(i, Y[i >> 2][i & 3]);
                    else ro.st16(i, f32_to_bf16_bits(Y[i >> 2][i & 3]));
                }
            }
        }
        // S_end = diag(E_L) S + Kd^T Delta
#pragma unroll
        for (int kt = 0; kt < 8; kt++) {
            f4 acc;
#pragma unroll
            for (int r = 0; r < 4; r++) acc[r] = RB[bEL + 16 * kt + 4 * r + g] * s[4 * kt + r];
#pragma unroll
            for (int m = 0; m < 16; m++) {
                acc = mfma4(RB[bKDT + cmap(kt, c) * RecF::PD + kmap(m, g)], D[m >> 2][m & 3], acc);
                if ((m & 7) == 7) sched_fence();
            }
#pragma unroll
            for (int r = 0; r < 4; r++) s[4 * kt + r] = acc[r];
        }
        if (QMODE != LA_QDQ_NONE && ((t0 + L) % p.qdq_interval == 0 || t0 + L == p.T))
            wave_quantize<32, QMODE, G, kChDk>(s, qsh, lane, w, qpar);
    }
    if (ST) {
#pragma unroll
        for (int m = 0; m < 32; m++) ST[soff + static_cast<size_t>(kmap(m, g0)) * dv] = s[m];
    }
}

template <int QMODE, int G>
hipError_t launch_chunk_state(const la_config& c, const ChunkParams& p, const ChunkIn& in, const float* S0, void* o,
                              float* ST, float* ckpts, const float* rec, hipStream_t s) {
    hipLaunchKernelGGL((chunk_fwd_kernel<QMODE, G>), dim3(chunk_tile_blocks(c.B * c.H, p.ntile)), dim3(kChThreads), 0,
                       s, p, in, S0, o, ST, ckpts, rec);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_prep(const la_config& c, const ChunkIn& in, float* rec, bool bwd, hipStream_t s) {
    const ChunkParams p = make_chunk_params(c);
    const dim3 grid(p.nch, c.H, c.B);
    const bool kda = c.gate == LA_GATE_KEY;
    if (bwd) {
        if (kda) hipLaunchKernelGGL((chunk_prep_kernel<true, true>), grid, dim3(kPrepT), 0, s, p, in, rec);
        else hipLaunchKernelGGL((chunk_prep_kernel<false, true>), grid, dim3(kPrepT), 0, s, p, in, rec);
    } else {
        if (kda) hipLaunchKernelGGL((chunk_prep_kernel<true, false>), grid, dim3(kPrepT), 0, s, p, in, rec);
        else hipLaunchKernelGGL((chunk_prep_kernel<false, false>), grid, dim3(kPrepT), 0, s, p, in, rec);
    }
    return hipGetLastError();
}

hipError_t launch_chunk_fwd(const la_config& c, const FwdArgs& a, float* rec, hipStream_t s) {
    const ChunkParams p = make_chunk_params(c);
    const ChunkIn in{a.q, a.k, a.v, a.g, a.beta};
    hipError_t e = launch_chunk_prep(c, in, rec, false, s);
    if (e != hipSuccess) return e;
    if (c.qdq == LA_QDQ_NONE) return launch_chunk_state<LA_QDQ_NONE, 1>(c, p, in, a.S0, a.o, a.ST, a.ckpts, rec, s);
    if (c.qdq == LA_QDQ_E4M3_TILE)
        return launch_chunk_state<LA_QDQ_E4M3_TILE, 64>(c, p, in, a.S0, a.o, a.ST, a.ckpts, rec, s);
    switch (c.group) {
        case 16: return launch_chunk_state<LA_QDQ_INT8_GROUP, 16>(c, p, in, a.S0, a.o, a.ST, a.ckpts, rec, s);
        case 32: return launch_chunk_state<LA_QDQ_INT8_GROUP, 32>(c, p, in, a.S0, a.o, a.ST, a.ckpts, rec, s);
        default: return launch_chunk_state<LA_QDQ_INT8_GROUP, 64>(c, p, in, a.S0, a.o, a.ST, a.ckpts, rec, s);
    }
}

}  // namespace la
