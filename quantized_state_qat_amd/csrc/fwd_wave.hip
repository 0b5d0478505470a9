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
// Per-key gates (KDA): each token's gates a = exp(g) arrive spread over the row group's lanes
// like its keys, and a third DPP pass scales the state rows (S~ = diag(a) S) before the two
// FMA passes; no rescale is carried (a per-row gate cannot be folded into one scalar), so
// every block runs the same way and the gate windows only supply beta.
#include "la_device.hpp"
#include "la_internal.hpp"
#include "la_recur.hpp"
#include "la_wave.hpp"

namespace la {

Params make_params(const la_config& c);

namespace {

constexpr int kWaveThreads = kWaveTileWaves * 64;
constexpr int kRing = 8;   // tokens per block and depth of the input ring
constexpr int kWin = 64;   // tokens per gate window
constexpr float kFoldLo = 0x1p-30f, kFoldHi = 0x1p30f;

}  // namespace

template <int DK, int QMODE, int G, bool BF16, bool GF32, bool OBF16, bool KDA>
__global__ __launch_bounds__(kWaveThreads) void fwd_wave_kernel(Params p, FwdArgs a) {
    constexpr int R = DK / 4;                       // state rows per lane
    constexpr int KPL = R >= 32 ? 2 : 1;            // key (query) values per lane
    constexpr int NW = (KPL == 2 && !BF16) ? 2 : 1; // raw words per lane per key row
    constexpr int IB = BF16 ? 2 : 4;                // input element bytes
    constexpr int OB = OBF16 ? 2 : 4;
    constexpr int GB = GF32 ? 4 : 2;
    constexpr int NWG = (KPL == 2 && GF32) ? 2 : 1;  // raw words per lane of a token's key gates (KDA)

    __shared__ WaveQdqShared<DK, QMODE, G> qsh;

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
    // scalar gates [B][T][H]; per-key gates [B][T][H][d_k]
    const auto rgt = make_rsrc(static_cast<const char*>(a.g) + seq0 * (KDA ? DK : 1) * GB, seq_tok * (KDA ? DK : 1) * GB);
    const auto rbt = make_rsrc(static_cast<const char*>(a.beta) + seq0 * GB, seq_tok * GB);
    const bool has_o = a.o != nullptr;
    const auto ro = make_rsrc(has_o ? static_cast<const char*>(a.o) + seq0 * DV * OB : nullptr,
                              has_o ? seq_tok * DV * OB : 0);
    // this lane's key element(s) within a token's row, its value column, its output slot
    const int voff_k = (KPL == 2 ? 2 * lane : rg * R + (c % R)) * IB;
    const int voff_gk = (KPL == 2 ? 2 * lane : rg * R + (c % R)) * GB;  // the same key rows' gates (KDA)
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
        uint32_t gk[NWG];  // KDA only
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
        if constexpr (KDA) {
            const int so_g = (tt * H + h) * (DK * GB);
            if (KPL == 2 && GF32) {
                r.gk[0] = __builtin_amdgcn_raw_buffer_load_b32(rgt, voff_gk, so_g, 0);
                r.gk[NWG - 1] = __builtin_amdgcn_raw_buffer_load_b32(rgt, voff_gk + 4, so_g, 0);
            } else if (KPL == 2 || GF32) {
                r.gk[0] = __builtin_amdgcn_raw_buffer_load_b32(rgt, voff_gk, so_g, 0);
            } else {
                r.gk[0] = __builtin_amdgcn_raw_buffer_load_b16(rgt, voff_gk, so_g, 0);
            }
        }
    };
    // a = exp(g) of this lane's key rows (a1 only for two rows per lane); tokens past the end
    // read g = 0 (and beta = 0, so they leave the state unchanged)
    auto key_gates = [&](const Raw& r, float& a0, float& a1) {
        float g0, g1 = 0.0f;
        if (GF32) {
            g0 = __uint_as_float(r.gk[0]);
            if (KPL == 2) g1 = __uint_as_float(r.gk[NWG - 1]);
        } else {
            g0 = __uint_as_float(r.gk[0] << 16);
            if (KPL == 2) g1 = __uint_as_float(r.gk[0] & 0xFFFF0000u);
        }
        a0 = expf(g0);
        a1 = KPL == 2 ? expf(g1) : 1.0f;
    };

    // ---------------------------------------------------------------- gate windows
    float eg_w = 1.0f, beta_w = 0.0f, cum_w = 1.0f, rcum_w = 1.0f, bmin_w = 1.0f, bmax_w = 1.0f;
    uint32_t graw = 0, braw = 0;  // raw gates of the next window, in flight
    auto fetch_window = [&](int w0n) {
        const int so = (w0n * H + h) * GB;  // wave-uniform part
        const int vo = lane * H * GB;       // lane i: token w0n + i
        if (GF32) {
            if (!KDA) graw = __builtin_amdgcn_raw_buffer_load_b32(rgt, vo, so, 0);
            braw = __builtin_amdgcn_raw_buffer_load_b32(rbt, vo, so, 0);
        } else {
            if (!KDA) graw = __builtin_amdgcn_raw_buffer_load_b16(rgt, vo, so, 0);
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
    auto quantize = [&]() { wave_quantize<R, QMODE, G>(s, qsh, lane, w, qpar); };

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

    if constexpr (KDA) {
        // S~ = diag(a) S, P = S~^T k, Q = S~^T q, delta = beta (v - P), S' = S~ + k delta^T,
        // o = Q + delta (k . q)
        auto token_kda = [&](const Keys& x, float a0, float a1, uint32_t vraw, float kq, float bt) {
            const float vj = BF16 ? __uint_as_float(vraw << 16) : __uint_as_float(vraw);
            decay_pass<R>(s, a0, a1);
            float pk, pq, P, Q;
            dot_pass<R>(s, x.k0, x.k1, x.q0, x.q1, pk, pq);
            rows_sum2(pk, pq, P, Q);
            const float delta = bt * (vj - P);
            const float o = __builtin_fmaf(delta, kq, Q);
            update_pass<R>(s, x.k0, x.k1, delta);
            return o;
        };
#pragma unroll 1
        for (int t = 0; t < T; t += kRing) {
            if (t == w_next) {
                w0 = t;
                w_next = t + kWin;
                open_window(w0);
                fetch_window(w_next);
            }
            if (t == ck_next) {
                float* dst = a.ckpts + (bh * p.nck + t / p.ckpt_interval) * DK * DV;
#pragma unroll
                for (int m = 0; m < R; m++) dst[static_cast<size_t>(rg * R + m) * DV + col] = s[m];
                ck_next += p.ckpt_interval;
            }
            const int tw = t - w0;
            float o_acc = 0.0f;
#pragma unroll
            for (int j0 = 0; j0 < kRing; j0 += 4) {
                __builtin_amdgcn_sched_barrier(0);
                Keys x[4];
                uint32_t vr[4];
                float ga[4], gb[4];
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    x[i] = widen(ring[j0 + i]);
                    vr[i] = ring[j0 + i].v;
                    key_gates(ring[j0 + i], ga[i], gb[i]);
                    fetch(ring[j0 + i], t + j0 + i + kRing);
                }
                const float kq4 = sum4_by_rows(kq_part(x[0]), kq_part(x[1]), kq_part(x[2]), kq_part(x[3]));
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const float o = token_kda(x[i], ga[i], gb[i], vr[i], kq4, lane_of(beta_w, tw + j0 + i));
                    o_acc = rg == i ? o : o_acc;
                }
                store_o(t + j0, o_acc);
            }
            if (min(t + kRing, T) - 1 == q_next) {
                quantize();
                q_next = q_next + qi <= T - 1 ? q_next + qi : (q_next < T - 1 ? T - 1 : T);
            }
        }
        if (a.ST) {
#pragma unroll
            for (int m = 0; m < R; m++) a.ST[state_off + static_cast<size_t>(rg * R + m) * DV + col] = s[m];
        }
        return;
    }

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

template <int DK, int QMODE, int G, bool BF16, bool GF32, bool KDA>
hipError_t launch_wave_k(const la_config& c, const FwdArgs& a, hipStream_t s) {
    dim3 grid(c.d_v / kTileCols, c.H, c.B);
    if (c.out_dtype == LA_BF16)
        hipLaunchKernelGGL((fwd_wave_kernel<DK, QMODE, G, BF16, GF32, true, KDA>), grid, dim3(kWaveThreads), 0, s,
                           make_params(c), a);
    else
        hipLaunchKernelGGL((fwd_wave_kernel<DK, QMODE, G, BF16, GF32, false, KDA>), grid, dim3(kWaveThreads), 0, s,
                           make_params(c), a);
    return hipGetLastError();
}

template <int DK, int QMODE, int G, bool BF16, bool GF32>
hipError_t launch_wave_o(const la_config& c, const FwdArgs& a, hipStream_t s) {
    if (c.gate == LA_GATE_KEY) return launch_wave_k<DK, QMODE, G, BF16, GF32, true>(c, a, s);
    return launch_wave_k<DK, QMODE, G, BF16, GF32, false>(c, a, s);
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
    if (c.replay && c.qdq_interval > 1) return false;  // encoded updates: token by token
    if (c.gate == LA_GATE_KEY) {
        // per-key gates: the scalar-gate kernels' rounding conditions, without the rescale
        if (c.hadamard) return false;
        if (c.qdq != LA_QDQ_NONE &&
            (c.qdq_interval < 2 || (c.ckpt_interval > 0 && c.qdq_interval % c.ckpt_interval != 0)))
            return false;
    } else if (!fwd_fast_eligible(c)) {
        return false;
    }
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
