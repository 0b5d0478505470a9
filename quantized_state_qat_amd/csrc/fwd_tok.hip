// Token forward: every configuration the regrouped kernels do not take (per-key gates,
// the Hadamard rotation, a rounding point after every token or at intervals that do not
// fall on their block ends).  The layout and the per-token step are those of la_tok.hpp.
//
// The tile is 64 or 32 value columns wide (TokShape).  Token inputs arrive in blocks of eight:
// wave w fetches token 8 J + w of block J two blocks ahead (raw words in registers),
// publishes it into the LDS ring one block ahead, and every
// wave reads its rows of a token's record at the end of the previous token.  The only
// barrier per token is the one inside tok_step (plus one more for an E4M3 rounding point).
#include "la_tok.hpp"

namespace la {

TokParams make_tok_params(const la_config& c) {
    TokParams p;
    p.B = c.B; p.T = c.T; p.H = c.H; p.dk = c.d_k; p.dv = c.d_v;
    p.qkv_dt = c.qkv_dtype; p.gate_dt = c.gate_dtype; p.out_dt = c.out_dtype;
    p.qdq_interval = c.qdq == LA_QDQ_NONE ? 1 : c.qdq_interval;
    p.ckpt_interval = c.ckpt_interval > 0 ? c.ckpt_interval : 1;
    p.nck = n_ckpts(c);
    p.rot = c.hadamard && c.state_rotated;
    p.replay = c.replay && c.qdq != LA_QDQ_NONE;
    p.ntok = static_cast<long>(c.B) * c.T * c.H;
    return p;
}

template <int DK, int QMODE, int G, bool HAD, bool KDA>
__global__ __launch_bounds__(kTokThreads) void fwd_tok_kernel(TokParams p, FwdArgs a) {
    using S = TokShape<DK, QMODE, G>;
    constexpr int R = S::R, TC = S::TC;
    // Hadamard mode: the scalar gate carries Y = Hu S (RC); per-key gates carry S and rotate
    // around each rounding point (RQ)
    constexpr bool RC = HAD && !KDA, RQ = HAD && KDA;
    __shared__ TokRing<S, KDA, false> ring;
    __shared__ float2 red[2][kTokWaves][TC];
    __shared__ TokQdqShared<S> qsh;
    __shared__ float tile[HAD ? 2 * DK * TC : 1];  // tok_rotate's two tiles

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int H = p.H, DV = p.dv;
    int T = p.T;
    size_t tok0 = static_cast<size_t>(b) * T * H + h;  // token 0 of this (b, h)
    size_t ck0 = (static_cast<size_t>(b) * H + h) * p.nck;  // its first checkpoint
    if (a.cu_seqlens) {
        // packed sequences: this one's tokens (or one part of them), clamped to the packed
        // length; checkpoints in the packed slot layout
        int t_begin, t_end;
        packed_range(a.cu_seqlens, a.split, a.split_part, b, p.T, t_begin, t_end);
        T = t_end - t_begin;
        tok0 = static_cast<size_t>(t_begin) * H + h;
        ck0 = static_cast<size_t>(h) * p.nck + b + t_begin / p.ckpt_interval;
    }
    const int col = blk * TC + lane % TC;
    const int r0 = tok_row0<S>(w, lane);
    const size_t bh = static_cast<size_t>(b) * H + h;
    const size_t state_off = bh * DK * DV;
    const TokInputs in{a.q, a.k, a.v, a.g, a.beta, nullptr};
    if (T == 0) {
        // an empty packed sequence hands its initial state through unchanged (no rotation
        // round trip); uniform over the workgroup
        if (a.ST) {
#pragma unroll
            for (int m = 0; m < R; m++) {
                const size_t e = state_off + static_cast<size_t>(r0 + m) * DV + col;
                a.ST[e] = a.S0 ? a.S0[e] : 0.0f;
            }
        }
        return;
    }

    TokFetch<S, KDA, false> f;
    auto fetch = [&](int u) __attribute__((always_inline)) {  // (a token past the end fetches the last; never published)
        f.fetch(in, p, tok0 + static_cast<size_t>(min(u, T - 1)) * H, col, lane);
    };
    auto publish = [&](int u) __attribute__((always_inline)) {
        if (u < T) f.template publish<RC>(ring, u % kTokRing, p, lane);
    };

    float s[R];
#pragma unroll
    for (int m = 0; m < R; m++)
        s[m] = a.S0 ? a.S0[state_off + static_cast<size_t>(r0 + m) * DV + col] : 0.0f;
    if (RC && !p.rot) tok_rotate<S>(s, tile, w, lane, 1.0f);

    fetch(w);
    publish(w);
    // Settle every load issued so far before the first prefetch: otherwise the compiler's
    // wait analysis keeps them pending around the token loop and waits for all memory
    // traffic, prefetches included, at every token.
    __builtin_amdgcn_s_waitcnt(0);
    fetch(kTokWaves + w);
    __syncthreads();

    // operands of token t are read at the end of token t - 1, into the other of two buffers
    TokOps<S, KDA> opA, opB;
    if (T > 0) tok_read<S, KDA, false>(opA, ring, 0, w, lane);
    int ck_next = a.ckpts ? 0 : T;                                        // next checkpoint token
    int q_next = QMODE != LA_QDQ_NONE ? min(p.qdq_interval, T) - 1 : T;  // next rounding token

    auto token = [&](int t, const TokOps<S, KDA>& op, TokOps<S, KDA>& op_next) __attribute__((always_inline)) {
        const size_t tok = tok0 + static_cast<size_t>(t) * H;
        if ((t & (kTokWaves - 1)) == kTokWaves - 2) {  // publish the next block, fetch the one after
            const int u = t + 2 + w;
            publish(u);
            fetch(u + kTokWaves);
        }
        if (t == ck_next) {
            // checkpoints hold the carried state as the loop carries it (rotated in Hadamard mode)
            float* dst = a.ckpts + (ck0 + t / p.ckpt_interval) * DK * DV;
#pragma unroll
            for (int m = 0; m < R; m++) dst[static_cast<size_t>(r0 + m) * DV + col] = s[m];
            ck_next += p.ckpt_interval;
        }
        float u, delta, o;
        tok_step<S, KDA, RC>(s, op, red[t & 1], w, lane, u, delta, o, p.replay && t != q_next);
        if (a.o && w == (t & (kTokWaves - 1)) && lane < TC) store_elem(a.o, tok * DV + col, p.out_dt, o);
        if (a.entries && w == (t & (kTokWaves - 1)) && lane < TC)
            a.entries[tok * DV + col] = static_cast<uint16_t>(__float_as_uint(bf16_rne(delta)) >> 16);
        if (t + 1 < T) tok_read<S, KDA, false>(op_next, ring, (t + 1) % kTokRing, w, lane);
        if (t == q_next) {
            q_next = min(q_next + p.qdq_interval, T - 1);
            if (q_next == t) q_next = T;
            tok_qdq_at<S, RQ>(s, qsh, tile, w, lane);
        }
    };
#pragma unroll 1
    for (int t = 0; t < T; t += 2) {
        token(t, opA, opB);
        if (t + 1 < T) token(t + 1, opB, opA);
    }
    if (a.ST) {
        if (RC && !p.rot) tok_rotate<S>(s, tile, w, lane, 1.0f / DK);
#pragma unroll
        for (int m = 0; m < R; m++) a.ST[state_off + static_cast<size_t>(r0 + m) * DV + col] = s[m];
    }
}

namespace {

template <int DK, int QMODE, int G, bool HAD, bool KDA>
hipError_t launch_tok_t(const la_config& c, const FwdArgs& a, hipStream_t s) {
    dim3 grid(c.d_v / tok_tile_cols(DK, QMODE, G), c.H, c.B);
    TokParams p = make_tok_params(c);
    if (a.cu_seqlens) {
        p.nck = varlen_ckpt_slots(c);
        p.ntok = static_cast<long>(c.T) * c.H;
    }
    hipLaunchKernelGGL((fwd_tok_kernel<DK, QMODE, G, HAD, KDA>), grid, dim3(kTokThreads), 0, s, p, a);
    return hipGetLastError();
}

template <int DK, bool HAD, bool KDA>
hipError_t launch_tok_q(const la_config& c, const FwdArgs& a, hipStream_t s) {
    if (!HAD) {
        if (c.qdq == LA_QDQ_NONE) return launch_tok_t<DK, LA_QDQ_NONE, 16, HAD, KDA>(c, a, s);
        if (c.qdq == LA_QDQ_E4M3_TILE) return launch_tok_t<DK, LA_QDQ_E4M3_TILE, 64, HAD, KDA>(c, a, s);
    }
    switch (c.group) {
        case 16: return launch_tok_t<DK, LA_QDQ_INT8_GROUP, 16, HAD, KDA>(c, a, s);
        case 32: return launch_tok_t<DK, LA_QDQ_INT8_GROUP, 32, HAD, KDA>(c, a, s);
        default: return launch_tok_t<DK, LA_QDQ_INT8_GROUP, 64, HAD, KDA>(c, a, s);
    }
}

template <int DK>
hipError_t launch_tok_dk(const la_config& c, const FwdArgs& a, hipStream_t s) {
    if (c.hadamard)
        return c.gate == LA_GATE_KEY ? launch_tok_q<DK, true, true>(c, a, s) : launch_tok_q<DK, true, false>(c, a, s);
    if (c.gate == LA_GATE_KEY) return launch_tok_q<DK, false, true>(c, a, s);
    return launch_tok_q<DK, false, false>(c, a, s);
}

}  // namespace

hipError_t launch_fwd_tok(const la_config& c, const FwdArgs& a, hipStream_t s) {
    switch (c.d_k) {
        case 16: return launch_tok_dk<16>(c, a, s);
        case 32: return launch_tok_dk<32>(c, a, s);
        case 64: return launch_tok_dk<64>(c, a, s);
        default: return launch_tok_dk<128>(c, a, s);
    }
}

}  // namespace la
