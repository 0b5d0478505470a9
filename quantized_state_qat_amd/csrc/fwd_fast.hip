// Long-sequence forward for the scalar gate when the state is not rounded every token
// (no quantizer, or INT8/E4M3 at an interval >= 2).  The FP32-VALU-bound path.
//
// One workgroup per (sequence, head, 64-column value tile): 8 waves, lane j = column j,
// wave w = key rows [w R, (w+1) R), R = d_k / 8, so two waves share each SIMD.  Per token:
//  * the state is carried rescaled, S = A * Shat, with A a wave-uniform scalar, so the
//    update S' = a S + k delta^T becomes one FMA per element: Shat += k (delta / A'), A' = a A;
//    A' is folded back into Shat (and reset to 1) when it leaves [2^-30, 2^30], at
//    quantization points, and never drifts past an exponent range fp32 represents exactly;
//  * the wave's rows of k and q are wave-uniform: scalar loads of bf16 (or fp32) words,
//    widened on the scalar unit, consumed as SGPR operands of the FMAs;
//  * one pass over Shat gives the partial sums of Shat^T k and Shat^T q; the 8 waves'
//    partials meet in LDS (double-buffered by token parity) behind a single barrier and are
//    summed in a fixed order; o = A' (Shat^T q) + delta (k . q) reads the state before
//    rounding;
//  * exp(g) and k . q of token t+2 are computed by wave (t+2) mod 8 and passed through a
//    small LDS ring, two barriers ahead of use.
#include "la_device.hpp"
#include "la_internal.hpp"
#include "la_recur.hpp"

namespace la {

Params make_params(const la_config& c);

constexpr int kFastWaves = 8;
constexpr int kFastThreads = kFastWaves * 64;

// Loads through the constant address space: the address is wave-uniform and the data are
// never written by the kernel, so they become scalar loads into SGPRs.
typedef const __attribute__((address_space(4))) uint32_t* cu32_ptr;

template <bool BF16>
__device__ __forceinline__ float vload(const void* p, size_t i) {
    if (BF16) return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
    return static_cast<const float*>(p)[i];
}

// Raw words of R keys (bf16 pairs or fp32), wave-uniform, fetched one token ahead.
template <int R, bool BF16>
struct KeyWords {
    static constexpr int N = BF16 ? R / 2 : R;
    uint32_t w[N];
    __device__ __forceinline__ void fetch(const void* p, size_t off) {
        cu32_ptr src = BF16 ? (cu32_ptr)(static_cast<const uint16_t*>(p) + off) : (cu32_ptr)(static_cast<const float*>(p) + off);
#pragma unroll
        for (int j = 0; j < N; j++) w[j] = src[j];
    }
    __device__ __forceinline__ void widen(float (&out)[R]) const {
#pragma unroll
        for (int j = 0; j < N; j++) {
            if (BF16) {
                out[2 * j] = __uint_as_float(w[j] << 16);
                out[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
            } else {
                out[j] = __uint_as_float(w[j]);
            }
        }
    }
};

template <int DK, int QMODE, int G, bool BF16, bool GF32>
__global__ __launch_bounds__(kFastThreads) void fwd_fast_kernel(Params p, FwdArgs a) {
    constexpr int NW = kFastWaves;
    constexpr int R = DK / NW;
    constexpr int RING = 16;  // token slots in flight (two blocks of NW tokens)
    __shared__ float2 red[2][NW][64];
    __shared__ float4 tsc[RING];       // (exp(g), k . q, beta, -) of token u at u % RING
    __shared__ float vring[RING][64];  // v of token u for this tile's columns
    __shared__ float amax_s[NW];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int T = p.T, H = p.H, DV = p.dv;
    const int col = blk * kTileCols + lane;
    const size_t bh = static_cast<size_t>(b) * H + h;
    const size_t state_off = bh * DK * DV;
    const size_t tok0 = static_cast<size_t>(b) * T * H + h;  // token 0 of this (b, h)

    // Token inputs arrive in blocks of NW tokens: wave w fetches token NW*J + w (one word of k
    // and of q per lane, g, beta, and this tile's v) a block ahead, then reduces k . q, takes
    // exp(g) and publishes the block through the LDS rings, all waves at the same iteration.
    // raw words in flight (widened only when published, so the loads are not waited on early)
    uint32_t sk = 0, sq = 0, sg = 0, sb = 0, sv = 0;
    uint32_t sk2 = 0, sq2 = 0;  // fp32 inputs with d_k = 128: second half of the row
    auto fetch = [&](int u) {
        if (u >= T) return;
        const size_t tk = tok0 + static_cast<size_t>(u) * H;
        if (BF16) {
            if (lane < DK / 2) {
                sk = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.k) + tk * DK)[lane];
                sq = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.q) + tk * DK)[lane];
            }
        } else {
            if (lane < DK) {
                sk = __float_as_uint(static_cast<const float*>(a.k)[tk * DK + lane]);
                sq = __float_as_uint(static_cast<const float*>(a.q)[tk * DK + lane]);
            }
            if (lane + 64 < DK) {
                sk2 = reinterpret_cast<const uint32_t*>(a.k)[tk * DK + lane + 64];
                sq2 = reinterpret_cast<const uint32_t*>(a.q)[tk * DK + lane + 64];
            }
        }
        sg = GF32 ? reinterpret_cast<const uint32_t*>(a.g)[tk] : static_cast<const uint16_t*>(a.g)[tk];
        sb = GF32 ? reinterpret_cast<const uint32_t*>(a.beta)[tk] : static_cast<const uint16_t*>(a.beta)[tk];
        sv = BF16 ? static_cast<const uint16_t*>(a.v)[tk * DV + col] : reinterpret_cast<const uint32_t*>(a.v)[tk * DV + col];
    };
    auto widen_word = [](uint32_t x, bool bf16) { return bf16 ? __uint_as_float(x << 16) : __uint_as_float(x); };
    // Warm the scalar cache with token u's key and query rows (one dword per 64-byte line);
    // the per-token scalar loads of those rows then hit it.  The loaded words are folded
    // into `touch` so the loads are kept.
    uint32_t touch = 0;
    auto ktouch = [&](int u) {
        if (u >= T) return;
        const size_t tk = tok0 + static_cast<size_t>(u) * H;
        constexpr int kBytes = DK * (BF16 ? 2 : 4);
        cu32_ptr kp = (cu32_ptr)(static_cast<const char*>(a.k) + tk * kBytes);
        cu32_ptr qp = (cu32_ptr)(static_cast<const char*>(a.q) + tk * kBytes);
#pragma unroll
        for (int j = 0; j < kBytes / 64; j++) touch ^= kp[j * 16] ^ qp[j * 16];
    };
    auto publish = [&](int u) {
        if (u >= T) return;
        float acc = 0.0f;
        if (BF16) {
            if (lane < DK / 2) {
                acc = __uint_as_float(sk << 16) * __uint_as_float(sq << 16);
                acc = __builtin_fmaf(__uint_as_float(sk & 0xFFFF0000u), __uint_as_float(sq & 0xFFFF0000u), acc);
            }
        } else {
            if (lane < DK) acc = __uint_as_float(sk) * __uint_as_float(sq);
            if (lane + 64 < DK) acc = __builtin_fmaf(__uint_as_float(sk2), __uint_as_float(sq2), acc);
        }
        acc = wave_sum(acc);
        if (lane == 0) tsc[u % RING] = make_float4(expf(widen_word(sg, !GF32)), acc, widen_word(sb, !GF32), 0.0f);
        vring[u % RING][lane] = widen_word(sv, BF16);
    };

    float s[R];
#pragma unroll
    for (int m = 0; m < R; m++)
        s[m] = a.S0 ? a.S0[state_off + static_cast<size_t>(w * R + m) * DV + col] : 0.0f;
    float A = 1.0f;

    fetch(w);
    publish(w);
    // Settle every load issued so far (the conditional state loads included) before the first
    // block prefetch: otherwise the compiler's wait analysis keeps them pending around the
    // token loop and waits for all memory traffic, prefetches included, at every token.
    __builtin_amdgcn_s_waitcnt(0);
    fetch(NW + w);
    ktouch(NW + w);
    __syncthreads();

    KeyWords<R, BF16> kw, qw;
    kw.fetch(a.k, tok0 * DK + w * R);
    qw.fetch(a.q, tok0 * DK + w * R);
    float4 sc = tsc[0];
    float vj = vring[0][lane];
    int ck_next = a.ckpts ? 0 : T;                                        // next checkpoint token
    int q_next = QMODE != LA_QDQ_NONE ? min(p.qdq_interval, T) - 1 : T;  // next rounding token
    size_t tok = tok0;

#pragma unroll 1
    for (int t = 0; t < T; t++, tok += H) {
        if ((t & (NW - 1)) == NW - 2) {  // publish the next block, fetch the one after
            const int u = t + 2 + w;
            publish(u);
            fetch(u + NW);
            ktouch(u + NW);
        }
        if (t == ck_next) {
            float* dst = a.ckpts + (bh * p.nck + t / p.ckpt_interval) * DK * DV;
#pragma unroll
            for (int m = 0; m < R; m++) dst[static_cast<size_t>(w * R + m) * DV + col] = A * s[m];
            ck_next += p.ckpt_interval;
        }
        float kr[R], qr[R];
        kw.widen(kr);
        qw.widen(qr);
        float Ap = A * sc.x;
        if (!(Ap >= 0x1p-30f && Ap <= 0x1p30f)) {  // fold the scale back into the state
#pragma unroll
            for (int m = 0; m < R; m++) s[m] *= Ap;
            Ap = 1.0f;
        }
        float pk = 0.0f, pq = 0.0f;
#pragma unroll
        for (int m = 0; m < R; m++) {
            pk = __builtin_fmaf(s[m], kr[m], pk);
            pq = __builtin_fmaf(s[m], qr[m], pq);
        }
        red[t & 1][w][lane] = make_float2(pk, pq);
        __syncthreads();
        float P = red[t & 1][0][lane].x, Q = red[t & 1][0][lane].y;
#pragma unroll
        for (int ww = 1; ww < NW; ww++) {
            const float2 x = red[t & 1][ww][lane];
            P += x.x;
            Q += x.y;
        }
        const float4 sc_t = sc;
        const float vj_t = vj;
        const float delta = sc_t.z * (vj_t - Ap * P);
        if (a.o && w == (t & (NW - 1)))
            store_elem(a.o, tok * DV + col, p.out_dt, __builtin_fmaf(delta, sc_t.y, Ap * Q));
        // the rescale is not a rounding decision: the hardware reciprocal suffices
        const float dd = delta * __builtin_amdgcn_rcpf(Ap);
#pragma unroll
        for (int m = 0; m < R; m++) s[m] = __builtin_fmaf(kr[m], dd, s[m]);
        A = Ap;
        // next token's inputs: keys/queries were brought into L2 by the block fetch
        if (t + 1 < T) {
            kw.fetch(a.k, (tok + H) * DK + w * R);
            qw.fetch(a.q, (tok + H) * DK + w * R);
            sc = tsc[(t + 1) % RING];
            vj = vring[(t + 1) % RING][lane];
        }

        if (t == q_next) {
            q_next = min(q_next + p.qdq_interval, T - 1);
            if (q_next == t) q_next = T;
#pragma unroll
            for (int m = 0; m < R; m++) s[m] *= A;
            A = 1.0f;
            if (QMODE == LA_QDQ_INT8_GROUP) {
#pragma unroll
                for (int m = 0; m < R; m++) {
                    float sc8, y;
                    const float c = int8_scale_recip(group_max_abs<G>(s[m]), sc8, y) ? int8_code_fast(s[m], sc8, y)
                                                                                     : int8_code(s[m], sc8);
                    s[m] = c * sc8;
                }
            } else if (QMODE == LA_QDQ_E4M3_TILE) {
                float mx = 0.0f;
#pragma unroll
                for (int m = 0; m < R; m++) mx = fmaxf(mx, fabsf(s[m]));
                mx = wave_max_abs(mx);
                if (lane == 0) amax_s[w] = mx;
                __syncthreads();
                float amax = amax_s[0];
#pragma unroll
                for (int ww = 1; ww < NW; ww++) amax = fmaxf(amax, amax_s[ww]);
                float sce, y;
                if (e4m3_scale_recip(amax, sce, y)) {
#pragma unroll
                    for (int m = 0; m < R; m++) s[m] = e4m3_round(quot_rn_fast(s[m], sce, y)) * sce;
                } else {
#pragma unroll
                    for (int m = 0; m < R; m++) s[m] = e4m3_round(s[m] / sce) * sce;
                }
                // amax_s is rewritten only after at least one more token barrier
            }
        }
    }
    if (a.ST) {
#pragma unroll
        for (int m = 0; m < R; m++) a.ST[state_off + static_cast<size_t>(w * R + m) * DV + col] = A * s[m];
    }
    // T >= 0 always (checked on the host); the store only keeps the cache-warming loads alive
    if (T < 0 && a.o && lane == 0) static_cast<uint32_t*>(a.o)[0] = touch;
}

template <int DK, int QMODE, int G>
static hipError_t launch_fast_t(const la_config& c, const FwdArgs& a, hipStream_t s) {
    dim3 grid(c.d_v / kTileCols, c.H, c.B);
    const bool bf = c.qkv_dtype == LA_BF16, gf = c.gate_dtype == LA_F32;
    if (bf && gf)
        hipLaunchKernelGGL((fwd_fast_kernel<DK, QMODE, G, true, true>), grid, dim3(kFastThreads), 0, s, make_params(c), a);
    else if (bf)
        hipLaunchKernelGGL((fwd_fast_kernel<DK, QMODE, G, true, false>), grid, dim3(kFastThreads), 0, s, make_params(c), a);
    else if (gf)
        hipLaunchKernelGGL((fwd_fast_kernel<DK, QMODE, G, false, true>), grid, dim3(kFastThreads), 0, s, make_params(c), a);
    else
        hipLaunchKernelGGL((fwd_fast_kernel<DK, QMODE, G, false, false>), grid, dim3(kFastThreads), 0, s, make_params(c), a);
    return hipGetLastError();
}

template <int DK>
static hipError_t launch_fast_dk(const la_config& c, const FwdArgs& a, hipStream_t s) {
    if (c.qdq == LA_QDQ_NONE) return launch_fast_t<DK, LA_QDQ_NONE, 1>(c, a, s);
    if (c.qdq == LA_QDQ_E4M3_TILE) return launch_fast_t<DK, LA_QDQ_E4M3_TILE, 64>(c, a, s);
    switch (c.group) {
        case 16: return launch_fast_t<DK, LA_QDQ_INT8_GROUP, 16>(c, a, s);
        case 32: return launch_fast_t<DK, LA_QDQ_INT8_GROUP, 32>(c, a, s);
        default: return launch_fast_t<DK, LA_QDQ_INT8_GROUP, 64>(c, a, s);
    }
}

bool fwd_fast_eligible(const la_config& c) {
    if (c.gate != LA_GATE_SCALAR || c.hadamard) return false;
    if (c.replay && c.qdq_interval > 1) return false;  // encoded updates: token by token
    if (c.qdq == LA_QDQ_NONE) return true;
    // no rounding decision may fall strictly inside a checkpoint chunk, so that a backward
    // recompute (which uses the general kernel) meets the same decisions at chunk ends
    if (c.qdq_interval < 2) return false;
    return c.ckpt_interval == 0 || c.qdq_interval % c.ckpt_interval == 0;
}

hipError_t launch_fwd_fast(const la_config& c, const FwdArgs& a, hipStream_t s) {
    switch (c.d_k) {
        case 16: return launch_fast_dk<16>(c, a, s);
        case 32: return launch_fast_dk<32>(c, a, s);
        case 64: return launch_fast_dk<64>(c, a, s);
        default: return launch_fast_dk<128>(c, a, s);
    }
}

}  // namespace la
