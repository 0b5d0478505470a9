// Forward recurrence kernel: one workgroup per (sequence, head, 64-column value tile),
// the tile's FP32 state resident in VGPRs for the whole token loop (la_recur.hpp).
#include "la_recur.hpp"

namespace la {

template <int DK, int QMODE, int G, bool HAD, bool KDA>
__global__ __launch_bounds__(kThreads) void fwd_kernel(Params p, FwdArgs a) {
    constexpr int R = DK / 4;
    __shared__ Smem<DK> sm;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int T = p.T, H = p.H, DV = p.dv;
    const int col = blk * kTileCols + lane;
    const size_t bh = static_cast<size_t>(b) * H + h;
    const size_t state_off = bh * DK * DV;

    float s[R];
#pragma unroll
    for (int m = 0; m < R; m++)
        s[m] = a.S0 ? a.S0[state_off + static_cast<size_t>(w * R + m) * DV + col] : 0.0f;
    if (HAD && !p.rot) rotate_state<DK>(sm, s, 1.0f);

#pragma unroll 1
    for (int t = 0; t < T; t++) {
        if (a.ckpts && (t % p.ckpt_interval) == 0) {
            // Hadamard mode stores the carried state in its rotated form Hu S (exactly what
            // the token loop carries), so a recompute resumes bit for bit.
            float* dst = a.ckpts + (bh * p.nck + t / p.ckpt_interval) * DK * DV;
#pragma unroll
            for (int m = 0; m < R; m++) dst[static_cast<size_t>(w * R + m) * DV + col] = s[m];
        }
        const size_t tok = (static_cast<size_t>(b) * T + t) * H + h;
        float vj = load_elem(a.v, tok * DV + col, p.qkv_dt);
        stage_token<DK, HAD, KDA>(sm, a.q, a.k, a.g, a.beta, tok, p.qkv_dt, p.gate_dt);
        float u, d, o;
        bool qnow = (QMODE != LA_QDQ_NONE) && is_qdq_point(t, T, p.qdq_interval);
        token_step<DK, QMODE, G>(sm, s, vj, qnow, u, d, o);
        if (a.o && w == 0) store_elem(a.o, tok * DV + col, p.out_dt, o);
    }
    if (a.ST) {
        if (HAD && !p.rot) rotate_state<DK>(sm, s, 1.0f / DK);
#pragma unroll
        for (int m = 0; m < R; m++) a.ST[state_off + static_cast<size_t>(w * R + m) * DV + col] = s[m];
    }
}

__global__ void copy_state_kernel(const float* __restrict__ src, float* __restrict__ dst, size_t n) {
    size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.0f;
}

Params make_params(const la_config& c) {
    Params p;
    p.B = c.B; p.T = c.T; p.H = c.H; p.dk = c.d_k; p.dv = c.d_v;
    p.qkv_dt = c.qkv_dtype; p.gate_dt = c.gate_dtype; p.out_dt = c.out_dtype;
    p.qdq_interval = c.qdq == LA_QDQ_NONE ? 1 : c.qdq_interval;
    p.ckpt_interval = c.ckpt_interval > 0 ? c.ckpt_interval : 1;
    p.nck = n_ckpts(c);
    p.rot = c.hadamard && c.state_rotated;
    return p;
}

template <int DK, int QMODE, int G, bool HAD, bool KDA>
static hipError_t launch_fwd_t(const la_config& c, const FwdArgs& a, hipStream_t s) {
    dim3 grid(c.d_v / kTileCols, c.H, c.B);
    hipLaunchKernelGGL((fwd_kernel<DK, QMODE, G, HAD, KDA>), grid, dim3(kThreads), 0, s,
                       make_params(c), a);
    return hipGetLastError();
}

template <int DK>
static hipError_t launch_fwd_dk(const la_config& c, const FwdArgs& a, hipStream_t s) {
    const bool kda = c.gate == LA_GATE_KEY;
    if (c.qdq == LA_QDQ_NONE)
        return kda ? launch_fwd_t<DK, LA_QDQ_NONE, 1, false, true>(c, a, s)
                   : launch_fwd_t<DK, LA_QDQ_NONE, 1, false, false>(c, a, s);
    if (c.qdq == LA_QDQ_E4M3_TILE)
        return kda ? launch_fwd_t<DK, LA_QDQ_E4M3_TILE, 64, false, true>(c, a, s)
                   : launch_fwd_t<DK, LA_QDQ_E4M3_TILE, 64, false, false>(c, a, s);
    if (c.hadamard) {
        switch (c.group) {
            case 16: return launch_fwd_t<DK, LA_QDQ_INT8_GROUP, 16, true, false>(c, a, s);
            case 32: return launch_fwd_t<DK, LA_QDQ_INT8_GROUP, 32, true, false>(c, a, s);
            default: return launch_fwd_t<DK, LA_QDQ_INT8_GROUP, 64, true, false>(c, a, s);
        }
    }
    switch (c.group) {
        case 16: return kda ? launch_fwd_t<DK, LA_QDQ_INT8_GROUP, 16, false, true>(c, a, s)
                            : launch_fwd_t<DK, LA_QDQ_INT8_GROUP, 16, false, false>(c, a, s);
        case 32: return kda ? launch_fwd_t<DK, LA_QDQ_INT8_GROUP, 32, false, true>(c, a, s)
                            : launch_fwd_t<DK, LA_QDQ_INT8_GROUP, 32, false, false>(c, a, s);
        default: return kda ? launch_fwd_t<DK, LA_QDQ_INT8_GROUP, 64, false, true>(c, a, s)
                            : launch_fwd_t<DK, LA_QDQ_INT8_GROUP, 64, false, false>(c, a, s);
    }
}

const char* fwd_kernel_name(const la_config& c) {
    if (fwd_mfma_eligible(c)) return "block";
    if (fwd_wave_eligible(c)) return "wave";
    if (fwd_fast_eligible(c)) return "fast";
    return "token";
}

hipError_t launch_fwd(const la_config& c, const FwdArgs& a, hipStream_t s) {
    if (fwd_mfma_eligible(c)) return launch_fwd_mfma(c, a, s);
    if (fwd_wave_eligible(c)) return launch_fwd_wave(c, a, s);
    if (fwd_fast_eligible(c)) return launch_fwd_fast(c, a, s);
    switch (c.d_k) {
        case 16: return launch_fwd_dk<16>(c, a, s);
        case 32: return launch_fwd_dk<32>(c, a, s);
        case 64: return launch_fwd_dk<64>(c, a, s);
        default: return launch_fwd_dk<128>(c, a, s);
    }
}

hipError_t launch_copy_state(const la_config& c, const float* src, float* dst, hipStream_t s) {
    size_t n = static_cast<size_t>(c.B) * c.H * c.d_k * c.d_v;
    if (n == 0) return hipSuccess;
    unsigned blocks = static_cast<unsigned>((n + 255) / 256);
    hipLaunchKernelGGL(copy_state_kernel, dim3(blocks), dim3(256), 0, s, src, dst, n);
    return hipGetLastError();
}

}  // namespace la
