// Forward dispatch: the first kernel whose conditions a configuration meets (fwd_mfma.hip,
// fwd_wave.hip, fwd_fast.hip), else the token kernel (fwd_tok.hip).  All of them compute the
// same recurrence and meet the same rounding points; they differ in the order of
// floating-point operations between rounding points.
#include "la_recur.hpp"

namespace la {

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

la_kernel fwd_kernel(const la_config& c) {
    // the Neumann solve defines a different function: the chunk kernel or nothing
    if (c.solve == LA_SOLVE_NEUMANN || c.kernel == LA_KERNEL_CHUNK)
        return chunk_eligible(c) ? LA_KERNEL_CHUNK : LA_KERNEL_AUTO;
    switch (c.kernel) {
        case LA_KERNEL_BLOCK: return fwd_mfma_eligible(c) ? LA_KERNEL_BLOCK : LA_KERNEL_AUTO;
        case LA_KERNEL_WAVE: return fwd_wave_eligible(c) ? LA_KERNEL_WAVE : LA_KERNEL_AUTO;
        case LA_KERNEL_FAST: return fwd_fast_eligible(c) ? LA_KERNEL_FAST : LA_KERNEL_AUTO;
        case LA_KERNEL_TOKEN: return LA_KERNEL_TOKEN;  // serves every valid configuration
        default: break;
    }
    if (fwd_mfma_eligible(c)) return LA_KERNEL_BLOCK;
    if (fwd_wave_eligible(c)) return LA_KERNEL_WAVE;
    if (fwd_fast_eligible(c)) return LA_KERNEL_FAST;
    return LA_KERNEL_TOKEN;
}

la_kernel bwd_kernel(const la_config& c) {
    if (fwd_kernel(c) == LA_KERNEL_CHUNK) return LA_KERNEL_CHUNK;
    if (bwd_mfma_eligible(c)) return LA_KERNEL_BLOCK;
    if (c.kernel != LA_KERNEL_TOKEN && c.ckpt_interval == kChunkTokens && chunk_eligible(c)) return LA_KERNEL_CHUNK;
    return LA_KERNEL_TOKEN;
}

const char* fwd_kernel_name(const la_config& c) {
    switch (fwd_kernel(c)) {
        case LA_KERNEL_BLOCK: return "block";
        case LA_KERNEL_WAVE: return "wave";
        case LA_KERNEL_FAST: return "fast";
        case LA_KERNEL_TOKEN: return "token";
        case LA_KERNEL_CHUNK: return "chunk";
        default: return "";
    }
}

hipError_t launch_fwd(const la_config& c, const FwdArgs& a, hipStream_t s) {
    switch (fwd_kernel(c)) {
        case LA_KERNEL_BLOCK: return launch_fwd_mfma(c, a, s);
        case LA_KERNEL_WAVE: return launch_fwd_wave(c, a, s);
        case LA_KERNEL_FAST: return launch_fwd_fast(c, a, s);
        case LA_KERNEL_TOKEN: return launch_fwd_tok(c, a, s);
        default: return hipErrorInvalidValue;  // rejected by the ABI before any launch
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
