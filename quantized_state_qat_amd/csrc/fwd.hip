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
    return launch_fwd_tok(c, a, s);
}

hipError_t launch_copy_state(const la_config& c, const float* src, float* dst, hipStream_t s) {
    size_t n = static_cast<size_t>(c.B) * c.H * c.d_k * c.d_v;
    if (n == 0) return hipSuccess;
    unsigned blocks = static_cast<unsigned>((n + 255) / 256);
    hipLaunchKernelGGL(copy_state_kernel, dim3(blocks), dim3(256), 0, s, src, dst, n);
    return hipGetLastError();
}

}  // namespace la
