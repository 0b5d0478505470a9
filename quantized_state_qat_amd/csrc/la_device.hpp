// Device helpers shared by the recurrence kernels: input widening, wave-level
// reductions and the two state codecs.  gfx950 (CDNA4), wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace la {

constexpr int kWave = 64;

// ------------------------------------------------------------------ input widening
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Element idx of a tensor stored as float32 (dtype 0) or bfloat16 (dtype 1).
__device__ __forceinline__ float load_elem(const void* p, size_t idx, int dtype) {
    if (dtype == 0) return static_cast<const float*>(p)[idx];
    return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[idx]);
}

// Round float32 to bfloat16 (nearest, ties to even) for bf16 outputs.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// The nearest BF16 value of x as a float (ties to even): the replay windows' encoding.
__device__ __forceinline__ float bf16_rne(float x) {
    return __uint_as_float(static_cast<uint32_t>(f32_to_bf16_bits(x)) << 16);
}

__device__ __forceinline__ void store_elem(void* p, size_t idx, int dtype, float x) {
    if (dtype == 0) static_cast<float*>(p)[idx] = x;
    else static_cast<uint16_t*>(p)[idx] = f32_to_bf16_bits(x);
}

// Buffer resource over `bytes` bytes at base: loads past the end return zero and stores there
// are dropped (raw buffer addressing, 32-bit offsets).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, size_t bytes) {
    const uint32_t n = bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : static_cast<uint32_t>(bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(n), 0x00020000);
}

// ------------------------------------------------------------------ cross-lane
// Lane exchanges use DPP (within rows of 16 lanes) and the gfx950 permlane swaps (across
// rows), never the LDS crossbar.  Every reduction step combines a lane with one partner
// in the complementary half of its group, and IEEE add/max are commutative, so all lanes of
// a group end with bit-identical results.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within 16

struct Pair {
    float a, b;
};
// (x of this lane, x of lane ^ 16)
__device__ __forceinline__ Pair swap16(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
// (x of this lane, x of lane ^ 32)
__device__ __forceinline__ Pair swap32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// Max over aligned groups of N lanes (N a power of two <= 64); result in every lane.
template <int N>
__device__ __forceinline__ float group_max(float x) {
    if (N >= 2) x = fmaxf(x, dpp<kDppXor1>(x));
    if (N >= 4) x = fmaxf(x, dpp<kDppXor2>(x));
    if (N >= 8) x = fmaxf(x, dpp<kDppHalfMirror>(x));
    if (N >= 16) x = fmaxf(x, dpp<kDppMirror>(x));
    if (N >= 32) { Pair p = swap16(x); x = fmaxf(p.a, p.b); }
    if (N >= 64) { Pair p = swap32(x); x = fmaxf(p.a, p.b); }
    return x;
}

// Max of |x| over aligned groups of N lanes (N a power of two <= 64), as the unsigned max of
// the sign-cleared bit patterns: for non-negative floats the integer order is the float order,
// and the integer max needs no canonicalizing moves after a cross-lane exchange.  DPP within
// rows of 16 lanes, then the permlane swaps.  Result (>= 0) in every lane of the group.
template <int N>
__device__ __forceinline__ float group_max_abs(float x) {
    uint32_t u = __float_as_uint(x) & 0x7FFFFFFFu;
    auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
    auto dp = [](uint32_t v, auto ctrl) {
        return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), decltype(ctrl)::value, 0xF, 0xF, true));
    };
    if (N >= 2) u = mx(u, dp(u, std::integral_constant<int, kDppXor1>{}));
    if (N >= 4) u = mx(u, dp(u, std::integral_constant<int, kDppXor2>{}));
    if (N >= 8) u = mx(u, dp(u, std::integral_constant<int, kDppHalfMirror>{}));
    if (N >= 16) u = mx(u, dp(u, std::integral_constant<int, kDppMirror>{}));
    if (N >= 32) {
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        u = mx(r[0], r[1]);
    }
    if (N >= 64) {
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        u = mx(r[0], r[1]);
    }
    return __uint_as_float(u);
}

// Sum over aligned groups of N lanes; result in every lane.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    if (N >= 2) x = x + dpp<kDppXor1>(x);
    if (N >= 4) x = x + dpp<kDppXor2>(x);
    if (N >= 8) x = x + dpp<kDppHalfMirror>(x);
    if (N >= 16) x = x + dpp<kDppMirror>(x);
    if (N >= 32) { Pair p = swap16(x); x = p.a + p.b; }
    if (N >= 64) { Pair p = swap32(x); x = p.a + p.b; }
    return x;
}

__device__ __forceinline__ float wave_sum(float x) { return group_sum<kWave>(x); }

// Sum over the four lanes {i, i^16, i^32, i^48}: the same position in each row of 16.
__device__ __forceinline__ float rows_sum(float x) {
    Pair p = swap16(x);
    x = p.a + p.b;
    p = swap32(x);
    return p.a + p.b;
}

// General lane exchange (LDS crossbar), for patterns the above do not cover.
__device__ __forceinline__ float xor_shfl(float x, int mask) { return __shfl_xor(x, mask, kWave); }

// ------------------------------------------------------------------ correctly rounded quotient
// x / s rounded to nearest even, given y = RN(1/s) (Markstein, "Computation of elementary
// functions on the IBM RISC System/6000 processor", IBM J. Res. Dev. 34(1), 1990): with y
// within half an ulp of 1/s, one residual correction brings q = RN(x y) within one ulp of
// x/s, and a second residual correction r = x - s q (exact by FMA) gives q + r y = RN(x/s).
// Valid when no intermediate underflows or overflows: callers use it for |x/s| <= 2^8 and
// s >= 2^-100 and fall back to the division otherwise.  The sign of a zero quotient is
// restored from x.
__device__ __forceinline__ float quot_rn(float x, float s, float y) {
    float q = x * y;
    float r = __builtin_fmaf(-s, q, x);
    q = __builtin_fmaf(r, y, q);
    r = __builtin_fmaf(-s, q, x);
    q = __builtin_fmaf(r, y, q);
    return copysignf(q, x);
}

// ------------------------------------------------------------------ INT8 group codec
// s = amax/127 (1 when amax == 0); code = clamp(rne(x / s), -127, 127).  x / s is the
// IEEE correctly rounded quotient (HIP's default float division).
__device__ __forceinline__ float int8_scale(float amax) { return amax > 0.0f ? amax / 127.0f : 1.0f; }

__device__ __forceinline__ float int8_code(float x, float s) {
    float r = rintf(x / s);
    return fminf(fmaxf(r, -127.0f), 127.0f);
}

// Same code from a precomputed y = RN(1/s) (see quot_rn; requires s >= 2^-100).
__device__ __forceinline__ float int8_code_y(float x, float s, float y) {
    float r = rintf(quot_rn(x, s, y));
    return fminf(fmaxf(r, -127.0f), 127.0f);
}

constexpr float kFastQuotMinScale = 0x1p-100f;      // INT8: decisions need |x/s| >= 1/2

// s = amax/127 (1 when amax == 0) and y = RN(1/s) without a division, both equal to the IEEE
// quotients for s >= 2^-100:
//  * s: RN(amax * c), c = RN(1/127), then one residual correction r = amax - 127 q (exact by
//    FMA), s = RN(q + r c) -- checked exhaustively against amax / 127 over all significands
//    in ten binades from 2^-95 to 2^100 (the map commutes with scaling by powers of two there);
//  * y: the hardware reciprocal refined by one Newton step, fma(fma(-s, r, 1), r, r) --
//    checked exhaustively against 1 / s on gfx950 in twelve binades from 2^-100 to 2^99.
// Returns false (and the IEEE s) when s < 2^-100; callers then use the division per element.
__device__ __forceinline__ bool int8_scale_recip(float amax, float& s, float& y) {
    constexpr float c127 = 1.0f / 127.0f;
    const float q0 = amax * c127;
    s = __builtin_fmaf(__builtin_fmaf(-127.0f, q0, amax), c127, q0);
    s = amax > 0.0f ? s : 1.0f;
    const bool fast = s >= kFastQuotMinScale;
    if (!fast) s = int8_scale(amax);
    const float r = __builtin_amdgcn_rcpf(s);
    y = __builtin_fmaf(__builtin_fmaf(-s, r, 1.0f), r, r);
    return fast;
}

// INT8 code of x for a scale s >= 2^-100 with y = RN(1/s): rint of the correctly rounded
// quotient x / s (quot_rn without the sign restore, which only decides the sign of an exactly
// zero quotient).  No clamp: with |x| <= amax and s = RN(amax/127), |x/s| <= 127 (1 + 2^-24),
// which rounds to at most 127.
__device__ __forceinline__ float int8_code_fast(float x, float s, float y) {
    float q = x * y;
    q = __builtin_fmaf(__builtin_fmaf(-s, q, x), y, q);
    q = __builtin_fmaf(__builtin_fmaf(-s, q, x), y, q);
    return rintf(q);
}

constexpr float kFastQuotMinScaleE4M3 = 0x1p-80f;   // E4M3: decisions down to |x/s| ~ 2^-10

// ------------------------------------------------------------------ E4M3FN codec
// Nearest OCP E4M3FN value to y (ties to even, saturating at +-448).  For |y| in the binade
// [2^e, 2^(e+1)) with e >= -6 the grid step is 2^(e-3); below 2^-6 (subnormals) the step is
// 2^-9.  Scaling by an exact power of two, rint (ties to even) and scaling back rounds onto
// that grid exactly; a carry into the next binade lands on a representable value.
__device__ __forceinline__ float e4m3_round(float y) {
    uint32_t ebits = (__float_as_uint(y) >> 23) & 0xFFu;  // biased exponent of |y|
    int e = static_cast<int>(ebits) - 127;
    e = e < -6 ? -6 : e;
    float up = __uint_as_float(static_cast<uint32_t>(127 + 3 - e) << 23);    // 2^(3-e)
    float down = __uint_as_float(static_cast<uint32_t>(127 - 3 + e) << 23);  // 2^(e-3)
    float r = rintf(y * up) * down;
    return fminf(fmaxf(r, -448.0f), 448.0f);
}

// e4m3_round of two values with the gfx950 conversion instructions (OCP E4M3FN, round to
// nearest even).  Inputs are clamped to +-448 first, where the conversion saturates the same
// way e4m3_round does; for every |y| <= 448 the two agree bit for bit.
__device__ __forceinline__ void e4m3_round2(float& a, float& b) {
    const float ya = fminf(fmaxf(a, -448.0f), 448.0f);
    const float yb = fminf(fmaxf(b, -448.0f), 448.0f);
    const int p = __builtin_amdgcn_cvt_pk_fp8_f32(ya, yb, 0, false);
    a = __builtin_amdgcn_cvt_f32_fp8(p, 0);
    b = __builtin_amdgcn_cvt_f32_fp8(p, 1);
}

// E4M3 tile scale s = amax/448 (1 when amax == 0) and y = RN(1/s) without a division, both
// equal to the IEEE quotients for s >= 2^-80 (the fast-quotient domain of E4M3 decisions):
// s from RN(amax * c), c = RN(1/448), and one residual correction -- checked exhaustively
// against amax / 448 over all significands in ten binades from 2^-95 to 2^100; y as in
// int8_scale_recip.  Returns false (and the IEEE s) when s < 2^-80.
__device__ __forceinline__ bool e4m3_scale_recip(float amax, float& s, float& y) {
    constexpr float c448 = 1.0f / 448.0f;
    const float q0 = amax * c448;
    s = __builtin_fmaf(__builtin_fmaf(-448.0f, q0, amax), c448, q0);
    s = amax > 0.0f ? s : 1.0f;
    const bool fast = s >= kFastQuotMinScaleE4M3;
    if (!fast) s = amax > 0.0f ? amax / 448.0f : 1.0f;
    const float r = __builtin_amdgcn_rcpf(s);
    y = __builtin_fmaf(__builtin_fmaf(-s, r, 1.0f), r, r);
    return fast;
}

// x / s correctly rounded from y = RN(1/s) (quot_rn without the sign restore, which only
// decides the sign of an exactly zero quotient; valid for s >= 2^-100).
__device__ __forceinline__ float quot_rn_fast(float x, float s, float y) {
    float q = x * y;
    q = __builtin_fmaf(__builtin_fmaf(-s, q, x), y, q);
    return __builtin_fmaf(__builtin_fmaf(-s, q, x), y, q);
}

// Max of |x| over the 64 lanes of the wave; result (>= 0) in every lane.
__device__ __forceinline__ float wave_max_abs(float x) { return group_max_abs<64>(x); }

// Bit pattern of an E4M3FN grid value v (|v| <= 448, v on the grid).
__device__ __forceinline__ uint8_t e4m3_bits(float v) {
    uint32_t u = __float_as_uint(v);
    uint32_t sign = (u >> 31) << 7;
    float a = fabsf(v);
    if (a < 0.015625f) {  // subnormal or zero: m * 2^-9
        return static_cast<uint8_t>(sign | static_cast<uint32_t>(a * 512.0f));
    }
    uint32_t au = __float_as_uint(a);
    uint32_t e = ((au >> 23) & 0xFFu) - 127u + 7u;
    uint32_t m = (au >> 20) & 7u;
    return static_cast<uint8_t>(sign | (e << 3) | m);
}

}  // namespace la
