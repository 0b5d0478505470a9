// Device helpers shared by the recurrence kernels: input widening, wave-level
// reductions and the two state codecs.  gfx950 (CDNA4), wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

__device__ __forceinline__ void store_elem(void* p, size_t idx, int dtype, float x) {
    if (dtype == 0) static_cast<float*>(p)[idx] = x;
    else static_cast<uint16_t*>(p)[idx] = f32_to_bf16_bits(x);
}

// ------------------------------------------------------------------ cross-lane
__device__ __forceinline__ float xor_shfl(float x, int mask) { return __shfl_xor(x, mask, kWave); }

// Max over aligned groups of `n` lanes (n a power of two <= 64); result in every lane.
template <int N>
__device__ __forceinline__ float group_max(float x) {
#pragma unroll
    for (int m = 1; m < N; m <<= 1) x = fmaxf(x, xor_shfl(x, m));
    return x;
}

// Sum over the whole wave with a fixed butterfly order; result in every lane.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) x += xor_shfl(x, m);
    return x;
}

// ------------------------------------------------------------------ INT8 group codec
// s = amax/127 (1 when amax == 0); code = clamp(rne(x / s), -127, 127).  x / s is the
// IEEE correctly rounded quotient (HIP's default float division).
__device__ __forceinline__ float int8_scale(float amax) { return amax > 0.0f ? amax / 127.0f : 1.0f; }

__device__ __forceinline__ float int8_code(float x, float s) {
    float r = rintf(x / s);
    return fminf(fmaxf(r, -127.0f), 127.0f);
}

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
