// Helpers of the matrix-core kernels (block forward and block backward): vector types, the
// state layout of a 16-column wave, and the exact three-part bf16 split of fp32 values.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

constexpr int kBlk = 16;  // tokens per block
// LDS row of one token's 128 keys, in bf16 elements: 320 bytes, so that the transposed reads of
// the update (four tokens 320 bytes apart, four 16-byte row offsets) hit distinct banks
constexpr int kKeyRow = 160;

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef short s4 __attribute__((ext_vector_type(4)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s4 lds_s4;

// x = hi + lo + lo2 exactly, each part a bf16 (nearest at each step): the residual of rounding
// an fp32 value to bf16 is exact in fp32 and has at most 16 significant bits, the residual of
// that at most 8, which bf16 holds exactly.  Products of exact bf16 inputs with the parts are
// exact in fp32, so an MFMA over the three parts forms fp32 products (summed in fp32).
// Two values at a time: one packed conversion per part, whose halves widen back by a shift
// and a mask (11 operations per pair).
__device__ __forceinline__ void split3_pair(float x0, float x1, uint32_t& hi, uint32_t& lo, uint32_t& lo2) {
    hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{x0, x1}, bf2));
    const float r0 = x0 - __uint_as_float(hi << 16), r1 = x1 - __uint_as_float(hi & 0xFFFF0000u);
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{r0, r1}, bf2));
    const float q0 = r0 - __uint_as_float(lo << 16), q1 = r1 - __uint_as_float(lo & 0xFFFF0000u);
    lo2 = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{q0, q1}, bf2));
}
template <int N, typename FV, typename BV>
__device__ __forceinline__ void split3(const FV& x, BV& hi, BV& lo, BV& lo2) {
    typedef uint32_t uv __attribute__((ext_vector_type(N / 2)));
    uv h, l, l2;
#pragma unroll
    for (int i = 0; i < N / 2; i++) {
        uint32_t a, b, c;
        split3_pair(x[2 * i], x[2 * i + 1], a, b, c);
        h[i] = a;
        l[i] = b;
        l2[i] = c;
    }
    hi = __builtin_bit_cast(BV, h);
    lo = __builtin_bit_cast(BV, l);
    lo2 = __builtin_bit_cast(BV, l2);
}

// Key row held in s[m] by lane group g of a 16-column wave (lane 16 g + c holds column c):
// rows 32 (m / 8) + 8 g + m % 8, so that slice i = s[8 i .. 8 i + 7] pairs with the lane's
// 16-byte load i of a token's keys (the four lane groups together one 64-byte line).
__device__ __forceinline__ int state_row(int m, int g) { return 32 * (m >> 3) + 8 * g + (m & 7); }

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }

// Offset (bf16 elements) of the gfx950 transposed LDS read that gives lane (g, c) the A
// operand of accumulator tile tau in the rank-16 update: within each group of 16 lanes, slot j
// of lane i is element i % 4 of the 8 bytes addressed by lane 4 j + i / 4.  The rows lanes
// 4 a .. 4 a + 3 need are consecutive (32 (tau / 2) + 8 a + 4 (tau % 2) + b), so lane s of
// group g addresses token 4 g + s / 4 at the first of lane group s % 4's rows, and slot j of
// lane c receives token 4 g + j at row(c).
__device__ __forceinline__ int tr_offset(int g, int c, int tau) {
    return (4 * g + (c >> 2)) * kKeyRow + 32 * (tau >> 1) + 8 * (c & 3) + 4 * (tau & 1);
}

}  // namespace la
