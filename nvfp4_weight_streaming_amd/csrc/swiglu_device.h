// SwiGLU arithmetic shared by the SwiGLU kernel and the gate_up epilogue that
// computes it in place of that kernel: h = silu(g) * up in fp64 from bf16
// inputs, rounded once to bf16 (the reading of the layer's non-GEMM step is
// described in swiglu.hip).
#pragma once

#include "common.h"

namespace nvfp4 {

// fp64 -> bf16 bits, rounded once to nearest, ties to even.  Overflow goes to
// infinity; NaN becomes the quiet NaN 0x7FC0 with the input's sign.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
    const unsigned long long b = (unsigned long long)__double_as_longlong(x);
    const uint16_t sign = (uint16_t)((b >> 63) << 15);
    const unsigned long long ax = b & 0x7FFFFFFFFFFFFFFFull;
    if (ax > 0x7FF0000000000000ull) return sign | 0x7FC0;  // NaN
    if (ax == 0x7FF0000000000000ull) return sign | 0x7F80;  // infinity
    if (ax == 0) return sign;
    int e = (int)(ax >> 52) - 1023;  // unbiased exponent (normal inputs)
    unsigned long long m = (ax & 0xFFFFFFFFFFFFFull) | (1ull << 52);
    if ((ax >> 52) == 0) return sign;  // fp64 subnormal: far below bf16's range
    // bf16 keeps 8 significant bits for e >= -126 (shift 45); below, the
    // subnormal grid of 2^-133 (shift 45 + (-126 - e)).
    const int shift = e >= -126 ? 45 : 45 + (-126 - e);
    if (shift >= 64) return sign;  // below half the smallest subnormal
    unsigned long long q = m >> shift;
    const unsigned long long rem = m & ((1ull << shift) - 1ull);
    const unsigned long long half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (q & 1ull))) ++q;
    if (e >= -126) {
        if (q == 256) {  // carried into the next binade
            q = 128;
            ++e;
        }
        if (e > 127) return sign | 0x7F80;
        return sign | (uint16_t)(((e + 127) << 7) | (int)(q & 127ull));
    }
    return sign | (uint16_t)q;  // subnormal, or 0x0080 after a carry: 2^-126
}

__device__ __forceinline__ double bf16_to_f64(uint16_t h) {
    return (double)__uint_as_float((unsigned int)h << 16);
}

// h = silu(g) * u = g u / (1 + e^-g), fp64 from the bf16 bits, one rounding.
__device__ __forceinline__ uint16_t swiglu_bf16(uint16_t g_bits, uint16_t u_bits) {
    const double g = bf16_to_f64(g_bits);
    const double u = bf16_to_f64(u_bits);
    return f64_to_bf16_rne(g * u / (1.0 + exp(-g)));
}

}  // namespace nvfp4
