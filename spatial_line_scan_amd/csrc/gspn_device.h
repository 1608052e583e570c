// Device helpers shared by the gfx950 kernels of libgspn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gspn {

// ------------------------------------------------------------ element access

__device__ __forceinline__ float load_elem(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float load_elem(const uint16_t* p, size_t i) {
    return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ void store_elem(float* p, size_t i, float v) { p[i] = v; }
__device__ __forceinline__ void store_elem(uint16_t* p, size_t i, float v) { p[i] = bf16_rne(v); }

// ------------------------------------------------------------ normalisation

// Logistic sigmoid from the hardware base-2 exponential and reciprocal:
// sigmoid(z) = 1 / (1 + 2^(-z log2 e)).  A very negative z makes the
// exponential +inf and the reciprocal exactly 0.
__device__ __forceinline__ float sigmoid_hw(float z) {
    const float e = __builtin_amdgcn_exp2f(z * -1.4426950408889634f);
    return __builtin_amdgcn_rcpf(1.0f + e);
}

// Row-stochastic three-tap weights of one destination position: taps whose
// source lies off the line get 0, the sum is clamped below by eps.
__device__ __forceinline__ void normalize3(float z0, float z1, float z2, bool has_left,
                                           bool has_right, float eps, float& w0, float& w1,
                                           float& w2) {
    const float s0 = has_left ? sigmoid_hw(z0) : 0.0f;
    const float s1 = sigmoid_hw(z1);
    const float s2 = has_right ? sigmoid_hw(z2) : 0.0f;
    const float r = __builtin_amdgcn_rcpf(fmaxf((s0 + s1) + s2, eps));
    w0 = s0 * r;
    w1 = s1 * r;
    w2 = s2 * r;
}

}  // namespace gspn
