// Wavefront-level helpers shared by the gfx950 line-scan kernels that keep a
// line in registers: lane shifts for the three-tap neighbourhood, buffer-
// resource window loads and bf16 window decoding.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gspn {
namespace lane {

constexpr float kNegLog2e = -1.4426950408889634f;
constexpr int kBufFlags = 0x00020000;  // raw buffer, 32-bit dwords

// Wave-wide lane shifts: lane l receives lane l - 1 (from_prev) or l + 1
// (from_next); lanes 0 and 63 receive 0.
__device__ __forceinline__ float from_prev(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x138, 0xf, 0xf, true));
}
__device__ __forceinline__ float from_next(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x130, 0xf, 0xf, true));
}

// The middle one of three unsigned values, as one v_med3_u32 (clamping a
// look-ahead offset to a plane's first and last lines).
__device__ __forceinline__ uint32_t umed3(uint32_t a, uint32_t b, uint32_t c) {
    uint32_t r;
    asm("v_med3_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// NW (1..4) consecutive dwords as one value, so that a prefetched window
// stays one register tuple from its load to its use.
template <int NW> struct Words { using type = uint32_t __attribute__((ext_vector_type(NW))); };
template <> struct Words<1> { using type = uint32_t; };
template <int NW> using words_t = typename Words<NW>::type;

// NW consecutive dwords at byte offset `off` of a buffer.
template <int NW>
__device__ __forceinline__ words_t<NW> load_words(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    static_assert(NW >= 1 && NW <= 4, "one load per window");
    if constexpr (NW == 1) return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    else if constexpr (NW == 2) return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    else if constexpr (NW == 3) return __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, 0);
    else return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// The same at byte offset `off` + `soff` (soff uniform: a scalar offset).
template <int NW>
__device__ __forceinline__ words_t<NW> load_words_so(__amdgpu_buffer_rsrc_t r, uint32_t off, int soff) {
    static_assert(NW >= 1 && NW <= 4, "one load per window");
    if constexpr (NW == 1) return __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0);
    else if constexpr (NW == 2) return __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, 0);
    else if constexpr (NW == 3) return __builtin_amdgcn_raw_buffer_load_b96(r, off, soff, 0);
    else return __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0);
}

template <int NW>
__device__ __forceinline__ uint32_t word(const words_t<NW>& w, int i) {
    if constexpr (NW == 1) return w;
    else return w[i];
}

// Dwords covering K consecutive elements starting at an element of parity
// `par` (bf16: the window starts at the even element below).
template <typename T, int K>
constexpr int window_words() {
    return sizeof(T) == 4 ? K : ((K % 2) ? (K + 1) / 2 : K / 2);
}

// Element j of a lane's window as fp32.
template <typename T, int K, int NW>
__device__ __forceinline__ float window_elem(const words_t<NW>& w, int j, uint32_t sel_even,
                                             uint32_t sel_odd) {
    if constexpr (sizeof(T) == 4) {
        return __uint_as_float(word<NW>(w, j));
    } else {
        const int a = j >> 1;
        const uint32_t lo = word<NW>(w, a);
        const uint32_t hi = (a + 1 < NW) ? word<NW>(w, a + 1) : lo;
        return __uint_as_float(__builtin_amdgcn_perm(hi, lo, (j & 1) ? sel_odd : sel_even));
    }
}

// v_perm selectors for a bf16 window element that ignore the memory: 0xff000000
// (-2^127, a logit whose sigmoid is exactly 0) and 0 (a value that adds
// nothing).
constexpr uint32_t kSelDropped = 0x0d0c0c0cu;
constexpr uint32_t kSelZero = 0x0c0c0c0cu;

// Two floats to packed bf16 (low, high), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

}  // namespace lane
}  // namespace gspn
