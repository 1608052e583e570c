// One-direction scan (gspn_scan_dir) for planes whose lambda x fits in LDS as
// fp32 (gfx950): one wavefront per (b, c) plane.
//
// Operator: "Scaling Parallel Sequence Models to Foundation-Scale Vision
// Encoders", §3 line-scan recurrence (standard GSPN form) and §4.3
// stream-based concurrency (directions run as separate passes); reading
// notes, method / overall framework (the top-down scan and the fused
// normalisation: sigmoid, local sum, clamp, divide).
//
// Work split.  The wavefront walks the NL lines of its direction in scan
// order; lane q holds positions Kq .. Kq+K-1 of the current line (K = 1..4
// for lines up to 64, 128, 192, 256) and the three-tap neighbour exchange is
// one whole-wavefront DPP shift each way (lanes 0 and 63 receive 0, which
// only dropped taps weigh).
//
// On-chip data: one fp32 plane in LDS.  A prologue fills it with b = lambda x
// from coalesced loads of x and lambda (row-major, whatever the direction);
// each step reads b of its line's pixels one step ahead and writes h in its
// place (b of a pixel is read once, at the step that updates it).  The
// epilogue writes y = u h, or adds u h to y, again row-major.  So x, lambda,
// u and y are never gathered along a column; the taps (line-major for every
// direction) stream one element a slot, 8 lines ahead.
//
// Taps: raw logits are normalised in registers (sigmoid; taps whose source
// lies outside the line dropped; sum clamped below by eps; divide);
// normalised taps are used as given, those outside the line weighing 0
// whatever their value.  Slots past a line's end read and write a dummy LDS
// word and weigh nothing.
#include "gspn_device.h"
#include "gspn_internal.h"
#include "gspn_lane.h"

#include <type_traits>

namespace gspn {
namespace {

using namespace lane;

constexpr int kPad = 16;   // bytes: the dummy word (and alignment) before the plane

template <typename V> using lds_t = __attribute__((address_space(3))) V;

template <typename V>
__device__ __forceinline__ lds_t<V>& lds_ref(uint32_t byte_off) {
    // the kernel's only LDS is its dynamic array, which starts at address 0
    return *reinterpret_cast<lds_t<V>*>(static_cast<uintptr_t>(byte_off));
}

__device__ __forceinline__ void lds_order() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
}

// Raw bits of one tap element and their fp32 value.  The bits keep the
// storage width, so that widening happens where they are used, not where
// they are loaded.
template <typename T> using tap_bits_t = std::conditional_t<sizeof(T) == 4, uint32_t, uint16_t>;
template <typename T>
__device__ __forceinline__ tap_bits_t<T> load_tap_bits(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
    if constexpr (sizeof(T) == 4) return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
    else return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}
template <typename T>
__device__ __forceinline__ float tap_value(tap_bits_t<T> bits) {
    if constexpr (sizeof(T) == 4) return __uint_as_float(bits);
    else return __uint_as_float(static_cast<uint32_t>(bits) << 16);
}

// ------------------------------------------------ whole-plane vector I/O
// V consecutive elements at element e (a multiple of V) of a plane's buffer,
// as fp32; past the buffer's end they read 0 (the buffer's range check).
template <typename T, int V>
__device__ __forceinline__ void load_vec(__amdgpu_buffer_rsrc_t r, int e, float (&v)[V]) {
    constexpr int NB = V * static_cast<int>(sizeof(T));
    const uint32_t off = static_cast<uint32_t>(e) * sizeof(T);
    if constexpr (NB == 2) {
        v[0] = __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0)) << 16);
    } else {
        const words_t<NB / 4> wv = load_words<NB / 4>(r, off);
#pragma unroll
        for (int i = 0; i < NB / 4; ++i) {
            const uint32_t wd = word<NB / 4>(wv, i);
            if constexpr (sizeof(T) == 4) {
                v[i] = __uint_as_float(wd);
            } else {
                v[2 * i] = __uint_as_float(wd << 16);
                v[2 * i + 1] = __uint_as_float(wd & 0xffff0000u);
            }
        }
    }
}

// Stores V fp32 values as T at element e; stores past the end are dropped.
template <typename T, int V>
__device__ __forceinline__ void store_vec(__amdgpu_buffer_rsrc_t r, int e, const float (&v)[V]) {
    constexpr int NB = V * static_cast<int>(sizeof(T));
    const uint32_t off = static_cast<uint32_t>(e) * sizeof(T);
    if constexpr (NB == 2) {
        __builtin_amdgcn_raw_buffer_store_b16(bf16_rne(v[0]), r, off, 0, 0);
    } else {
        uint32_t wd[NB / 4];
#pragma unroll
        for (int i = 0; i < NB / 4; ++i)
            wd[i] = sizeof(T) == 4 ? __float_as_uint(v[i])
                                   : static_cast<uint32_t>(bf16_rne(v[2 * i])) |
                                         (static_cast<uint32_t>(bf16_rne(v[2 * i + 1])) << 16);
        if constexpr (NB == 4) {
            __builtin_amdgcn_raw_buffer_store_b32(wd[0], r, off, 0, 0);
        } else if constexpr (NB == 8) {
            const words_t<2> q = {wd[0], wd[1]};
            __builtin_amdgcn_raw_buffer_store_b64(q, r, off, 0, 0);
        } else {
            const words_t<4> q = {wd[0], wd[1], wd[2], wd[3]};
            __builtin_amdgcn_raw_buffer_store_b128(q, r, off, 0, 0);
        }
    }
}

// b = lambda x of the whole plane into LDS (fp32 at byte kPad + 4 e), V
// elements a lane and U vectors a lane in flight.
template <typename T, int V>
__device__ __forceinline__ void fill_b(__amdgpu_buffer_rsrc_t xr, __amdgpu_buffer_rsrc_t lr, int HW) {
    constexpr int U = 8;
    const int lane = threadIdx.x;
    for (int e0 = V * lane; e0 < HW; e0 += 64 * V * U) {
        float xv[U][V], lv[U][V];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            load_vec<T, V>(xr, e0 + 64 * V * k, xv[k]);
            load_vec<T, V>(lr, e0 + 64 * V * k, lv[k]);
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int e = e0 + 64 * V * k;
            if (e < HW) {
#pragma unroll
                for (int i = 0; i < V; ++i) lds_ref<float>(kPad + 4u * (e + i)) = lv[k][i] * xv[k][i];
            }
        }
    }
}

// y = u h (or y += u h) of the whole plane, h from LDS.
template <typename T, int V>
__device__ __forceinline__ void emit_y(__amdgpu_buffer_rsrc_t ur, __amdgpu_buffer_rsrc_t yr, int HW,
                                       bool accumulate) {
    constexpr int U = 8;
    const int lane = threadIdx.x;
    for (int e0 = V * lane; e0 < HW; e0 += 64 * V * U) {
        float uv[U][V], yv[U][V];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            load_vec<T, V>(ur, e0 + 64 * V * k, uv[k]);
            if (accumulate) {
                load_vec<T, V>(yr, e0 + 64 * V * k, yv[k]);
            } else {
#pragma unroll
                for (int i = 0; i < V; ++i) yv[k][i] = 0.0f;
            }
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int e = e0 + 64 * V * k;
            if (e < HW) {
                float o[V];
#pragma unroll
                for (int i = 0; i < V; ++i) {
                    const float t = uv[k][i] * lds_ref<float>(kPad + 4u * (e + i));
                    o[i] = accumulate ? yv[k][i] + t : t;
                }
                store_vec<T, V>(yr, e, o);
            }
        }
    }
}

// T: float or bf16 bits (uint16_t).  K: positions a lane.  D: lines of taps
// in flight.  RAW: taps are logits to normalise.
template <typename T, int K, int D, bool RAW>
__global__ void __launch_bounds__(64)
scan_dir_fast_kernel(const T* __restrict__ x, const T* __restrict__ lam, const T* __restrict__ u,
                     const T* __restrict__ w, float eps, T* __restrict__ y, int accumulate,
                     int H, int W, int dir, int vec) {
    const int lane = threadIdx.x;
    const int HW = H * W;
    const size_t plane = blockIdx.x;
    const size_t pix0 = plane * static_cast<size_t>(HW);
    const bool rows = dir < 2;
    const bool fwd = (dir & 1) == 0;
    const int NL = rows ? H : W;
    const int L = rows ? W : H;

    // ------------------------------------------------ b = lambda x into LDS
    // vec: elements a lane moves at once in the whole-plane passes (every
    // plane's x, lambda, u and y start on a multiple of vec elements)
    const int pbytes = HW * static_cast<int>(sizeof(T));
    auto plane_rsrc = [&](const T* base) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(base + pix0), 0, pbytes, kBufFlags);
    };
    if (lane == 0) lds_ref<float>(0) = 0.0f;
    {
        const __amdgpu_buffer_rsrc_t xr = plane_rsrc(x), lr = plane_rsrc(lam);
        if (vec == 1) fill_b<T, 1>(xr, lr, HW);
        else if (vec == 2) fill_b<T, 2>(xr, lr, HW);
        else if (sizeof(T) == 4 || vec == 4) fill_b<T, 4>(xr, lr, HW);
        else fill_b<T, 16 / sizeof(T)>(xr, lr, HW);
    }
    lds_order();

    // ------------------------------------------------ taps: first D lines
    // slot j of lane q: position p = Kq + j of the line; tap k of (line i,
    // position p) at element (k NL + i) L + p of the plane's taps.  Loads
    // keep the raw bits (converted where used, D steps later, so that no
    // instruction waits on a load in the step that issues it); a slot past
    // the line's end reads the line's last element and weighs nothing.
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T*>(w + plane * 3 * static_cast<size_t>(HW)), 0,
        static_cast<int>(3 * HW * sizeof(T)), kBufFlags);
    uint32_t voff[K];
    bool valid[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const int p = K * lane + j;
        valid[j] = p < L;
        voff[j] = static_cast<uint32_t>((valid[j] ? p : L - 1) * static_cast<int>(sizeof(T)));
    }
    tap_bits_t<T> tap[D][3][K];
    const int line = fwd ? 0 : NL - 1;
    const int dline = fwd ? 1 : -1;
    auto load_line = [&](int d, int ln) {
        // a line past the scan's end repeats its last line (in bounds; unused)
        const int lc = ln < 0 ? 0 : (ln >= NL ? NL - 1 : ln);
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const int so = (k * NL + lc) * L * static_cast<int>(sizeof(T));
#pragma unroll
            for (int j = 0; j < K; ++j) tap[d][k][j] = load_tap_bits<T>(wr, voff[j], so);
        }
    };
#pragma unroll
    for (int d = 0; d < D; ++d) load_line(d, line + d * dline);

    // per slot: LDS address of its pixel on the current line and its change
    // a step (slots past the line's end stay on the dummy word)
    uint32_t aS[K];
    int dS[K];
    float keep[3][K];   // 1 where a tap's source is in the line, else 0
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const int p = K * lane + j;
        const int e = rows ? line * W + p : p * W + line;
        aS[j] = valid[j] ? static_cast<uint32_t>(kPad + 4 * e) : 0u;
        dS[j] = valid[j] ? 4 * (rows ? dline * W : dline) : 0;
        keep[0][j] = (valid[j] && p > 0) ? 1.0f : 0.0f;
        keep[1][j] = valid[j] ? 1.0f : 0.0f;
        keep[2][j] = (valid[j] && p < L - 1) ? 1.0f : 0.0f;
    }
    float h[K], bv[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        h[j] = 0.0f;
        bv[j] = lds_ref<float>(aS[j]);
    }

    auto step = [&](int s, int d) {
        float w0[K], w1[K], w2[K];
        if constexpr (RAW) {
            float r[K];
#pragma unroll
            for (int j = 0; j < K; ++j) {
                // a dropped tap's sigmoid is 0: exp2 of +inf
                const float z0 = keep[0][j] != 0.0f ? tap_value<T>(tap[d][0][j]) * kNegLog2e : __builtin_inff();
                const float z1 = keep[1][j] != 0.0f ? tap_value<T>(tap[d][1][j]) * kNegLog2e : __builtin_inff();
                const float z2 = keep[2][j] != 0.0f ? tap_value<T>(tap[d][2][j]) * kNegLog2e : __builtin_inff();
                w0[j] = __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(z0) + 1.0f);
                w1[j] = __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(z1) + 1.0f);
                w2[j] = __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(z2) + 1.0f);
                r[j] = __builtin_amdgcn_rcpf(fmaxf((w0[j] + w1[j]) + w2[j], eps));
            }
#pragma unroll
            for (int j = 0; j < K; ++j) {
                w0[j] *= r[j];
                w1[j] *= r[j];
                w2[j] *= r[j];
            }
        } else {
            // given weights; out-of-line taps weigh 0 whatever their value
#pragma unroll
            for (int j = 0; j < K; ++j) {
                w0[j] = keep[0][j] != 0.0f ? tap_value<T>(tap[d][0][j]) : 0.0f;
                w1[j] = keep[1][j] != 0.0f ? tap_value<T>(tap[d][1][j]) : 0.0f;
                w2[j] = keep[2][j] != 0.0f ? tap_value<T>(tap[d][2][j]) : 0.0f;
            }
        }
        // refill slot d with the line D steps on, once it has been read
        load_line(d, line + (s + D) * dline);

        const float hl0 = from_prev(h[K - 1]);
        const float hrK = from_next(h[0]);
        float hn[K];
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const float hl = j > 0 ? h[j - 1] : hl0;
            const float hr = j < K - 1 ? h[j + 1] : hrK;
            // the first line has no line before it: h = lambda x
            hn[j] = s == 0 ? bv[j] : fmaf(w2[j], hr, fmaf(w0[j], hl, fmaf(w1[j], h[j], bv[j])));
            // slots past the line's end hold 0
            hn[j] = valid[j] ? hn[j] : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < K; ++j) {
            h[j] = hn[j];
            lds_ref<float>(aS[j]) = hn[j];
            aS[j] += dS[j];
            bv[j] = lds_ref<float>(aS[j]);   // the next line's b (read after this write)
        }
    };

    int s0 = 0;
    for (; s0 + D <= NL; s0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) step(s0 + d, d);
    }
#pragma unroll
    for (int d = 0; d < D; ++d)
        if (s0 + d < NL) step(s0 + d, d);
    lds_order();

    // ------------------------------------------------ y = u h (or y += u h)
    {
        const __amdgpu_buffer_rsrc_t ur = plane_rsrc(u), yr = plane_rsrc(y);
        const bool acc = accumulate != 0;
        if (vec == 1) emit_y<T, 1>(ur, yr, HW, acc);
        else if (vec == 2) emit_y<T, 2>(ur, yr, HW, acc);
        else if (sizeof(T) == 4 || vec == 4) emit_y<T, 4>(ur, yr, HW, acc);
        else emit_y<T, 16 / sizeof(T)>(ur, yr, HW, acc);
    }
}

template <typename T, int K, bool RAW>
hipError_t launch_tk(const void* x, const void* lam, const void* u, const void* w, float eps,
                     void* y, int accumulate, int64_t planes, int64_t H, int64_t W, int dir,
                     hipStream_t stream) {
    // loads in flight (3 K D) stay within the 63 the wave's counter tracks
    constexpr int D = K <= 2 ? 8 : (K == 3 ? 6 : 5);
    const size_t lds = kPad + 4 * static_cast<size_t>(H * W);
    auto kern = scan_dir_fast_kernel<T, K, D, RAW>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(lds));
        if (e != hipSuccess) return e;
    }
    // widest vector (up to 16 bytes) that divides the plane and on which every
    // plane of x, lambda, u and y starts
    int vec = 16 / static_cast<int>(sizeof(T));
    const uintptr_t any = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(lam) |
                          reinterpret_cast<uintptr_t>(u) | reinterpret_cast<uintptr_t>(y);
    while (vec > 1 && ((H * W) % vec != 0 || any % (vec * sizeof(T)) != 0)) vec /= 2;
    kern<<<dim3(static_cast<unsigned>(planes)), dim3(64), lds, stream>>>(
        static_cast<const T*>(x), static_cast<const T*>(lam), static_cast<const T*>(u),
        static_cast<const T*>(w), eps, static_cast<T*>(y), accumulate, static_cast<int>(H),
        static_cast<int>(W), dir, vec);
    return hipGetLastError();
}

template <typename T, bool RAW>
hipError_t launch_t(const void* x, const void* lam, const void* u, const void* w, float eps,
                    void* y, int accumulate, int64_t planes, int64_t H, int64_t W, int dir,
                    hipStream_t stream) {
    const int64_t L = dir < 2 ? W : H;
    if (L <= 64) return launch_tk<T, 1, RAW>(x, lam, u, w, eps, y, accumulate, planes, H, W, dir, stream);
    if (L <= 128) return launch_tk<T, 2, RAW>(x, lam, u, w, eps, y, accumulate, planes, H, W, dir, stream);
    if (L <= 192) return launch_tk<T, 3, RAW>(x, lam, u, w, eps, y, accumulate, planes, H, W, dir, stream);
    return launch_tk<T, 4, RAW>(x, lam, u, w, eps, y, accumulate, planes, H, W, dir, stream);
}

}  // namespace

bool scan_dir_fast_eligible(int64_t H, int64_t W, int dir) {
    const int64_t L = dir < 2 ? W : H;
    if (L > 256) return false;
    return kPad + 4 * H * W <= kLdsBytes;
}

hipError_t launch_scan_dir_fast(const void* x, const void* lam, const void* u, const void* w,
                                int w_is_raw, float eps, void* y, int accumulate, int dtype,
                                int64_t planes, int64_t H, int64_t W, int dir, hipStream_t stream) {
    if (dtype == 0)
        return w_is_raw ? launch_t<float, true>(x, lam, u, w, eps, y, accumulate, planes, H, W, dir, stream)
                        : launch_t<float, false>(x, lam, u, w, eps, y, accumulate, planes, H, W, dir, stream);
    return w_is_raw ? launch_t<uint16_t, true>(x, lam, u, w, eps, y, accumulate, planes, H, W, dir, stream)
                    : launch_t<uint16_t, false>(x, lam, u, w, eps, y, accumulate, planes, H, W, dir, stream);
}

}  // namespace gspn
