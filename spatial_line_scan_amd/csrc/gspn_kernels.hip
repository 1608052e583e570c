// gfx950 kernels of the GSPN line-scan propagation.
//
// Operator: "Scaling Parallel Sequence Models to Foundation-Scale Vision
// Encoders", §3 line-scan recurrence (standard GSPN form h_i = w_i h_{i-1} +
// lambda_i x_i, output u_i h_i), §4.1 single-kernel design (all line steps in
// one launch, hidden line kept on chip), §5.1 fused normalisation (sigmoid,
// local sum, clamp, divide); reading notes of the same paper, method /
// overall framework (three-tap tridiagonal neighbourhood, row-stochastic
// normalisation, four scan directions).
//
// This file holds the general kernels: one workgroup owns one (b, c) plane,
// its threads cover the positions of a line, and the hidden line lives in
// LDS between the steps of the scan.
#include "gspn_device.h"
#include "gspn_internal.h"

#include <algorithm>

namespace gspn {
namespace {

constexpr int kThreads = 256;

template <typename T>
__global__ void __launch_bounds__(kThreads)
normalize_kernel(const T* __restrict__ w_raw, T* __restrict__ w_norm, int64_t planes, int H,
                 int W, int dir0, int ndir, float eps) {
    const int64_t npix = static_cast<int64_t>(H) * W;
    const int64_t per_dir = planes * npix;
    const int64_t total = per_dir * ndir;
    for (int64_t idx = blockIdx.x * static_cast<int64_t>(kThreads) + threadIdx.x; idx < total;
         idx += static_cast<int64_t>(gridDim.x) * kThreads) {
        const int64_t dd = idx / per_dir;
        const int64_t rem = idx - dd * per_dir;
        const int64_t plane = rem / npix;
        const int64_t t = rem - plane * npix;  // offset inside [NL][L]
        const int dir = dir0 + static_cast<int>(dd);
        const int L = dir < 2 ? W : H;
        const int p = static_cast<int>(t % L);
        const size_t base = static_cast<size_t>((dd * planes + plane) * 3 * npix + t);
        float w0, w1, w2;
        normalize3(load_elem(w_raw, base), load_elem(w_raw, base + npix),
                   load_elem(w_raw, base + 2 * npix), p > 0, p < L - 1, eps, w0, w1, w2);
        store_elem(w_norm, base, w0);
        store_elem(w_norm, base + npix, w1);
        store_elem(w_norm, base + 2 * npix, w2);
    }
}

// ------------------------------------------------------------ one scan pass

// Scans direction `dir` of the plane whose inputs start at xp/lp/up/wp.  For
// every produced value h at pixel `pix`, calls sink(pix, h).  h_prev and
// h_next are LDS lines of at least L floats.  Ends with a barrier.
// The lines are scanned in segments of `seg` lines (seg = NL: one global
// scan); the first line of a segment in scan order is lambda x.
template <typename T, typename Sink>
__device__ __forceinline__ void scan_plane(const T* __restrict__ xp, const T* __restrict__ lp,
                                           const T* __restrict__ wp, bool w_is_raw, float eps,
                                           int H, int W, int dir, int seg, float* h_prev,
                                           float* h_next, Sink sink) {
    const bool rows = dir < 2;
    const int NL = rows ? H : W;
    const int L = rows ? W : H;
    const bool forward = (dir == 0 || dir == 2);
    const size_t npix = static_cast<size_t>(H) * W;
    for (int step = 0; step < NL; ++step) {
        const int i = forward ? step : NL - 1 - step;
        const bool restart = forward ? i % seg == 0 : (i == NL - 1 || (i + 1) % seg == 0);
        for (int p = threadIdx.x; p < L; p += kThreads) {
            const int r = rows ? i : p;
            const int c = rows ? p : i;
            const size_t pix = static_cast<size_t>(r) * W + c;
            const float bx = load_elem(lp, pix) * load_elem(xp, pix);
            float h = bx;
            if (!restart) {
                const size_t ti = static_cast<size_t>(i) * L + p;
                const bool has_left = p > 0;
                const bool has_right = p < L - 1;
                float w0 = load_elem(wp, ti);
                float w1 = load_elem(wp, ti + npix);
                float w2 = load_elem(wp, ti + 2 * npix);
                if (w_is_raw) normalize3(w0, w1, w2, has_left, has_right, eps, w0, w1, w2);
                float m = w1 * h_prev[p];
                if (has_left) m = fmaf(w0, h_prev[p - 1], m);
                if (has_right) m = fmaf(w2, h_prev[p + 1], m);
                h = m + bx;
            }
            h_next[p] = h;
            sink(pix, h);
        }
        __syncthreads();
        float* t = h_prev;
        h_prev = h_next;
        h_next = t;
    }
}

template <typename T>
__global__ void __launch_bounds__(kThreads)
scan_dir_kernel(const T* __restrict__ x, const T* __restrict__ lam, const T* __restrict__ u,
                const T* __restrict__ w, int w_is_raw, float eps, T* __restrict__ y,
                int accumulate, int H, int W, int dir) {
    extern __shared__ float lds[];
    const int L = dir < 2 ? W : H;
    const size_t npix = static_cast<size_t>(H) * W;
    const size_t plane = blockIdx.x;
    const T* up = u + plane * npix;
    T* yp = y + plane * npix;
    scan_plane(x + plane * npix, lam + plane * npix, w + plane * 3 * npix, w_is_raw != 0, eps, H,
               W, dir, dir < 2 ? H : W, lds, lds + L, [&](size_t pix, float h) {
                   float o = load_elem(up, pix) * h;
                   if (accumulate) o = load_elem(yp, pix) + o;
                   store_elem(yp, pix, o);
               });
}

// Four directions of one plane per workgroup.  The sum of the directional
// states is kept in `acc`: LDS when it fits, otherwise the fp32 output itself
// or, for bf16 output, the fp32 plane of `accg` (a workspace of one float per
// pixel-channel).
template <typename T, bool kAccInLds>
__global__ void __launch_bounds__(kThreads)
prop2d_plane_kernel(const T* __restrict__ x, const T* __restrict__ lam, const T* __restrict__ u,
                    const T* __restrict__ w4, float eps, T* __restrict__ y, int64_t planes, int H,
                    int W, int64_t cpg, int k_chunk, float* __restrict__ accg) {
    extern __shared__ float lds[];
    const int Lmax = H > W ? H : W;
    const size_t npix = static_cast<size_t>(H) * W;
    const size_t plane = blockIdx.x;
    float* acc;
    if constexpr (kAccInLds) {
        acc = lds + 2 * Lmax;
    } else if constexpr (sizeof(T) == sizeof(float)) {
        acc = reinterpret_cast<float*>(y + plane * npix);
    } else {
        acc = accg + plane * npix;
    }
    // tap plane of this plane: its channel group's
    const size_t tap_planes = static_cast<size_t>(planes / cpg);
    const size_t tplane = plane / static_cast<size_t>(cpg);
    const int seg_rows = (H + k_chunk - 1) / k_chunk;
    const int seg_cols = (W + k_chunk - 1) / k_chunk;
    for (int dir = 0; dir < 4; ++dir) {
        const T* wp = w4 + (static_cast<size_t>(dir) * tap_planes + tplane) * 3 * npix;
        const int seg = dir < 2 ? seg_rows : seg_cols;
        if (dir == 0) {
            scan_plane(x + plane * npix, lam + plane * npix, wp, true, eps, H, W, dir, seg, lds,
                       lds + Lmax, [&](size_t pix, float h) { acc[pix] = h; });
        } else {
            scan_plane(x + plane * npix, lam + plane * npix, wp, true, eps, H, W, dir, seg, lds,
                       lds + Lmax, [&](size_t pix, float h) { acc[pix] += h; });
        }
    }
    const T* up = u + plane * npix;
    T* yp = y + plane * npix;
    for (size_t pix = threadIdx.x; pix < npix; pix += kThreads)
        store_elem(yp, pix, load_elem(up, pix) * acc[pix]);
}

// Dynamic LDS above the default per-launch limit has to be opted into once
// per kernel.
template <typename K>
hipError_t allow_lds(K kernel, size_t bytes) {
    if (bytes <= 64 * 1024) return hipSuccess;
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize,
                               static_cast<int>(bytes));
}

template <typename T>
hipError_t normalize_t(const void* w_raw, void* w_norm, int64_t planes, int64_t H, int64_t W,
                       int dir0, int ndir, float eps, hipStream_t stream) {
    const int64_t total = planes * H * W * ndir;
    const int64_t blocks = std::min<int64_t>((total + kThreads - 1) / kThreads, 256 * 64);
    normalize_kernel<T><<<dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream>>>(
        static_cast<const T*>(w_raw), static_cast<T*>(w_norm), planes, static_cast<int>(H),
        static_cast<int>(W), dir0, ndir, eps);
    return hipGetLastError();
}

template <typename T>
hipError_t scan_dir_t(const void* x, const void* lam, const void* u, const void* w,
                      int w_is_raw, float eps, void* y, int accumulate, int64_t planes,
                      int64_t H, int64_t W, int dir, hipStream_t stream) {
    const int64_t L = dir < 2 ? W : H;
    const size_t lds = 2 * L * sizeof(float);
    hipError_t e = allow_lds(scan_dir_kernel<T>, lds);
    if (e != hipSuccess) return e;
    scan_dir_kernel<T><<<dim3(static_cast<unsigned>(planes)), dim3(kThreads), lds, stream>>>(
        static_cast<const T*>(x), static_cast<const T*>(lam), static_cast<const T*>(u),
        static_cast<const T*>(w), w_is_raw, eps, static_cast<T*>(y), accumulate,
        static_cast<int>(H), static_cast<int>(W), dir);
    return hipGetLastError();
}

size_t prop2d_lds_bytes(int64_t H, int64_t W) {
    return static_cast<size_t>(2 * std::max(H, W) + H * W) * sizeof(float);
}

template <typename T>
hipError_t prop2d_t(const void* x, const void* lam, const void* u, const void* w4, float eps,
                    void* y, int64_t planes, int64_t H, int64_t W, const PropOpts& o,
                    hipStream_t stream) {
    const size_t lds_acc = prop2d_lds_bytes(H, W);
    const bool in_lds = static_cast<int64_t>(lds_acc) <= kLdsBytes;
    const dim3 grid(static_cast<unsigned>(planes));
    if (in_lds) {
        hipError_t e = allow_lds(prop2d_plane_kernel<T, true>, lds_acc);
        if (e != hipSuccess) return e;
        prop2d_plane_kernel<T, true><<<grid, dim3(kThreads), lds_acc, stream>>>(
            static_cast<const T*>(x), static_cast<const T*>(lam), static_cast<const T*>(u),
            static_cast<const T*>(w4), eps, static_cast<T*>(y), planes, static_cast<int>(H),
            static_cast<int>(W), o.cpg, static_cast<int>(o.k_chunk), nullptr);
    } else {
        if constexpr (sizeof(T) != sizeof(float)) {
            return hipErrorInvalidValue;  // rejected earlier by prop2d_max_plane
        } else {
            const size_t lds = 2 * std::max(H, W) * sizeof(float);
            hipError_t e = allow_lds(prop2d_plane_kernel<T, false>, lds);
            if (e != hipSuccess) return e;
            prop2d_plane_kernel<T, false><<<grid, dim3(kThreads), lds, stream>>>(
                static_cast<const T*>(x), static_cast<const T*>(lam), static_cast<const T*>(u),
                static_cast<const T*>(w4), eps, static_cast<T*>(y), planes,
                static_cast<int>(H), static_cast<int>(W), o.cpg, static_cast<int>(o.k_chunk), nullptr);
        }
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_normalize(const void* w_raw, void* w_norm, int dtype, int64_t planes,
                            int64_t H, int64_t W, int dir0, int ndir, float eps,
                            hipStream_t stream) {
    return dtype == 0 ? normalize_t<float>(w_raw, w_norm, planes, H, W, dir0, ndir, eps, stream)
                      : normalize_t<uint16_t>(w_raw, w_norm, planes, H, W, dir0, ndir, eps,
                                              stream);
}

hipError_t launch_scan_dir(const void* x, const void* lam, const void* u, const void* w,
                           int w_is_raw, float eps, void* y, int accumulate, int dtype,
                           int64_t planes, int64_t H, int64_t W, int dir, hipStream_t stream) {
    if (scan_dir_fast_eligible(H, W, dir))
        return launch_scan_dir_fast(x, lam, u, w, w_is_raw, eps, y, accumulate, dtype, planes, H,
                                    W, dir, stream);
    return dtype == 0 ? scan_dir_t<float>(x, lam, u, w, w_is_raw, eps, y, accumulate, planes, H,
                                          W, dir, stream)
                      : scan_dir_t<uint16_t>(x, lam, u, w, w_is_raw, eps, y, accumulate,
                                             planes, H, W, dir, stream);
}

hipError_t launch_prop2d(const void* x, const void* lam, const void* u, const void* w4,
                         float eps, void* y, int dtype, int64_t planes, int64_t H, int64_t W,
                         const PropOpts& o, hipStream_t stream) {
    // square bf16 planes: one wavefront a plane up to 80, except when there
    // are too few planes to fill the CUs, where a wavefront a direction
    // finishes sooner (sides 66..80: 128 planes of 74 x 74 take 0.025 ms
    // against 0.037); two wavefronts a plane for sides 82..96, four for
    // 98..150 and odd 97..149
    const bool few = planes <= kFewPlanes && H > 64;
    if (!few && prop2d_quad_eligible(dtype, planes, H, W, o, x, lam, u, w4, y))
        return launch_prop2d_quad(x, lam, u, w4, eps, y, planes, H, o, stream);
    if (prop2d_duo_eligible(dtype, planes, H, W, o, x, lam, u, w4, y))
        return launch_prop2d_duo(x, lam, u, w4, eps, y, planes, H, o, stream);
    if (prop2d_phase_eligible(dtype, planes, H, W, x, lam, u, w4, y))
        return launch_prop2d_phase(x, lam, u, w4, eps, y, dtype, planes, H, W, o, stream);
    if (prop2d_pair_eligible(dtype, planes, H, W, x, lam, u, w4, y))
        return launch_prop2d_pair(x, lam, u, w4, eps, y, dtype, planes, H, W, o, stream);
    if (prop2d_wide_eligible(dtype, planes, H, W, x, lam, u, w4, y))
        return launch_prop2d_wide(x, lam, u, w4, eps, y, planes, H, W, o, stream);
    return dtype == 0 ? prop2d_t<float>(x, lam, u, w4, eps, y, planes, H, W, o, stream)
                      : prop2d_t<uint16_t>(x, lam, u, w4, eps, y, planes, H, W, o, stream);
}

int64_t prop2d_max_plane(int dtype, int64_t H, int64_t W) {
    if (dtype == 0) return INT64_MAX;  // fp32 output doubles as the accumulator
    return kLdsBytes / static_cast<int64_t>(sizeof(float)) - 2 * std::max(H, W);
}

int64_t prop2d_global_acc_bytes(int dtype, int64_t planes, int64_t H, int64_t W) {
    if (dtype != 1 || H * W <= prop2d_max_plane(dtype, H, W)) return 0;
    return (planes * H * W * static_cast<int64_t>(sizeof(float)) + 255) & ~static_cast<int64_t>(255);
}

hipError_t launch_prop2d_global_acc(const void* x, const void* lam, const void* u, const void* w4,
                                    float eps, void* y, int64_t planes, int64_t H, int64_t W,
                                    const PropOpts& o, float* acc, hipStream_t stream) {
    const size_t lds = 2 * std::max(H, W) * sizeof(float);
    hipError_t e = allow_lds(prop2d_plane_kernel<uint16_t, false>, lds);
    if (e != hipSuccess) return e;
    prop2d_plane_kernel<uint16_t, false><<<dim3(static_cast<unsigned>(planes)), dim3(kThreads), lds, stream>>>(
        static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(lam), static_cast<const uint16_t*>(u),
        static_cast<const uint16_t*>(w4), eps, static_cast<uint16_t*>(y), planes, static_cast<int>(H),
        static_cast<int>(W), o.cpg, static_cast<int>(o.k_chunk), acc);
    return hipGetLastError();
}

}  // namespace gspn
