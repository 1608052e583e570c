// Gradient of the four-direction propagation (gfx950).
//
// Operator: "Scaling Parallel Sequence Models to Foundation-Scale Vision
// Encoders", §3 line-scan recurrence and §5.1 fused normalisation (forward);
// §6.1 reports backward kernels without describing them, so this is the exact
// derivative of the forward definition:
//
//   adjoint of direction d, lines in reverse scan order:
//     g_last = u * gy,   g_i = u * gy + (W_{i+1})^T g_{i+1}
//   where (W^T g)[p] = sum_k wn_k(q) g[q] over the destinations q = p - k + 1
//   of the next line whose tap k reads position p;
//   gx = lambda * sum_d g_d,  glambda = x * sum_d g_d,  gu = gy * sum_d h_d;
//   gwn_k(i, p) = g_i[p] h_{i-1}[p + k - 1] (0 on the first line and for
//   dropped taps); through the normalisation s = sigmoid(z), T = sum s:
//     T > eps : gs_m = (gwn_m - sum_k gwn_k wn_k) / T,   else gs_m = gwn_m / eps
//     (evaluated as sum_{k != m} wn_k (gwn_m - gwn_k) / T, equal since the
//     unclamped taps sum to one)
//     gz_m = gs_m s_m (1 - s_m) for in-line taps.
//
// One workgroup owns one (b, c) plane and runs the four directions in turn:
// a forward pass that keeps every line of h (in the line-major order of the
// direction), then the adjoint pass.  The three fp32 planes (h of the current
// direction, sum_d h, sum_d g) live in LDS when they fit, else in a workspace
// the caller passes; the current, previous and next lines and the next line's
// normalised taps are LDS lines.
#include "gspn_device.h"
#include <algorithm>
#include "gspn_internal.h"

namespace gspn {
namespace {

constexpr int kBwdThreads = 256;

// Sigmoids, sum and normalised taps of one destination position (forward
// normalisation, kept for the Jacobian).
struct TapNorm {
    float s[3], wn[3], T;
};

__device__ __forceinline__ TapNorm tap_norm(float z0, float z1, float z2, bool has_left,
                                            bool has_right, float eps) {
    TapNorm t;
    t.s[0] = has_left ? sigmoid_hw(z0) : 0.0f;
    t.s[1] = sigmoid_hw(z1);
    t.s[2] = has_right ? sigmoid_hw(z2) : 0.0f;
    t.T = (t.s[0] + t.s[1]) + t.s[2];
    const float r = __builtin_amdgcn_rcpf(fmaxf(t.T, eps));
    for (int k = 0; k < 3; ++k) t.wn[k] = t.s[k] * r;
    return t;
}

template <typename T>
__device__ __forceinline__ void store_f(T* p, size_t i, float v) {
    store_elem(p, i, v);
}

// GT: type of the tap gradients written, per channel ([4][planes][3][..][..]):
// T straight into gw4 when every channel has its own taps, fp32 into a
// workspace that a group reduction then sums when channels share them.
// cpg: channels per tap group; k_chunk: segments per scan.
template <typename T, typename GT>
__global__ void __launch_bounds__(kBwdThreads)
prop2d_backward_kernel(const T* __restrict__ x, const T* __restrict__ lam,
                       const T* __restrict__ u, const T* __restrict__ w4,
                       const T* __restrict__ gy, float eps, T* __restrict__ gx,
                       T* __restrict__ glam, T* __restrict__ gu, GT* __restrict__ gwd,
                       float* __restrict__ ws, int64_t planes, int H, int W, int cpg, int k_chunk) {
    extern __shared__ float lds[];
    const int tid = threadIdx.x;
    const int Lmax = H > W ? H : W;
    const size_t npix = static_cast<size_t>(H) * W;
    const size_t plane = blockIdx.x;
    // LDS lines: h (2), g (2), normalised taps of the next line (3)
    float* hline = lds;                  // [2][Lmax]
    float* gline = hline + 2 * Lmax;     // [2][Lmax]
    float* wnext = gline + 2 * Lmax;     // [3][Lmax]
    float* planes3;
    if (ws == nullptr) planes3 = wnext + 3 * Lmax;   // [3][npix] in LDS
    else planes3 = ws + plane * 3 * npix;
    float* hd = planes3;                 // h of the current direction, [NL][L]
    float* hs = planes3 + npix;          // sum_d h, pixel order
    float* gs = planes3 + 2 * npix;      // sum_d g, pixel order

    const T* xp = x + plane * npix;
    const T* lp = lam + plane * npix;
    const T* up = u + plane * npix;
    const T* gyp = gy + plane * npix;
    for (size_t e = tid; e < npix; e += kBwdThreads) {
        hs[e] = 0.0f;
        gs[e] = 0.0f;
    }
    __syncthreads();

    for (int dir = 0; dir < 4; ++dir) {
        const bool rows = dir < 2;
        const bool fwd = dir == 0 || dir == 2;
        const int NL = rows ? H : W;
        const int L = rows ? W : H;
        const T* wp = w4 + (static_cast<size_t>(dir) * (planes / cpg) + plane / cpg) * 3 * npix;
        GT* gwp = gwd + (static_cast<size_t>(dir) * planes + plane) * 3 * npix;
        auto pix = [&](int i, int p) -> size_t {
            return rows ? static_cast<size_t>(i) * W + p : static_cast<size_t>(p) * W + i;
        };
        auto line_of = [&](int step) { return fwd ? step : NL - 1 - step; };
        // the first line of each segment in scan order reads no line before it
        const int seg = (NL + k_chunk - 1) / k_chunk;
        auto restarts = [&](int i) { return fwd ? i % seg == 0 : (i == NL - 1 || (i + 1) % seg == 0); };

        // ---------------------------------------------- forward, keeping h
        for (int step = 0; step < NL; ++step) {
            const int i = line_of(step);
            const float* hprev = hline + ((step + 1) & 1) * Lmax;
            float* hnew = hline + (step & 1) * Lmax;
            for (int p = tid; p < L; p += kBwdThreads) {
                const size_t px = pix(i, p);
                float h = load_elem(lp, px) * load_elem(xp, px);
                if (!restarts(i)) {
                    const size_t t = static_cast<size_t>(i) * L + p;
                    const TapNorm tn = tap_norm(load_elem(wp, t), load_elem(wp, t + npix),
                                                load_elem(wp, t + 2 * npix), p > 0, p < L - 1, eps);
                    float m = tn.wn[1] * hprev[p];
                    if (p > 0) m = fmaf(tn.wn[0], hprev[p - 1], m);
                    if (p < L - 1) m = fmaf(tn.wn[2], hprev[p + 1], m);
                    h += m;
                }
                hnew[p] = h;
                hd[static_cast<size_t>(i) * L + p] = h;
                hs[px] += h;
            }
            __syncthreads();
        }

        // ---------------------------------------------- adjoint, reverse order
        for (int step = NL - 1; step >= 0; --step) {
            const int i = line_of(step);
            const int iprev = step > 0 ? line_of(step - 1) : i;
            const float* gold = gline + ((step + 1) & 1) * Lmax;   // line scanned after i
            float* gnew = gline + (step & 1) * Lmax;
            const bool next_reads_i = step < NL - 1 && !restarts(line_of(step + 1));
            const bool reads_prev = !restarts(i);
            float wcur[3][4];   // normalised taps of line i for this thread's positions
            int slot = 0;
            for (int p = tid; p < L; p += kBwdThreads, ++slot) {
                const size_t px = pix(i, p);
                float v = load_elem(up, px) * load_elem(gyp, px);
                if (next_reads_i) {
                    // destinations q = p + 1, p, p - 1 of the next line read p
                    // through their taps 0, 1, 2
                    v = fmaf(wnext[Lmax + p], gold[p], v);
                    if (p + 1 < L) v = fmaf(wnext[p + 1], gold[p + 1], v);
                    if (p > 0) v = fmaf(wnext[2 * Lmax + p - 1], gold[p - 1], v);
                }
                gnew[p] = v;
                gs[px] += v;

                const size_t t = static_cast<size_t>(i) * L + p;
                const TapNorm tn = tap_norm(load_elem(wp, t), load_elem(wp, t + npix),
                                            load_elem(wp, t + 2 * npix), p > 0, p < L - 1, eps);
                if (slot < 4)
                    for (int k = 0; k < 3; ++k) wcur[k][slot] = tn.wn[k];
                float gz[3] = {0.0f, 0.0f, 0.0f};
                if (reads_prev) {
                    const float* hp = hd + static_cast<size_t>(iprev) * L;
                    float gwn[3];
                    gwn[0] = p > 0 ? v * hp[p - 1] : 0.0f;
                    gwn[1] = v * hp[p];
                    gwn[2] = p < L - 1 ? v * hp[p + 1] : 0.0f;
                    // Unclamped, the taps sum to one, so gwn_m - sum_k gwn_k wn_k
                    // = sum_{k != m} wn_k (gwn_m - gwn_k): the same value without
                    // the cancellation (a lone in-line tap gets exactly 0).
                    const bool unclamped = tn.T > eps;
                    const float rT = __builtin_amdgcn_rcpf(unclamped ? tn.T : eps);
                    for (int m = 0; m < 3; ++m) {
                        float num = gwn[m];
                        if (unclamped) {
                            num = 0.0f;
                            for (int k = 0; k < 3; ++k)
                                if (k != m) num = fmaf(tn.wn[k], gwn[m] - gwn[k], num);
                        }
                        gz[m] = num * rT * tn.s[m] * (1.0f - tn.s[m]);
                    }
                    if (p == 0) gz[0] = 0.0f;
                    if (p == L - 1) gz[2] = 0.0f;
                }
                store_f(gwp, t, gz[0]);
                store_f(gwp, t + npix, gz[1]);
                store_f(gwp, t + 2 * npix, gz[2]);
            }
            __syncthreads();   // every read of wnext and gold of this step is done
            slot = 0;
            for (int p = tid; p < L; p += kBwdThreads, ++slot) {
                if (slot < 4) {
                    for (int k = 0; k < 3; ++k) wnext[k * Lmax + p] = wcur[k][slot];
                } else {
                    const size_t t = static_cast<size_t>(i) * L + p;
                    const TapNorm tn = tap_norm(load_elem(wp, t), load_elem(wp, t + npix),
                                                load_elem(wp, t + 2 * npix), p > 0, p < L - 1, eps);
                    for (int k = 0; k < 3; ++k) wnext[k * Lmax + p] = tn.wn[k];
                }
            }
            __syncthreads();
        }
    }

    for (size_t e = tid; e < npix; e += kBwdThreads) {
        const float g = gs[e];
        store_f(gx + plane * npix, e, load_elem(lp, e) * g);
        store_f(glam + plane * npix, e, load_elem(xp, e) * g);
        store_f(gu + plane * npix, e, load_elem(gyp, e) * hs[e]);
    }
}

size_t bwd_line_floats(int64_t H, int64_t W) { return 7 * static_cast<size_t>(H > W ? H : W); }

template <typename T, typename GT>
hipError_t backward_t(const void* x, const void* lam, const void* u, const void* w4,
                      const void* gy, float eps, void* gx, void* glam, void* gu, void* gwd,
                      void* ws, int64_t planes, int64_t H, int64_t W, const PropOpts& o,
                      hipStream_t stream) {
    const size_t lines = bwd_line_floats(H, W) * sizeof(float);
    const size_t lds = ws ? lines : lines + 3 * static_cast<size_t>(H * W) * sizeof(float);
    auto kern = prop2d_backward_kernel<T, GT>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(lds));
        if (e != hipSuccess) return e;
    }
    kern<<<dim3(static_cast<unsigned>(planes)), dim3(kBwdThreads), lds, stream>>>(
        static_cast<const T*>(x), static_cast<const T*>(lam), static_cast<const T*>(u),
        static_cast<const T*>(w4), static_cast<const T*>(gy), eps, static_cast<T*>(gx),
        static_cast<T*>(glam), static_cast<T*>(gu), static_cast<GT*>(gwd),
        static_cast<float*>(ws), planes, static_cast<int>(H), static_cast<int>(W),
        static_cast<int>(o.cpg), static_cast<int>(o.k_chunk));
    return hipGetLastError();
}

// Workspace of this kernel: its three fp32 planes when they do not fit in LDS.
int64_t plane_kernel_workspace_bytes(int64_t planes, int64_t H, int64_t W) {
    const int64_t lds = static_cast<int64_t>(bwd_line_floats(H, W) + 3 * H * W) * 4;
    return lds <= kLdsBytes ? 0 : planes * 3 * H * W * 4;
}

// Per-channel fp32 tap gradients of channels that share taps, [4][planes][3][H W].
// Channels sharing taps: their fp32 tap gradients (or partial sums of tap
// products), then the group's normalised weights (pair kernel).
int64_t group_grad_bytes(int64_t planes, int64_t H, int64_t W, int64_t cpg) {
    return cpg > 1 ? ((12 * planes * H * W * 4 + 255) & ~static_cast<int64_t>(255)) +
                         prop2d_backward_pair_shared_weights_bytes(planes, H, W, cpg)
                   : 0;
}

// Tap gradient of each group: the sum over its channels, in channel order.
// gwc is [4][B][G][cpg][3 HW] read as [..][cpg][plane3]; gw4 is [4][B][G][3 HW].
template <typename T>
__global__ void __launch_bounds__(256)
group_sum_kernel(const float* __restrict__ gwc, T* __restrict__ gw4, int64_t n_out, int64_t plane3,
                 int cpg) {
    for (int64_t o = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; o < n_out;
         o += static_cast<int64_t>(gridDim.x) * 256) {
        const int64_t grp = o / plane3, r = o - grp * plane3;
        const float* src = gwc + grp * cpg * plane3 + r;
        float acc = 0.0f;
        for (int c = 0; c < cpg; ++c) acc += src[c * plane3];
        store_elem(gw4, static_cast<size_t>(o), acc);
    }
}

// The same sum, four adjacent outputs a thread (plane3 a multiple of 4;
// gwc 16-byte and gw4 4-output aligned): 16-byte loads, eight channels'
// loads issued before their adds, which stay in channel order.
template <typename T>
__global__ void __launch_bounds__(256)
group_sum4_kernel(const float* __restrict__ gwc, T* __restrict__ gw4, int64_t n_out4, int64_t plane3,
                  int cpg) {
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    for (int64_t o4 = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; o4 < n_out4;
         o4 += static_cast<int64_t>(gridDim.x) * 256) {
        const int64_t o = 4 * o4;
        const int64_t grp = o / plane3, r = o - grp * plane3;
        const f32x4_t* src = reinterpret_cast<const f32x4_t*>(gwc + grp * cpg * plane3 + r);
        const int64_t stride = plane3 / 4;
        f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
        int c = 0;
        for (; c + 8 <= cpg; c += 8) {
            f32x4_t v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] = src[(c + k) * stride];
#pragma unroll
            for (int k = 0; k < 8; ++k) acc += v[k];
        }
        for (; c < cpg; ++c) acc += src[c * stride];
        if constexpr (sizeof(T) == 4) {
            *reinterpret_cast<f32x4_t*>(gw4 + o) = acc;
        } else {
            // store_elem's rounding, two outputs a dword
            auto bf = [](float lo, float hi) {
                return static_cast<uint32_t>(bf16_rne(lo)) | (static_cast<uint32_t>(bf16_rne(hi)) << 16);
            };
            *reinterpret_cast<u32x2_t*>(gw4 + o) = u32x2_t{bf(acc.x, acc.y), bf(acc.z, acc.w)};
        }
    }
}

}  // namespace

int64_t prop2d_backward_workspace_bytes(int64_t planes, int64_t H, int64_t W, int64_t cpg) {
    const int64_t general = plane_kernel_workspace_bytes(planes, H, W);
    const int64_t pair = prop2d_backward_pair_shape(planes, H, W)
                             ? prop2d_backward_pair_workspace_bytes(planes, H, W) : 0;
    return group_grad_bytes(planes, H, W, cpg) + (general > pair ? general : pair);
}

int64_t prop2d_backward_max_line() { return kLdsBytes / 4 / 7; }

hipError_t launch_prop2d_backward(const void* x, const void* lam, const void* u, const void* w4,
                                  const void* gy, float eps, void* gx, void* glam, void* gu,
                                  void* gw4, void* ws, int dtype, int64_t planes, int64_t H,
                                  int64_t W, const PropOpts& o, hipStream_t stream) {
    // channels that share taps write their own fp32 tap gradients first, at
    // the start of the workspace; the kernels' own scratch follows
    const bool grouped = o.cpg > 1;
    void* gdst = grouped ? ws : gw4;
    void* rest = ws ? static_cast<char*>(ws) + group_grad_bytes(planes, H, W, o.cpg) : nullptr;
    const void* ptrs[] = {x, lam, u, w4, gy, gx, glam, gu, gw4};
    hipError_t e;
    // bytes the workspace query reserved after the tap gradients
    const int64_t general = plane_kernel_workspace_bytes(planes, H, W);
    const int64_t pair = prop2d_backward_pair_shape(planes, H, W)
                             ? prop2d_backward_pair_workspace_bytes(planes, H, W) : 0;
    const int64_t avail = ws ? (general > pair ? general : pair) : 0;
    if (prop2d_backward_pair_eligible(dtype, planes, H, W, ptrs, 9, rest)) {
        if (grouped) {
            // partial sums at the start of the workspace, the weights after
            // the per-channel region
            float* part = static_cast<float*>(ws);
            float* wpre = reinterpret_cast<float*>(
                static_cast<char*>(ws) + ((12 * planes * H * W * 4 + 255) & ~static_cast<int64_t>(255)));
            return launch_prop2d_backward_pair_shared(x, lam, u, w4, gy, eps, gx, glam, gu, gw4, part, wpre,
                                                      rest, dtype, planes, H, W, o, stream);
        }
        e = launch_prop2d_backward_pair(x, lam, u, w4, gy, eps, gx, glam, gu, gdst, grouped, rest,
                                        dtype, planes, H, W, o, stream);
    } else if (prop2d_backward_wide_eligible(dtype, planes, H, W, ptrs, 9, rest, avail)) {
        e = launch_prop2d_backward_wide(x, lam, u, w4, gy, eps, gx, glam, gu, gdst, rest, planes, H, W, o,
                                        stream);
    } else {
        // this kernel takes a workspace only when its planes leave LDS
        void* pws = plane_kernel_workspace_bytes(planes, H, W) == 0 ? nullptr : rest;
        if (dtype == 0)
            e = backward_t<float, float>(x, lam, u, w4, gy, eps, gx, glam, gu, gdst, pws, planes, H, W, o,
                                         stream);
        else if (grouped)
            e = backward_t<uint16_t, float>(x, lam, u, w4, gy, eps, gx, glam, gu, gdst, pws, planes, H, W,
                                            o, stream);
        else
            e = backward_t<uint16_t, uint16_t>(x, lam, u, w4, gy, eps, gx, glam, gu, gdst, pws, planes, H,
                                               W, o, stream);
    }
    if (e != hipSuccess || !grouped) return e;
    const int64_t plane3 = 3 * H * W;
    const int64_t n_out = 4 * (planes / o.cpg) * plane3;
    const uintptr_t out_align = dtype == 0 ? 15u : 7u;
    if (plane3 % 4 == 0 && (reinterpret_cast<uintptr_t>(ws) & 15u) == 0 &&
        (reinterpret_cast<uintptr_t>(gw4) & out_align) == 0) {
        const int64_t n_out4 = n_out / 4;
        const int64_t blocks4 = std::min<int64_t>((n_out4 + 255) / 256, 16384);
        if (dtype == 0)
            group_sum4_kernel<float><<<dim3(static_cast<unsigned>(blocks4)), dim3(256), 0, stream>>>(
                static_cast<const float*>(ws), static_cast<float*>(gw4), n_out4, plane3, static_cast<int>(o.cpg));
        else
            group_sum4_kernel<uint16_t><<<dim3(static_cast<unsigned>(blocks4)), dim3(256), 0, stream>>>(
                static_cast<const float*>(ws), static_cast<uint16_t*>(gw4), n_out4, plane3,
                static_cast<int>(o.cpg));
        return hipGetLastError();
    }
    const int64_t blocks = std::min<int64_t>((n_out + 255) / 256, 16384);
    if (dtype == 0)
        group_sum_kernel<float><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream>>>(
            static_cast<const float*>(ws), static_cast<float*>(gw4), n_out, plane3, static_cast<int>(o.cpg));
    else
        group_sum_kernel<uint16_t><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream>>>(
            static_cast<const float*>(ws), static_cast<uint16_t*>(gw4), n_out, plane3, static_cast<int>(o.cpg));
    return hipGetLastError();
}

}  // namespace gspn
