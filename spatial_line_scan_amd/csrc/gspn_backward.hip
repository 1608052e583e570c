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

// ------------------------------------------------------------ odd sides
// A plane with an odd side is run as the plane one row and/or column larger,
// which the pair kernel takes.  The copy adds a zero row below and a zero
// column to the right of x, lambda, u and gy; in every direction's taps the
// added line's taps are 0 and so are those of the added position of each
// line, and the tap that reaches from a line's last position to the added
// one gets logit -inf, whose sigmoid is exactly 0.  Then every real
// position's weights are the ones of the plane as it is, the added positions
// never reach a real one (weight 0 times a finite value), a scan that starts
// on the added line gives the first real line h = lambda x exactly as the
// plane's own first line, and with gy = 0 there the adjoint carries nothing
// out of it; the tap gradient of the -inf tap is 0 (s (1 - s) = 0), as for a
// dropped tap.  So the real part of the padded gradients is the gradient of
// the plane.  A chunked scan keeps its segments as long as ceil(NL / k) does
// not change with the added line (not when k divides an odd NL).

// Division of n < 2^31 by a fixed d (1 <= d < 2^31): q = (umulhi(n, m) + n) >> s
// with s = ceil(log2 d) and m = floor(2^32 (2^s - d) / d) + 1 (the
// round-up method of Granlund and Montgomery, "Division by invariant
// integers using multiplication").
struct FastDiv {
    uint32_t d, m, s;
    FastDiv() = default;
    explicit FastDiv(uint32_t div) : d(div), s(0) {
        while ((1ull << s) < div) ++s;
        m = static_cast<uint32_t>(((1ull << 32) * ((1ull << s) - div)) / div + 1);
    }
    __device__ __forceinline__ uint32_t div(uint32_t n) const { return (__umulhi(n, m) + n) >> s; }
};

// Up to four line-plane tensors ([n][NL][L]) and their padded copies
// ([n][NLp][Lp], Lp even); blockIdx.y picks the tensor.  One thread per
// element pair of the padded copies (a 4- or 8-byte store: padded lines
// start on even elements).  taps: plane j is tap j % 3 of its position, and
// tap 2 of each line's last real position gets neg_inf when the line was
// lengthened.
template <typename T>
struct PadArgs {
    const T* src[4];
    T* dst[4];
    int n, NL, L, NLp, Lp;
    FastDiv per_plane, per_line;     // NLp * Lp / 2, Lp / 2 (pairs)
    bool taps;
    T neg_inf;
};

template <typename T> struct Pair2;
template <> struct Pair2<float> { typedef float __attribute__((ext_vector_type(2))) type; };
template <> struct Pair2<uint16_t> { typedef uint16_t __attribute__((ext_vector_type(2))) type; };

template <typename T>
__global__ void __launch_bounds__(256)
pad_lines_kernel(PadArgs<T> a) {
    const uint32_t total = static_cast<uint32_t>(a.n) * a.per_plane.d;
    const uint32_t i = blockIdx.x * 256u + threadIdx.x;
    if (i >= total) return;
    const uint32_t pl = a.per_plane.div(i);
    const uint32_t e = i - pl * a.per_plane.d;
    const uint32_t line = a.per_line.div(e);
    const uint32_t p0 = 2 * (e - line * a.per_line.d);
    const T* src = a.src[blockIdx.y] + (static_cast<int64_t>(pl) * a.NL + line) * a.L;
    const bool real_line = line < static_cast<uint32_t>(a.NL);
    T v[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const uint32_t p = p0 + j;
        v[j] = T(0);
        if (real_line && p < static_cast<uint32_t>(a.L))
            v[j] = (a.taps && pl % 3 == 2 && p == static_cast<uint32_t>(a.L - 1) && a.Lp > a.L) ? a.neg_inf : src[p];
    }
    typedef typename Pair2<T>::type P2;
    reinterpret_cast<P2*>(a.dst[blockIdx.y])[i] = P2{v[0], v[1]};
}

// The real lines of padded copies: dst[y] ([n][NL][L]) from src[y]
// ([n][NLp][Lp]); one thread per element pair of the padded copy (an
// aligned 4- or 8-byte load), storing its real elements.
template <typename T>
struct CropArgs {
    const T* src[4];
    T* dst[4];
    int n, NL, L, NLp, Lp;
    FastDiv per_plane, per_line;     // NLp * Lp / 2, Lp / 2 (pairs)
};

template <typename T>
__global__ void __launch_bounds__(256)
crop_lines_kernel(CropArgs<T> a) {
    const uint32_t total = static_cast<uint32_t>(a.n) * a.per_plane.d;
    const uint32_t i = blockIdx.x * 256u + threadIdx.x;
    if (i >= total) return;
    const uint32_t pl = a.per_plane.div(i);
    const uint32_t e = i - pl * a.per_plane.d;
    const uint32_t line = a.per_line.div(e);
    if (line >= static_cast<uint32_t>(a.NL)) return;
    const uint32_t p0 = 2 * (e - line * a.per_line.d);
    typedef typename Pair2<T>::type P2;
    const P2 v = reinterpret_cast<const P2*>(a.src[blockIdx.y])[i];
    T* dst = a.dst[blockIdx.y] + (static_cast<int64_t>(pl) * a.NL + line) * a.L;
    if (p0 < static_cast<uint32_t>(a.L)) dst[p0] = v.x;
    if (p0 + 1 < static_cast<uint32_t>(a.L)) dst[p0 + 1] = v.y;
}

// The padded problem: inputs and taps copied in, the pair path run on it,
// the real part of the gradients copied out.  buf: padded x, lambda, u, gy,
// gx, glambda, gu, taps, tap gradients.
template <typename T>
hipError_t run_padded(const void* x, const void* lam, const void* u, const void* w4, const void* gy,
                      float eps, void* gx, void* glam, void* gu, void* gw4, void* ws, void* const* buf,
                      int dtype, int64_t planes, int64_t H, int64_t W, int64_t Hp, int64_t Wp,
                      const PropOpts& o, hipStream_t stream) {
    const int64_t tp = planes / o.cpg;
    const int64_t HW = H * W, HWp = Hp * Wp;
    auto blocks = [](int64_t n, int ny) { return dim3(static_cast<unsigned>((n + 255) / 256), ny); };
    T neg_inf;
    if constexpr (sizeof(T) == 4) neg_inf = -__builtin_inff();
    else neg_inf = static_cast<T>(0xff80u);   // bf16 -inf
    hipError_t e;
    {   // x, lambda, u, gy: lines are rows
        PadArgs<T> a{};
        const void* in[4] = {x, lam, u, gy};
        for (int i = 0; i < 4; ++i) {
            a.src[i] = static_cast<const T*>(in[i]);
            a.dst[i] = static_cast<T*>(buf[i]);
        }
        a.n = static_cast<int>(planes);
        a.NL = static_cast<int>(H); a.L = static_cast<int>(W); a.NLp = static_cast<int>(Hp); a.Lp = static_cast<int>(Wp);
        a.per_plane = FastDiv(static_cast<uint32_t>(HWp / 2));
        a.per_line = FastDiv(static_cast<uint32_t>(Wp / 2));
        a.taps = false;
        a.neg_inf = neg_inf;
        pad_lines_kernel<T><<<blocks(planes * HWp / 2, 4), dim3(256), 0, stream>>>(a);
    }
    // taps: the row directions' 6 tp planes (lines are rows), then the column
    // directions' (lines are columns)
    for (int part = 0; part < 2; ++part) {
        PadArgs<T> a{};
        a.src[0] = static_cast<const T*>(w4) + part * 6 * tp * HW;
        a.dst[0] = static_cast<T*>(buf[7]) + part * 6 * tp * HWp;
        a.n = static_cast<int>(6 * tp);
        a.NL = static_cast<int>(part ? W : H); a.L = static_cast<int>(part ? H : W);
        a.NLp = static_cast<int>(part ? Wp : Hp); a.Lp = static_cast<int>(part ? Hp : Wp);
        a.per_plane = FastDiv(static_cast<uint32_t>(HWp / 2));
        a.per_line = FastDiv(static_cast<uint32_t>(a.Lp / 2));
        a.taps = true;
        a.neg_inf = neg_inf;
        pad_lines_kernel<T><<<blocks(6 * tp * HWp / 2, 1), dim3(256), 0, stream>>>(a);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    e = launch_prop2d_backward(buf[0], buf[1], buf[2], buf[7], buf[3], eps, buf[4], buf[5], buf[6], buf[8], ws,
                               dtype, planes, Hp, Wp, o, stream);
    if (e != hipSuccess) return e;
    {
        CropArgs<T> a{};
        void* out[3] = {gx, glam, gu};
        for (int i = 0; i < 3; ++i) {
            a.src[i] = static_cast<const T*>(buf[4 + i]);
            a.dst[i] = static_cast<T*>(out[i]);
        }
        a.n = static_cast<int>(planes);
        a.NL = static_cast<int>(H); a.L = static_cast<int>(W); a.NLp = static_cast<int>(Hp); a.Lp = static_cast<int>(Wp);
        a.per_plane = FastDiv(static_cast<uint32_t>(HWp / 2));
        a.per_line = FastDiv(static_cast<uint32_t>(Wp / 2));
        crop_lines_kernel<T><<<blocks(planes * HWp / 2, 3), dim3(256), 0, stream>>>(a);
    }
    for (int part = 0; part < 2; ++part) {
        CropArgs<T> a{};
        a.src[0] = static_cast<const T*>(buf[8]) + part * 6 * tp * HWp;
        a.dst[0] = static_cast<T*>(gw4) + part * 6 * tp * HW;
        a.n = static_cast<int>(6 * tp);
        a.NL = static_cast<int>(part ? W : H); a.L = static_cast<int>(part ? H : W);
        a.NLp = static_cast<int>(part ? Wp : Hp); a.Lp = static_cast<int>(part ? Hp : Wp);
        a.per_plane = FastDiv(static_cast<uint32_t>(HWp / 2));
        a.per_line = FastDiv(static_cast<uint32_t>(a.Lp / 2));
        crop_lines_kernel<T><<<blocks(6 * tp * HWp / 2, 1), dim3(256), 0, stream>>>(a);
    }
    return hipGetLastError();
}

int64_t a256(int64_t v) { return (v + 255) & ~static_cast<int64_t>(255); }

// Bytes of the padded copies (storage up to 4 bytes): x, lambda, u, gy, gx,
// glambda, gu and the taps and their gradients.
int64_t padded_copy_bytes(int64_t planes, int64_t Hp, int64_t Wp, int64_t cpg) {
    const int64_t n = planes * Hp * Wp * 4;
    return 7 * a256(n) + 2 * a256(12 * (planes / cpg) * Hp * Wp * 4);
}

bool odd_shape(int64_t H, int64_t W) { return (H & 1) || (W & 1); }

// Whether the padded plane takes the pair kernel (workspace sizing).
bool padded_pair_shape(int64_t planes, int64_t H, int64_t W) {
    return odd_shape(H, W) && prop2d_backward_pair_shape(planes, H + (H & 1), W + (W & 1));
}

int64_t direct_workspace_bytes(int64_t planes, int64_t H, int64_t W, int64_t cpg) {
    const int64_t general = plane_kernel_workspace_bytes(planes, H, W);
    const int64_t pair = prop2d_backward_pair_shape(planes, H, W)
                             ? prop2d_backward_pair_workspace_bytes(planes, H, W) : 0;
    return group_grad_bytes(planes, H, W, cpg) + (general > pair ? general : pair);
}

// ceil(NL / k) with the added line.
bool segments_keep(int64_t NL, int64_t k) {
    if (!(NL & 1) || k <= 1) return true;
    return (NL + 1 + k - 1) / k == (NL + k - 1) / k;
}

}  // namespace

int64_t prop2d_backward_workspace_bytes(int64_t planes, int64_t H, int64_t W, int64_t cpg) {
    const int64_t direct = direct_workspace_bytes(planes, H, W, cpg);
    if (!padded_pair_shape(planes, H, W)) return direct;
    const int64_t Hp = H + (H & 1), Wp = W + (W & 1);
    const int64_t padded = direct_workspace_bytes(planes, Hp, Wp, cpg) + padded_copy_bytes(planes, Hp, Wp, cpg);
    return padded > direct ? padded : direct;
}

int64_t prop2d_backward_max_line() { return kLdsBytes / 4 / 7; }

hipError_t launch_prop2d_backward(const void* x, const void* lam, const void* u, const void* w4,
                                  const void* gy, float eps, void* gx, void* glam, void* gu,
                                  void* gw4, void* ws, int dtype, int64_t planes, int64_t H,
                                  int64_t W, const PropOpts& o, hipStream_t stream) {
    // square bf16 planes of odd side with per-channel taps take the pair
    // kernel's odd form directly; other odd shapes that fit it padded run
    // padded
    const bool odd = odd_shape(H, W);
    const void* ptrs0[] = {x, lam, u, w4, gy, gx, glam, gu, gw4};
    const bool odd_direct =
        odd && dtype == 1 && o.cpg == 1 && ws &&
        prop2d_backward_pair_eligible(dtype, planes, H, W, ptrs0, 9,
                                      static_cast<char*>(ws) + group_grad_bytes(planes, H, W, o.cpg));
    if (!odd_direct && ws && padded_pair_shape(planes, H, W) && segments_keep(H, o.k_chunk) &&
        segments_keep(W, o.k_chunk)) {
        const int64_t Hp = H + (H & 1), Wp = W + (W & 1);
        const int64_t n = planes * Hp * Wp, nt = 12 * (planes / o.cpg) * Hp * Wp;
        char* p = static_cast<char*>(ws) + direct_workspace_bytes(planes, Hp, Wp, o.cpg);
        void* buf[9];
        for (int i = 0; i < 7; ++i) {
            buf[i] = p;
            p += a256(n * 4);
        }
        buf[7] = p;                      // taps
        p += a256(nt * 4);
        buf[8] = p;                      // tap gradients
        return dtype == 0 ? run_padded<float>(x, lam, u, w4, gy, eps, gx, glam, gu, gw4, ws, buf, dtype, planes,
                                              H, W, Hp, Wp, o, stream)
                          : run_padded<uint16_t>(x, lam, u, w4, gy, eps, gx, glam, gu, gw4, ws, buf, dtype,
                                                 planes, H, W, Hp, Wp, o, stream);
    }
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
    if (!(odd && grouped) && prop2d_backward_pair_eligible(dtype, planes, H, W, ptrs, 9, rest)) {
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
