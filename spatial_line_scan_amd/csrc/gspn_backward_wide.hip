// Gradient of the four-direction propagation for large fp32 planes (sides up
// to 256, a multiple of 4), gfx950.
//
// Operator: "Scaling Parallel Sequence Models to Foundation-Scale Vision
// Encoders", §3 line-scan recurrence and §5.1 fused normalisation; the pages
// report backward kernels (§6.1) without describing them, so this is the exact
// derivative of the forward definition, the same as the general backward
// kernel's:
//   adjoint of a direction, lines in reverse scan order:
//     g_last = u gy,   g_i = u gy + (W_{i+1})^T g_{i+1};
//   gwn_k(i, p) = g_i[p] h_{i-1}[p + k - 1], taken through the normalisation
//   (s = sigmoid(z), T = s_0 + s_1 + s_2, wn = s / max(T, eps));
//   gx = lambda sum_d g_d,  glambda = x sum_d g_d,  gu = gy sum_d h_d.
//
// A 256 x 256 fp32 plane's sums do not fit in LDS, so one wavefront per (b, c)
// plane works through HBM, without any barrier: for each direction in the
// order TD, BU, LR, RL, a forward pass recomputes h and keeps every line of it
// in a workspace plane (line-major), then the adjoint pass runs in reverse
// scan order, reading h of the line before.  sum_d h and sum_d g accumulate in
// gu and gx themselves, in that direction order, and the last direction's
// passes turn them into the three gradients as they complete them.  Passes
// are ordered by workgroup-scope fences: a pass reads what other lanes of the
// wavefront wrote in an earlier one.
// As in the wide forward kernel, lane l holds positions K l .. K l + K - 1 of
// a line (neighbours through one DPP shift each way), row passes stream row
// windows, and column passes walk strips of 32 columns (whole 128-byte lines)
// whose pixel-order input (lambda x, or u gy) is staged transposed in LDS and
// replaced in place by the pass's result, then added into the accumulator a
// strip at a time.
#include "gspn_device.h"
#include "gspn_internal.h"
#include "gspn_lane.h"

namespace gspn {
namespace {

using namespace lane;

constexpr int kSW = 32;           // columns per strip
constexpr int kCQ = kSW / 4;      // 16-byte chunks per strip row
constexpr int kBatch = 16;        // strip chunks a lane loads per batch
constexpr int kD = 4;             // lines prefetched ahead
constexpr int kMaxSideBwdWide = 256;

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3_t __attribute__((ext_vector_type(3)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// LDS row pitch of a strip (floats), = 2 mod 16 so that a batch's transposed
// accesses (8 rows x 8 chunks) fall on distinct banks.
__host__ __device__ inline int strip_pitch(int H) { return ((H + 13) & ~15) + 2; }

__device__ __forceinline__ void lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup", "local");
}

__device__ __forceinline__ void pass_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const float* p, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p), 0, bytes, kBufFlags);
}

// A lane's K floats at byte offset off: one vector store when all are in the
// line, else one store per position in it.
template <int K>
__device__ __forceinline__ void store_window(__amdgpu_buffer_rsrc_t r, uint32_t off, const float (&v)[K],
                                             const bool (&valid)[K]) {
    if (valid[K - 1]) {
        if constexpr (K == 1) {
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[0]), r, off, 0, 0);
        } else if constexpr (K == 2) {
            __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{__float_as_uint(v[0]), __float_as_uint(v[1])}, r,
                                                  off, 0, 0);
        } else if constexpr (K == 3) {
            __builtin_amdgcn_raw_buffer_store_b96(
                u32x3_t{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2])}, r, off, 0, 0);
        } else {
            __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{__float_as_uint(v[0]), __float_as_uint(v[1]),
                                                           __float_as_uint(v[2]), __float_as_uint(v[3])},
                                                   r, off, 0, 0);
        }
    } else {
#pragma unroll
        for (int j = 0; j < K; ++j)
            if (valid[j]) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[j]), r, off + 4 * j, 0, 0);
    }
}

template <int K>
__device__ __forceinline__ float wf(const words_t<K>& w, int j) {
    return __uint_as_float(word<K>(w, j));
}

// What every pass of a plane needs.
struct Ctx {
    __amdgpu_buffer_rsrc_t xs, ls, us, gys, hs, gxs, gus, gls;   // plane-sized, pixel order (hs: line-major h)
    const float* w4;
    float* gwd;
    int planes, tap_planes, cpg, k_chunk, plane, H, W;
    float eps;
};

// One pass over the plane: the forward recompute (Adj = false) or the adjoint
// (Adj = true) of direction Dir.
template <int K, int Dir, bool Adj, bool Chunked>
__device__ __forceinline__ void bwd_pass(const Ctx& c, float* strip) {
    constexpr bool kRows = Dir < 2;
    constexpr bool kFwd = Dir == 0 || Dir == 2;   // the direction's own order: ascending lines
    constexpr bool kAsc = kFwd != Adj;            // this pass's order
    const int H = c.H, W = c.W, HW = H * W;
    const int NL = kRows ? H : W;
    const int L = kRows ? W : H;
    const int lane = threadIdx.x;
    const int plane_bytes = HW * 4;
    const size_t tap0 = (static_cast<size_t>(Dir) * c.tap_planes + c.plane / c.cpg) * 3 * HW;
    const size_t gw0 = (static_cast<size_t>(Dir) * c.planes + c.plane) * 3 * HW;
    __amdgpu_buffer_rsrc_t taps[3], gws[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        taps[k] = rsrc(c.w4 + tap0 + static_cast<size_t>(k) * HW, plane_bytes);
        if constexpr (Adj) gws[k] = rsrc(c.gwd + gw0 + static_cast<size_t>(k) * HW, plane_bytes);
    }
    // in the line: p < L; taps reading outside it are dropped
    bool valid[K], has_l[K], has_r[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const int p = K * lane + j;
        valid[j] = p < L;
        has_l[j] = valid[j] && p > 0;
        has_r[j] = valid[j] && p < L - 1;
    }
    const float eps = c.eps;
    const int seg = Chunked ? (NL + c.k_chunk - 1) / c.k_chunk : NL;
    auto fline = [&](int step) { return kFwd ? step : NL - 1 - step; };   // forward step -> line
    auto restarts = [&](int i) { return kFwd ? i % seg == 0 : (i == NL - 1 || (i + 1) % seg == 0); };
    // forward step of this pass's step s
    auto fstep = [&](int s) { return Adj ? NL - 1 - s : s; };
    const uint32_t win = static_cast<uint32_t>(K * lane) * 4;
    auto line_off = [&](int i) { return static_cast<uint32_t>(i * L) * 4 + win; };

    // prefetch ring, slot d: taps of the step's line; rows: its pixel-order
    // windows; adjoint: h of the line before it
    constexpr int kPix = kRows ? kD : 1;
    constexpr int kPrev = Adj ? kD : 1;
    words_t<K> tbuf[kD][3], abuf[kPix], bbuf[kPix], accbuf[kPix], hbuf[kPrev];
    auto load_step = [&](int s, int d) {
        const int sc = s < NL ? s : NL - 1;
        const int f = fstep(sc);
        const uint32_t lo = line_off(fline(f));
#pragma unroll
        for (int k = 0; k < 3; ++k) tbuf[d][k] = load_words<K>(taps[k], lo);
        if constexpr (kRows) {
            abuf[d] = load_words<K>(Adj ? c.us : c.ls, lo);
            bbuf[d] = load_words<K>(Adj ? c.gys : c.xs, lo);
            if constexpr (Dir == 1) accbuf[d] = load_words<K>(Adj ? c.gxs : c.gus, lo);
        }
        if constexpr (Adj) hbuf[d] = load_words<K>(c.hs, line_off(fline(f > 0 ? f - 1 : 0)));
    };
#pragma unroll
    for (int d = 0; d < kD; ++d) load_step(d, d);

    // carried state: forward h of the last line; adjoint g and normalised
    // taps of the line processed last (the one after, in forward order)
    float h[K], gold[K], wx0[K], wx1[K], wx2[K];
#pragma unroll
    for (int j = 0; j < K; ++j) h[j] = gold[j] = wx0[j] = wx1[j] = wx2[j] = 0.0f;

    // one step: b[] is lambda x (forward) or u gy (adjoint) of the lane's
    // positions; out[] receives h or g
    auto step = [&](int s, int d, const float (&b)[K], float (&out)[K]) {
        const int f = fstep(s);
        const int i = fline(f);
        if constexpr (!Adj) {
            const bool restart = restarts(i);
            float m[K];
#pragma unroll
            for (int j = 0; j < K; ++j) h[j] = restart ? 0.0f : h[j];
            const float hl0 = from_prev(h[K - 1]);
            const float hrK = from_next(h[0]);
#pragma unroll
            for (int j = 0; j < K; ++j) {
                float w0, w1, w2;
                normalize3(wf<K>(tbuf[d][0], j), wf<K>(tbuf[d][1], j), wf<K>(tbuf[d][2], j), has_l[j],
                           has_r[j], eps, w0, w1, w2);
                const float hl = j > 0 ? h[j - 1] : hl0;
                const float hr = j < K - 1 ? h[j + 1] : hrK;
                m[j] = w1 * h[j];
                m[j] = has_l[j] ? fmaf(w0, hl, m[j]) : m[j];
                m[j] = has_r[j] ? fmaf(w2, hr, m[j]) : m[j];
            }
#pragma unroll
            for (int j = 0; j < K; ++j) {
                out[j] = valid[j] ? (restart ? b[j] : b[j] + m[j]) : 0.0f;
                h[j] = out[j];
            }
            store_window<K>(c.hs, line_off(i), out, valid);
        } else {
            // g_i = u gy + contributions of the next line's destinations
            // q = p + 1, p, p - 1, which read p through taps 0, 1, 2
            const bool next_reads_i = s > 0 && !restarts(fline(f + 1));
            const float g_r = from_next(gold[0]), w0_r = from_next(wx0[0]);
            const float g_l = from_prev(gold[K - 1]), w2_l = from_prev(wx2[K - 1]);
            float v[K];
#pragma unroll
            for (int j = 0; j < K; ++j) {
                float a = b[j];
                if (next_reads_i) {
                    const float gp1 = j < K - 1 ? gold[j + 1] : g_r;
                    const float w0p1 = j < K - 1 ? wx0[j + 1] : w0_r;
                    const float gm1 = j > 0 ? gold[j - 1] : g_l;
                    const float w2m1 = j > 0 ? wx2[j - 1] : w2_l;
                    a = fmaf(wx1[j], gold[j], a);
                    a = fmaf(w0p1, gp1, a);
                    a = fmaf(w2m1, gm1, a);
                }
                v[j] = valid[j] ? a : 0.0f;
            }
            // tap gradients of line i through the normalisation
            const bool reads_prev = !restarts(i);
            const float hl0 = from_prev(wf<K>(hbuf[d], K - 1));
            const float hrK = from_next(wf<K>(hbuf[d], 0));
            float gz0[K], gz1[K], gz2[K];
#pragma unroll
            for (int j = 0; j < K; ++j) {
                const float s0 = has_l[j] ? sigmoid_hw(wf<K>(tbuf[d][0], j)) : 0.0f;
                const float s1 = valid[j] ? sigmoid_hw(wf<K>(tbuf[d][1], j)) : 0.0f;
                const float s2 = has_r[j] ? sigmoid_hw(wf<K>(tbuf[d][2], j)) : 0.0f;
                const float T = (s0 + s1) + s2;
                const float r = __builtin_amdgcn_rcpf(fmaxf(T, eps));
                const float wn[3] = {s0 * r, s1 * r, s2 * r};
                const float sg[3] = {s0, s1, s2};
                float gz[3] = {0.0f, 0.0f, 0.0f};
                if (reads_prev) {
                    const float hp = wf<K>(hbuf[d], j);
                    const float hm1 = j > 0 ? wf<K>(hbuf[d], j - 1) : hl0;
                    const float hp1 = j < K - 1 ? wf<K>(hbuf[d], j + 1) : hrK;
                    float gwn[3];
                    gwn[0] = has_l[j] ? v[j] * hm1 : 0.0f;
                    gwn[1] = v[j] * hp;
                    gwn[2] = has_r[j] ? v[j] * hp1 : 0.0f;
                    // unclamped, the taps sum to one, so gwn_m - sum_k gwn_k wn_k
                    // = sum_{k != m} wn_k (gwn_m - gwn_k), without the cancellation
                    const bool unclamped = T > eps;
                    const float rT = __builtin_amdgcn_rcpf(unclamped ? T : eps);
#pragma unroll
                    for (int mm = 0; mm < 3; ++mm) {
                        float num = gwn[mm];
                        if (unclamped) {
                            num = 0.0f;
#pragma unroll
                            for (int k = 0; k < 3; ++k)
                                if (k != mm) num = fmaf(wn[k], gwn[mm] - gwn[k], num);
                        }
                        gz[mm] = num * rT * sg[mm] * (1.0f - sg[mm]);
                    }
                    if (!has_l[j]) gz[0] = 0.0f;
                    if (!has_r[j]) gz[2] = 0.0f;
                }
                gz0[j] = gz[0];
                gz1[j] = gz[1];
                gz2[j] = gz[2];
                wx0[j] = wn[0];
                wx1[j] = wn[1];
                wx2[j] = wn[2];
            }
            const uint32_t lo = line_off(i);
            store_window<K>(gws[0], lo, gz0, valid);
            store_window<K>(gws[1], lo, gz1, valid);
            store_window<K>(gws[2], lo, gz2, valid);
#pragma unroll
            for (int j = 0; j < K; ++j) {
                gold[j] = v[j];
                out[j] = v[j];
            }
        }
    };

    if constexpr (kRows) {
        // accumulator: sum h in gu (forward), sum g in gx (adjoint)
        const __amdgpu_buffer_rsrc_t acc = Adj ? c.gxs : c.gus;
        for (int s0 = 0; s0 < NL; s0 += kD) {
#pragma unroll
            for (int d = 0; d < kD; ++d) {
                const int s = s0 + d;
                if (s < NL) {
                    float b[K], out[K], av[K];
#pragma unroll
                    for (int j = 0; j < K; ++j) {
                        b[j] = wf<K>(abuf[d], j) * wf<K>(bbuf[d], j);
                        av[j] = Dir == 1 ? wf<K>(accbuf[d], j) : 0.0f;
                    }
                    step(s, d, b, out);
                    const uint32_t lo = line_off(fline(fstep(s)));
                    load_step(s + kD, d);
                    float nv[K];
#pragma unroll
                    for (int j = 0; j < K; ++j) nv[j] = Dir == 0 ? out[j] : av[j] + out[j];
                    store_window<K>(acc, lo, nv, valid);
                }
            }
        }
    } else {
        const int pitch = strip_pitch(H);
        float* bs = strip;                          // [column][row]: lambda x or u gy, then h or g
        const int T = (W + kSW - 1) / kSW;
        const int units = H * kCQ;                  // (row, 4-column chunk) pairs of a strip
        const __amdgpu_buffer_rsrc_t pa = Adj ? c.us : c.ls;
        const __amdgpu_buffer_rsrc_t pb = Adj ? c.gys : c.xs;
        const __amdgpu_buffer_rsrc_t acc = Adj ? c.gxs : c.gus;
        int s = 0;
        for (int tt = 0; tt < T; ++tt) {
            const int t = kAsc ? tt : T - 1 - tt;
            const int cb = t * kSW;
            const int width = W - cb < kSW ? W - cb : kSW;   // a multiple of 4
            for (int f0 = 0; f0 < units; f0 += 64 * kBatch) {
                f32x4_t av[kBatch], bv[kBatch];
#pragma unroll
                for (int a = 0; a < kBatch; ++a) {
                    const int f = f0 + 64 * a + lane;
                    const int row = f / kCQ, cq = 4 * (f % kCQ);
                    av[a] = bv[a] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
                    if (f < units && cq < width) {
                        const uint32_t o = static_cast<uint32_t>(row * W + cb + cq) * 4;
                        av[a] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(pa, o, 0, 0));
                        bv[a] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(pb, o, 0, 0));
                    }
                }
#pragma unroll
                for (int a = 0; a < kBatch; ++a) {
                    const int f = f0 + 64 * a + lane;
                    const int row = f / kCQ, cq = 4 * (f % kCQ);
                    if (f < units) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) bs[(cq + e) * pitch + row] = av[a][e] * bv[a][e];
                    }
                }
            }
            lds_sync();
            for (int q0 = 0; q0 < kSW; q0 += kD) {
#pragma unroll
                for (int d = 0; d < kD; ++d) {
                    const int q = q0 + d;
                    if (q < width) {
                        // strips start at multiples of kD steps (widths are
                        // multiples of 4), so this step's ring slot is d;
                        // positions past H touch no LDS
                        const int cl = kAsc ? q : width - 1 - q;
                        float b[K], out[K];
#pragma unroll
                        for (int j = 0; j < K; ++j) b[j] = valid[j] ? bs[cl * pitch + K * lane + j] : 0.0f;
                        step(s, d, b, out);
                        load_step(s + kD, d);
#pragma unroll
                        for (int j = 0; j < K; ++j)
                            if (valid[j]) bs[cl * pitch + K * lane + j] = out[j];
                        ++s;
                    }
                }
            }
            lds_sync();
            // acc += the strip; the last direction completes the sums, so
            // its passes write the gradients instead: gu = gy sum h, and
            // gx = lambda sum g, glambda = x sum g
            for (int f0 = 0; f0 < units; f0 += 64 * kBatch) {
                f32x4_t yv[kBatch], m0[kBatch], m1[kBatch];
#pragma unroll
                for (int a = 0; a < kBatch; ++a) {
                    const int f = f0 + 64 * a + lane;
                    const int row = f / kCQ, cq = 4 * (f % kCQ);
                    if (f < units && cq < width) {
                        const uint32_t o = static_cast<uint32_t>(row * W + cb + cq) * 4;
                        yv[a] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(acc, o, 0, 0));
                        if constexpr (Dir == 3) {
                            m0[a] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                                    Adj ? c.ls : c.gys, o, 0, 0));
                            if constexpr (Adj)
                                m1[a] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(c.xs, o, 0, 0));
                        }
                    }
                }
#pragma unroll
                for (int a = 0; a < kBatch; ++a) {
                    const int f = f0 + 64 * a + lane;
                    const int row = f / kCQ, cq = 4 * (f % kCQ);
                    if (f < units && cq < width) {
                        f32x4_t v;
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] = yv[a][e] + bs[(cq + e) * pitch + row];
                        const uint32_t o = static_cast<uint32_t>(row * W + cb + cq) * 4;
                        if constexpr (Dir == 3) {
                            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, m0[a] * v), acc, o, 0, 0);
                            if constexpr (Adj)
                                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, m1[a] * v), c.gls, o, 0,
                                                                       0);
                        } else {
                            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), acc, o, 0, 0);
                        }
                    }
                }
            }
            lds_sync();
        }
    }
}

template <int K, bool Chunked>
__global__ void __launch_bounds__(64)
prop2d_backward_wide_kernel(const float* __restrict__ x, const float* __restrict__ lam,
                            const float* __restrict__ u, const float* __restrict__ w4,
                            const float* __restrict__ gy, float eps, float* __restrict__ gx,
                            float* __restrict__ glam, float* __restrict__ gu, float* __restrict__ gwd,
                            float* __restrict__ hws, int planes, int H, int W, int cpg, int k_chunk) {
    extern __shared__ __attribute__((aligned(16))) float strip[];
    const int HW = H * W;
    const size_t pix0 = static_cast<size_t>(blockIdx.x) * HW;
    const int pb = HW * 4;
    Ctx c;
    c.xs = rsrc(x + pix0, pb);
    c.ls = rsrc(lam + pix0, pb);
    c.us = rsrc(u + pix0, pb);
    c.gys = rsrc(gy + pix0, pb);
    c.hs = rsrc(hws + pix0, pb);
    c.gxs = rsrc(gx + pix0, pb);
    c.gus = rsrc(gu + pix0, pb);
    c.gls = rsrc(glam + pix0, pb);
    c.w4 = w4;
    c.gwd = gwd;
    c.planes = planes;
    c.tap_planes = planes / cpg;
    c.cpg = cpg;
    c.k_chunk = k_chunk;
    c.plane = blockIdx.x;
    c.H = H;
    c.W = W;
    c.eps = eps;
    bwd_pass<K, 0, false, Chunked>(c, strip);
    pass_sync();
    bwd_pass<K, 0, true, Chunked>(c, strip);
    pass_sync();
    bwd_pass<K, 1, false, Chunked>(c, strip);
    pass_sync();
    bwd_pass<K, 1, true, Chunked>(c, strip);
    pass_sync();
    bwd_pass<K, 2, false, Chunked>(c, strip);
    pass_sync();
    bwd_pass<K, 2, true, Chunked>(c, strip);
    pass_sync();
    bwd_pass<K, 3, false, Chunked>(c, strip);
    pass_sync();
    bwd_pass<K, 3, true, Chunked>(c, strip);
}

template <int K>
hipError_t launch_k(const float* x, const float* lam, const float* u, const float* w4, const float* gy,
                    float eps, float* gx, float* glam, float* gu, float* gwd, float* hws, int64_t planes,
                    int64_t H, int64_t W, const PropOpts& o, hipStream_t stream) {
    const size_t lds = kSW * static_cast<size_t>(strip_pitch(static_cast<int>(H))) * 4;
    auto run = [&](auto kern) -> hipError_t {
        if (lds > 64 * 1024) {
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
            if (e != hipSuccess) return e;
        }
        kern<<<dim3(static_cast<unsigned>(planes)), dim3(64), lds, stream>>>(
            x, lam, u, w4, gy, eps, gx, glam, gu, gwd, hws, static_cast<int>(planes), static_cast<int>(H),
            static_cast<int>(W), static_cast<int>(o.cpg), static_cast<int>(o.k_chunk));
        return hipGetLastError();
    };
    return o.k_chunk > 1 ? run(prop2d_backward_wide_kernel<K, true>) : run(prop2d_backward_wide_kernel<K, false>);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

int64_t prop2d_backward_wide_workspace_bytes(int64_t planes, int64_t H, int64_t W) {
    return planes * H * W * 4;
}

bool prop2d_backward_wide_eligible(int dtype, int64_t planes, int64_t H, int64_t W,
                                   const void* const* ptrs, int nptrs, const void* ws,
                                   int64_t ws_bytes) {
    if (dtype != 0) return false;                                   // fp32: the outputs accumulate
    if (H > kMaxSideBwdWide || W > kMaxSideBwdWide || (H & 3) || (W & 3)) return false;
    if (planes > 0x7fffffff) return false;
    if (ws == nullptr || !aligned16(ws) || ws_bytes < prop2d_backward_wide_workspace_bytes(planes, H, W))
        return false;
    for (int i = 0; i < nptrs; ++i)
        if (!aligned16(ptrs[i])) return false;
    return true;
}

hipError_t launch_prop2d_backward_wide(const void* x_, const void* lam_, const void* u_, const void* w4_,
                                       const void* gy_, float eps, void* gx_, void* glam_, void* gu_,
                                       void* gwd_, void* ws, int64_t planes, int64_t H, int64_t W,
                                       const PropOpts& o, hipStream_t stream) {
    const float* x = static_cast<const float*>(x_);
    const float* lam = static_cast<const float*>(lam_);
    const float* u = static_cast<const float*>(u_);
    const float* w4 = static_cast<const float*>(w4_);
    const float* gy = static_cast<const float*>(gy_);
    float* gx = static_cast<float*>(gx_);
    float* glam = static_cast<float*>(glam_);
    float* gu = static_cast<float*>(gu_);
    float* gwd = static_cast<float*>(gwd_);
    float* hws = static_cast<float*>(ws);
    const int64_t L = H > W ? H : W;
    if (L <= 64) return launch_k<1>(x, lam, u, w4, gy, eps, gx, glam, gu, gwd, hws, planes, H, W, o, stream);
    if (L <= 128) return launch_k<2>(x, lam, u, w4, gy, eps, gx, glam, gu, gwd, hws, planes, H, W, o, stream);
    if (L <= 192) return launch_k<3>(x, lam, u, w4, gy, eps, gx, glam, gu, gwd, hws, planes, H, W, o, stream);
    return launch_k<4>(x, lam, u, w4, gy, eps, gx, glam, gu, gwd, hws, planes, H, W, o, stream);
}

}  // namespace gspn
