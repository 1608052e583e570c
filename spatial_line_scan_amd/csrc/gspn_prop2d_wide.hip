// Four-direction propagation of large planes (sides up to 256, a multiple
// of 4): fp32, and bf16 planes whose direction sum does not fit on chip
// (sides 196..256, four positions a lane), gfx950.
//
// Operator: "Scaling Parallel Sequence Models to Foundation-Scale Vision
// Encoders", §3 line-scan recurrence, §4.1 all steps of a scan in one launch,
// §5.1 fused normalisation (sigmoid, local sum, clamp, divide); reading
// notes, method / overall framework.
//
// A plane's direction sum does not fit in LDS, so it is kept in global
// memory: in the fp32 output y itself, or for bf16 in an fp32 plane of the
// caller's workspace (acc), from which the last pass writes y.  One launch, one wavefront per (b, c) plane, which runs four
// passes over its plane in turn (ordered by workgroup-scope fences: a pass
// reads y that other lanes wrote in the previous one); lane l holds
// positions K l .. K l + K - 1 of the current line (K = ceil(L / 64)), and
// the neighbour exchange is one wave-wide DPP shift each way:
//   TD  acc = h_TD                rows top-down
//   BU  acc = acc + h_BU          rows bottom-up
//   LR  acc = acc + h_LR          columns left-right
//   RL  y = u (acc + h_RL)        columns right-left
// so the four terms of a pixel are summed in the fixed order TD, BU, LR, RL.
// Every direction's taps are line-major, so a tap window is contiguous in
// both kinds of pass, and taps are prefetched D lines ahead.
//   Row passes read x, lambda (and y) as row windows, prefetched with the
//   taps, and write y rows.
//   Column passes walk the plane in strips of 32 columns, so that each row
//   of a strip is one whole 128-byte line of x, lambda, y and u (narrower
//   strips fetch every line twice: its other half is evicted before the
//   next strip).  A strip's b = lambda x is read with row-contiguous 16-byte
//   loads and staged in LDS transposed ([column][row], 33 KB at 256 rows);
//   the strip's columns are then scanned from LDS, each column's h taking
//   the place of its b, and the strip's y is read, added to (and in the last
//   pass multiplied by u) and written back in rows.  Reading along columns
//   straight from memory would fetch a cache line per element.
// Chunked scans restart h at the first line of each segment of
// ceil(NL / k_chunk) lines; the tap plane of plane p is p / cpg.
#include "gspn_device.h"
#include "gspn_internal.h"
#include "gspn_lane.h"

namespace gspn {
namespace {

using namespace lane;

constexpr int kSW = 32;           // columns per strip: 128-byte rows of x, lambda, y, u
constexpr int kCQ = kSW / 4;      // 16-byte chunks per strip row
constexpr int kBatch = 16;        // strip chunks a lane loads per batch
constexpr int kMaxSideWide = 256;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
template <typename V> using lds_t = __attribute__((address_space(3))) V;

// LDS row pitch of a strip (floats): a column of H rows plus a pad, with
// pitch = 2 mod 16 so that the transposed accesses of one batch (8 rows x 8
// chunks of 4 columns) fall on distinct banks.
__host__ __device__ inline int strip_pitch(int H) { return ((H + 13) & ~15) + 2; }

// Orders this wavefront's LDS accesses before the fence against those after
// it (one wavefront per workgroup: no barrier).
__device__ __forceinline__ void lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup", "local");
}

// Orders this wavefront's global stores of one pass before the next pass's
// loads, which other lanes of the wavefront issue.
__device__ __forceinline__ void pass_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Element j of a window of K consecutive values (fp32 words, or bf16 pairs
// from an even element) as fp32.
template <typename T, int KW>
__device__ __forceinline__ float wide_elem(const words_t<KW>& w, int j) {
    if constexpr (sizeof(T) == 4) {
        return __uint_as_float(word<KW>(w, j));
    } else {
        const uint32_t v = word<KW>(w, j >> 1);
        return __uint_as_float((j & 1) ? (v & 0xffff0000u) : (v << 16));
    }
}

// One direction's pass over plane blockIdx.x; strip is the column passes' LDS.
// T: storage type of x, lambda, u, the taps and y; acc: the fp32 direction
// sum (y itself for fp32).
template <typename T, int K, int D, int Dir, bool Chunked>
__device__ __forceinline__ void wide_pass(const T* __restrict__ x, const T* __restrict__ lam,
                                          const T* __restrict__ u, const T* __restrict__ w4,
                                          float eps, float* __restrict__ y, T* __restrict__ yout,
                                          int planes, int H, int W, int cpg, int k_chunk, float* strip) {
    constexpr bool kRows = Dir < 2;
    constexpr bool kFwd = Dir == 0 || Dir == 2;
    constexpr int ES = sizeof(T);
    static_assert(ES == 4 || K % 2 == 0, "bf16 windows of whole dwords");
    constexpr int KW = ES == 4 ? K : K / 2;   // dwords of a lane's window
    static_assert(kSW % D == 0 && 4 % D == 0, "strip steps stay aligned to the prefetch ring");
    const int HW = H * W;
    const int NL = kRows ? H : W;
    const int L = kRows ? W : H;
    const int lane = threadIdx.x;
    const int plane = blockIdx.x;
    const size_t pix0 = static_cast<size_t>(plane) * HW;
    // one buffer resource per plane (offsets within a plane; loads past its
    // end return 0), so the tensors themselves may exceed 2 GiB
    const int plane_bytes = HW * ES;
    const int acc_bytes = HW * 4;
    const __amdgpu_buffer_rsrc_t xs = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(x + pix0), 0, plane_bytes, kBufFlags);
    const __amdgpu_buffer_rsrc_t ls = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(lam + pix0), 0, plane_bytes, kBufFlags);
    const __amdgpu_buffer_rsrc_t ys = __builtin_amdgcn_make_buffer_rsrc(y + pix0, 0, acc_bytes, kBufFlags);
    __amdgpu_buffer_rsrc_t taps[3];
    const int tap_planes = planes / cpg;
    const size_t tap0 = (static_cast<size_t>(Dir) * tap_planes + plane / cpg) * 3 * HW;
#pragma unroll
    for (int k = 0; k < 3; ++k)
        taps[k] = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(w4 + tap0 + static_cast<size_t>(k) * HW), 0,
                                                    plane_bytes, kBufFlags);

    float c0[K], c1[K], c2[K];
    bool valid[K];
    const float inf = __builtin_inff();
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const int p = K * lane + j;
        valid[j] = p < L;
        c0[j] = (valid[j] && p > 0) ? 1.0f : inf;
        c1[j] = valid[j] ? 1.0f : inf;
        c2[j] = (valid[j] && p < L - 1) ? 1.0f : inf;
    }
    const int seg = Chunked ? (NL + k_chunk - 1) / k_chunk : NL;
    auto line_of = [&](int s) { return kFwd ? s : NL - 1 - s; };
    auto restarts = [&](int i) {
        return kFwd ? i % seg == 0 : (i == NL - 1 || (i + 1) % seg == 0);
    };
    // byte offsets of the lane's window: storage type, and the fp32 sum
    const uint32_t win = static_cast<uint32_t>(K * lane) * ES;
    const uint32_t wina = static_cast<uint32_t>(K * lane) * 4;

    // ---- prefetch ring: taps (and for rows x, lambda, y) of line line_of(s)
    words_t<KW> tbuf[D][3], xbuf[kRows ? D : 1], lbuf[kRows ? D : 1];
    words_t<K> ybuf[kRows ? D : 1];
    auto load_line = [&](int s, int d) {
        const int i = line_of(s < NL ? s : NL - 1);
        const uint32_t lo = static_cast<uint32_t>(i * L) * ES + win;
#pragma unroll
        for (int k = 0; k < 3; ++k) tbuf[d][k] = load_words<KW>(taps[k], lo);
        if constexpr (kRows) {
            const uint32_t xo = static_cast<uint32_t>(i * W) * ES + win;
            xbuf[d] = load_words<KW>(xs, xo);
            lbuf[d] = load_words<KW>(ls, xo);
            if constexpr (Dir == 1) ybuf[d] = load_words<K>(ys, static_cast<uint32_t>(i * W) * 4 + wina);
        }
    };
#pragma unroll
    for (int d = 0; d < D; ++d) load_line(d, d);

    float h[K];
#pragma unroll
    for (int j = 0; j < K; ++j) h[j] = 0.0f;

    // one step of the scan: line line_of(s), prefetch slot d; b[] is lambda x
    // of the lane's positions, out[] receives the new states
    auto advance = [&](int s, int d, const float (&b)[K], float (&hn)[K]) {
        float s0[K], s1[K], s2[K], r[K];
#pragma unroll
        for (int j = 0; j < K; ++j) {
            s0[j] = __builtin_amdgcn_exp2f(wide_elem<T, KW>(tbuf[d][0], j) * kNegLog2e);
            s1[j] = __builtin_amdgcn_exp2f(wide_elem<T, KW>(tbuf[d][1], j) * kNegLog2e);
            s2[j] = __builtin_amdgcn_exp2f(wide_elem<T, KW>(tbuf[d][2], j) * kNegLog2e);
        }
#pragma unroll
        for (int j = 0; j < K; ++j) {
            s0[j] = __builtin_amdgcn_rcpf(s0[j] + c0[j]);
            s1[j] = __builtin_amdgcn_rcpf(s1[j] + c1[j]);
            s2[j] = __builtin_amdgcn_rcpf(s2[j] + c2[j]);
            r[j] = __builtin_amdgcn_rcpf(fmaxf((s0[j] + s1[j]) + s2[j], eps));
        }
        const bool restart = restarts(line_of(s));
#pragma unroll
        for (int j = 0; j < K; ++j) h[j] = restart ? 0.0f : h[j];
        const float hl0 = from_prev(h[K - 1]);
        const float hrK = from_next(h[0]);
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const float hl = j > 0 ? h[j - 1] : hl0;
            const float hr = j < K - 1 ? h[j + 1] : hrK;
            float m = s1[j] * h[j];
            m = fmaf(s0[j], hl, m);
            m = fmaf(s2[j], hr, m);
            hn[j] = fmaf(m, r[j], b[j]);
        }
#pragma unroll
        for (int j = 0; j < K; ++j) h[j] = hn[j];
    };

    if constexpr (kRows) {
        for (int s0 = 0; s0 < NL; s0 += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int s = s0 + d;
                if (s < NL) {
                    float b[K], hn[K];
#pragma unroll
                    for (int j = 0; j < K; ++j)
                        b[j] = wide_elem<T, KW>(lbuf[d], j) * wide_elem<T, KW>(xbuf[d], j);
                    float yv[K];
                    if constexpr (Dir == 1) {
#pragma unroll
                        for (int j = 0; j < K; ++j) yv[j] = __uint_as_float(word<K>(ybuf[d], j));
                    }
                    advance(s, d, b, hn);
                    const int i = line_of(s);
                    float* yr = y + pix0 + static_cast<size_t>(i) * W + K * lane;
                    load_line(s + D, d);
#pragma unroll
                    for (int j = 0; j < K; ++j)
                        if (valid[j]) yr[j] = Dir == 0 ? hn[j] : yv[j] + hn[j];
                }
            }
        }
    } else {
        // strips of kSW columns: LR takes them left to right, RL right to left
        const int pitch = strip_pitch(H);
        float* bs = strip;                          // [column][row]: b = lambda x, then h
        const int nstrips = (W + kSW - 1) / kSW;
        const int units = H * kCQ;                  // (row, 4-column chunk) pairs of a strip
        const __amdgpu_buffer_rsrc_t us =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(u + pix0), 0, plane_bytes, kBufFlags);
        // four consecutive values of a storage-type plane at element e
        auto load4 = [&](__amdgpu_buffer_rsrc_t r, int e) -> f32x4_t {
            if constexpr (ES == 4) {
                return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<uint32_t>(e) * 4, 0, 0));
            } else {
                const words_t<2> v = load_words<2>(r, static_cast<uint32_t>(e) * 2);
                return f32x4_t{wide_elem<T, 2>(v, 0), wide_elem<T, 2>(v, 1), wide_elem<T, 2>(v, 2), wide_elem<T, 2>(v, 3)};
            }
        };
        int s = 0;                                  // scan step
        for (int tt = 0; tt < nstrips; ++tt) {
            const int t = kFwd ? tt : nstrips - 1 - tt;
            const int cb = t * kSW;                 // first column of the strip
            const int width = W - cb < kSW ? W - cb : kSW;   // a multiple of 4
            // b of the strip: unit f = row f / kCQ, columns cb + 4 (f % kCQ) ..
            for (int f0 = 0; f0 < units; f0 += 64 * kBatch) {
                f32x4_t xv[kBatch], lv[kBatch];
#pragma unroll
                for (int a = 0; a < kBatch; ++a) {
                    const int f = f0 + 64 * a + lane;
                    const int row = f / kCQ, cq = 4 * (f % kCQ);
                    xv[a] = lv[a] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
                    if (f < units && cq < width) {
                        xv[a] = load4(xs, row * W + cb + cq);
                        lv[a] = load4(ls, row * W + cb + cq);
                    }
                }
#pragma unroll
                for (int a = 0; a < kBatch; ++a) {
                    const int f = f0 + 64 * a + lane;
                    const int row = f / kCQ, cq = 4 * (f % kCQ);
                    if (f < units) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) bs[(cq + e) * pitch + row] = lv[a][e] * xv[a][e];
                    }
                }
            }
            lds_sync();
            // scan the strip's columns; each column's h replaces its b
            for (int q0 = 0; q0 < kSW; q0 += D) {
#pragma unroll
                for (int d = 0; d < D; ++d) {
                    const int q = q0 + d;                    // step within the strip
                    if (q < width) {
                        const int cl = kFwd ? q : width - 1 - q;   // column within the strip
                        // strips start at multiples of D steps (widths are
                        // multiples of 4), so this step's ring slot is d;
                        // positions past H (their taps are dropped) take b = 0
                        // and touch no LDS: they would reach the next column
                        float b[K], hn[K];
#pragma unroll
                        for (int j = 0; j < K; ++j) b[j] = valid[j] ? bs[cl * pitch + K * lane + j] : 0.0f;
                        advance(s, d, b, hn);
                        load_line(s + D, d);
#pragma unroll
                        for (int j = 0; j < K; ++j)
                            if (valid[j]) bs[cl * pitch + K * lane + j] = hn[j];
                        ++s;
                    }
                }
            }
            lds_sync();
            // y of the strip = y + h (times u in the last pass), written back in rows
            for (int f0 = 0; f0 < units; f0 += 64 * kBatch) {
                f32x4_t yv[kBatch], uv[kBatch];
#pragma unroll
                for (int a = 0; a < kBatch; ++a) {
                    const int f = f0 + 64 * a + lane;
                    const int row = f / kCQ, cq = 4 * (f % kCQ);
                    if (f < units && cq < width) {
                        const uint32_t o = static_cast<uint32_t>(row * W + cb + cq) * 4;
                        yv[a] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ys, o, 0, 0));
                        if constexpr (Dir == 3) uv[a] = load4(us, row * W + cb + cq);
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
                        if constexpr (Dir == 3) v = v * uv[a];
                        const size_t e = pix0 + static_cast<size_t>(row) * W + cb + cq;
                        if constexpr (Dir == 3 && ES == 2) {
                            typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
                            *reinterpret_cast<u32x2_t*>(yout + e) =
                                u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                        } else {
                            *reinterpret_cast<f32x4_t*>(y + e) = v;
                        }
                    }
                }
            }
            lds_sync();
        }
    }
}

// The four passes of one plane, in the summation order TD, BU, LR, RL; KR
// and KC are the positions a lane holds on a row and on a column.
template <typename T, int KR, int KC, bool Chunked>
__global__ void __launch_bounds__(64)
prop2d_wide_kernel(const T* __restrict__ x, const T* __restrict__ lam, const T* __restrict__ u,
                   const T* __restrict__ w4, float eps, float* __restrict__ y, T* __restrict__ yout,
                   int planes, int H, int W, int cpg, int k_chunk) {
    extern __shared__ __attribute__((aligned(16))) float strip[];
    constexpr int D = 4;
    wide_pass<T, KR, D, 0, Chunked>(x, lam, u, w4, eps, y, yout, planes, H, W, cpg, k_chunk, strip);
    pass_sync();
    wide_pass<T, KR, D, 1, Chunked>(x, lam, u, w4, eps, y, yout, planes, H, W, cpg, k_chunk, strip);
    pass_sync();
    wide_pass<T, KC, D, 2, Chunked>(x, lam, u, w4, eps, y, yout, planes, H, W, cpg, k_chunk, strip);
    pass_sync();
    wide_pass<T, KC, D, 3, Chunked>(x, lam, u, w4, eps, y, yout, planes, H, W, cpg, k_chunk, strip);
}

// y: the fp32 direction sum (the output itself for fp32); yout: the output.
template <typename T, int KR, int KC>
hipError_t launch_k(const T* x, const T* lam, const T* u, const T* w4, float eps, float* y, T* yout,
                    int64_t planes, int64_t H, int64_t W, const PropOpts& o, hipStream_t stream) {
    const size_t lds = kSW * static_cast<size_t>(strip_pitch(static_cast<int>(H))) * 4;
    auto run = [&](auto kern) -> hipError_t {
        if (lds > 64 * 1024) {
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
            if (e != hipSuccess) return e;
        }
        kern<<<dim3(static_cast<unsigned>(planes)), dim3(64), lds, stream>>>(
            x, lam, u, w4, eps, y, yout, static_cast<int>(planes), static_cast<int>(H),
            static_cast<int>(W), static_cast<int>(o.cpg), static_cast<int>(o.k_chunk));
        return hipGetLastError();
    };
    return o.k_chunk > 1 ? run(prop2d_wide_kernel<T, KR, KC, true>) : run(prop2d_wide_kernel<T, KR, KC, false>);
}

// K = ceil(L / 64) positions a lane, L up to 256
template <int KR>
hipError_t launch_kc(const float* x, const float* lam, const float* u, const float* w4, float eps,
                     float* y, int64_t planes, int64_t H, int64_t W, const PropOpts& o,
                     hipStream_t stream) {
    if (H <= 64) return launch_k<float, KR, 1>(x, lam, u, w4, eps, y, y, planes, H, W, o, stream);
    if (H <= 128) return launch_k<float, KR, 2>(x, lam, u, w4, eps, y, y, planes, H, W, o, stream);
    if (H <= 192) return launch_k<float, KR, 3>(x, lam, u, w4, eps, y, y, planes, H, W, o, stream);
    return launch_k<float, KR, 4>(x, lam, u, w4, eps, y, y, planes, H, W, o, stream);
}

// bf16 planes take this kernel only when their direction sum leaves LDS
// (above about 40,500 pixels, so both sides above 158): K = 4 on both lines
// (sides 196..256, multiples of 4); other sizes take the general kernel
bool wide_bf16_side(int64_t L) { return L > 192 && L <= kMaxSideWide; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

bool prop2d_wide_bf16_eligible(int64_t planes, int64_t H, int64_t W, const void* x, const void* lam,
                               const void* u, const void* w4, const void* y, const void* acc) {
    if ((H & 3) || (W & 3) || !wide_bf16_side(H) || !wide_bf16_side(W)) return false;
    if (planes > 0x7fffffff || 12 * H * W * 2 > 0x7fffffff) return false;
    return aligned16(x) && aligned16(lam) && aligned16(u) && aligned16(w4) && aligned16(y) && aligned16(acc);
}

hipError_t launch_prop2d_wide_bf16(const void* x_, const void* lam_, const void* u_, const void* w4_,
                                   float eps, void* y_, int64_t planes, int64_t H, int64_t W,
                                   const PropOpts& o, float* acc, hipStream_t stream) {
    const uint16_t* x = static_cast<const uint16_t*>(x_);
    const uint16_t* lam = static_cast<const uint16_t*>(lam_);
    const uint16_t* u = static_cast<const uint16_t*>(u_);
    const uint16_t* w4 = static_cast<const uint16_t*>(w4_);
    uint16_t* y = static_cast<uint16_t*>(y_);
    if (!wide_bf16_side(H) || !wide_bf16_side(W)) return hipErrorInvalidValue;
    return launch_k<uint16_t, 4, 4>(x, lam, u, w4, eps, acc, y, planes, H, W, o, stream);
}

bool prop2d_wide_eligible(int dtype, int64_t planes, int64_t H, int64_t W, const void* x,
                          const void* lam, const void* u, const void* w4, const void* y) {
    if (dtype != 0) return false;                                   // fp32: y is the accumulator
    if (H > kMaxSideWide || W > kMaxSideWide || (H & 3) || (W & 3)) return false;
    if (planes > 0x7fffffff) return false;                          // one workgroup a plane
    return aligned16(x) && aligned16(lam) && aligned16(u) && aligned16(w4) && aligned16(y);
}

hipError_t launch_prop2d_wide(const void* x_, const void* lam_, const void* u_, const void* w4_,
                              float eps, void* y_, int64_t planes, int64_t H, int64_t W,
                              const PropOpts& o, hipStream_t stream) {
    const float* x = static_cast<const float*>(x_);
    const float* lam = static_cast<const float*>(lam_);
    const float* u = static_cast<const float*>(u_);
    const float* w4 = static_cast<const float*>(w4_);
    float* y = static_cast<float*>(y_);
    if (W <= 64) return launch_kc<1>(x, lam, u, w4, eps, y, planes, H, W, o, stream);
    if (W <= 128) return launch_kc<2>(x, lam, u, w4, eps, y, planes, H, W, o, stream);
    if (W <= 192) return launch_kc<3>(x, lam, u, w4, eps, y, planes, H, W, o, stream);
    return launch_kc<4>(x, lam, u, w4, eps, y, planes, H, W, o, stream);
}

}  // namespace gspn
