// Four-direction propagation, two wavefronts per (b, c) plane (gfx950).
//
// Operator: "Scaling Parallel Sequence Models to Foundation-Scale Vision
// Encoders", §3 line-scan recurrence (standard GSPN form), §4.1 single-kernel
// design, §4.3 coalesced access with the hidden state kept on chip, §5.1
// fused normalisation (sigmoid, local sum, clamp, divide); reading notes,
// method / overall framework (three-tap neighbourhood, row-stochastic taps,
// four directions).
//
// Work split.  A workgroup of two wavefronts owns one plane.  Wavefront 0
// scans the rows: lanes 0-31 top-down, lanes 32-63 bottom-up.  Wavefront 1
// scans the columns: lanes 0-31 left-right, lanes 32-63 right-left.  Within a
// 32-lane half, lane q holds the K consecutive positions Kq .. Kq+K-1 of the
// current line in registers; the tridiagonal neighbour exchange is one
// wave-wide DPP shift in each direction (across the boundary between the two
// halves the shifted value meets a dropped tap of weight exactly 0).
//
// Sums.  LDS holds two fp32 planes: R (row-major) receives h_TD + h_BU and
// C (column-major) receives h_LR + h_RL; each plane is written by one
// wavefront only, and each of its lines is visited twice (once per
// direction): the first visit writes, the second reads (issued one step
// ahead), adds and writes.  Every pixel's sum therefore has a fixed order.
// After both scans y = u * (R + C).
//
// Streams.  Taps are line-major for every direction, so each half reads its
// line's taps contiguously; x and lambda rows are contiguous for the row
// scans; the column scans read x and lambda in chunks of D columns of their
// K rows, which stay resident in L2 while the plane is being scanned.  All
// streams are prefetched D steps ahead with buffer loads, which return 0
// outside the tensor (offsets below its start wrap to large values and read
// as 0 too).
//
// Normalisation: s_k = 1 / (2^(-z_k log2 e) + c_k) with c_k = 1 for in-line
// taps and +inf for dropped ones (s_k exactly 0), r = 1 / max(s_0 + s_1 + s_2,
// eps), h = r (s_0 h_l + s_1 h_c + s_2 h_r) + lambda x.
#include "gspn_device.h"
#include "gspn_internal.h"

#include <type_traits>

namespace gspn {
namespace {

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

// NW consecutive dwords at byte offset `off` of a buffer.
template <int NW>
__device__ __forceinline__ void load_words(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t* dst) {
    int w = 0;
#pragma unroll
    for (; w + 4 <= NW; w += 4) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off + 4 * w, 0, 0);
        dst[w] = v[0]; dst[w + 1] = v[1]; dst[w + 2] = v[2]; dst[w + 3] = v[3];
    }
    if constexpr (NW % 4 == 3) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b96(r, off + 4 * w, 0, 0);
        dst[w] = v[0]; dst[w + 1] = v[1]; dst[w + 2] = v[2];
    } else if constexpr (NW % 4 == 2) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off + 4 * w, 0, 0);
        dst[w] = v[0]; dst[w + 1] = v[1];
    } else if constexpr (NW % 4 == 1) {
        dst[w] = __builtin_amdgcn_raw_buffer_load_b32(r, off + 4 * w, 0, 0);
    }
}

// Dwords covering K consecutive elements starting at an element of parity
// `par` (bf16: the window starts at the even element below).
template <typename T, int K>
constexpr int window_words() {
    return sizeof(T) == 4 ? K : ((K % 2) ? (K + 1) / 2 : K / 2);
}

// Element j of a lane's window as fp32.
template <typename T, int K, int NW>
__device__ __forceinline__ float window_elem(const uint32_t (&w)[NW], int j, uint32_t sel_even,
                                             uint32_t sel_odd) {
    if constexpr (sizeof(T) == 4) {
        return __uint_as_float(w[j]);
    } else {
        const int a = j >> 1;
        const uint32_t lo = w[a];
        const uint32_t hi = (a + 1 < NW) ? w[a + 1] : lo;
        return __uint_as_float(__builtin_amdgcn_perm(hi, lo, (j & 1) ? sel_odd : sel_even));
    }
}

template <typename T, int K, int D>
__global__ void __launch_bounds__(128)
prop2d_pair_kernel(const T* __restrict__ x, const T* __restrict__ lam, const T* __restrict__ u,
                   const T* __restrict__ w4, int w4_bytes, int xl_bytes, float eps,
                   T* __restrict__ y, int planes, int H, int W) {
    constexpr bool kBf16 = sizeof(T) == 2;
    constexpr int ES = sizeof(T);
    constexpr int NW = window_words<T, K>();
    constexpr int CW = D * ES / 4;        // dwords of one D-column chunk
    static_assert(D % 2 == 0 && CW >= 1, "chunks are whole dwords");
    extern __shared__ float lds[];
    const int HW = H * W;
    float* const R = lds;                // [H][W]
    float* const Cp = lds + HW;          // [W][H]

    const int wv = threadIdx.x >> 6;     // 0: rows, 1: columns
    const int lane = threadIdx.x & 63;
    const int half = lane >> 5;          // 0: forward (TD, LR), 1: backward (BU, RL)
    const int q = lane & 31;
    const bool rows = wv == 0;
    const int g = 2 * wv + half;         // direction TD, BU, LR, RL
    const int L = rows ? W : H;
    const int NL = rows ? H : W;
    const bool fwd = half == 0;
    const int plane = blockIdx.x;
    const size_t pix0 = static_cast<size_t>(plane) * HW;

    // ------------------------------------------------ u, prefetched for the end
    constexpr int kUPer = 24;            // per-thread dwords of u kept in registers
    const int u_words = kBf16 ? HW / 2 : HW;
    uint32_t ureg[kUPer];
    const uint32_t* u32 = reinterpret_cast<const uint32_t*>(u + pix0);
#pragma unroll
    for (int k = 0; k < kUPer; ++k) {
        const int f = static_cast<int>(threadIdx.x) + 128 * k;
        ureg[k] = f < u_words ? u32[f] : 0u;
    }

    // ------------------------------------------------------- per-lane constants
    float c0[K], c1[K], c2[K];
    bool valid[K];
    const float inf = __builtin_inff();
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const int p = K * q + j;
        valid[j] = p < L;
        c0[j] = (valid[j] && p > 0) ? 1.0f : inf;
        c1[j] = valid[j] ? 1.0f : inf;
        c2[j] = (valid[j] && p < L - 1) ? 1.0f : inf;
    }

    const __amdgpu_buffer_rsrc_t taps =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(w4), 0, w4_bytes, kBufFlags);
    const __amdgpu_buffer_rsrc_t xs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(x), 0, xl_bytes, kBufFlags);
    const __amdgpu_buffer_rsrc_t ls =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(lam), 0, xl_bytes, kBufFlags);

    // Lane window inside a line: K elements from K q, read from the even
    // element at or below it (bf16).
    const int par = kBf16 ? ((K * q) & 1) : 0;
    const uint32_t win_b = static_cast<uint32_t>(K * q - par) * ES;
    const uint32_t sel_even = par ? 0x03020c0cu : 0x01000c0cu;
    const uint32_t sel_odd = par ? 0x05040c0cu : 0x03020c0cu;
    const uint32_t line_b = static_cast<uint32_t>(L) * ES;
    uint32_t tap_b[3];
#pragma unroll
    for (int k = 0; k < 3; ++k)
        tap_b[k] = static_cast<uint32_t>((((g * planes + plane) * 3 + k) * HW)) * ES + win_b;
    // Row scans: x and lambda of the current row, same window.
    const uint32_t xl_row_b = static_cast<uint32_t>(pix0) * ES + win_b;
    // Column scans: x and lambda of rows K q + j, D columns per chunk.
    uint32_t xl_col_b[K];
#pragma unroll
    for (int j = 0; j < K; ++j)
        xl_col_b[j] = static_cast<uint32_t>(pix0 + static_cast<size_t>(K * q + j) * W) * ES;

    // The scan of one wavefront; the row and column scans differ only in
    // where x and lambda come from and in which sum plane they fill.
    auto scan = [&](auto rows_tag) {
        constexpr bool kRows = decltype(rows_tag)::value;
        // Tap and x/lambda streams for the line of step s (D steps ahead).
        uint32_t lo = fwd ? 0u : static_cast<uint32_t>(NL - 1) * line_b;
        const uint32_t dlo = fwd ? line_b : 0u - line_b;
        uint32_t tbuf[D][3][NW];
        uint32_t xbuf[kRows ? D : 1][NW], lbuf[kRows ? D : 1][NW];
        auto load_line = [&](int d) {
    #pragma unroll
            for (int k = 0; k < 3; ++k) load_words<NW>(taps, tap_b[k] + lo, tbuf[d][k]);
            if constexpr (kRows) {
                load_words<NW>(xs, xl_row_b + lo, xbuf[d]);
                load_words<NW>(ls, xl_row_b + lo, lbuf[d]);
            }
            lo += dlo;
        };
        // Column-scan chunks: the D columns a block of steps visits, for each
        // of the lane's K rows, one dword per load.  Dword w holds the
        // columns of steps EPD w .. EPD w + EPD - 1 in visiting order: forward
        // scans read ascending addresses, backward scans descending ones, so
        // both index a step's element by the same static position.  The last
        // chunk of a backward scan reaches left of column 0; those dwords
        // lie below the row (first row of the tensor: below its start, where
        // the offset wraps and the load reads 0) and are never used.
        constexpr int EPD = 4 / ES;            // elements per dword
        constexpr int KC = kRows ? 1 : K;     // chunk rows (unused by the row scans)
        uint32_t xc0[KC][CW], lc0[KC][CW], xc1[KC][CW], lc1[KC][CW];
        const int cstep = fwd ? 4 : -4;
        auto load_chunk = [&](int s0, uint32_t (&cx)[KC][CW], uint32_t (&cl)[KC][CW]) {
            const int cfirst = fwd ? s0 : W - EPD - s0;   // column of dword 0
#pragma unroll
            for (int j = 0; j < KC; ++j) {
                const uint32_t off = xl_col_b[j] + static_cast<uint32_t>(cfirst * ES);
#pragma unroll
                for (int w = 0; w < CW; ++w) {
                    const uint32_t o = off + static_cast<uint32_t>(cstep * w);
                    cx[j][w] = __builtin_amdgcn_raw_buffer_load_b32(xs, o, 0, 0);
                    cl[j][w] = __builtin_amdgcn_raw_buffer_load_b32(ls, o, 0, 0);
                }
            }
        };
        // bf16 half of a chunk dword visited at even / odd steps
        const uint32_t csel_even = fwd ? 0x01000c0cu : 0x03020c0cu;
        const uint32_t csel_odd = fwd ? 0x03020c0cu : 0x01000c0cu;

    #pragma unroll
        for (int d = 0; d < D; ++d) load_line(d);
        if constexpr (!kRows) load_chunk(0, xc0, lc0);

        // This wave's sum plane, line-major in its own orientation.
        float* const P = kRows ? R : Cp;
        const int i0 = fwd ? 0 : NL - 1;
        float* pl = P + i0 * L + K * q;                       // slot 0 of the current line
        const int dpl = fwd ? L : -L;
        float prev[K];                                        // second-visit reads, one step ahead

        float h[K];
    #pragma unroll
        for (int j = 0; j < K; ++j) {
            h[j] = 0.0f;
            prev[j] = 0.0f;
        }

        // One block of D steps; cx/cl hold this block's column chunks and the
        // next block's are loaded into nx/nl.
        auto run_block = [&](int s0, const uint32_t (&cx)[KC][CW], const uint32_t (&cl)[KC][CW],
                             uint32_t (&nx)[KC][CW], uint32_t (&nl)[KC][CW]) {
            if constexpr (!kRows) {
                if (s0 + D < NL) load_chunk(s0 + D, nx, nl);
            }
    #pragma unroll
            for (int d = 0; d < D; ++d) {
                const int s = s0 + d;
                if (s >= NL) break;
                float z[3][K], b[K];
    #pragma unroll
                for (int j = 0; j < K; ++j) {
    #pragma unroll
                    for (int k = 0; k < 3; ++k)
                        z[k][j] = window_elem<T, K, NW>(tbuf[d][k], j, sel_even, sel_odd);
                    float xv, lv;
                    if constexpr (kRows) {
                        xv = window_elem<T, K, NW>(xbuf[d], j, sel_even, sel_odd);
                        lv = window_elem<T, K, NW>(lbuf[d], j, sel_even, sel_odd);
                    } else {
                        if constexpr (kBf16) {
                            const uint32_t sel = (d & 1) ? csel_odd : csel_even;
                            xv = __uint_as_float(__builtin_amdgcn_perm(cx[j][d >> 1], cx[j][d >> 1], sel));
                            lv = __uint_as_float(__builtin_amdgcn_perm(cl[j][d >> 1], cl[j][d >> 1], sel));
                        } else {
                            xv = __uint_as_float(cx[j][d]);
                            lv = __uint_as_float(cl[j][d]);
                        }
                    }
                    b[j] = lv * xv;
                }
                load_line(d);

                const float hl0 = from_prev(h[K - 1]);
                const float hrK = from_next(h[0]);
                float hn[K];
    #pragma unroll
                for (int j = 0; j < K; ++j) {
                    const float hl = j > 0 ? h[j - 1] : hl0;
                    const float hr = j < K - 1 ? h[j + 1] : hrK;
                    const float s0v = __builtin_amdgcn_rcpf(
                        __builtin_amdgcn_exp2f(z[0][j] * kNegLog2e) + c0[j]);
                    const float s1v = __builtin_amdgcn_rcpf(
                        __builtin_amdgcn_exp2f(z[1][j] * kNegLog2e) + c1[j]);
                    const float s2v = __builtin_amdgcn_rcpf(
                        __builtin_amdgcn_exp2f(z[2][j] * kNegLog2e) + c2[j]);
                    const float r = __builtin_amdgcn_rcpf(fmaxf((s0v + s1v) + s2v, eps));
                    float m = s1v * h[j];
                    m = fmaf(s0v, hl, m);
                    m = fmaf(s2v, hr, m);
                    hn[j] = fmaf(m, r, b[j]);
                }
    #pragma unroll
                for (int j = 0; j < K; ++j) h[j] = hn[j];

                // Visits of this line: first (2s < NL-1) write, second (2s > NL-1)
                // add to the value read one step ahead; the middle line of an odd
                // scan is visited by both halves in this step: forward writes,
                // then backward reads it back and adds.
                const int twice = 2 * s;
                if (twice < NL - 1) {
    #pragma unroll
                    for (int j = 0; j < K; ++j)
                        if (valid[j]) pl[j] = h[j];
                } else if (twice > NL - 1) {
    #pragma unroll
                    for (int j = 0; j < K; ++j)
                        if (valid[j]) pl[j] = prev[j] + h[j];
                } else {
                    if (fwd) {
    #pragma unroll
                        for (int j = 0; j < K; ++j)
                            if (valid[j]) pl[j] = h[j];
                    }
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                    __builtin_amdgcn_wave_barrier();
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                    if (!fwd) {
    #pragma unroll
                        for (int j = 0; j < K; ++j)
                            if (valid[j]) pl[j] = pl[j] + h[j];
                    }
                }
                pl += dpl;
                if (2 * (s + 1) > NL - 1 && s + 1 < NL) {
    #pragma unroll
                    for (int j = 0; j < K; ++j) prev[j] = valid[j] ? pl[j] : 0.0f;
                }
            }
        };
        for (int s0 = 0; s0 < NL; s0 += 2 * D) {
            run_block(s0, xc0, lc0, xc1, lc1);
            if (s0 + D < NL) run_block(s0 + D, xc1, lc1, xc0, lc0);
        }
    };
    if (rows) scan(std::true_type{});
    else scan(std::false_type{});
    __syncthreads();

    // ------------------------------------------------------- y = u * (R + C)
    if constexpr (kBf16) {
        uint32_t* y32 = reinterpret_cast<uint32_t*>(y + pix0);
#pragma unroll
        for (int k = 0; k < kUPer; ++k) {
            const int f = static_cast<int>(threadIdx.x) + 128 * k;
            if (f < u_words) {
                const int p0 = 2 * f;                         // even pixel, same row as p0 + 1
                const int r0 = p0 / W, c0i = p0 - r0 * W;
                const float a0 = R[p0] + Cp[c0i * H + r0];
                const float a1 = R[p0 + 1] + Cp[(c0i + 1) * H + r0];
                const uint32_t uv = ureg[k];
                const uint32_t lo16 = bf16_rne(__uint_as_float(uv << 16) * a0);
                const uint32_t hi16 = bf16_rne(__uint_as_float(uv & 0xffff0000u) * a1);
                y32[f] = lo16 | (hi16 << 16);
            }
        }
        for (int f = static_cast<int>(threadIdx.x) + 128 * kUPer; f < u_words; f += 128) {
            const int p0 = 2 * f;
            const int r0 = p0 / W, c0i = p0 - r0 * W;
            const float a0 = R[p0] + Cp[c0i * H + r0];
            const float a1 = R[p0 + 1] + Cp[(c0i + 1) * H + r0];
            const uint32_t uv = u32[f];
            y32[f] = bf16_rne(__uint_as_float(uv << 16) * a0) |
                     (static_cast<uint32_t>(bf16_rne(__uint_as_float(uv & 0xffff0000u) * a1)) << 16);
        }
    } else {
        float* yp = reinterpret_cast<float*>(y + pix0);
#pragma unroll
        for (int k = 0; k < kUPer; ++k) {
            const int f = static_cast<int>(threadIdx.x) + 128 * k;
            if (f < u_words) {
                const int r0 = f / W, c0i = f - r0 * W;
                yp[f] = __uint_as_float(ureg[k]) * (R[f] + Cp[c0i * H + r0]);
            }
        }
        for (int f = static_cast<int>(threadIdx.x) + 128 * kUPer; f < u_words; f += 128) {
            const int r0 = f / W, c0i = f - r0 * W;
            yp[f] = __uint_as_float(u32[f]) * (R[f] + Cp[c0i * H + r0]);
        }
    }
}

template <typename T, int K>
hipError_t launch_k(const void* x, const void* lam, const void* u, const void* w4, float eps,
                    void* y, int64_t planes, int64_t H, int64_t W, hipStream_t stream) {
    constexpr int D = 8;
    const size_t lds = static_cast<size_t>(2 * H * W) * sizeof(float);
    auto kern = prop2d_pair_kernel<T, K, D>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(lds));
        if (e != hipSuccess) return e;
    }
    const int64_t n = planes * H * W;
    kern<<<dim3(static_cast<unsigned>(planes)), dim3(128), lds, stream>>>(
        static_cast<const T*>(x), static_cast<const T*>(lam), static_cast<const T*>(u),
        static_cast<const T*>(w4), static_cast<int>(12 * n * sizeof(T)),
        static_cast<int>(n * sizeof(T)), eps, static_cast<T*>(y), static_cast<int>(planes),
        static_cast<int>(H), static_cast<int>(W));
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const void* x, const void* lam, const void* u, const void* w4, float eps,
                    void* y, int64_t planes, int64_t H, int64_t W, hipStream_t stream) {
    const int64_t Lmax = H > W ? H : W;
    if (Lmax <= 32) return launch_k<T, 1>(x, lam, u, w4, eps, y, planes, H, W, stream);
    if (Lmax <= 64) return launch_k<T, 2>(x, lam, u, w4, eps, y, planes, H, W, stream);
    return launch_k<T, 3>(x, lam, u, w4, eps, y, planes, H, W, stream);
}

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

}  // namespace

bool prop2d_pair_eligible(int dtype, int64_t planes, int64_t H, int64_t W, const void* x,
                          const void* lam, const void* u, const void* w4, const void* y) {
    if (H > 96 || W > 96) return false;
    if (2 * H * W * 4 > kLdsBytes) return false;
    // all stream offsets are 32-bit byte offsets into one buffer resource
    const int64_t es = dtype == 0 ? 4 : 2;
    if (12 * planes * H * W * es > 0x7fffffff) return false;
    if (dtype == 1) {  // bf16: whole dwords per line, per plane and per chunk
        if ((H & 1) || (W & 1)) return false;
        if (!aligned4(x) || !aligned4(lam) || !aligned4(u) || !aligned4(w4) || !aligned4(y))
            return false;
    }
    return true;
}

hipError_t launch_prop2d_pair(const void* x, const void* lam, const void* u, const void* w4,
                              float eps, void* y, int dtype, int64_t planes, int64_t H, int64_t W,
                              hipStream_t stream) {
    return dtype == 0 ? launch_t<float>(x, lam, u, w4, eps, y, planes, H, W, stream)
                      : launch_t<uint16_t>(x, lam, u, w4, eps, y, planes, H, W, stream);
}

}  // namespace gspn
