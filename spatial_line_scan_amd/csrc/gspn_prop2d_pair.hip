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
// Sums.  LDS holds two fp32 planes, zeroed first: R (row-major) receives
// h_TD + h_BU and C (column-major) receives h_LR + h_RL.  Each plane is
// written by one wavefront only.  Every step adds h to the value of its line
// that was read right after the previous step's writes, and writes it back;
// the in-order LDS makes the other half's earlier writes visible to that
// read, so a pixel's two terms are added in a fixed order and the step body
// has no branches.  Padding lines before and after each plane keep the
// look-ahead reads in bounds; slots past the end of a line use a dummy word
// of their lane.  When a scan has an odd number of lines both halves reach
// the middle line in the same step: the forward half writes first, then the
// backward half adds.  After both scans y = u * (R + C).
//
// Streams.  Taps are line-major for every direction, so each half reads its
// line's taps contiguously; x and lambda rows are contiguous for the row
// scans; the column scans read x and lambda in chunks of D columns (16 bytes
// or more) of each of their K rows, loaded a block ahead, which stay resident
// in L2 while the plane is being scanned.  All streams are prefetched D steps
// ahead with buffer loads, which return 0 for every dword outside the tensor
// (offsets below its start wrap to large values and read as 0 too).
//
// Tap groups: plane p = b C + c reads the taps of tap plane p / (C / G) =
// b G + c / (C / G) (channel-shared weights, paper text §4.2).  Chunked
// scans (Chunked): the lines of a scan restart from h = 0 at the first line
// of each segment of ceil(NL / k_chunk) lines in scan order, so that line is
// lambda x (paper text §4.1, chunk index of the grid).
//
// Normalisation: s_k = 1 / (2^(-z_k log2 e) + c_k) with c_k = 1 for in-line
// taps and +inf for dropped ones (s_k exactly 0), r = 1 / max(s_0 + s_1 + s_2,
// eps), h = r (s_0 h_l + s_1 h_c + s_2 h_r) + lambda x.
#include "gspn_device.h"
#include "gspn_internal.h"
#include "gspn_lane.h"

#include <type_traits>

namespace gspn {
namespace {

using namespace lane;

__device__ __forceinline__ float& lds_at(float* lds, uint32_t byte_off) {
    return *reinterpret_cast<float*>(reinterpret_cast<char*>(lds) + byte_off);
}

// LDS layout in floats: [pad W][R: H x W][pad W] [pad H][C: W x H][pad H]
// [dummy: 2 x 64] (one dummy word per lane of each wavefront); the row and
// column regions each start at a multiple of 4 floats.
struct PairLayout {
    int rows_end, r0, c0, cols_end, dummy, words;
    __host__ __device__ PairLayout(int H, int W) {
        r0 = W;
        rows_end = (H * W + 2 * W + 3) & ~3;
        c0 = rows_end + H;
        cols_end = (rows_end + H * W + 2 * H + 3) & ~3;
        dummy = cols_end;
        words = dummy + 128;
    }
};

// OddH / OddW: the row / column scans have an odd number of lines.
// Chunked: k_chunk > 1.
template <typename T, int K, int D, bool OddH, bool OddW, bool Chunked>
// Two wavefronts per SIMD: at most 256 VGPRs, so that three planes share a CU.
__global__ void __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2)))
prop2d_pair_kernel(const T* __restrict__ x, const T* __restrict__ lam, const T* __restrict__ u,
                   const T* __restrict__ w4, int w4_bytes, int xl_bytes, float eps,
                   T* __restrict__ y, int planes, int H, int W, int cpg, int k_chunk) {
    constexpr bool kBf16 = sizeof(T) == 2;
    constexpr int ES = sizeof(T);
    constexpr int NW = window_words<T, K>();
    constexpr int CW = D * ES / 4;        // dwords of one D-column chunk
    static_assert(CW % 4 == 0, "chunks are whole 16-byte pieces");
    extern __shared__ float lds[];
    const int HW = H * W;
    const PairLayout lay(H, W);
    float* const R = lds + lay.r0;       // [H][W]
    float* const Cp = lds + lay.c0;      // [W][H]

    // 0: rows, 1: columns (read from lane 0, so that branches on it are uniform)
    const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
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

    // ------------------------------- zero this wavefront's plane and its pads
    {
        const int first = rows ? 0 : lay.rows_end;
        const int count = rows ? lay.rows_end : lay.cols_end - lay.rows_end;
        float4* z4 = reinterpret_cast<float4*>(lds + first);
        for (int f = lane; f < count / 4; f += 64) z4[f] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
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

    // one resource per tap plane k, based k planes into the tap tensor, so
    // that the three tap loads of a step share one offset register
    __amdgpu_buffer_rsrc_t taps[3];
#pragma unroll
    for (int k = 0; k < 3; ++k)
        taps[k] = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(w4 + static_cast<size_t>(k) * HW), 0,
                                                    w4_bytes - k * HW * ES, kBufFlags);
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
    // offset of this lane's window in tap plane 0 of its direction
    const int tap_planes = planes / cpg;
    const uint32_t tap_b =
        static_cast<uint32_t>(((g * tap_planes + plane / cpg) * 3) * HW) * ES + win_b;
    // Row scans: x and lambda of the current row, same window.
    const uint32_t xl_row_b = static_cast<uint32_t>(pix0) * ES + win_b;
    // Column scans: x and lambda of rows K q + j, D columns per chunk.
    uint32_t xl_col_b[K];
#pragma unroll
    for (int j = 0; j < K; ++j)
        xl_col_b[j] = static_cast<uint32_t>(pix0 + static_cast<size_t>(K * q + j) * W) * ES;

    // The scan of one wavefront; the row and column scans differ only in
    // where x and lambda come from and in which sum plane they fill.
    auto scan = [&](auto rows_tag, auto odd_tag) {
        constexpr bool kRows = decltype(rows_tag)::value;
        constexpr bool kOdd = decltype(odd_tag)::value;   // odd number of lines
        // Tap and x/lambda streams for the line of step s (D steps ahead).
        const uint32_t lo0 = fwd ? 0u : static_cast<uint32_t>(NL - 1) * line_b;
        const uint32_t dlo = fwd ? line_b : 0u - line_b;
        uint32_t lo = tap_b + lo0;                  // taps of the line loaded next
        uint32_t xo = xl_row_b + lo0;               // x and lambda (row scans)
        words_t<NW> tbuf[D][3];
        words_t<NW> xbuf[kRows ? D : 1], lbuf[kRows ? D : 1];
        auto load_line = [&](int d) {
#pragma unroll
            for (int k = 0; k < 3; ++k) tbuf[d][k] = load_words<NW>(taps[k], lo);
            lo += dlo;
            if constexpr (kRows) {
                xbuf[d] = load_words<NW>(xs, xo);
                lbuf[d] = load_words<NW>(ls, xo);
                xo += dlo;
            }
        };
        // Column scans: x and lambda of the lane's rows K q + j for the D
        // columns of a block, as CW dwords in ascending address order (one
        // 16-byte load per 4 dwords): forward lanes take a block's columns
        // s0 .. s0+D-1, backward lanes W-D-s0 .. W-1-s0, and one byte permute
        // of (forward word, backward word) decodes both.  Two chunk buffers
        // alternate between blocks; a block's buffer is filled at the start
        // of the previous block.  A backward chunk that would start left of
        // column 0 (the partial last block) starts at column 0 instead; its
        // words are moved into place before that block.
        constexpr int KC = kRows ? 1 : K;
        constexpr int CQ = CW / 4;             // 16-byte pieces per chunk
        using chunk_t = words_t<4>[KC][CQ];
        chunk_t xcA, lcA, xcB, lcB;
        uint32_t xl_col_b[KC];
#pragma unroll
        for (int j = 0; j < KC; ++j)
            xl_col_b[j] = static_cast<uint32_t>(pix0 + static_cast<size_t>(K * q + j) * W) * ES;
        auto load_chunk = [&](int s0, chunk_t& cx, chunk_t& cl) {
            int c0 = fwd ? s0 : W - D - s0;
            c0 = c0 < 0 ? 0 : c0;
            // an empty asm orders the load after the decodes of the previous
            // block, which read the same registers
            uint32_t cofs = static_cast<uint32_t>(c0 * ES);
            asm volatile("" : "+v"(cofs));
#pragma unroll
            for (int j = 0; j < KC; ++j) {
                const uint32_t o = xl_col_b[j] + cofs;
#pragma unroll
                for (int i = 0; i < CQ; ++i) {
                    cx[j][i] = load_words<4>(xs, o + 16 * i);
                    cl[j][i] = load_words<4>(ls, o + 16 * i);
                }
            }
        };
        // chunk word holding the column of step d of a block
        auto fwd_word = [](int d) { return (d * ES) / 4; };
        auto bwd_word = [](int d) { return ((D - 1 - d) * ES) / 4; };
        // byte selectors: forward word from the first operand, backward word
        // (other half for bf16) from the second
        const uint32_t csel_even = kBf16 ? (fwd ? 0x05040c0cu : 0x03020c0cu) : (fwd ? 0x07060504u : 0x03020100u);
        const uint32_t csel_odd = kBf16 ? (fwd ? 0x07060c0cu : 0x01000c0cu) : csel_even;

        // Prologue: slots in step order, as the loop refills them (the wait
        // counts inside the loop are derived from this order as well).
        if constexpr (!kRows) load_chunk(0, xcA, lcA);
#pragma unroll
        for (int d = 0; d < D; ++d) {
            load_line(d);
            __builtin_amdgcn_sched_barrier(0);
        }

        // LDS byte offset of each slot in this wavefront's sum plane (line-major
        // in its own orientation) and its change per step; a slot past the
        // line end stays on its lane's dummy word.
        const int base = kRows ? lay.r0 : lay.c0;
        const int i0 = fwd ? 0 : NL - 1;
        uint32_t addr[K];
        uint32_t dstep[K];
#pragma unroll
        for (int j = 0; j < K; ++j) {
            addr[j] = 4u * static_cast<uint32_t>(valid[j] ? base + i0 * L + K * q + j
                                                          : lay.dummy + 64 * wv + lane);
            dstep[j] = valid[j] ? (fwd ? 4u * L : 0u - 4u * L) : 0u;
        }
        float h[K], acc[K];
#pragma unroll
        for (int j = 0; j < K; ++j) {
            h[j] = 0.0f;
            acc[j] = lds_at(lds, addr[j]);      // the zeroes stored above
        }
        // Odd scans: both halves reach the middle line in step mid; there the
        // backward half's slots are moved by mid_off to the padding line after
        // the plane, which starts zeroed.
        const int mid = (NL - 1) / 2;
        // Chunked scans: step of the next restart after step 0 (where h is
        // still 0).  Forward lines restart at multiples of the segment
        // length; backward ones at s = 0 and where NL - s is a multiple of it.
        int seg = NL, next_restart = NL;
        if constexpr (Chunked) {
            seg = (NL + k_chunk - 1) / k_chunk;
            next_restart = fwd ? seg : NL - ((NL - 1) / seg) * seg;
        }
        uint32_t mid_off[K];
#pragma unroll
        for (int j = 0; j < K; ++j)
            mid_off[j] = (valid[j] && !fwd) ? 4u * static_cast<uint32_t>((NL - mid) * L) : 0u;

        // Step s with its streams in slot d: decode them, refill slot d for
        // step s + D, advance h and add it into the sum plane.
        auto step = [&](int s, int d, chunk_t& cx, chunk_t& cl) {
            // The slot's words pass through an empty asm here, so that no
            // decode of them is scheduled before this step (it would wait for
            // the most recent loads).
            asm volatile("" : "+v"(tbuf[d][0]), "+v"(tbuf[d][1]), "+v"(tbuf[d][2]));
            if constexpr (kRows) {
                asm volatile("" : "+v"(xbuf[d]), "+v"(lbuf[d]));
            } else {
#pragma unroll
                for (int j = 0; j < KC; ++j) {
                    asm volatile("" : "+v"(cx[j][fwd_word(d) / 4]), "+v"(cl[j][fwd_word(d) / 4]));
                    if (bwd_word(d) / 4 != fwd_word(d) / 4)
                        asm volatile("" : "+v"(cx[j][bwd_word(d) / 4]), "+v"(cl[j][bwd_word(d) / 4]));
                }
            }
            // Everything that does not depend on h: normalised taps and lambda x.
            float s0v[K], s1v[K], s2v[K], r[K], b[K];
#pragma unroll
            for (int j = 0; j < K; ++j) {
                const float z0 = window_elem<T, K, NW>(tbuf[d][0], j, sel_even, sel_odd);
                const float z1 = window_elem<T, K, NW>(tbuf[d][1], j, sel_even, sel_odd);
                const float z2 = window_elem<T, K, NW>(tbuf[d][2], j, sel_even, sel_odd);
                float xv, lv;
                if constexpr (kRows) {
                    xv = window_elem<T, K, NW>(xbuf[d], j, sel_even, sel_odd);
                    lv = window_elem<T, K, NW>(lbuf[d], j, sel_even, sel_odd);
                } else {
                    const int fw = fwd_word(d), bw = bwd_word(d);
                    const uint32_t sel = (d & 1) ? csel_odd : csel_even;
                    xv = __uint_as_float(__builtin_amdgcn_perm(cx[j][fw / 4][fw % 4], cx[j][bw / 4][bw % 4], sel));
                    lv = __uint_as_float(__builtin_amdgcn_perm(cl[j][fw / 4][fw % 4], cl[j][bw / 4][bw % 4], sel));
                }
                b[j] = lv * xv;
                s0v[j] = __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(z0 * kNegLog2e) + c0[j]);
                s1v[j] = __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(z1 * kNegLog2e) + c1[j]);
                s2v[j] = __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(z2 * kNegLog2e) + c2[j]);
                r[j] = __builtin_amdgcn_rcpf(fmaxf((s0v[j] + s1v[j]) + s2v[j], eps));
            }
            // Slot d is refilled only after it has been decoded: the refill
            // offsets pass through an empty asm that takes the decoded values,
            // so no load can move above the decode (two live copies of a slot
            // would need register copies that wait for the load).
#pragma unroll
            for (int j = 0; j < K; ++j) {
                if constexpr (kRows)
                    asm volatile("" : "+v"(lo), "+v"(xo)
                                 : "v"(s0v[j]), "v"(s1v[j]), "v"(s2v[j]), "v"(r[j]), "v"(b[j]));
                else
                    asm volatile("" : "+v"(lo)
                                 : "v"(s0v[j]), "v"(s1v[j]), "v"(s2v[j]), "v"(r[j]), "v"(b[j]));
            }
            load_line(d);

            if constexpr (Chunked) {
                // lanes at a segment start go on from h = 0 (values that
                // cross between the two halves meet dropped taps of weight 0)
                const bool restart = s == next_restart;
                next_restart = restart ? next_restart + seg : next_restart;
#pragma unroll
                for (int j = 0; j < K; ++j) h[j] = restart ? 0.0f : h[j];
            }
            const float hl0 = from_prev(h[K - 1]);
            const float hrK = from_next(h[0]);
            float hn[K];
#pragma unroll
            for (int j = 0; j < K; ++j) {
                const float hl = j > 0 ? h[j - 1] : hl0;
                const float hr = j < K - 1 ? h[j + 1] : hrK;
                float m = s1v[j] * h[j];
                m = fmaf(s0v[j], hl, m);
                m = fmaf(s2v[j], hr, m);
                hn[j] = fmaf(m, r[j], b[j]);
            }
            // slots past the line end hold 0: their windows read the next
            // line, or the next plane, whose values may not be finite, and
            // dropped taps weigh them by 0
#pragma unroll
            for (int j = 0; j < K; ++j) h[j] = valid[j] ? hn[j] : 0.0f;

            // On the middle line of an odd scan the backward half writes to
            // the padding line after the plane instead (added in afterwards).
            const bool at_mid = kOdd && s == mid;
#pragma unroll
            for (int j = 0; j < K; ++j)
                lds_at(lds, at_mid ? addr[j] + mid_off[j] : addr[j]) = acc[j] + h[j];
            // the next line, read after this step's writes
#pragma unroll
            for (int j = 0; j < K; ++j) {
                addr[j] += dstep[j];
                acc[j] = lds_at(lds, addr[j]);
            }
        };

        // Whole blocks of D steps, two per iteration so that the chunk buffers
        // alternate; the streams are refilled unconditionally (past the end
        // they read unused data or 0), so that no branch drains the prefetch
        // queue.  Then the partial last block.
        auto block = [&](int s0, chunk_t& cx, chunk_t& cl, chunk_t& nx, chunk_t& nl) {
            if constexpr (!kRows) load_chunk(s0 + D, nx, nl);
#pragma unroll
            for (int d = 0; d < D; ++d) step(s0 + d, d, cx, cl);
        };
        int s0 = 0;
        for (; s0 + 2 * D <= NL; s0 += 2 * D) {
            block(s0, xcA, lcA, xcB, lcB);
            block(s0 + D, xcB, lcB, xcA, lcA);
        }
        if (s0 + D <= NL) {
            block(s0, xcA, lcA, xcB, lcB);
            s0 += D;
            if constexpr (!kRows) {
#pragma unroll
                for (int j = 0; j < KC; ++j)
#pragma unroll
                    for (int i = 0; i < CQ; ++i) {
                        xcA[j][i] = xcB[j][i];
                        lcA[j][i] = lcB[j][i];
                    }
            }
        }
        if (s0 < NL) {
            if constexpr (!kRows) {
                // The backward chunk of this block starts at column 0 rather
                // than D - T columns to its left (T steps remain): move its words
                // up by that many columns.
                const int sh = ((D - (NL - s0)) * ES) / 4;
                for (int i = 0; i < sh; ++i) {
#pragma unroll
                    for (int j = 0; j < KC; ++j)
#pragma unroll
                        for (int w = CW - 1; w >= 1; --w) {
                            const uint32_t xp = xcA[j][(w - 1) / 4][(w - 1) % 4];
                            const uint32_t lp = lcA[j][(w - 1) / 4][(w - 1) % 4];
                            if (!fwd) {
                                xcA[j][w / 4][w % 4] = xp;
                                lcA[j][w / 4][w % 4] = lp;
                            }
                        }
                }
            }
#pragma unroll
            for (int d = 0; d < D; ++d)
                if (s0 + d < NL) step(s0 + d, d, xcA, lcA);
        }
        if constexpr (kOdd) {
            // the middle line receives the backward half's term last
            if (!fwd) {
#pragma unroll
                for (int j = 0; j < K; ++j) {
                    const uint32_t a = 4u * static_cast<uint32_t>(base + mid * L + K * q + j);
                    if (valid[j]) lds_at(lds, a) = lds_at(lds, a) + lds_at(lds, a + mid_off[j]);
                }
            }
        }
    };
    if (rows) scan(std::true_type{}, std::bool_constant<OddH>{});
    else scan(std::false_type{}, std::bool_constant<OddW>{});
    __syncthreads();

    // ------------------------------------------------------- y = u * (R + C)
    // Thread slot f walks the plane in strides of 128 words; its pixel
    // position advances by whole rows and a remainder instead of a division.
    if constexpr (kBf16) {
        uint32_t* y32 = reinterpret_cast<uint32_t*>(y + pix0);
        const int dq = 256 / W, dr = 256 - dq * W;   // 128 pixel pairs
        int f = threadIdx.x;
        int r0 = (2 * f) / W, c0i = 2 * f - r0 * W;
        auto emit = [&](uint32_t uv) {
            // W is even: the pair (r0, c0i), (r0, c0i + 1) lies in one row
            const float2 rr = *reinterpret_cast<const float2*>(R + r0 * W + c0i);
            const float a0 = rr.x + Cp[c0i * H + r0];
            const float a1 = rr.y + Cp[(c0i + 1) * H + r0];
            y32[f] = pack_bf16x2(__uint_as_float(uv << 16) * a0, __uint_as_float(uv & 0xffff0000u) * a1);
        };
        auto advance = [&]() {
            f += 128;
            c0i += dr;
            r0 += dq;
            if (c0i >= W) { c0i -= W; ++r0; }
        };
#pragma unroll
        for (int k = 0; k < kUPer; ++k) {
            if (f < u_words) emit(ureg[k]);
            advance();
        }
        for (; f < u_words; advance()) emit(u32[f]);
    } else {
        float* yp = reinterpret_cast<float*>(y + pix0);
        const int dq = 128 / W, dr = 128 - dq * W;
        int f = threadIdx.x;
        int r0 = f / W, c0i = f - r0 * W;
        auto advance = [&]() {
            f += 128;
            c0i += dr;
            r0 += dq;
            if (c0i >= W) { c0i -= W; ++r0; }
        };
#pragma unroll
        for (int k = 0; k < kUPer; ++k) {
            if (f < u_words) yp[f] = __uint_as_float(ureg[k]) * (R[f] + Cp[c0i * H + r0]);
            advance();
        }
        for (; f < u_words; advance()) yp[f] = __uint_as_float(u32[f]) * (R[f] + Cp[c0i * H + r0]);
    }
}

template <typename T, int K, bool OddH, bool OddW, bool Chunked>
hipError_t launch_k(const void* x, const void* lam, const void* u, const void* w4, float eps,
                    void* y, int64_t planes, int64_t H, int64_t W, const PropOpts& o,
                    hipStream_t stream) {
    // prefetch depth: D steps of every stream in registers
    constexpr int D = (sizeof(T) == 4 && K == 3) ? 4 : 8;
    const size_t lds =
        static_cast<size_t>(PairLayout(static_cast<int>(H), static_cast<int>(W)).words) * sizeof(float);
    auto kern = prop2d_pair_kernel<T, K, D, OddH, OddW, Chunked>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(lds));
        if (e != hipSuccess) return e;
    }
    const int64_t n = planes * H * W;
    kern<<<dim3(static_cast<unsigned>(planes)), dim3(128), lds, stream>>>(
        static_cast<const T*>(x), static_cast<const T*>(lam), static_cast<const T*>(u),
        static_cast<const T*>(w4), static_cast<int>(12 * (n / o.cpg) * sizeof(T)),
        static_cast<int>(n * sizeof(T)), eps, static_cast<T*>(y), static_cast<int>(planes),
        static_cast<int>(H), static_cast<int>(W), static_cast<int>(o.cpg),
        static_cast<int>(o.k_chunk));
    return hipGetLastError();
}

template <typename T, int K, bool Chunked>
hipError_t launch_parity(const void* x, const void* lam, const void* u, const void* w4, float eps,
                         void* y, int64_t planes, int64_t H, int64_t W, const PropOpts& o,
                         hipStream_t stream) {
    if constexpr (sizeof(T) == 2) {  // bf16 shapes are even (eligibility)
        return launch_k<T, K, false, false, Chunked>(x, lam, u, w4, eps, y, planes, H, W, o, stream);
    } else {
        const bool oh = H & 1, ow = W & 1;
        if (!oh && !ow)
            return launch_k<T, K, false, false, Chunked>(x, lam, u, w4, eps, y, planes, H, W, o, stream);
        if (oh && ow)
            return launch_k<T, K, true, true, Chunked>(x, lam, u, w4, eps, y, planes, H, W, o, stream);
        if (oh)
            return launch_k<T, K, true, false, Chunked>(x, lam, u, w4, eps, y, planes, H, W, o, stream);
        return launch_k<T, K, false, true, Chunked>(x, lam, u, w4, eps, y, planes, H, W, o, stream);
    }
}

template <typename T, bool Chunked>
hipError_t launch_c(const void* x, const void* lam, const void* u, const void* w4, float eps,
                    void* y, int64_t planes, int64_t H, int64_t W, const PropOpts& o,
                    hipStream_t stream) {
    const int64_t Lmax = H > W ? H : W;
    if (Lmax <= 32) return launch_parity<T, 1, Chunked>(x, lam, u, w4, eps, y, planes, H, W, o, stream);
    if (Lmax <= 64) return launch_parity<T, 2, Chunked>(x, lam, u, w4, eps, y, planes, H, W, o, stream);
    return launch_parity<T, 3, Chunked>(x, lam, u, w4, eps, y, planes, H, W, o, stream);
}

template <typename T>
hipError_t launch_t(const void* x, const void* lam, const void* u, const void* w4, float eps,
                    void* y, int64_t planes, int64_t H, int64_t W, const PropOpts& o,
                    hipStream_t stream) {
    return o.k_chunk > 1 ? launch_c<T, true>(x, lam, u, w4, eps, y, planes, H, W, o, stream)
                         : launch_c<T, false>(x, lam, u, w4, eps, y, planes, H, W, o, stream);
}

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

}  // namespace

bool prop2d_pair_eligible(int dtype, int64_t planes, int64_t H, int64_t W, const void* x,
                          const void* lam, const void* u, const void* w4, const void* y) {
    if (H > 96 || W > 96) return false;
    if (4 * static_cast<int64_t>(PairLayout(static_cast<int>(H), static_cast<int>(W)).words) >
        kLdsBytes)
        return false;
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
                              const PropOpts& o, hipStream_t stream) {
    return dtype == 0 ? launch_t<float>(x, lam, u, w4, eps, y, planes, H, W, o, stream)
                      : launch_t<uint16_t>(x, lam, u, w4, eps, y, planes, H, W, o, stream);
}

}  // namespace gspn
