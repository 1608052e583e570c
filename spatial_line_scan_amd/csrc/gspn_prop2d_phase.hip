// Four-direction propagation of bf16 planes with sides up to 160, one
// workgroup per (b, c) plane in two phases (gfx950).  fp32 planes take the
// two-wavefront kernel: their 4-byte lambda x would not leave room for four
// planes per CU.
//
// Operator: "Scaling Parallel Sequence Models to Foundation-Scale Vision
// Encoders", §3 line-scan recurrence (standard GSPN form), §4.1 single-kernel
// design, §4.3 hidden state kept on chip, §5.1 fused normalisation (sigmoid,
// local sum, clamp, divide); reading notes, method / overall framework.
//
// Work split.  One workgroup owns one plane and scans it twice: first the
// rows (one half of its lanes top-down, the other bottom-up), then the
// columns (left-right, right-left).  The halves are either the two 32-lane
// halves of one wavefront or two whole wavefronts (when fewer than four
// planes per CU are resident, or there are fewer planes than SIMDs): within
// a half, lane q holds positions Kq .. Kq+K-1 of the current line in
// registers and the neighbour exchange is one wave-wide DPP shift each way
// (across the 32-lane halves the shifted value meets a dropped tap of weight
// 0).  K = 1 .. 5 for lines up to 32, 64, 96, 128, 160 positions (32-lane
// halves) or 1 .. 3 for lines up to 64, 128, 192 (64-lane halves); a 148 x
// 148 plane takes 155 KB of LDS, one plane per CU.
//
// On-chip data.  LDS holds, per plane:
//   S  fp32 [H][W]: the sum of the four directional states, zeroed first;
//      every step adds h into the value of its line read one step earlier.
//      With one wavefront all the adds run in program order; two wavefronts
//      meet at one barrier a phase, at its middle step, which separates the
//      two updates every pixel gets in the phase.  Either way the four terms
//      of a pixel are summed in a fixed order (TD or BU first, then LR or
//      RL) and no two lanes ever update one word at once.
//   b = lambda x of every pixel, computed once from coalesced loads of x and
//      lambda: the exact product of two bf16 values has at most 16
//      significant bits, so its fp32 pattern ends in 8 zero bits and it is
//      kept as 24 bits, the upper 16 in one array and the next 8 in another
//      (3 bytes a pixel instead of 4).
// With b on chip, the scans stream only the taps (line-major for every
// direction, one coalesced window load per tap and step); x and lambda are
// read once, whole, and never along a column.  At 74 x 74 bf16 a plane takes
// 39 KB, so four planes share a CU, one wavefront per SIMD.
//
// Padding.  S and the b arrays are surrounded by pads of one longest line,
// so that the one-step-ahead reads past either end of a scan stay inside the
// allocation; slots past the end of a line all read and write dummy words at
// LDS address 0 (zeroed; such a slot's taps are all dropped, so no
// in-line position ever weighs its state).  With an even number of lines the
// two halves of a scan never meet on one line in the same step.
//
// Tap groups and chunked scans as in the two-wavefront kernel: the tap plane
// of plane p is p / cpg, and a chunked scan restarts h at the first line of
// each segment of ceil(NL / k_chunk) lines.
#include "gspn_device.h"
#include "gspn_internal.h"
#include "gspn_lane.h"

#include <type_traits>

namespace gspn {
namespace {

using namespace lane;

// LDS layout in bytes (all offsets multiples of 16):
//   [S dummy: 16][b dummy: 16][pad Lmax][S: H W][pad Lmax][side: Lmax] fp32,
//   [pad][b_hi: H W][pad] u16, [pad][b_lo: H W][pad] u8
// Slots past a line end all use the dummies: their S reads and writes go to
// the S dummy, their b reads in the column scan to the b dummy (zero, never
// written) and their b writes in the row scan to the pads before the b
// arrays.  Their taps are all dropped, so no in-line position ever weighs
// their (finite) states.
// side: one line of fp32 where, with an odd number of lines, the backward
// scan order puts its terms of the middle line (both orders reach it in the
// same step); zeroed with S, added into S after the phase.
struct PhaseLayout {
    int s, side, bh, bl, bytes;
    static constexpr int dum = 0, bdum = 16;
    __host__ __device__ static int a16(int v) { return (v + 15) & ~15; }
    __host__ __device__ PhaseLayout(int H, int W) {
        const int lmax = H > W ? H : W;
        const int hw = H * W;
        s = a16(32 + 4 * lmax);
        side = a16(s + 4 * hw + 4 * lmax);
        bh = a16(side + 4 * lmax + 2 * lmax);
        bl = a16(bh + 2 * (hw + lmax) + lmax);
        bytes = a16(bl + hw + lmax);
    }
};

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
template <typename V> using lds_t = __attribute__((address_space(3))) V;

// Orders this wavefront's LDS accesses before the fence against those after
// it (one wavefront per workgroup: no barrier, and global loads in flight
// are not waited for).
__device__ __forceinline__ void lds_order() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
}

// Two wavefronts: their LDS accesses before this point complete before
// either wavefront's after it (LDS only: global loads in flight stay so).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <typename V>
__device__ __forceinline__ lds_t<V>& lds_ref(uint32_t byte_off) {
    // the kernel's only LDS is its dynamic array, which starts at address 0
    return *reinterpret_cast<lds_t<V>*>(static_cast<uintptr_t>(byte_off));
}

// T: bf16 bits (uint16_t).  Chunked: k_chunk > 1.  NH: lanes a scan order
// takes: 32 (the two halves of one wavefront) or 64 (one wavefront each).
// Odd: H or W may be odd (then lines and planes start at any element; see
// the window notes in phase()).
template <typename T, int K, int D, bool Chunked, int NH, bool Odd>
__global__ void __launch_bounds__(2 * NH)
prop2d_phase_kernel(const T* __restrict__ x, const T* __restrict__ lam, const T* __restrict__ u,
                    const T* __restrict__ w4, int w4_bytes, float eps, T* __restrict__ y,
                    int planes, int H, int W, int cpg, int k_chunk) {
    static_assert(sizeof(T) == 2, "bf16 planes only");
    static_assert(!Odd || D % 2 == 0, "odd lines: the window parity alternates with the ring slot");
    constexpr int ES = sizeof(T);
    // words a window decodes from, and words loaded for it: with Odd a
    // window is loaded from the even element at or below its first and
    // shifted into place, which for even K takes one more word
    constexpr int NW = Odd ? (K + 1) / 2 : window_words<T, K>();
    constexpr int NWL = Odd && (K % 2 == 0) ? NW + 1 : NW;
    const int HW = H * W;
    const PhaseLayout lay(H, W);
    constexpr int NT = 2 * NH;           // threads of the workgroup
    constexpr bool kTwo = NH == 64;
    const int tid = threadIdx.x;
    const int half = tid / NH;           // 0: forward (TD, LR), 1: backward (BU, RL)
    const int q = tid % NH;
    const bool fwd = half == 0;
    // orders the LDS accesses of the scan orders' lanes
    auto sync = [&]() {
        if constexpr (kTwo) lds_barrier();
        else lds_order();
    };
    const int plane = blockIdx.x;
    const size_t pix0 = static_cast<size_t>(plane) * HW;

    // ---------------------------------------- zero S, its pads and dummies
    // [0, bh): the dummy words, S with its pads, and the pad before b_hi
    for (int f = tid; f < lay.bh / 16; f += NT) lds_ref<u32x4_t>(16u * f) = u32x4_t{0u, 0u, 0u, 0u};

    const int words = HW / 2;     // two pixels a dword (Odd: and a last pixel)
    // u for the end, in dword pairs, loaded now so that it arrives during
    // the scans (a trailing odd dword is loaded at the end).  With Odd a
    // plane may start at any element: the pairs are then 2-byte aligned,
    // which global loads and stores allow.
    constexpr int kUPer = kTwo ? 12 : 24;
    const int pairs = words / 2;
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    // (the attribute is kept only on the named type: no template may carry
    // it, or the compiler takes the 8-byte alignment back)
    typedef uint32_t u32x2_u __attribute__((ext_vector_type(2), aligned(2)));
    const u32x2_u* u64p = reinterpret_cast<const u32x2_u*>(u + pix0);
    u32x2_t ureg[kUPer];
#pragma unroll
    for (int k = 0; k < kUPer; ++k) {
        const int f = tid + NT * k;
        ureg[k] = f < pairs ? u64p[f] : u32x2_t{0u, 0u};
    }
    sync();

    // LDS address of b at element index e
    auto b_addr_hi = [&](int e) { return static_cast<uint32_t>(lay.bh + 2 * e); };
    auto b_addr_lo = [&](int e) { return static_cast<uint32_t>(lay.bl + e); };

    // one resource per tap plane k, based k planes into the tap tensor (with
    // Odd one, at the tensor, and the planes at scalar offsets).  Sizes are
    // rounded up to whole dwords: an odd element count ends inside an aligned
    // dword whose other half the windows never use.
    const int xbytes = static_cast<int>((static_cast<int64_t>(planes) * HW * ES + 3) & ~int64_t{3});
    const __amdgpu_buffer_rsrc_t xs = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(x), 0, xbytes, kBufFlags);
    const __amdgpu_buffer_rsrc_t ls = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(lam), 0, xbytes, kBufFlags);
    __amdgpu_buffer_rsrc_t taps[3];
#pragma unroll
    for (int k = 0; k < 3; ++k)
        taps[k] = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(w4 + (Odd ? 0 : static_cast<size_t>(k) * HW)),
                                                    0, ((w4_bytes + 3) & ~3) - (Odd ? 0 : k * HW * ES), kBufFlags);
    const int tap_planes = planes / cpg;
    const int par = Odd ? 0 : (K * q) & 1;
    const uint32_t win_b = Odd ? 0u : static_cast<uint32_t>(K * q - par) * ES;
    const uint32_t sel_even = par ? 0x03020c0cu : 0x01000c0cu;
    const uint32_t sel_odd = par ? 0x05040c0cu : 0x03020c0cu;

    auto phase = [&](auto rows_tag) {
        constexpr bool kRows = decltype(rows_tag)::value;
        const int L = kRows ? W : H;
        const int NL = kRows ? H : W;
        const int g = (kRows ? 0 : 2) + half;        // direction TD, BU, LR, RL
        // per slot and tap, the byte selector of its element in the window;
        // a dropped tap (or any tap of a slot past the line end) decodes to
        // -2^127, whose sigmoid is exactly 0 whatever the memory holds, and x
        // and lambda of a slot past the line end decode to 0
        uint32_t st[3][K], sx[K];
        bool valid[K];
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const int p = K * q + j;
            valid[j] = p < L;
            const uint32_t s_in = (j & 1) ? sel_odd : sel_even;
            st[0][j] = (valid[j] && p > 0) ? s_in : kSelDropped;
            st[1][j] = valid[j] ? s_in : kSelDropped;
            st[2][j] = (valid[j] && p < L - 1) ? s_in : kSelDropped;
            sx[j] = valid[j] ? s_in : kSelZero;
        }
        const uint32_t line_b = static_cast<uint32_t>(L) * ES;
        const uint32_t lo0 = fwd ? 0u : static_cast<uint32_t>(NL - 1) * line_b;
        const uint32_t dlo = fwd ? line_b : 0u - line_b;
        uint32_t lo = static_cast<uint32_t>(((g * tap_planes + plane / cpg) * 3) * HW) * ES + win_b + lo0;
        // row scan: x and lambda of the current row, same window as the taps
        uint32_t xo = static_cast<uint32_t>(pix0) * ES + win_b + lo0;
        // Odd: a window starts at element E (its first position Kq on the
        // line); it is loaded from element E & ~1 and shifted right by 16 bits
        // when E is odd.  Along a scan E moves by +-L, so with L odd its
        // parity alternates from step to step: slot d of the ring (steps of
        // d's parity, D even) uses the shift and the offset increment of its
        // parity, both fixed per lane.  Tap plane 2 lies 2 HW elements after
        // plane 0 (same parity: a scalar offset); plane 1 lies HW after it,
        // which with HW odd flips the parity (a scalar offset plus 4 bytes on
        // the steps where plane 0's window starts odd).
        uint32_t incE = dlo, incO = dlo, shE = 0, shO = 0, add1E = 0, add1O = 0, sh1E = 0, sh1O = 0;
        uint32_t xincE = dlo, xincO = dlo, xshE = 0, xshO = 0;
        int so1 = HW * ES, so2 = 2 * HW * ES;
        if constexpr (Odd) {
            const int lodd = L & 1, hodd = HW & 1;
            const int line0 = fwd ? 0 : NL - 1;
            const int dl = fwd ? L : -L;
            const int e0 = ((g * tap_planes + plane / cpg) * 3) * HW + line0 * L + K * q;
            const int p0 = e0 & 1, p1 = p0 ^ lodd;
            lo = static_cast<uint32_t>(e0 - p0) * ES;
            incE = static_cast<uint32_t>(2 * dl - 2 * lodd + 4 * lodd * p0);
            incO = static_cast<uint32_t>(2 * dl - 2 * lodd + 4 * lodd * p1);
            shE = 16u * p0;
            shO = 16u * p1;
            add1E = 4u * (p0 & hodd);
            add1O = 4u * (p1 & hodd);
            sh1E = shE ^ (16u * hodd);
            sh1O = shO ^ (16u * hodd);
            so1 = 2 * HW - 2 * hodd;
            so2 = 4 * HW;
            const int ex = static_cast<int>(pix0) + line0 * L + K * q;
            const int px0 = ex & 1, px1 = px0 ^ lodd;
            xo = static_cast<uint32_t>(ex - px0) * ES;
            xincE = static_cast<uint32_t>(2 * dl - 2 * lodd + 4 * lodd * px0);
            xincO = static_cast<uint32_t>(2 * dl - 2 * lodd + 4 * lodd * px1);
            xshE = 16u * px0;
            xshO = 16u * px1;
        }
        words_t<NWL> tbuf[D][3];
        words_t<NWL> xbuf[kRows ? D : 1], lbuf[kRows ? D : 1];
        auto load_line = [&](int d) {
            if constexpr (Odd) {
                const bool od = (d & 1) != 0;
                tbuf[d][0] = load_words_so<NWL>(taps[0], lo, 0);
                tbuf[d][1] = load_words_so<NWL>(taps[0], lo + (od ? add1O : add1E), so1);
                tbuf[d][2] = load_words_so<NWL>(taps[0], lo, so2);
                lo += od ? incO : incE;
                if constexpr (kRows) {
                    xbuf[d] = load_words<NWL>(xs, xo);
                    lbuf[d] = load_words<NWL>(ls, xo);
                    xo += od ? xincO : xincE;
                }
            } else {
#pragma unroll
                for (int k = 0; k < 3; ++k) tbuf[d][k] = load_words<NW>(taps[k], lo);
                lo += dlo;
                if constexpr (kRows) {
                    xbuf[d] = load_words<NW>(xs, xo);
                    lbuf[d] = load_words<NW>(ls, xo);
                    xo += dlo;
                }
            }
        };
        // the NW words a window decodes from (Odd: shifted into place)
        auto window = [&](const words_t<NWL>& w, uint32_t sh) -> words_t<NW> {
            if constexpr (Odd) {
                words_t<NW> r;
#pragma unroll
                for (int i = 0; i < NW; ++i) {
                    const uint32_t lo_w = word<NWL>(w, i);
                    const uint32_t hi_w = word<NWL>(w, i + 1 < NWL ? i + 1 : NWL - 1);
                    const uint32_t v = __builtin_amdgcn_alignbit(hi_w, lo_w, sh);
                    if constexpr (NW == 1) r = v;
                    else r[i] = v;
                }
                return r;
            } else {
                return w;
            }
        };
#pragma unroll
        for (int d = 0; d < D; ++d) {
            load_line(d);
            __builtin_amdgcn_sched_barrier(0);
        }

        // Per slot: element index of its pixel on the current line, and its
        // change per step (0 for slots past the line end, which stay on the
        // lane's dummy words).
        const int i0 = fwd ? 0 : NL - 1;
        const int de = kRows ? (fwd ? W : -W) : (fwd ? 1 : -1);
        uint32_t aS[K], aH[K], aL[K];
        const int dS = 4 * de, dH = 2 * de, dL = de;
        int dSj[K], dHj[K], dLj[K];
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const int p = K * q + j;
            const int e = kRows ? i0 * W + p : p * W + i0;
            if (valid[j]) {
                aS[j] = static_cast<uint32_t>(lay.s + 4 * e);
                aH[j] = b_addr_hi(e);
                aL[j] = b_addr_lo(e);
            } else if (kRows) {
                // b writes of the row scan land in the pads before the b arrays
                aS[j] = PhaseLayout::dum;
                aH[j] = static_cast<uint32_t>(lay.bh - 2 * (j + 1));
                aL[j] = static_cast<uint32_t>(lay.bl - (j + 1));
            } else {
                aS[j] = PhaseLayout::dum;
                aH[j] = aL[j] = PhaseLayout::bdum;
            }
            dSj[j] = valid[j] ? dS : 0;
            dHj[j] = valid[j] ? dH : 0;
            dLj[j] = valid[j] ? dL : 0;
        }
        auto read_b = [&](int j) -> float {
            const uint32_t hi = lds_ref<uint16_t>(aH[j]);
            const uint32_t lo8 = lds_ref<uint8_t>(aL[j]);
            // bytes (hi.1, hi.0, lo.0, 0)
            return __uint_as_float(__builtin_amdgcn_perm(hi, lo8, 0x0504000cu));
        };
        // Odd number of lines: both scan orders reach middle line m in step m;
        // there the backward order reads and writes the side line instead
        const bool mid = Odd && !fwd && (NL & 1);
        const int m = NL / 2;
        uint32_t sideJ[Odd ? K : 1];
        if constexpr (Odd) {
#pragma unroll
            for (int j = 0; j < K; ++j)
                sideJ[j] = valid[j] ? static_cast<uint32_t>(lay.side + 4 * (K * q + j)) : PhaseLayout::dum;
        }
        auto sum_addr = [&](int j, int st) -> uint32_t {
            if constexpr (Odd) return (mid && st == m) ? sideJ[j] : aS[j];
            else return aS[j];
        };
        float h[K], acc[K], bv[K];
#pragma unroll
        for (int j = 0; j < K; ++j) {
            h[j] = 0.0f;
            acc[j] = lds_ref<float>(sum_addr(j, 0));
            if constexpr (!kRows) bv[j] = read_b(j);
        }
        int seg = NL, next_restart = NL;
        if constexpr (Chunked) {
            seg = (NL + k_chunk - 1) / k_chunk;
            next_restart = fwd ? seg : NL - ((NL - 1) / seg) * seg;
        }

        auto step = [&](int s, int d) {
            asm volatile("" : "+v"(tbuf[d][0]), "+v"(tbuf[d][1]), "+v"(tbuf[d][2]));
            if constexpr (kRows) asm volatile("" : "+v"(xbuf[d]), "+v"(lbuf[d]));
            const bool od = (d & 1) != 0;
            const words_t<NW> w0 = window(tbuf[d][0], od ? shO : shE);
            const words_t<NW> w1 = window(tbuf[d][1], od ? sh1O : sh1E);
            const words_t<NW> w2 = window(tbuf[d][2], od ? shO : shE);
            words_t<NW> wx{}, wl{};
            if constexpr (kRows) {
                wx = window(xbuf[d], od ? xshO : xshE);
                wl = window(lbuf[d], od ? xshO : xshE);
            }
            float s0v[K], s1v[K], s2v[K], r[K];
#pragma unroll
            for (int j = 0; j < K; ++j) {
                if constexpr (kRows) {
                    // b = lambda x from the row's windows, also kept for the column scan
                    bv[j] = window_elem<T, K, NW>(wl, j, sx[j], sx[j]) *
                            window_elem<T, K, NW>(wx, j, sx[j], sx[j]);
                }
                s0v[j] = window_elem<T, K, NW>(w0, j, st[0][j], st[0][j]) * kNegLog2e;
                s1v[j] = window_elem<T, K, NW>(w1, j, st[1][j], st[1][j]) * kNegLog2e;
                s2v[j] = window_elem<T, K, NW>(w2, j, st[2][j], st[2][j]) * kNegLog2e;
            }
            // breadth first over the 3 K taps: each dependent operation finds
            // its operand several instructions back
#pragma unroll
            for (int j = 0; j < K; ++j) {
                s0v[j] = __builtin_amdgcn_exp2f(s0v[j]);
                s1v[j] = __builtin_amdgcn_exp2f(s1v[j]);
                s2v[j] = __builtin_amdgcn_exp2f(s2v[j]);
            }
#pragma unroll
            for (int j = 0; j < K; ++j) {
                s0v[j] += 1.0f;
                s1v[j] += 1.0f;
                s2v[j] += 1.0f;
            }
#pragma unroll
            for (int j = 0; j < K; ++j) {
                s0v[j] = __builtin_amdgcn_rcpf(s0v[j]);
                s1v[j] = __builtin_amdgcn_rcpf(s1v[j]);
                s2v[j] = __builtin_amdgcn_rcpf(s2v[j]);
            }
#pragma unroll
            for (int j = 0; j < K; ++j) r[j] = s0v[j] + s1v[j];
#pragma unroll
            for (int j = 0; j < K; ++j) r[j] = fmaxf(r[j] + s2v[j], eps);
#pragma unroll
            for (int j = 0; j < K; ++j) r[j] = __builtin_amdgcn_rcpf(r[j]);
            // refill slot d only after it has been decoded
#pragma unroll
            for (int j = 0; j < K; ++j) {
                if constexpr (kRows)
                    asm volatile("" : "+v"(lo), "+v"(xo)
                                 : "v"(s0v[j]), "v"(s1v[j]), "v"(s2v[j]), "v"(r[j]), "v"(bv[j]));
                else
                    asm volatile("" : "+v"(lo) : "v"(s0v[j]), "v"(s1v[j]), "v"(s2v[j]), "v"(r[j]));
            }
            load_line(d);
            if constexpr (kRows) {
#pragma unroll
                for (int j = 0; j < K; ++j) {
                    const uint32_t bb = __float_as_uint(bv[j]);
                    lds_ref<uint16_t>(aH[j]) = static_cast<uint16_t>(bb >> 16);
                    lds_ref<uint8_t>(aL[j]) = static_cast<uint8_t>(bb >> 8);
                }
            }

            if constexpr (Chunked) {
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
                hn[j] = fmaf(m, r[j], bv[j]);
            }
#pragma unroll
            for (int j = 0; j < K; ++j) h[j] = hn[j];

#pragma unroll
            for (int j = 0; j < K; ++j) lds_ref<float>(sum_addr(j, s)) = acc[j] + h[j];
            // Each pixel of the phase is updated once per scan order.  The
            // order that reaches it first does so by step NL / 2 - 1; the
            // other reads it one step ahead, at step NL / 2 - 1 or later.  So
            // one barrier there, between this step's writes and its
            // read-ahead, orders every pair of updates (with NL odd the
            // middle line, reached by both at step NL / 2, goes to the side
            // line for the backward order).
            if constexpr (kTwo)
                if (s == NL / 2 - 1) lds_barrier();
            // the next line, read after this step's writes
#pragma unroll
            for (int j = 0; j < K; ++j) {
                aS[j] += dSj[j];
                aH[j] += dHj[j];
                aL[j] += dLj[j];
                acc[j] = lds_ref<float>(sum_addr(j, s + 1));
                if constexpr (!kRows) bv[j] = read_b(j);
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
    };
    // with an odd number of lines, the backward order's terms of the middle
    // line are added after the forward order's, and the side line cleared
    auto fold = [&](bool rows) {
        const int NL = rows ? H : W, L = rows ? W : H;
        if (!(NL & 1)) return;
        const int m = NL / 2;
        for (int p = tid; p < L; p += NT) {
            const uint32_t a = static_cast<uint32_t>(lay.s + 4 * (rows ? m * W + p : p * W + m));
            lds_ref<float>(a) = lds_ref<float>(a) + lds_ref<float>(lay.side + 4 * p);
            lds_ref<float>(lay.side + 4 * p) = 0.0f;
        }
        sync();
    };
    phase(std::true_type{});
    sync();
    if constexpr (Odd) fold(true);
    phase(std::false_type{});
    sync();
    if constexpr (Odd) fold(false);

    // --------------------------------------------------------- y = u * S
    // (S is read as four floats per dword pair, 16-byte aligned since the
    // pair starts at an even dword)
    uint32_t* y32 = reinterpret_cast<uint32_t*>(y + pix0);
    const uint32_t* u32 = reinterpret_cast<const uint32_t*>(u + pix0);
    u32x2_u* y64p = reinterpret_cast<u32x2_u*>(y + pix0);
    auto emit_word = [&](int f, uint32_t uv) -> uint32_t {
        const f32x2_t sv = lds_ref<f32x2_t>(lay.s + 8u * f);
        return pack_bf16x2(__uint_as_float(uv << 16) * sv.x, __uint_as_float(uv & 0xffff0000u) * sv.y);
    };
    auto emit_pair = [&](int f, u32x2_t uv) {
        const u32x2_t o = {emit_word(2 * f, uv.x), emit_word(2 * f + 1, uv.y)};
        if constexpr (Odd) y64p[f] = o;
        else reinterpret_cast<u32x2_t*>(y + pix0)[f] = o;
    };
#pragma unroll
    for (int k = 0; k < kUPer; ++k) {
        const int f = tid + NT * k;
        if (f < pairs) emit_pair(f, ureg[k]);
    }
    // the rest of u (planes over 6144 pixels), eight loads in flight at a time
    for (int f0 = tid + NT * kUPer; f0 < pairs; f0 += NT * 8) {
        u32x2_t uv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (f0 + NT * j < pairs) uv[j] = u64p[f0 + NT * j];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (f0 + NT * j < pairs) emit_pair(f0 + NT * j, uv[j]);
    }
    if constexpr (Odd) {
        // the last HW mod 4 pixels one by one, 16 bits each (a plane may
        // start at any element)
        const int i = 4 * pairs + tid;
        if (i < HW) {
            const float v = __uint_as_float(static_cast<uint32_t>(u[pix0 + i]) << 16) *
                            lds_ref<float>(lay.s + 4u * i);
            y[pix0 + i] = static_cast<T>(pack_bf16x2(v, v) & 0xffffu);
        }
    } else {
        if ((words & 1) && tid == 0) y32[words - 1] = emit_word(words - 1, u32[words - 1]);
    }
}

template <int K, bool Chunked, int NH, bool Odd = false>
hipError_t launch_k(const void* x, const void* lam, const void* u, const void* w4, float eps,
                    void* y, int64_t planes, int64_t H, int64_t W, const PropOpts& o,
                    hipStream_t stream) {
    using T = uint16_t;
    constexpr int D = 8;   // taps prefetched D steps ahead
    const size_t lds = PhaseLayout(static_cast<int>(H), static_cast<int>(W)).bytes;
    auto kern = prop2d_phase_kernel<T, K, D, Chunked, NH, Odd>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(lds));
        if (e != hipSuccess) return e;
    }
    const int64_t n = planes * H * W;
    kern<<<dim3(static_cast<unsigned>(planes)), dim3(2 * NH), lds, stream>>>(
        static_cast<const T*>(x), static_cast<const T*>(lam), static_cast<const T*>(u),
        static_cast<const T*>(w4), static_cast<int>(12 * (n / o.cpg) * sizeof(T)), eps,
        static_cast<T*>(y), static_cast<int>(planes), static_cast<int>(H), static_cast<int>(W),
        static_cast<int>(o.cpg), static_cast<int>(o.k_chunk));
    return hipGetLastError();
}

// gfx950 (MI355X): compute units, four SIMDs each.
constexpr int64_t kComputeUnits = 256;

// Two wavefronts a plane (one per scan order, K = ceil(L / 64)) or one (32
// lanes a scan order, K = ceil(L / 32)).  One wavefront a plane keeps every
// SIMD busy once LDS holds four planes per CU and there is a plane for every
// SIMD (latent1k: 0.115 ms against 0.129 with two, whose 64-lane lines leave
// more slots idle); with fewer planes resident two wavefronts keep twice the
// SIMDs busy (148 x 148: one plane per CU, 0.099 ms against 0.164).
bool phase_two_waves(int64_t planes, int64_t H, int64_t W) {
    const int64_t per_cu = kLdsBytes / PhaseLayout(static_cast<int>(H), static_cast<int>(W)).bytes;
    return per_cu < 4 || planes < 4 * kComputeUnits;
}

template <bool Chunked>
hipError_t launch_c(const void* x, const void* lam, const void* u, const void* w4, float eps,
                    void* y, int64_t planes, int64_t H, int64_t W, const PropOpts& o,
                    hipStream_t stream) {
    const int64_t Lmax = H > W ? H : W;
    // an odd side takes the two-wavefront form (its windows need the
    // registers the one-wavefront form has no room for)
    if ((H & 1) || (W & 1)) {
        if (Lmax <= 64) return launch_k<1, Chunked, 64, true>(x, lam, u, w4, eps, y, planes, H, W, o, stream);
        if (Lmax <= 128) return launch_k<2, Chunked, 64, true>(x, lam, u, w4, eps, y, planes, H, W, o, stream);
        return launch_k<3, Chunked, 64, true>(x, lam, u, w4, eps, y, planes, H, W, o, stream);
    }
    if (phase_two_waves(planes, H, W)) {
        if (Lmax <= 64) return launch_k<1, Chunked, 64>(x, lam, u, w4, eps, y, planes, H, W, o, stream);
        if (Lmax <= 128) return launch_k<2, Chunked, 64>(x, lam, u, w4, eps, y, planes, H, W, o, stream);
        return launch_k<3, Chunked, 64>(x, lam, u, w4, eps, y, planes, H, W, o, stream);
    }
    if (Lmax <= 32) return launch_k<1, Chunked, 32>(x, lam, u, w4, eps, y, planes, H, W, o, stream);
    if (Lmax <= 64) return launch_k<2, Chunked, 32>(x, lam, u, w4, eps, y, planes, H, W, o, stream);
    if (Lmax <= 96) return launch_k<3, Chunked, 32>(x, lam, u, w4, eps, y, planes, H, W, o, stream);
    if (Lmax <= 128) return launch_k<4, Chunked, 32>(x, lam, u, w4, eps, y, planes, H, W, o, stream);
    return launch_k<5, Chunked, 32>(x, lam, u, w4, eps, y, planes, H, W, o, stream);
}

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

}  // namespace

bool prop2d_phase_eligible(int dtype, int64_t planes, int64_t H, int64_t W, const void* x,
                           const void* lam, const void* u, const void* w4, const void* y) {
    if (dtype != 1) return false;                         // bf16 planes only
    if (H > 160 || W > 160) return false;                 // K <= 5 positions a lane
    if (PhaseLayout(static_cast<int>(H), static_cast<int>(W)).bytes > kLdsBytes) return false;
    if (12 * planes * H * W * 2 > 0x7fffffff) return false;
    return aligned4(x) && aligned4(lam) && aligned4(u) && aligned4(w4) && aligned4(y);
}

hipError_t launch_prop2d_phase(const void* x, const void* lam, const void* u, const void* w4,
                               float eps, void* y, int dtype, int64_t planes, int64_t H, int64_t W,
                               const PropOpts& o, hipStream_t stream) {
    if (dtype != 1) return hipErrorInvalidValue;
    return o.k_chunk > 1 ? launch_c<true>(x, lam, u, w4, eps, y, planes, H, W, o, stream)
                         : launch_c<false>(x, lam, u, w4, eps, y, planes, H, W, o, stream);
}

}  // namespace gspn
