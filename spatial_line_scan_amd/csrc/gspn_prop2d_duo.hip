// Four-direction propagation of square bf16 planes with even sides 66..150
// and odd sides 97..149, all four directions in the same step, with the two row scans and the two
// column scans in different wavefronts of one workgroup (gfx950).
//
// Operator: "Scaling Parallel Sequence Models to Foundation-Scale Vision
// Encoders", §3 line-scan recurrence (standard GSPN form), §4.1 single-kernel
// design, §4.3 hidden state kept on chip, §5.1 fused normalisation (sigmoid,
// local sum, clamp, divide); reading notes, method / overall framework.
//
// Work split, two forms:
//   - 32 lanes a direction (two wavefronts a plane): wavefront 0 scans rows,
//     lanes 0..31 top-down (row s at step s), lanes 32..63 bottom-up (row
//     L-1-s); wavefront 1 scans columns, lanes 0..31 left-right (column s),
//     lanes 32..63 right-left (column L-1-s).  The value a half's first or
//     last lane receives from the other half only meets a dropped tap
//     (weight exactly 0).
//   - 64 lanes a direction (four wavefronts a plane): top-down, bottom-up,
//     left-right, right-left.  The only form for odd sides.
// Lane q holds positions Kq .. Kq+K-1 of its line; the neighbour exchange is
// one whole-wavefront DPP shift each way.
//
// When they pay: a plane's sums and products fill about 40 KB of LDS at
// 74 x 74 (four planes a CU) and about 157 KB at 148 x 148 (one).  The
// one-wavefront-a-plane kernel leaves SIMDs idle when planes are few or
// large; more wavefronts a plane shorten each one's step (128 planes of
// 74 x 74: 0.025 ms with four wavefronts, 0.029 with two, 0.037 with one;
// 256 planes of 148 x 148: 0.061 ms, 0.086 and 0.099 for the rows-then-
// columns kernel).  On a full GPU at 74 x 74 the SIMDs' issue is the limit
// and the one-wavefront kernel's 80 slots a line (against 96 or 128 here)
// win.
//
// On-chip data, per plane (as one wavefront a plane would keep it):
//   S   fp32 [L][L]: the sum of the four directional states.
//   b = lambda x of every pixel, computed before the scan, kept as 24 bits
//       (the exact product of two bf16 values has at most 16 significant
//       bits): the upper 16 in one array, the next 8 in another.
//   side fp32 [4][L]: the column scans' terms of the four pixels where a row
//       scan and a column scan meet in the same step.
//
// Ordering.  Pixel (i, j) is updated by the row wavefront at steps i and
// L-1-i and by the column wavefront at steps j and L-1-j.  The wavefronts
// meet at a barrier after every step's writes, and every step reads its
// pixels after that barrier, so two updates of one pixel in different steps
// are ordered.  In one step the two wavefronts meet only at (s, s),
// (s, L-1-s), (L-1-s, s) and (L-1-s, L-1-s); there the column scan adds its
// state into a side word indexed by the step, and the side words are added
// into the diagonals after the scan.  Row scans never meet each other
// (L even), nor do column scans.  With L odd the two row scans both reach
// the middle row m = (L-1)/2 at step m (and the column scans the middle
// column): there the bottom-up and right-left scans write their terms into
// separate mid lines, added in after the scan.  Each pixel's four terms are
// therefore summed in a fixed order and the result is bitwise reproducible.
//
// Slots past the end of a line (positions >= L) read and write dummy words,
// decode every tap to -2^127 (weight exactly 0) and hold h = 0; lanes whose
// whole window lies past the line load nothing.
#include "gspn_device.h"
#include "gspn_internal.h"
#include "gspn_lane.h"

namespace gspn {
namespace {

using namespace lane;

// LDS layout in bytes (offsets multiples of 16):
//   [S dummy: 16][b dummy: 16][pad: 4 L][S: L L fp32][side: 4 L fp32]
//   [b_hi: L L + 8 u16][b_lo: L L + L + 8 u8]
// The last step's read-ahead goes one line past every scan: one row before S
// (the pad), one row after it (side), and for b the neighbouring arrays or
// b_lo's spare row.  b_hi and b_lo have 8 spare entries for the second half
// of the plane's last 16-byte chunk when L L is not a multiple of 8.
// mid fp32 [2][L]: with L odd, where the bottom-up scan puts its terms of the
// middle row and the right-left scan its terms of the middle column (each
// pair of scans reaches its middle line in the same step); added into S
// after the scan.
struct DuoLayout {
    int s, side, mid, bh, bl, bytes;
    static constexpr int sdum = 0, bdum = 16;
    __host__ __device__ static int a16(int v) { return (v + 15) & ~15; }
    __host__ __device__ explicit DuoLayout(int L) {
        const int n = L * L;
        s = a16(32 + 4 * L);
        side = a16(s + 4 * n);
        mid = a16(side + 16 * L);
        bh = a16(mid + 8 * L);
        bl = a16(bh + 2 * (n + 8));
        bytes = a16(bl + n + L + 8);
    }
};

constexpr int kMaxSide = 150;       // the layout's LDS at 150 x 150: 157 KB
constexpr int kMinOddSide = 97;     // odd sides: a wavefront a direction, 97..149
// 16-byte chunks of a plane's bf16 values a thread loads at once (a 96 x 96
// plane in one batch)
constexpr int kBatch = 9;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_u __attribute__((ext_vector_type(4), aligned(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
template <typename V> using lds_t = __attribute__((address_space(3))) V;

template <typename V>
__device__ __forceinline__ lds_t<V>& lds_ref(uint32_t byte_off) {
    // the kernel's only LDS is its dynamic array, which starts at address 0
    return *reinterpret_cast<lds_t<V>*>(static_cast<uintptr_t>(byte_off));
}

// Both wavefronts' LDS writes before the call are visible to both after it.
// Only LDS is ordered: global loads in flight (prefetched taps) stay in
// flight.
__device__ __forceinline__ void block_lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// bf16 of the low / high half of a dword as fp32
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

struct DuoArgs {
    const uint16_t* w4;
    int w4_bytes;
    float eps;
    int planes, L, cpg, plane;
};

// Zeroes S, side and the dummies, writes b = lambda x, and meets the other
// wavefront (every thread of the block calls it once).
template <int NT>
__device__ __forceinline__ void fill_plane(const DuoLayout& lay, int tid, int nchunk, __amdgpu_buffer_rsrc_t xs,
                                           __amdgpu_buffer_rsrc_t ls, uint32_t plane_b) {
    for (int f = tid; f < lay.bh / 16; f += NT) lds_ref<u32x4_t>(16u * f) = u32x4_t{0u, 0u, 0u, 0u};
    for (int f0 = 0; f0 < nchunk; f0 += NT * kBatch) {
    // x and lambda of a batch of chunks, all loads before any use
    u32x4_t xv[kBatch], lv[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
        const int f = f0 + tid + NT * k;
        const uint32_t off = plane_b + 16u * static_cast<uint32_t>(f);
        xv[k] = f < nchunk ? __builtin_amdgcn_raw_buffer_load_b128(xs, off, 0, 0) : u32x4_t{0u, 0u, 0u, 0u};
        lv[k] = f < nchunk ? __builtin_amdgcn_raw_buffer_load_b128(ls, off, 0, 0) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
        const int f = f0 + tid + NT * k;
        if (f < nchunk) {
            uint32_t bb[8];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                bb[2 * m] = __float_as_uint(bf_lo(lv[k][m]) * bf_lo(xv[k][m]));
                bb[2 * m + 1] = __float_as_uint(bf_hi(lv[k][m]) * bf_hi(xv[k][m]));
            }
            u32x4_t hi;
#pragma unroll
            for (int m = 0; m < 4; ++m) hi[m] = __builtin_amdgcn_perm(bb[2 * m + 1], bb[2 * m], 0x07060302u);
            u32x2_t lo8;
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const uint32_t t01 = __builtin_amdgcn_perm(bb[4 * m + 1], bb[4 * m], 0x0c0c0501u);
                const uint32_t t23 = __builtin_amdgcn_perm(bb[4 * m + 3], bb[4 * m + 2], 0x05010c0cu);
                lo8[m] = t01 | t23;
            }
            lds_ref<u32x4_t>(lay.bh + 16u * f) = hi;
            lds_ref<u32x2_t>(lay.bl + 8u * f) = lo8;
        }
    }
    }
    block_lds_barrier();
}

// The two scans of one wavefront (ROWS: top-down and bottom-up; else
// left-right and right-left) over the whole plane: prefetch of the first D
// lines of taps, the plane fill (shared with the other wavefront), then L
// steps, each ending at a barrier with the other wavefront.
// K: positions a lane; R = (L - 1) mod K; D: steps a block (a multiple of K),
// also the number of lines of taps prefetched ahead.
// LANES: lanes a direction (32: a wavefront holds both scans of the pair,
// one per half; 64: a wavefront per scan, `half` says which).  NT: threads
// of the workgroup.
// Odd: L odd (lines and planes start at any element; see the window notes
// below), a wavefront a direction.
template <int K, int R, int D, bool ROWS, int LANES, int NT, bool Odd>
__device__ __forceinline__ void scan_pair(const DuoArgs& a, const DuoLayout& lay, int tid, int lane,
                                          int wave_half, int nchunk, __amdgpu_buffer_rsrc_t xs,
                                          __amdgpu_buffer_rsrc_t ls, uint32_t plane_b) {
    static_assert(D % K == 0, "blocks of whole slot cycles");
    static_assert(!Odd || (D % 2 == 0 && LANES == 64), "odd lines: window parity alternates with the ring slot");
    // words a window decodes from, and words loaded for it: with Odd a window
    // is loaded from the even element at or below its first and shifted into
    // place, which for even K takes one more word
    constexpr int NW = Odd ? (K + 1) / 2 : window_words<uint16_t, K>();
    constexpr int NWL = Odd && (K % 2 == 0) ? NW + 1 : NW;
    const int L = a.L;
    const int n = L * L;
    const int half = LANES == 32 ? lane >> 5 : wave_half;
    const int g = (ROWS ? 0 : 2) + half;   // 0 TD, 1 BU, 2 LR, 3 RL
    const int q = LANES == 32 ? lane & 31 : lane;
    const bool fwd = half == 0;

    // ------------------------------------------------ taps: first D lines
    const int tap_planes = a.planes / a.cpg;
    __amdgpu_buffer_rsrc_t taps[3];
#pragma unroll
    for (int k = 0; k < 3; ++k)
        taps[k] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.w4) + static_cast<size_t>(k) * n,
                                                    0, a.w4_bytes - k * n * 2, kBufFlags);
    const int par = Odd ? 0 : (K * q) & 1;
    const bool lane_live = K * q < L;
    const uint32_t line_b = static_cast<uint32_t>(L) * 2u;
    const uint32_t tap_base =
        static_cast<uint32_t>((g * tap_planes + a.plane / a.cpg) * 3) * static_cast<uint32_t>(n) * 2u +
        static_cast<uint32_t>(K * q - par) * 2u;
    const uint32_t lo_min = lane_live ? tap_base : 0x80000000u;
    const uint32_t lo_max = lane_live ? tap_base + static_cast<uint32_t>(L - 1) * line_b : 0x80000000u;
    uint32_t lo = fwd ? lo_min : lo_max;
    const uint32_t dlo = lane_live ? (fwd ? line_b : 0u - line_b) : 0u;
    // Odd: a window starts at element E (its first position Kq on the line);
    // it is loaded from element E & ~1 and shifted right by 16 bits when E is
    // odd.  Along a scan E moves by +-L, so its parity alternates from step to
    // step: ring slot d (steps of d's parity, D even) uses the shift and the
    // offset increment of its parity.  Tap plane 2 lies 2 n elements after
    // plane 0 (same parity: a scalar offset); plane 1 lies n after it, which
    // with n odd flips the parity (a scalar offset plus 4 bytes on the steps
    // where plane 0's window starts odd).  Reads past a scan's end run on
    // into the next lines or past the tensor (0); they are never used.
    __amdgpu_buffer_rsrc_t tall = taps[0];
    uint32_t incE = 0, incO = 0, shE = 0, shO = 0, add1E = 0, add1O = 0, sh1E = 0, sh1O = 0;
    int so1 = 0, so2 = 0;
    if constexpr (Odd) {
        tall = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.w4), 0, (a.w4_bytes + 3) & ~3, kBufFlags);
        const int line0 = fwd ? 0 : L - 1;
        const int dl = fwd ? L : -L;
        const int e0 = ((g * tap_planes + a.plane / a.cpg) * 3) * n + line0 * L + K * q;
        const int p0 = e0 & 1, p1 = p0 ^ 1;
        lo = static_cast<uint32_t>(e0 - p0) * 2u;
        incE = static_cast<uint32_t>(2 * dl - 2 + 4 * p0);
        incO = static_cast<uint32_t>(2 * dl - 2 + 4 * p1);
        shE = 16u * p0;
        shO = 16u * p1;
        add1E = 4u * p0;
        add1O = 4u * p1;
        sh1E = shE ^ 16u;
        sh1O = shO ^ 16u;
        so1 = 2 * n - 2;
        so2 = 4 * n;
    }
    words_t<NWL> tbuf[D][3];
    auto load_line = [&](int d) {
        if constexpr (Odd) {
            const bool od = (d & 1) != 0;
            tbuf[d][0] = load_words_so<NWL>(tall, lo, 0);
            tbuf[d][1] = load_words_so<NWL>(tall, lo + (od ? add1O : add1E), so1);
            tbuf[d][2] = load_words_so<NWL>(tall, lo, so2);
            lo += od ? incO : incE;
        } else {
#pragma unroll
            for (int k = 0; k < 3; ++k) tbuf[d][k] = load_words<NW>(taps[k], lo);
            const uint32_t nx = lo + dlo;
            lo = umed3(nx, lo_min, lo_max);
        }
    };
    // the NW words a window decodes from (Odd: shifted into place)
    auto window = [&](const words_t<NWL>& w, uint32_t sh) -> words_t<NW> {
        if constexpr (Odd) {
            words_t<NW> rv;
#pragma unroll
            for (int i = 0; i < NW; ++i) {
                const uint32_t lo_w = word<NWL>(w, i);
                const uint32_t hi_w = word<NWL>(w, i + 1 < NWL ? i + 1 : NWL - 1);
                const uint32_t v = __builtin_amdgcn_alignbit(hi_w, lo_w, sh);
                if constexpr (NW == 1) rv = v;
                else rv[i] = v;
            }
            return rv;
        } else {
            return w;
        }
    };
#pragma unroll
    for (int d = 0; d < D; ++d) {
        load_line(d);
        __builtin_amdgcn_sched_barrier(0);
    }

    fill_plane<NT>(lay, tid, nchunk, xs, ls, plane_b);

    // ------------------------------------------------ per-slot constants
    const int i0 = fwd ? 0 : L - 1;
    const int de = ROWS ? (fwd ? L : -L) : (fwd ? 1 : -1);
    uint32_t aS[K], aH[K], aL[K];
    int dSj[K], dHj[K], dLj[K];
    uint32_t sel[3][K];
    const uint32_t sel_even = par ? 0x03020c0cu : 0x01000c0cu;
    const uint32_t sel_odd = par ? 0x05040c0cu : 0x03020c0cu;
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const int p = K * q + j;
        const bool valid = p < L;
        const int e = ROWS ? i0 * L + p : p * L + i0;
        aS[j] = valid ? static_cast<uint32_t>(lay.s + 4 * e) : DuoLayout::sdum;
        aH[j] = valid ? static_cast<uint32_t>(lay.bh + 2 * e) : DuoLayout::bdum;
        aL[j] = valid ? static_cast<uint32_t>(lay.bl + e) : DuoLayout::bdum;
        dSj[j] = valid ? 4 * de : 0;
        dHj[j] = valid ? 2 * de : 0;
        dLj[j] = valid ? de : 0;
        const uint32_t s_in = (j & 1) ? sel_odd : sel_even;
        sel[0][j] = (valid && p > 0) ? s_in : kSelDropped;
        sel[1][j] = valid ? s_in : kSelDropped;
        sel[2][j] = (valid && p < L - 1) ? s_in : kSelDropped;
    }
    // Odd: the backward scan of the pair (bottom-up, right-left) puts its
    // terms of the middle line (step m) into the mid lines
    const bool mid_scan = Odd && !fwd;
    const int m = L / 2;
    uint32_t aM[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const int p = K * q + j;
        aM[j] = p < L ? static_cast<uint32_t>(lay.mid + 4 * (ROWS ? 0 : L) + 4 * p) : DuoLayout::sdum;
    }
    // the S word of slot j at step s (the mid line at the middle step)
    auto base = [&](int j, int s) -> uint32_t {
        if constexpr (Odd) return (mid_scan && s == m) ? aM[j] : aS[j];
        else return aS[j];
    };
    // column slots that meet a row scan go to side words
    const uint32_t side1 = static_cast<uint32_t>(lay.side + 4 * L * (g == 3 ? 1 : 0));
    const uint32_t side2 = static_cast<uint32_t>(lay.side + 4 * L * (g == 3 ? 3 : 2));
    const uint32_t key = static_cast<uint32_t>(q);

    float h[K], acc[K];
    uint32_t bhr[K], blr[K];
    uint32_t ra1 = 0, ra2 = 0;   // addresses of this step's two meeting slots (columns)
    float s0v[K], s1v[K], s2v[K], r[K];   // the next step's weights

    // Reads the sums of step s = s0 + t of a block starting at s0 (a multiple
    // of K; t a compile-time value).  Column slots that meet a row scan are
    // rows s (slot t mod K, lanes q1) and L-1-s (slot (R - t) mod K, lanes
    // q2), with q1 = s0 / K + t / K and q2 = (L-1-R-s0) / K + floor((R - t) / K).
    auto read_sums = [&](int t, int s, int qb1, int qb2) {
        const int j1 = t % K;
        const int j2 = ((R - t) % K + K) % K;
        if constexpr (!ROWS) {
            const uint32_t q1 = static_cast<uint32_t>(qb1 + t / K);
            const uint32_t q2 =
                static_cast<uint32_t>(qb2 + (R - t >= 0 ? (R - t) / K : -((t - R + K - 1) / K)));
            uint32_t m1 = base(j1, s), m2 = base(j2, s);
            m1 = key == q1 ? side1 + 4u * s : m1;
            if (j2 == j1) m2 = m1;
            m2 = key == q2 ? side2 + 4u * s : m2;
            if (j2 == j1) m1 = m2;
            ra1 = m1;
            ra2 = m2;
        }
#pragma unroll
        for (int j = 0; j < K; ++j) {
            uint32_t ad = base(j, s);
            if constexpr (!ROWS) ad = j == j1 ? ra1 : (j == j2 ? ra2 : ad);
            acc[j] = lds_ref<float>(ad);
        }
    };
    // b of the next step's pixels (written before the scan, never after)
    auto read_b = [&]() {
#pragma unroll
        for (int j = 0; j < K; ++j) {
            bhr[j] = lds_ref<uint16_t>(aH[j]);
            blr[j] = lds_ref<uint8_t>(aL[j]);
            aH[j] += dHj[j];
            aL[j] += dLj[j];
            asm volatile("" : "+v"(aH[j]), "+v"(aL[j]));
        }
    };
    // weights of the step whose taps are in ring slot d, in two halves:
    // decode and exponentials, then the sigmoids, their sum and its inverse
    auto weights_a = [&](int d) {
        asm volatile("" : "+v"(tbuf[d][0]), "+v"(tbuf[d][1]), "+v"(tbuf[d][2]));
        const bool od = (d & 1) != 0;
        const words_t<NW> w0 = window(tbuf[d][0], od ? shO : shE);
        const words_t<NW> w1 = window(tbuf[d][1], od ? sh1O : sh1E);
        const words_t<NW> w2 = window(tbuf[d][2], od ? shO : shE);
#pragma unroll
        for (int j = 0; j < K; ++j) {
            s0v[j] = window_elem<uint16_t, K, NW>(w0, j, sel[0][j], sel[0][j]) * kNegLog2e;
            s1v[j] = window_elem<uint16_t, K, NW>(w1, j, sel[1][j], sel[1][j]) * kNegLog2e;
            s2v[j] = window_elem<uint16_t, K, NW>(w2, j, sel[2][j], sel[2][j]) * kNegLog2e;
        }
#pragma unroll
        for (int j = 0; j < K; ++j) {
            s0v[j] = __builtin_amdgcn_exp2f(s0v[j]);
            s1v[j] = __builtin_amdgcn_exp2f(s1v[j]);
            s2v[j] = __builtin_amdgcn_exp2f(s2v[j]);
        }
        // refill slot d only after it has been decoded
#pragma unroll
        for (int j = 0; j < K; ++j)
            asm volatile("" : "+v"(lo) : "v"(s0v[j]), "v"(s1v[j]), "v"(s2v[j]));
        load_line(d);
    };
    auto weights_b = [&]() {
#pragma unroll
        for (int j = 0; j < K; ++j) {
            s0v[j] = __builtin_amdgcn_rcpf(s0v[j] + 1.0f);
            s1v[j] = __builtin_amdgcn_rcpf(s1v[j] + 1.0f);
            s2v[j] = __builtin_amdgcn_rcpf(s2v[j] + 1.0f);
        }
#pragma unroll
        for (int j = 0; j < K; ++j) r[j] = s0v[j] + s1v[j];
#pragma unroll
        for (int j = 0; j < K; ++j) r[j] = fmaxf(r[j] + s2v[j], a.eps);
#pragma unroll
        for (int j = 0; j < K; ++j) r[j] = __builtin_amdgcn_rcpf(r[j]);
    };

#pragma unroll
    for (int j = 0; j < K; ++j) h[j] = 0.0f;
    read_b();
    weights_a(0);
    weights_b();

    // Step s (ring slot d): the sums are read after the previous step's
    // barrier; h is updated; the next step's exponentials cover the reads'
    // latency; the sums are written; the next step's b is read; the rest of
    // the next step's weights covers the writes' latency; barrier.
    auto step = [&](int s, int d, int qb1, int qb2) {
        read_sums(d, s, qb1, qb2);
        float bv[K];
#pragma unroll
        for (int j = 0; j < K; ++j) bv[j] = __uint_as_float(__builtin_amdgcn_perm(bhr[j], blr[j], 0x0504000cu));
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
        __builtin_amdgcn_sched_barrier(0);

        weights_a((d + 1) % D);
        __builtin_amdgcn_sched_barrier(0);

        const int t = d % K;
        const int j1 = t;
        const int j2 = ((R - t) % K + K) % K;
#pragma unroll
        for (int j = 0; j < K; ++j) {
            uint32_t ad = base(j, s);
            if constexpr (!ROWS) ad = j == j1 ? ra1 : (j == j2 ? ra2 : ad);
            lds_ref<float>(ad) = acc[j] + h[j];
        }
        // the pins keep each address one add a step instead of base +
        // multiple of the step
#pragma unroll
        for (int j = 0; j < K; ++j) {
            aS[j] += dSj[j];
            asm volatile("" : "+v"(aS[j]));
        }
        read_b();
        __builtin_amdgcn_sched_barrier(0);

        weights_b();
        block_lds_barrier();
    };

    int s0 = 0;
    for (; s0 + D <= L; s0 += D) {
        const int qb1 = s0 / K, qb2 = (L - 1 - R - s0) / K;
#pragma unroll
        for (int d = 0; d < D; ++d) step(s0 + d, d, qb1, qb2);
    }
    {
        const int qb1 = s0 / K, qb2 = (L - 1 - R - s0) / K;
#pragma unroll
        for (int d = 0; d < D; ++d)
            if (s0 + d < L) step(s0 + d, d, qb1, qb2);
    }
}

template <int K, int R, int D, int LANES, bool Odd>
__global__ void __launch_bounds__(LANES == 32 ? 128 : 256)
prop2d_duo_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ lam,
                  const uint16_t* __restrict__ u, const uint16_t* __restrict__ w4, int w4_bytes,
                  float eps, uint16_t* __restrict__ y, int planes, int L, int cpg) {
    const int n = L * L;
    const DuoLayout lay(L);
    constexpr int NT = LANES == 32 ? 128 : 256;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int plane = blockIdx.x;
    const uint32_t plane_b = static_cast<uint32_t>(plane) * static_cast<uint32_t>(n) * 2u;
    const int nchunk = (2 * n + 15) / 16;   // 16-byte chunks of a plane's bf16 values
    // Odd L: planes start at any element, so a plane's 16-byte chunks are not
    // dword aligned; a dword that straddles a buffer's end reads as 0, so the
    // bound reaches past the dword holding the last element (2 bytes at most
    // past the tensor, never used)
    const int bytes = static_cast<int>(static_cast<int64_t>(planes) * n * 2);
    const int span = Odd ? ((bytes + 2 + 3) & ~3) : bytes;

    // ------------------------------------------------ u: the first batch, prefetched for the end
    const __amdgpu_buffer_rsrc_t us = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(u), 0, span, kBufFlags);
    u32x4_t uv[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
        const int f = tid + NT * k;
        uv[k] = f < nchunk ? __builtin_amdgcn_raw_buffer_load_b128(us, plane_b + 16u * static_cast<uint32_t>(f), 0, 0)
                           : u32x4_t{0u, 0u, 0u, 0u};
    }
    // x and lambda are loaded by the plane fill, in batches
    const __amdgpu_buffer_rsrc_t xs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), 0, span, kBufFlags);
    const __amdgpu_buffer_rsrc_t ls = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(lam), 0, span, kBufFlags);

    const DuoArgs a{w4, w4_bytes, eps, planes, L, cpg, plane};
    // LANES 32: wavefront 0 the rows, 1 the columns; 64: wavefronts 0..3
    // top-down, bottom-up, left-right, right-left
    const bool rows = LANES == 32 ? wave == 0 : wave < 2;
    const int wave_half = LANES == 32 ? 0 : (wave & 1);
    if (rows)
        scan_pair<K, R, D, true, LANES, NT, Odd>(a, lay, tid, lane, wave_half, nchunk, xs, ls, plane_b);
    else
        scan_pair<K, R, D, false, LANES, NT, Odd>(a, lay, tid, lane, wave_half, nchunk, xs, ls, plane_b);
    block_lds_barrier();

    // ------------------------------------------------ meeting pixels
    // (t, t) += LR's side word of step t + RL's of step L-1-t;
    // (t, L-1-t) += RL's of step t + LR's of step L-1-t.
    // Odd L: the middle row and column get the mid lines; of their pixels
    // only (m, m) is also on a diagonal, and its thread adds both.
    for (int t = tid; t < L; t += NT) {
        const uint32_t sd = static_cast<uint32_t>(lay.s + 4 * (t * L + t));
        const uint32_t sa = static_cast<uint32_t>(lay.s + 4 * (t * L + L - 1 - t));
        const float d0 = lds_ref<float>(lay.side + 4 * t);
        const float d1 = lds_ref<float>(lay.side + 4 * (3 * L + L - 1 - t));
        const float a0 = lds_ref<float>(lay.side + 4 * (L + t));
        const float a1 = lds_ref<float>(lay.side + 4 * (2 * L + L - 1 - t));
        lds_ref<float>(sd) = (lds_ref<float>(sd) + d0) + d1;
        lds_ref<float>(sa) = (lds_ref<float>(sa) + a0) + a1;
        if constexpr (Odd) {
            const int m = L / 2;
            const float mr = lds_ref<float>(lay.mid + 4 * t);
            const float mc = lds_ref<float>(lay.mid + 4 * (L + t));
            if (t == m) {
                lds_ref<float>(sd) = (lds_ref<float>(sd) + mr) + mc;
            } else {
                const uint32_t sr = static_cast<uint32_t>(lay.s + 4 * (m * L + t));
                const uint32_t sc = static_cast<uint32_t>(lay.s + 4 * (t * L + m));
                lds_ref<float>(sr) = lds_ref<float>(sr) + mr;
                lds_ref<float>(sc) = lds_ref<float>(sc) + mc;
            }
        }
    }
    block_lds_barrier();

    // ------------------------------------------------ y = u * S
    const __amdgpu_buffer_rsrc_t ys = __builtin_amdgcn_make_buffer_rsrc(y, 0, span, kBufFlags);
    const int nfull = (2 * n) / 16;   // whole chunks of the plane
    for (int f0 = 0; f0 < nchunk; f0 += NT * kBatch) {
    if (f0 > 0) {
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const int f = f0 + tid + NT * k;
            uv[k] = f < nchunk ? __builtin_amdgcn_raw_buffer_load_b128(us, plane_b + 16u * static_cast<uint32_t>(f), 0, 0)
                               : u32x4_t{0u, 0u, 0u, 0u};
        }
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
        const int f = f0 + tid + NT * k;
        if (f < nchunk) {
            const f32x4_t sa = lds_ref<f32x4_t>(lay.s + 32u * f);
            const f32x4_t sb = lds_ref<f32x4_t>(lay.s + 32u * f + 16u);
            u32x4_t o;
            o[0] = pack_bf16x2(bf_lo(uv[k][0]) * sa[0], bf_hi(uv[k][0]) * sa[1]);
            o[1] = pack_bf16x2(bf_lo(uv[k][1]) * sa[2], bf_hi(uv[k][1]) * sa[3]);
            o[2] = pack_bf16x2(bf_lo(uv[k][2]) * sb[0], bf_hi(uv[k][2]) * sb[1]);
            o[3] = pack_bf16x2(bf_lo(uv[k][3]) * sb[2], bf_hi(uv[k][3]) * sb[3]);
            const uint32_t yo = plane_b + 16u * static_cast<uint32_t>(f);
            if constexpr (Odd) {
                // planes start at any element: whole chunks as one unaligned
                // store, the last one element by element (never into the next
                // plane, which another workgroup writes)
                uint16_t* yp = y + static_cast<size_t>(plane) * n + 8 * f;
                if (f < nfull) {
                    *reinterpret_cast<u32x4_u*>(yp) = o;
                } else {
                    const int rest = n - 8 * f;
#pragma unroll
                    for (int e = 0; e < 7; ++e)
                        if (e < rest) yp[e] = static_cast<uint16_t>(o[e >> 1] >> (16 * (e & 1)));
                }
            } else if (f < nfull) {
                __builtin_amdgcn_raw_buffer_store_b128(o, ys, yo, 0, 0);
            } else {  // a plane of L L = 4 mod 8 values ends half way into its last chunk
                __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{o[0], o[1]}, ys, yo, 0, 0);
            }
        }
    }
    }
}

template <int K, int R, int LANES, bool Odd>
hipError_t launch_kr(const void* x, const void* lam, const void* u, const void* w4, float eps,
                     void* y, int64_t planes, int64_t L, const PropOpts& o, hipStream_t stream) {
    // lines of taps in flight: a multiple of K, at least 8 up to K = 3 (the
    // ring of 3-dword windows stays within the registers for K = 4, 5); odd
    // L: also even
    constexpr int DM = Odd && (K % 2) ? 2 * K : K;
    constexpr int D = K <= 3 ? DM * ((8 + DM - 1) / DM) : DM;
    const size_t lds = DuoLayout(static_cast<int>(L)).bytes;
    auto kern = prop2d_duo_kernel<K, R, D, LANES, Odd>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(lds));
        if (e != hipSuccess) return e;
    }
    const int64_t n = planes * L * L;
    kern<<<dim3(static_cast<unsigned>(planes)), dim3(LANES == 32 ? 128 : 256), lds, stream>>>(
        static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(lam), static_cast<const uint16_t*>(u),
        static_cast<const uint16_t*>(w4), static_cast<int>(12 * (n / o.cpg) * 2), eps,
        static_cast<uint16_t*>(y), static_cast<int>(planes), static_cast<int>(L), static_cast<int>(o.cpg));
    return hipGetLastError();
}

template <int K, int LANES, bool Odd = false, int R = K - 1>
hipError_t launch_k(const void* x, const void* lam, const void* u, const void* w4, float eps,
                    void* y, int64_t planes, int64_t L, const PropOpts& o, hipStream_t stream) {
    // R = (L - 1) mod K
    if ((L - 1) % K == R) return launch_kr<K, R, LANES, Odd>(x, lam, u, w4, eps, y, planes, L, o, stream);
    if constexpr (R > 0) return launch_k<K, LANES, Odd, R - 1>(x, lam, u, w4, eps, y, planes, L, o, stream);
    return hipErrorInvalidValue;
}

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

}  // namespace

bool prop2d_duo_eligible(int dtype, int64_t planes, int64_t H, int64_t W, const PropOpts& o,
                         const void* x, const void* lam, const void* u, const void* w4,
                         const void* y) {
    if (dtype != 1 || H != W || H <= 64 || H > kMaxSide) return false;
    if ((H & 1) && H < kMinOddSide) return false;
    if (o.k_chunk != 1) return false;
    if (DuoLayout(static_cast<int>(H)).bytes > kLdsBytes) return false;
    if (12 * planes * H * W * 2 > 0x7fffffff) return false;
    return aligned4(x) && aligned4(lam) && aligned4(u) && aligned4(w4) && aligned4(y);
}

hipError_t launch_prop2d_duo(const void* x, const void* lam, const void* u, const void* w4,
                             float eps, void* y, int64_t planes, int64_t L, const PropOpts& o,
                             hipStream_t stream) {
    // A wavefront a direction (64 lanes, K = 2 up to 128, 3 up to 150) where
    // SIMDs would idle: sides 98..150 (one plane a CU) and the small launches
    // of sides up to 80 that reach this kernel.  Two wavefronts a plane (32
    // lanes a direction, K = 3, 96 slots a line) for sides 82..96, where
    // their fuller lines win (96 x 96: 0.041 ms against 0.045 with 64 lanes,
    // 256 planes).
    if (L & 1)
        return L <= 128 ? launch_k<2, 64, true>(x, lam, u, w4, eps, y, planes, L, o, stream)
                        : launch_k<3, 64, true>(x, lam, u, w4, eps, y, planes, L, o, stream);
    if (L <= 80) return launch_k<2, 64>(x, lam, u, w4, eps, y, planes, L, o, stream);
    if (L <= 96) return launch_k<3, 32>(x, lam, u, w4, eps, y, planes, L, o, stream);
    if (L <= 128) return launch_k<2, 64>(x, lam, u, w4, eps, y, planes, L, o, stream);
    return launch_k<3, 64>(x, lam, u, w4, eps, y, planes, L, o, stream);
}

}  // namespace gspn
