// Four-direction propagation of square bf16 planes with even sides up to 80,
// all four scan orders at once: one wavefront per (b, c) plane, one 16-lane
// row of the wavefront per direction (gfx950).
//
// Operator: "Scaling Parallel Sequence Models to Foundation-Scale Vision
// Encoders", §3 line-scan recurrence (standard GSPN form), §4.1 single-kernel
// design, §4.3 hidden state kept on chip, §5.1 fused normalisation (sigmoid,
// local sum, clamp, divide); reading notes, method / overall framework.
//
// Work split.  Lanes 16 g .. 16 g + 15 scan direction g (0 top-down, 1
// bottom-up, 2 left-right, 3 right-left) of the same plane, all in the same
// step: at step s, TD is on row s, BU on row L-1-s, LR on column s and RL on
// column L-1-s.  Lane q of a row holds positions Kq .. Kq+K-1 of its line in
// registers (K = 1..5 for sides up to 16, 32, 48, 64, 80), and the
// neighbour exchange is one DPP shift each way inside the 16-lane row (its
// first and last lanes receive 0, which only dropped taps weigh).  Compared
// with scanning rows and then columns with two directions a wavefront, a
// 74-position line fills 74 of 80 slots instead of 74 of 96, and the plane
// takes one pass of L steps instead of two.
//
// On-chip data, per plane:
//   S   fp32 [L][L]: the sum of the four directional states.  Every step
//       adds h into the value of its pixel read one step earlier.
//   b = lambda x of every pixel, computed before the scan from coalesced
//       loads of x and lambda.  The exact product of two bf16 values has at
//       most 16 significant bits, so its fp32 pattern ends in 8 zero bits:
//       it is kept as 24 bits, the upper 16 in one array and the next 8 in
//       another (3 bytes a pixel).
//   side fp32 [4][L]: the column scans' terms of the pixels where a row scan
//       and a column scan meet in the same step.
// At 74 x 74 a plane takes 39.5 KB, so four planes share a CU.
//
// Meeting pixels.  Any row line and column line cross, so in every step the
// column scans reach four pixels that a row scan updates in the same step:
// (s, s), (s, L-1-s), (L-1-s, s), (L-1-s, L-1-s).  There the column scan
// adds its state into a side word indexed by the step instead of into S (a
// column slot's row is Kq + j, so the meeting rows s and L-1-s fall in slots
// s mod K and (L-1-s) mod K, both fixed for each step of a block of
// K-aligned steps once (L-1) mod K is a template constant).  After the scan
// the side words are added into the diagonal and anti-diagonal pixels.  Row
// scans never meet each other (L even), nor do column scans; every other
// pair of updates of one pixel falls in different steps, and each step reads
// its pixels' sums after the previous step's writes.  One wavefront does all
// adds in program order, so every pixel's four terms are summed in a fixed
// order and the result is bitwise reproducible.
//
// Grid.  The launch has as many workgroups as the CUs keep resident at once
// (four 74 x 74 planes a CU), each walking planes blockIdx.x + i gridDim.x:
// a workgroup issues its next plane's x, lambda and first tap lines as soon
// as the current plane's scan ends, so they arrive while it adds the meeting
// pixels' side words and writes y, instead of every workgroup of a second
// round waiting for them at once.
//
// Slots past the end of a line (positions >= L) read and write dummy words,
// decode every tap to -2^127 (weight exactly 0) and hold h = 0; lanes whose
// whole window lies past the line load nothing (an offset past the buffer).
// So no value outside the plane enters it.
#include "gspn_device.h"
#include "gspn_internal.h"
#include "gspn_lane.h"

#include <mutex>
#include <type_traits>

namespace gspn {
namespace {

using namespace lane;

// LDS layout in bytes (offsets multiples of 16):
//   [S dummy: 16][b dummy: 16][pad: 4 L][S: L L fp32][side: 4 L fp32]
//   [b_hi: L L + 8 u16][b_lo: L L + L + 8 u8]
// The last step's read-ahead goes one line past every scan: one row before S
// (the pad), one row after it (side), and for b the neighbouring arrays or
// b_lo's spare row.
// b_hi and b_lo have 8 spare entries for the second half of the plane's last
// 16-byte chunk when L L is not a multiple of 8.  A workgroup of several
// planes gives each its own copy, `bytes` apart; the offsets below include
// the copy's base.
struct QuadLayout {
    int base, sdum, bdum, s, side, bh, bl, bytes;
    __host__ __device__ static int a16(int v) { return (v + 15) & ~15; }
    __host__ __device__ explicit QuadLayout(int L, int copy = 0) {
        const int n = L * L;
        bytes = a16(a16(a16(a16(32 + 4 * L) + 4 * n) + 16 * L) + 2 * (n + 8)) + n + L + 8;
        bytes = a16(bytes);
        base = copy * bytes;
        sdum = base;
        bdum = base + 16;
        s = base + a16(32 + 4 * L);
        side = a16(s + 4 * n);
        bh = a16(side + 16 * L);
        bl = a16(bh + 2 * (n + 8));
    }
};

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
template <typename V> using lds_t = __attribute__((address_space(3))) V;

template <typename V>
__device__ __forceinline__ lds_t<V>& lds_ref(uint32_t byte_off) {
    // the kernel's only LDS is its dynamic array, which starts at address 0
    return *reinterpret_cast<lds_t<V>*>(static_cast<uintptr_t>(byte_off));
}

// Orders this wavefront's LDS accesses before the fence against those after
// it (one wavefront per workgroup; global loads in flight are not waited for).
__device__ __forceinline__ void lds_order() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
}

// Shifts inside each 16-lane row: lane l receives lane l - 1 (from_prev) or
// l + 1 (from_next) of its row; a row's first (last) lane receives 0.
__device__ __forceinline__ float row_prev(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, true));
}
__device__ __forceinline__ float row_next(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x101, 0xf, 0xf, true));
}

// bf16 of the low / high half of a dword as fp32
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// K: positions a lane; R = (L - 1) mod K; D: steps a block (a multiple of K),
// also the number of lines of taps prefetched ahead.
// Floats of prepared weights a lane keeps a line: three a position, padded
// to whole 16-byte loads.
constexpr int prepared_floats(int K) { return (3 * K + 3) / 4 * 4; }

// Weights of taps shared by a group of channels, normalised once for all of
// them (paper §4.2, channel-shared weights; §5.1 fused normalisation: sigmoid,
// local sum, clamp, divide).  For position p = Kq + j of the line the scan
// reaches at a step (lane q of the 16 a direction takes, slot j), w_k =
// s_k / max(s_0 + s_1 + s_2, eps) with
// s_k the sigmoid of raw tap k, 0 for taps whose source lies outside the line
// and for positions past its end.  Output [4][tap planes][L steps][16][KP]
// fp32, position j's taps at 3 j .. 3 j + 2; the same arithmetic as the
// fused kernels (hardware exp2 and reciprocal).
template <int K>
__global__ void __launch_bounds__(256)
quad_prepare_kernel(const uint16_t* __restrict__ w4, float* __restrict__ wp, float eps, int tap_planes,
                    int L) {
    // one thread per (direction and tap plane, step, slot Kq + j of the 16 K
    // a line has): its three weights, and the lane's padding after its last
    // slot
    constexpr int KP = prepared_floats(K);
    constexpr int NS = 16 * K;
    const int64_t total = static_cast<int64_t>(4) * tap_planes * L * NS;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (t >= total) return;
    const int p = static_cast<int>(t % NS);
    const int64_t ls = t / NS;                              // (direction, tap plane, step)
    const int step = static_cast<int>(ls % L);
    const int64_t dp = ls / L;                              // direction * tap_planes + tap plane
    const int dir = static_cast<int>(dp / tap_planes);
    const int line = (dir & 1) == 0 ? step : L - 1 - step;
    const int q = p / K, j = p - q * K;
    float* dst = wp + (ls * 16 + q) * KP + 3 * j;
    if (j == K - 1) {
#pragma unroll
        for (int e = 3 * K; e < KP; ++e) wp[(ls * 16 + q) * KP + e] = 0.0f;
    }
    if (p >= L) {
        dst[0] = dst[1] = dst[2] = 0.0f;
        return;
    }
    const int64_t n = static_cast<int64_t>(L) * L;
    const uint16_t* src = w4 + dp * 3 * n + static_cast<int64_t>(line) * L + p;
    float sv[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const bool dropped = (k == 0 && p == 0) || (k == 2 && p == L - 1);
        const float z = __uint_as_float(static_cast<uint32_t>(src[k * n]) << 16);
        sv[k] = dropped ? 0.0f : __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(z * kNegLog2e) + 1.0f);
    }
    const float r = __builtin_amdgcn_rcpf(fmaxf((sv[0] + sv[1]) + sv[2], eps));
#pragma unroll
    for (int k = 0; k < 3; ++k) dst[k] = sv[k] * r;
}

// PRE: w4 holds the weights quad_prepare_kernel wrote (fp32, normalised, in
// scan order, KP a lane a line) instead of raw bf16 taps.
// WPB: planes (wavefronts) a workgroup, 1 or (with prepared weights) 4.
template <int K, int R, int D, bool PRE, int WPB>
__global__ void __launch_bounds__(64 * WPB)
prop2d_quad_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ lam,
                   const uint16_t* __restrict__ u, const uint16_t* __restrict__ w4, int w4_bytes,
                   float eps, uint16_t* __restrict__ y, int planes, int L, int cpg) {
    static_assert(D % K == 0, "blocks of whole slot cycles");
    constexpr int NW = window_words<uint16_t, K>();
    constexpr int KP = prepared_floats(K);
    constexpr int NV = KP / 4;
    static_assert(WPB == 1 || (WPB == 4 && PRE), "four planes a workgroup share prepared weights");
    const int n = L * L;
    const int lane = WPB == 1 ? static_cast<int>(threadIdx.x) : static_cast<int>(threadIdx.x) & 63;
    const int wave = WPB == 1 ? 0 : static_cast<int>(threadIdx.x) >> 6;
    const QuadLayout lay(L, wave);
    const int g = lane >> 4;             // 0 TD, 1 BU, 2 LR, 3 RL
    const int q = lane & 15;
    const bool rows = g < 2;
    const bool fwd = (g & 1) == 0;
    // A workgroup takes plane slots v = blockIdx.x, blockIdx.x + gridDim.x,
    // ... (the grid holds at most as many workgroups as the CUs keep
    // resident): the next slot's x, lambda and first tap lines are loaded
    // while the current plane's sums are finished and written out.  gridDim.x
    // is a multiple of 8 or the whole slot count, so v and blockIdx.x share an
    // XCD.  A slot is WPB consecutive planes, one a wavefront.
    // With shared taps, consecutive workgroups go to the 8 XCDs in turn, and
    // slot v is chosen so that XCD x walks tap groups x, x + 8, ...: every
    // channel of a group reads its weights through one L2, and the
    // wavefronts of a workgroup (channels of one group, at about the same
    // step) through one L1.  Any plane order gives the same results.
    const int slots = (planes + WPB - 1) / WPB;
    auto plane_of = [&](int v) -> int {
        if constexpr (PRE) {
            const int spg = cpg / WPB;     // slots a tap group
            if (cpg % WPB == 0 && planes % (8 * cpg) == 0) {
                const int x8 = v & 7, sl = v >> 3;
                return (((sl / spg) * 8 + x8) * spg + sl % spg) * WPB + wave;
            }
        }
        return v * WPB + wave;
    };
    const int nchunk = (2 * n + 15) / 16;  // 16-byte chunks of a plane's bf16 values

    // ------------------------------------------------ u, prefetched for the end
    // (it arrives while the plane is scanned; kU 16-byte chunks a lane)
    constexpr int kU = (2 * (16 * K) * (16 * K) / 16 + 63) / 64;   // sides up to 16 K
    const __amdgpu_buffer_rsrc_t us = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(u), 0, static_cast<int>(static_cast<int64_t>(planes) * n * 2), kBufFlags);
    u32x4_t uv[kU];

    // ------------------------------------------------ x and lambda, all at once
    const __amdgpu_buffer_rsrc_t xs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(x), 0, static_cast<int>(static_cast<int64_t>(planes) * n * 2), kBufFlags);
    const __amdgpu_buffer_rsrc_t ls = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(lam), 0, static_cast<int>(static_cast<int64_t>(planes) * n * 2), kBufFlags);
    u32x4_t xv[kU], lv[kU];

    // ------------------------------------------------ taps: first D lines
    const int tap_planes = planes / cpg;
    __amdgpu_buffer_rsrc_t taps[3];
    const int par = (K * q) & 1;
    const bool lane_live = K * q < L;
    const uint32_t line_b = static_cast<uint32_t>(L) * 2u;
    uint32_t lo = 0, lo_min = 0, lo_max = 0, dlo = 0;
    words_t<NW> tbuf[PRE ? 1 : D][3];
    // prepared weights: this lane's KP floats of the direction's step 0, then
    // one line of 16 lanes a step
    u32x4_t pbuf[PRE ? D : 1][NV];
    const __amdgpu_buffer_rsrc_t wpr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(w4), 0, w4_bytes, kBufFlags);
    uint32_t po = 0;
    constexpr uint32_t dpo = 16u * KP * 4u;
    if constexpr (!PRE) {
#pragma unroll
        for (int k = 0; k < 3; ++k)
            taps[k] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(w4) + static_cast<size_t>(k) * n,
                                                        0, w4_bytes - k * n * 2, kBufFlags);
    }
    // a plane's first tap line of this lane's direction
    auto tap_start = [&](int plane) {
        if constexpr (PRE) {
            po = (static_cast<uint32_t>(g * tap_planes + plane / cpg) * static_cast<uint32_t>(L) * 16u +
                  static_cast<uint32_t>(q)) * (KP * 4u);
        } else {
            const uint32_t tap_base =
                static_cast<uint32_t>((g * tap_planes + plane / cpg) * 3) * static_cast<uint32_t>(n) * 2u +
                static_cast<uint32_t>(K * q - par) * 2u;
            lo_min = lane_live ? tap_base : 0x80000000u;
            lo_max = lane_live ? tap_base + static_cast<uint32_t>(L - 1) * line_b : 0x80000000u;
            lo = fwd ? lo_min : lo_max;
            dlo = lane_live ? (fwd ? line_b : 0u - line_b) : 0u;
        }
    };
    auto load_line = [&](int d) {
        if constexpr (PRE) {
            // a step past the scan reads the next block or past the buffer
            // (0); its weights are never used
#pragma unroll
            for (int v = 0; v < NV; ++v) pbuf[d][v] = __builtin_amdgcn_raw_buffer_load_b128(wpr, po + 16u * v, 0, 0);
            po += dpo;
        } else {
#pragma unroll
            for (int k = 0; k < 3; ++k) tbuf[d][k] = load_words<NW>(taps[k], lo);
            const uint32_t nx = lo + dlo;
            lo = umed3(nx, lo_min, lo_max);
        }
    };
    // x, lambda and the first D tap lines of a plane
    auto issue_plane = [&](int plane) {
        const uint32_t pb = static_cast<uint32_t>(plane) * static_cast<uint32_t>(n) * 2u;
#pragma unroll
        for (int k = 0; k < kU; ++k) {
            const int f = lane + 64 * k;
            const uint32_t off = pb + 16u * static_cast<uint32_t>(f);
            xv[k] = f < nchunk ? __builtin_amdgcn_raw_buffer_load_b128(xs, off, 0, 0) : u32x4_t{0u, 0u, 0u, 0u};
            lv[k] = f < nchunk ? __builtin_amdgcn_raw_buffer_load_b128(ls, off, 0, 0) : u32x4_t{0u, 0u, 0u, 0u};
        }
        tap_start(plane);
#pragma unroll
        for (int d = 0; d < D; ++d) {
            load_line(d);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    issue_plane(plane_of(static_cast<int>(blockIdx.x)));

    for (int v = static_cast<int>(blockIdx.x); v < slots; v += static_cast<int>(gridDim.x)) {
        const int plane = plane_of(v);
        if constexpr (WPB > 1) {
            if (plane >= planes) continue;   // the last slot's spare wavefronts (no barrier anywhere)
        }
        const uint32_t plane_b = static_cast<uint32_t>(plane) * static_cast<uint32_t>(n) * 2u;
        // ------------------------------------------------ u, for the end
        // (it arrives while the plane is scanned; kU 16-byte chunks a lane)
#pragma unroll
        for (int k = 0; k < kU; ++k) {
            const int f = lane + 64 * k;
            uv[k] = f < nchunk ? __builtin_amdgcn_raw_buffer_load_b128(us, plane_b + 16u * static_cast<uint32_t>(f), 0, 0)
                               : u32x4_t{0u, 0u, 0u, 0u};
        }

        // ------------------------------------------------ zero S, side, dummies
        // (after the previous plane's last reads of S)
        lds_order();
        for (int f = lane; f < (lay.bh - lay.base) / 16; f += 64)
            lds_ref<u32x4_t>(static_cast<uint32_t>(lay.base) + 16u * f) = u32x4_t{0u, 0u, 0u, 0u};

        // ------------------------------------------------ b = lambda x into LDS
#pragma unroll
        for (int k = 0; k < kU; ++k) {
            const int f = lane + 64 * k;
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
        lds_order();

        // ------------------------------------------------ per-slot constants
        const int i0 = fwd ? 0 : L - 1;
        const int de = rows ? (fwd ? L : -L) : (fwd ? 1 : -1);
        uint32_t aS[K], aH[K], aL[K];
        int dSj[K], dHj[K], dLj[K];
        uint32_t sel[3][K];
        const uint32_t sel_even = par ? 0x03020c0cu : 0x01000c0cu;
        const uint32_t sel_odd = par ? 0x05040c0cu : 0x03020c0cu;
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const int p = K * q + j;
            const bool valid = p < L;
            const int e = rows ? i0 * L + p : p * L + i0;
            aS[j] = valid ? static_cast<uint32_t>(lay.s + 4 * e) : static_cast<uint32_t>(lay.sdum);
            aH[j] = valid ? static_cast<uint32_t>(lay.bh + 2 * e) : static_cast<uint32_t>(lay.bdum);
            aL[j] = valid ? static_cast<uint32_t>(lay.bl + e) : static_cast<uint32_t>(lay.bdum);
            dSj[j] = valid ? 4 * de : 0;
            dHj[j] = valid ? 2 * de : 0;
            dLj[j] = valid ? de : 0;
            const uint32_t s_in = (j & 1) ? sel_odd : sel_even;
            sel[0][j] = (valid && p > 0) ? s_in : kSelDropped;
            sel[1][j] = valid ? s_in : kSelDropped;
            sel[2][j] = (valid && p < L - 1) ? s_in : kSelDropped;
        }
        // column slots that meet a row scan: key q for the column rows, none else
        const uint32_t key = rows ? 0xffu : static_cast<uint32_t>(q);
        const uint32_t side1 = static_cast<uint32_t>(lay.side + 4 * L * (g == 3 ? 1 : 0));
        const uint32_t side2 = static_cast<uint32_t>(lay.side + 4 * L * (g == 3 ? 3 : 2));

        float h[K], acc[K];
        uint32_t bhr[K], blr[K];
        uint32_t ra1 = 0, ra2 = 0;   // addresses of this step's two meeting slots

        // S address of slot j at step s, for a step whose meeting slots are j1
        // (row s, lanes q1) and j2 (row L-1-s, lanes q2)
        auto meet_addr = [&](int j, int j1, int j2, uint32_t q1, uint32_t q2, int s) -> uint32_t {
            uint32_t a = aS[j];
            if (j == j1) a = key == q1 ? side1 + 4u * s : a;
            if (j == j2) a = key == q2 ? side2 + 4u * s : a;
            return a;
        };
        // Meeting slots of step s = s0 + t of a block starting at s0 (a multiple
        // of K; t a compile-time value): rows s (slot t mod K, lanes q1) and
        // L-1-s (slot (R - t) mod K, lanes q2), with q1 = s0 / K + t / K and q2 =
        // (L-1-R-s0) / K + floor((R - t) / K).
        auto read_ahead = [&](int t, int s, int qb1, int qb2) {
            const int j1 = t % K;
            const int j2 = ((R - t) % K + K) % K;
            const uint32_t q1 = static_cast<uint32_t>(qb1 + t / K);
            const uint32_t q2 = static_cast<uint32_t>(qb2 + (R - t >= 0 ? (R - t) / K : -((t - R + K - 1) / K)));
            ra1 = meet_addr(j1, j1, j2, q1, q2, s);
            ra2 = meet_addr(j2, j1, j2, q1, q2, s);
#pragma unroll
            for (int j = 0; j < K; ++j) {
                const uint32_t a = j == j1 ? ra1 : (j == j2 ? ra2 : aS[j]);
                acc[j] = lds_ref<float>(a);
                bhr[j] = lds_ref<uint16_t>(aH[j]);
                blr[j] = lds_ref<uint8_t>(aL[j]);
            }
        };
#pragma unroll
        for (int j = 0; j < K; ++j) h[j] = 0.0f;
        read_ahead(0, 0, 0, (L - 1 - R) / K);

        auto step = [&](int s, int d, int qb1, int qb2) {
            float hn[K];
            if constexpr (PRE) {
                asm volatile("" : "+v"(pbuf[d][0]));
                float wv[3 * K];
#pragma unroll
                for (int e = 0; e < 3 * K; ++e) wv[e] = __uint_as_float(pbuf[d][e / 4][e % 4]);
                // refill slot d only after it has been read
#pragma unroll
                for (int e = 0; e < 3 * K; ++e) asm volatile("" : "+v"(po) : "v"(wv[e]));
                load_line(d);
                float bv[K];
#pragma unroll
                for (int j = 0; j < K; ++j) bv[j] = __uint_as_float(__builtin_amdgcn_perm(bhr[j], blr[j], 0x0504000cu));
                const float hl0 = row_prev(h[K - 1]);
                const float hrK = row_next(h[0]);
#pragma unroll
                for (int j = 0; j < K; ++j) {
                    const float hl = j > 0 ? h[j - 1] : hl0;
                    const float hr = j < K - 1 ? h[j + 1] : hrK;
                    hn[j] = fmaf(wv[3 * j + 2], hr, fmaf(wv[3 * j], hl, fmaf(wv[3 * j + 1], h[j], bv[j])));
                }
            } else {
            asm volatile("" : "+v"(tbuf[d][0]), "+v"(tbuf[d][1]), "+v"(tbuf[d][2]));
            float s0v[K], s1v[K], s2v[K], r[K];
#pragma unroll
            for (int j = 0; j < K; ++j) {
                s0v[j] = window_elem<uint16_t, K, NW>(tbuf[d][0], j, sel[0][j], sel[0][j]) * kNegLog2e;
                s1v[j] = window_elem<uint16_t, K, NW>(tbuf[d][1], j, sel[1][j], sel[1][j]) * kNegLog2e;
                s2v[j] = window_elem<uint16_t, K, NW>(tbuf[d][2], j, sel[2][j], sel[2][j]) * kNegLog2e;
            }
#pragma unroll
            for (int j = 0; j < K; ++j) {
                s0v[j] = __builtin_amdgcn_exp2f(s0v[j]);
                s1v[j] = __builtin_amdgcn_exp2f(s1v[j]);
                s2v[j] = __builtin_amdgcn_exp2f(s2v[j]);
            }
#pragma unroll
            for (int j = 0; j < K; ++j) {
                s0v[j] = __builtin_amdgcn_rcpf(s0v[j] + 1.0f);
                s1v[j] = __builtin_amdgcn_rcpf(s1v[j] + 1.0f);
                s2v[j] = __builtin_amdgcn_rcpf(s2v[j] + 1.0f);
            }
#pragma unroll
            for (int j = 0; j < K; ++j) r[j] = s0v[j] + s1v[j];
#pragma unroll
            for (int j = 0; j < K; ++j) r[j] = fmaxf(r[j] + s2v[j], eps);
#pragma unroll
            for (int j = 0; j < K; ++j) r[j] = __builtin_amdgcn_rcpf(r[j]);
            // refill slot d only after it has been decoded
#pragma unroll
            for (int j = 0; j < K; ++j)
                asm volatile("" : "+v"(lo) : "v"(s0v[j]), "v"(s1v[j]), "v"(s2v[j]), "v"(r[j]));
            load_line(d);

            float bv[K];
#pragma unroll
            for (int j = 0; j < K; ++j) bv[j] = __uint_as_float(__builtin_amdgcn_perm(bhr[j], blr[j], 0x0504000cu));
            const float hl0 = row_prev(h[K - 1]);
            const float hrK = row_next(h[0]);
#pragma unroll
            for (int j = 0; j < K; ++j) {
                const float hl = j > 0 ? h[j - 1] : hl0;
                const float hr = j < K - 1 ? h[j + 1] : hrK;
                float m = s1v[j] * h[j];
                m = fmaf(s0v[j], hl, m);
                m = fmaf(s2v[j], hr, m);
                hn[j] = fmaf(m, r[j], bv[j]);
            }
            }
#pragma unroll
            for (int j = 0; j < K; ++j) h[j] = hn[j];

            const int t = d % K;
            const int j1 = t;
            const int j2 = ((R - t) % K + K) % K;
#pragma unroll
            for (int j = 0; j < K; ++j) {
                const uint32_t a = j == j1 ? ra1 : (j == j2 ? ra2 : aS[j]);
                lds_ref<float>(a) = acc[j] + h[j];
            }
            // the next step's pixels, read after this step's writes (the pins keep
            // each address one add a step instead of base + multiple of the step)
#pragma unroll
            for (int j = 0; j < K; ++j) {
                aS[j] += dSj[j];
                aH[j] += dHj[j];
                aL[j] += dLj[j];
                asm volatile("" : "+v"(aS[j]), "+v"(aH[j]), "+v"(aL[j]));
            }
            read_ahead(d + 1, s + 1, qb1, qb2);
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
        // the next plane's inputs and first tap lines, while this one finishes
        if (v + static_cast<int>(gridDim.x) < slots) issue_plane(plane_of(v + static_cast<int>(gridDim.x)));
        lds_order();

        // ------------------------------------------------ meeting pixels
        // (t, t) += LR's side word of step t + RL's of step L-1-t;
        // (t, L-1-t) += RL's of step t + LR's of step L-1-t
        for (int t = lane; t < L; t += 64) {
            const uint32_t sd = static_cast<uint32_t>(lay.s + 4 * (t * L + t));
            const uint32_t sa = static_cast<uint32_t>(lay.s + 4 * (t * L + L - 1 - t));
            const float d0 = lds_ref<float>(lay.side + 4 * t);                    // LR, row = col = t
            const float d1 = lds_ref<float>(lay.side + 4 * (3 * L + L - 1 - t));  // RL at step L-1-t
            const float a0 = lds_ref<float>(lay.side + 4 * (L + t));              // RL, (t, L-1-t)
            const float a1 = lds_ref<float>(lay.side + 4 * (2 * L + L - 1 - t));  // LR at step L-1-t
            lds_ref<float>(sd) = (lds_ref<float>(sd) + d0) + d1;
            lds_ref<float>(sa) = (lds_ref<float>(sa) + a0) + a1;
        }
        lds_order();

        // ------------------------------------------------ y = u * S
        {
            const __amdgpu_buffer_rsrc_t ys = __builtin_amdgcn_make_buffer_rsrc(
                y, 0, static_cast<int>(static_cast<int64_t>(planes) * n * 2), kBufFlags);
            const int nfull = (2 * n) / 16;   // whole chunks of the plane
#pragma unroll
            for (int k = 0; k < kU; ++k) {
                const int f = lane + 64 * k;
                if (f < nchunk) {
                    const f32x4_t sa = lds_ref<f32x4_t>(lay.s + 32u * f);
                    const f32x4_t sb = lds_ref<f32x4_t>(lay.s + 32u * f + 16u);
                    u32x4_t o;
                    o[0] = pack_bf16x2(bf_lo(uv[k][0]) * sa[0], bf_hi(uv[k][0]) * sa[1]);
                    o[1] = pack_bf16x2(bf_lo(uv[k][1]) * sa[2], bf_hi(uv[k][1]) * sa[3]);
                    o[2] = pack_bf16x2(bf_lo(uv[k][2]) * sb[0], bf_hi(uv[k][2]) * sb[1]);
                    o[3] = pack_bf16x2(bf_lo(uv[k][3]) * sb[2], bf_hi(uv[k][3]) * sb[3]);
                    const uint32_t yo = plane_b + 16u * static_cast<uint32_t>(f);
                    if (f < nfull)
                        __builtin_amdgcn_raw_buffer_store_b128(o, ys, yo, 0, 0);
                    else  // a plane of L L = 4 mod 8 values ends half way into its last chunk
                        __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{o[0], o[1]}, ys, yo, 0, 0);
                }
            }
        }
    }  // planes of this workgroup
}

// Workgroups of `threads` threads with `lds` bytes of LDS each that the
// device keeps resident at once: its CUs times the smaller of the kernel's
// own limit per CU (registers; queried once per kernel) and the LDS limit.
template <typename F>
hipError_t resident_workgroups(F* kern, int threads, size_t lds, int64_t* out) {
    static std::once_flag once;
    static int per_cu = 0;
    static hipError_t err = hipSuccess;
    std::call_once(once, [kern, threads] {
        err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern), threads, 0);
    });
    if (err != hipSuccess) return err;
    int cus = 1;
    const hipError_t e = device_cu_count(&cus);
    if (e != hipSuccess) return e;
    int64_t w = per_cu > 0 ? per_cu : 1;
    const int64_t by_lds = lds > 0 ? static_cast<int64_t>(kLdsBytes / static_cast<int64_t>(lds)) : w;
    w = by_lds < w ? (by_lds > 0 ? by_lds : 1) : w;
    *out = w * cus;
    return hipSuccess;
}

// D: lines of taps in flight; with prepared weights a line takes KP
// registers instead of 3 window words, so fewer are kept.
template <int K, bool PRE> constexpr int depth() { return PRE ? K * ((5 + K - 1) / K) : K * ((8 + K - 1) / K); }

template <int K, int R, bool PRE, int WPB>
hipError_t launch_krw(const void* x, const void* lam, const void* u, const void* w4, int64_t w4_bytes,
                      float eps, void* y, int64_t planes, int64_t L, const PropOpts& o, hipStream_t stream) {
    constexpr int D = depth<K, PRE>();
    const size_t lds = static_cast<size_t>(WPB) * QuadLayout(static_cast<int>(L)).bytes;
    auto kern = prop2d_quad_kernel<K, R, D, PRE, WPB>;
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 static_cast<int>(lds));
        if (e != hipSuccess) return e;
    }
    // as many workgroups as the CUs keep resident at once (each walks its
    // share of the plane slots), or one a slot when there are fewer slots
    int64_t resident = 0;
    const hipError_t e = resident_workgroups(kern, 64 * WPB, lds, &resident);
    if (e != hipSuccess) return e;
    const int64_t slots = (planes + WPB - 1) / WPB;
    // a multiple of 8 (whole rounds of the XCDs) below the slot count
    const int64_t grid = slots <= resident ? slots : (resident & ~int64_t{7}) > 0 ? (resident & ~int64_t{7}) : resident;
    kern<<<dim3(static_cast<unsigned>(grid)), dim3(64 * WPB), lds, stream>>>(
        static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(lam), static_cast<const uint16_t*>(u),
        static_cast<const uint16_t*>(w4), static_cast<int>(w4_bytes), eps,
        static_cast<uint16_t*>(y), static_cast<int>(planes), static_cast<int>(L), static_cast<int>(o.cpg));
    return hipGetLastError();
}

// With prepared weights, four channels of one tap group a workgroup when
// their four layouts fit in LDS (the weights they read at the same steps
// then come through one L1).
template <int K, int R, bool PRE>
hipError_t launch_kr(const void* x, const void* lam, const void* u, const void* w4, int64_t w4_bytes,
                     float eps, void* y, int64_t planes, int64_t L, const PropOpts& o, hipStream_t stream) {
    if constexpr (PRE) {
        if (o.cpg % 4 == 0 && 4 * static_cast<int64_t>(QuadLayout(static_cast<int>(L)).bytes) <= kLdsBytes)
            return launch_krw<K, R, PRE, 4>(x, lam, u, w4, w4_bytes, eps, y, planes, L, o, stream);
    }
    return launch_krw<K, R, PRE, 1>(x, lam, u, w4, w4_bytes, eps, y, planes, L, o, stream);
}

template <int K, bool PRE>
hipError_t launch_k(const void* x, const void* lam, const void* u, const void* w4, int64_t w4_bytes,
                    float eps, void* y, int64_t planes, int64_t L, const PropOpts& o, hipStream_t stream) {
    switch ((L - 1) % K) {
        case 0: return launch_kr<K, 0, PRE>(x, lam, u, w4, w4_bytes, eps, y, planes, L, o, stream);
        case 1: if constexpr (K > 1) return launch_kr<K, 1 % K, PRE>(x, lam, u, w4, w4_bytes, eps, y, planes, L, o, stream);
                [[fallthrough]];
        case 2: if constexpr (K > 2) return launch_kr<K, 2 % K, PRE>(x, lam, u, w4, w4_bytes, eps, y, planes, L, o, stream);
                [[fallthrough]];
        case 3: if constexpr (K > 3) return launch_kr<K, 3 % K, PRE>(x, lam, u, w4, w4_bytes, eps, y, planes, L, o, stream);
                [[fallthrough]];
        default: if constexpr (K > 4) return launch_kr<K, 4 % K, PRE>(x, lam, u, w4, w4_bytes, eps, y, planes, L, o, stream);
    }
    return hipErrorInvalidValue;
}

int quad_k(int64_t L) { return L <= 16 ? 1 : L <= 32 ? 2 : L <= 48 ? 3 : L <= 64 ? 4 : 5; }

template <bool PRE>
hipError_t launch_any(const void* x, const void* lam, const void* u, const void* w4, int64_t w4_bytes,
                      float eps, void* y, int64_t planes, int64_t L, const PropOpts& o, hipStream_t stream) {
    switch (quad_k(L)) {
        case 1: return launch_k<1, PRE>(x, lam, u, w4, w4_bytes, eps, y, planes, L, o, stream);
        case 2: return launch_k<2, PRE>(x, lam, u, w4, w4_bytes, eps, y, planes, L, o, stream);
        case 3: return launch_k<3, PRE>(x, lam, u, w4, w4_bytes, eps, y, planes, L, o, stream);
        case 4: return launch_k<4, PRE>(x, lam, u, w4, w4_bytes, eps, y, planes, L, o, stream);
        default: return launch_k<5, PRE>(x, lam, u, w4, w4_bytes, eps, y, planes, L, o, stream);
    }
}

template <int K>
hipError_t launch_prepare(const void* w4, void* wp, float eps, int64_t tap_planes, int64_t L,
                          hipStream_t stream) {
    const int64_t total = 4 * tap_planes * L * 16 * K;
    quad_prepare_kernel<K><<<dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, stream>>>(
        static_cast<const uint16_t*>(w4), static_cast<float*>(wp), eps, static_cast<int>(tap_planes),
        static_cast<int>(L));
    return hipGetLastError();
}

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

}  // namespace

bool prop2d_quad_eligible(int dtype, int64_t planes, int64_t H, int64_t W, const PropOpts& o,
                          const void* x, const void* lam, const void* u, const void* w4,
                          const void* y) {
    if (dtype != 1 || H != W || (H & 1) || H > 80) return false;
    if (o.k_chunk != 1) return false;
    if (QuadLayout(static_cast<int>(H)).bytes > kLdsBytes) return false;
    if (12 * planes * H * W * 2 > 0x7fffffff) return false;
    return aligned4(x) && aligned4(lam) && aligned4(u) && aligned4(w4) && aligned4(y);
}

hipError_t launch_prop2d_quad(const void* x, const void* lam, const void* u, const void* w4,
                              float eps, void* y, int64_t planes, int64_t L, const PropOpts& o,
                              hipStream_t stream) {
    const int64_t w4_bytes = 12 * (planes / o.cpg) * L * L * 2;
    return launch_any<false>(x, lam, u, w4, w4_bytes, eps, y, planes, L, o, stream);
}

int64_t prop2d_quad_shared_workspace_bytes(int64_t planes, int64_t L, int64_t cpg) {
    return 4 * (planes / cpg) * L * 16 * prepared_floats(quad_k(L)) * 4;
}

bool prop2d_quad_shared_eligible(int dtype, int64_t planes, int64_t H, int64_t W, const PropOpts& o,
                                 const void* x, const void* lam, const void* u, const void* w4,
                                 const void* y) {
    if (o.cpg < 2) return false;
    if (!prop2d_quad_eligible(dtype, planes, H, W, o, x, lam, u, w4, y)) return false;
    return prop2d_quad_shared_workspace_bytes(planes, H, o.cpg) <= 0x7fffffff;
}

hipError_t launch_prop2d_quad_shared(const void* x, const void* lam, const void* u, const void* w4,
                                     float eps, void* y, int64_t planes, int64_t L,
                                     const PropOpts& o, void* ws, hipStream_t stream) {
    const int64_t tap_planes = planes / o.cpg;
    hipError_t e;
    switch (quad_k(L)) {
        case 1: e = launch_prepare<1>(w4, ws, eps, tap_planes, L, stream); break;
        case 2: e = launch_prepare<2>(w4, ws, eps, tap_planes, L, stream); break;
        case 3: e = launch_prepare<3>(w4, ws, eps, tap_planes, L, stream); break;
        case 4: e = launch_prepare<4>(w4, ws, eps, tap_planes, L, stream); break;
        default: e = launch_prepare<5>(w4, ws, eps, tap_planes, L, stream); break;
    }
    if (e != hipSuccess) return e;
    return launch_any<true>(x, lam, u, ws, prop2d_quad_shared_workspace_bytes(planes, L, o.cpg), eps, y,
                            planes, L, o, stream);
}

}  // namespace gspn
