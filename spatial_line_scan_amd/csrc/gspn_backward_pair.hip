// Gradient of the four-direction propagation, one workgroup per (b, c) plane
// and direction pair, a wavefront per direction (gfx950), for planes of even
// sides up to 160 (bf16; fp32 up to 128, while its wider layout fits in LDS).
//
// Operator: the exact derivative of the forward definition ("Scaling Parallel
// Sequence Models to Foundation-Scale Vision Encoders", §3 line-scan
// recurrence, §5.1 fused normalisation; §6.1 reports backward kernels without
// describing them), with the same formulas as the general backward kernel:
//   adjoint, lines in reverse scan order: g_last = u gy,
//     g_i[p] = u gy + sum_k wn_k(i+1, p-k+1) g_{i+1}[p-k+1];
//   gx = lambda G, glambda = x G, gu = gy S with G = sum_d g_d, S = sum_d h_d;
//   tap gradient gwn_k(i, p) = g_i[p] h_{i-1}[p+k-1] (0 on a scan's first
//   line), then through s = sigmoid(z), T = sum s, r = 1 / max(T, eps):
//     T > eps: gs_m = r sum_{k != m} wn_k (gwn_m - gwn_k), else gs_m = r gwn_m;
//     gz_m = gs_m s_m (1 - s_m); dropped taps have s = 0 and get 0.
//
// Work split.  The row pair (top-down, bottom-up) and the column pair
// (left-right, right-left) are two launches of one kernel that sees the lines
// of its pair as the rows of a line-major plane: the row launch reads x,
// lambda, u and gy as they are, the column launch reads copies transposed by
// transpose4_kernel.  Every direction's taps are line-major already.  The
// first wavefront takes the direction that scans lines 0 .. NL-1, the second
// the other; lane q holds positions Kq .. Kq+K-1 of its line (K = ceil(L /
// 64)), and the three-tap neighbourhood is one DPP lane shift each way, as in
// the forward kernels.  The wavefronts meet only between passes (LDS-only
// barriers).
//   1. Forward: h line by line (taps normalised in registers, b = lambda x
//      from the line's windows); every line of h goes to an fp32 LDS plane of
//      the wavefront.
//   2. S pass: S = h_a + h_b per pixel.  Row launch: to the workspace.
//      Column launch: added to the row launch's S, and gu = gy S written.
//   3. Adjoint, in reverse scan order.  The transposed products of line i+1
//      (wn_k g per destination) stay in registers from the previous step and
//      reach their source positions by lane shifts; the tap gradients of line
//      i take h_{i-1} from the LDS plane, read one step ahead, and go to gw4
//      as they are produced.  g_i overwrites h_i, which was last read one step
//      earlier.
//   4. G pass: G = g_a + g_b per pixel.  Row launch: to the workspace.
//      Column launch: added to the row launch's G, and gx, glambda written.
// Sums run in a fixed order (row pair before column pair, wavefront 0's
// direction before wavefront 1's), so the result is the same on every run.
#include "gspn_device.h"
#include "gspn_internal.h"
#include "gspn_lane.h"

#include <algorithm>
#include <type_traits>

namespace gspn {
namespace {

using namespace lane;

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
template <typename V> using lds_t = __attribute__((address_space(3))) V;

template <typename V>
__device__ __forceinline__ lds_t<V>& lds_at(uint32_t byte_off) {
    // the kernel's only LDS is its dynamic array, which starts at address 0
    return *reinterpret_cast<lds_t<V>*>(static_cast<uintptr_t>(byte_off));
}

// Two wavefronts: their LDS accesses before this point complete before
// either wavefront's after it (LDS only: global loads in flight stay so).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// LDS layout in bytes (offsets multiples of 16):
//   [dummy: 16 per wavefront][2 lines][A: NL x L][B: NL x L][2 lines] ... [staging: 6 x 64 K]
// A is the plane of the first direction's lanes, B that of the second's.
// The line before A and the line after B are zero: the h before a scan's
// first line.  The outer lines only absorb the read-ahead past the last
// adjoint step.  Slots past a line's end read and write the dummy words (16
// bytes, one set per wavefront).
// fp32 data: one array of fp32 values.  bf16 data (narrow): two arrays laid
// out this way, the upper 16 bits and the next 8 bits of each fp32 value
// rounded to nearest even at bit 8 (a 16-bit significand; the gradients are
// rounded to bf16's 8 bits in the end), so that four planes share a CU at
// 74 x 74.
struct PairBwdLayout {
    int a, b, la, lb, stage, bytes;   // line 0 of A and B: fp32 or upper-16-bit array; low-8-bit
                                      // array; tap-gradient staging lines
    static constexpr int dum = 0, ldum = 8;
    __host__ __device__ static int a16(int v) { return (v + 15) & ~15; }
    // gsize: bytes of a staged tap gradient; nstage: staging sets (two when
    // the workgroup's planes add their tap gradients)
    __host__ __device__ PairBwdLayout(int NL, int L, bool narrow, int gsize, int nstage = 1) {
        constexpr int nh = 64;   // lanes a direction takes
        const int w = narrow ? 2 : 4;
        a = a16(32 + 2 * w * L);   // 16 dummy bytes per wavefront
        b = a16(a + w * NL * L);
        int end = b + w * (NL + 2) * L;
        la = lb = 0;
        if (narrow) {
            la = a16(end + 2 * L);
            lb = a16(la + NL * L);
            end = lb + (NL + 2) * L;
        }
        stage = a16(end);
        bytes = stage + nstage * 6 * nh * ((L + nh - 1) / nh) * gsize;   // K = ceil(L / nh) slots a lane
    }
};

// Tap gradients of one adjoint step go out through LDS: each lane puts the
// values of its K slots into a staging line per (wavefront, tap), 64 K
// elements long so that slots past a line's end land in the padding, and the
// wavefront then writes the six lines as whole dwords (stores of a few bytes
// at a 6-byte stride cost far more).  kDrop pushes the offset of an unused
// dword store past the tensor; the hardware drops it.
constexpr uint32_t kDrop = 0x80000000u;

template <typename T, int K>
__device__ __forceinline__ void stage_put(uint32_t line, int q, const float (&v)[K]) {
    typedef __attribute__((address_space(3))) uint32_t lds_u32;
    typedef __attribute__((address_space(3))) uint16_t lds_u16;
    auto w32 = [](uint32_t a, uint32_t x) { *reinterpret_cast<lds_u32*>(static_cast<uintptr_t>(a)) = x; };
    auto w16 = [](uint32_t a, uint32_t x) {
        *reinterpret_cast<lds_u16*>(static_cast<uintptr_t>(a)) = static_cast<uint16_t>(x);
    };
    if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int j = 0; j < K; ++j) w32(line + 4u * (K * q + j), __float_as_uint(v[j]));
    } else if constexpr (K == 1) {
        w16(line + 2u * q, pack_bf16x2(v[0], v[0]));
    } else if constexpr (K == 2) {
        w32(line + 4u * q, pack_bf16x2(v[0], v[1]));
    } else if constexpr (K == 4) {
        w32(line + 8u * q, pack_bf16x2(v[0], v[1]));
        w32(line + 8u * q + 4u, pack_bf16x2(v[2], v[3]));
    } else if constexpr (K == 5) {
        // even q: dwords (5q, 5q+1), (5q+2, 5q+3), short 5q+4; odd q: short 5q,
        // dwords (5q+1, 5q+2), (5q+3, 5q+4)
        const bool even = (q & 1) == 0;
        const uint32_t b0 = 10u * q;
        w32(b0 + (even ? 0u : 2u) + line, even ? pack_bf16x2(v[0], v[1]) : pack_bf16x2(v[1], v[2]));
        w32(b0 + (even ? 4u : 6u) + line, even ? pack_bf16x2(v[2], v[3]) : pack_bf16x2(v[3], v[4]));
        w16(b0 + (even ? 8u : 0u) + line, even ? pack_bf16x2(v[4], v[4]) : pack_bf16x2(v[0], v[0]));
    } else {
        static_assert(K == 3, "one to five slots a lane");
        // even q: dword (3q, 3q+1), short 3q+2; odd q: short 3q, dword (3q+1, 3q+2)
        const bool even = (q & 1) == 0;
        const float a = even ? v[0] : v[1];
        const float b = even ? v[1] : v[2];
        const float c = even ? v[2] : v[0];
        w32(line + (even ? 6u * q : 6u * q + 2u), pack_bf16x2(a, b));
        w16(line + (even ? 6u * q + 4u : 6u * q), pack_bf16x2(c, c));
    }
}

// Two consecutive pixels of an output plane.
template <typename T>
__device__ __forceinline__ void store_pair(T* p, size_t e, float v0, float v1) {
    if constexpr (sizeof(T) == 4) *reinterpret_cast<f32x2_t*>(p + e) = f32x2_t{v0, v1};
    else *reinterpret_cast<uint32_t*>(p + e) = pack_bf16x2(v0, v1);
}
template <typename T>
__device__ __forceinline__ f32x2_t load_pair(const T* p, size_t e) {
    if constexpr (sizeof(T) == 4) {
        return *reinterpret_cast<const f32x2_t*>(p + e);
    } else {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(p + e);
        return f32x2_t{__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u)};
    }
}

// A buffer resource whose fields the compiler is told are uniform.  Values
// computed from the kernel's arguments can still be taken as varying across
// the wavefront when the compiler places their computation inside a loop
// with a per-lane trip count (the plane's zeroing loops); a resource held in
// vector registers then costs a loop over the distinct values on every load.
template <typename P>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const P* p, int num_records) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint64_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(a)));
    const uint64_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(a >> 32)));
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((hi << 32) | lo), 0,
                                             __builtin_amdgcn_readfirstlane(num_records), kBufFlags);
}

// Odd line lengths (bf16): a window of K elements starting at element E is
// loaded from the even element at or below E and shifted right by 16 bits
// when E is odd.  Along a scan E moves by +-L, so with L odd its parity
// alternates from line to line, and a ring of D (even) prefetched lines
// gives every slot a fixed parity.  A stream's state: the byte offset of
// the next load, the increments after a load of even and of odd parity (in
// the slot order of the scan's first line), and the shift of even slots.
struct OddStream {
    uint32_t off, incE, incO, shE;
};
__device__ __forceinline__ OddStream odd_stream(int e0, int dl) {
    const int p0 = e0 & 1;
    return {static_cast<uint32_t>(e0 - p0) * 2u, static_cast<uint32_t>(2 * dl - 2 + 4 * p0),
            static_cast<uint32_t>(2 * dl - 2 + 4 * (p0 ^ 1)), 16u * static_cast<uint32_t>(p0)};
}
// The NW words a window decodes from: with Odd, the NWL loaded words shifted
// right by sh bits (0 or 16).
template <bool Odd, int NW, int NWL>
__device__ __forceinline__ words_t<NW> odd_window(const words_t<NWL>& w, uint32_t sh) {
    if constexpr (!Odd) {
        return w;
    } else {
        words_t<NW> rv;
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            const uint32_t v = __builtin_amdgcn_alignbit(word<NWL>(w, i + 1 < NWL ? i + 1 : NWL - 1),
                                                         word<NWL>(w, i), sh);
            if constexpr (NW == 1) rv = v;
            else rv[i] = v;
        }
        return rv;
    }
}
// Two bf16 values at any element (a 4-byte load at 2-byte alignment).
typedef uint32_t u32_u __attribute__((aligned(2)));

// Cols = false: the row pair (NL = H, L = W), inputs as they are; writes S and
// G of the pair to s_ws, g_ws ([planes][H][W] fp32).
// Cols = true: the column pair (NL = W, L = H), inputs transposed; adds the
// row pair's S and G and writes gu, gx, glam.
// Taps are read from group plane p / cpg (w4: w4_bytes); the tap gradients
// are written per channel, as GT, to gwd ([4][planes][3][..][..], gw_bytes).
// Chunked: k_chunk > 1.  A wavefront per direction; they meet only between
// passes.
// Pre (channels sharing taps): the workgroup holds cc planes of one tap
// group, a wavefront pair each.  The weights come normalised in fp32 from
// wpre ([4][planes / cpg][3][..][..], wpre_bytes), so no step evaluates a
// transcendental, and the adjoint produces the tap products
// e_k(i, p) = g_i[p] h_{i-1}[p+k-1] in place of the tap gradients: the cc
// planes' products of a line are added on chip in plane order, and the sum
// goes to gwd as fp32, one plane of partial sums per workgroup
// ([4][planes / cc][3][..][..]).  The normalisation's Jacobian is applied
// once per group afterwards.
// Odd (bf16, per-channel taps, square planes of odd side): lines and planes
// start at any element (windows as OddStream describes); tap gradients go
// out one element a lane per store; S and G of the row pair are kept at a
// plane stride of HW rounded up to 4; the column pair's outputs are written
// in pixel pairs of unaligned dwords, a plane's odd last pixel alone.
template <typename T, typename GT, int K, int D, bool Cols, bool Chunked, bool Pre, int CC, bool Odd>
__global__ void __launch_bounds__(128 * CC)
prop2d_backward_pair_kernel(const T* __restrict__ xl, const T* __restrict__ laml,
                            const T* __restrict__ ul, const T* __restrict__ gyl,
                            const T* __restrict__ w4, int w4_bytes, GT* __restrict__ gwd,
                            int gw_bytes, int cpg, int k_chunk,
                            float eps, int planes, int NL, int L, int dir0,
                            float* __restrict__ s_ws, float* __restrict__ g_ws,
                            const T* __restrict__ x, const T* __restrict__ lam,
                            const T* __restrict__ gy, T* __restrict__ gx, T* __restrict__ glam,
                            T* __restrict__ gu, const float* __restrict__ wpre, int wpre_bytes) {
    static_assert(!Pre || sizeof(GT) == 4, "partial sums of tap products are fp32");
    static_assert(CC == 1 || Pre, "planes are added only with prepared weights");
    static_assert(!Odd || (sizeof(T) == 2 && sizeof(GT) == 2 && !Pre && D % 2 == 0),
                  "odd lines: bf16, per-channel taps, slots of fixed parity");
    constexpr int cc = CC;
    constexpr int ES = sizeof(T);
    // words a window decodes from, and words loaded for it (Odd: one more
    // for even K, which the shift needs)
    constexpr int NW = Odd ? (K + 1) / 2 : window_words<T, K>();
    constexpr int NWL = Odd && (K % 2 == 0) ? NW + 1 : NW;
    constexpr int TW = Pre ? K : NWL;       // words loaded for a tap window: fp32 weights or raw taps
    constexpr bool kNarrow = ES == 2;
    constexpr int VW = kNarrow ? 2 : 4;     // bytes of a value in the A / B array
    const int HW = NL * L;
    // plane stride of the row pair's S and G (fp32, workspace)
    const int HWa = Odd ? (HW + 3) & ~3 : HW;
    constexpr int GS = sizeof(GT);
    PairBwdLayout lay(NL, L, kNarrow, GS, CC > 1 ? 2 : 1);
    constexpr int NT = 128;                 // threads of a plane's wavefront pair
    const int pslot = Pre ? static_cast<int>(threadIdx.x >> 7) : 0;   // the workgroup's plane
    const int tid = Pre ? static_cast<int>(threadIdx.x & 127) : static_cast<int>(threadIdx.x);
    const int lane = tid & 63;
    const int half = tid >> 6;              // the wavefront: its direction
    const int q = lane;
    const bool fwd = half == 0;
    // each plane of the workgroup has its own copy of the layout
    const int pstride = lay.bytes;
    const uint32_t stage0 = static_cast<uint32_t>(lay.stage);   // plane 0's staging
    {
        const int pb = pslot * pstride;
        lay.a += pb;
        lay.b += pb;
        lay.la += pb;
        lay.lb += pb;
        lay.stage += pb;
    }
    // orders the LDS accesses of the workgroup's wavefronts
    auto sync = [&]() { lds_barrier(); };
    const int plane = Pre ? static_cast<int>(blockIdx.x) * cc + pslot : static_cast<int>(blockIdx.x);
    const size_t pix0 = static_cast<size_t>(plane) * HW;

    // each wavefront zeroes its own dummy words before it uses them: the
    // values that slots past a line's end leave there (finite, and weighed
    // only by dropped taps) then follow that wavefront's program order alone,
    // so even the signs of the zero tap gradients they touch are the same
    // from run to run
    const uint32_t dum0 = static_cast<uint32_t>(pslot * pstride) + 16u * half;
    if (lane < 4) lds_at<float>(dum0 + 4u * lane) = 0.0f;
    // zero lines: h before a scan's first line
    for (int f = tid; f < L; f += NT) {
        if constexpr (kNarrow) {
            lds_at<uint16_t>(lay.a - 2 * L + 2 * f) = 0;
            lds_at<uint16_t>(lay.b + 2 * HW + 2 * f) = 0;
            lds_at<uint8_t>(lay.la - L + f) = 0;
            lds_at<uint8_t>(lay.lb + HW + f) = 0;
        } else {
            lds_at<float>(lay.a - 4 * L + 4 * f) = 0.0f;
            lds_at<float>(lay.b + 4 * HW + 4 * f) = 0.0f;
        }
    }
    // one value of a plane: fp32, or its upper 24 bits (rounded to nearest
    // even) in the two narrow arrays
    auto put = [&](uint32_t ah, uint32_t al, float v) {
        if constexpr (kNarrow) {
            uint32_t w = __float_as_uint(v);
            w += 0x7fu + ((w >> 8) & 1u);
            lds_at<uint16_t>(ah) = static_cast<uint16_t>(w >> 16);
            lds_at<uint8_t>(al) = static_cast<uint8_t>(w >> 8);
        } else {
            lds_at<float>(ah) = v;
        }
    };
    auto get = [&](uint32_t ah, uint32_t al) -> float {
        if constexpr (kNarrow)
            return __uint_as_float(__builtin_amdgcn_perm(static_cast<uint32_t>(lds_at<uint16_t>(ah)),
                                                         static_cast<uint32_t>(lds_at<uint8_t>(al)),
                                                         0x0504000cu));
        else
            return lds_at<float>(ah);
    };
    // four consecutive values from array offset (in values) e4 * 4
    auto get4 = [&](int base, int lbase, int e4) -> f32x4_t {
        if constexpr (kNarrow) {
            const u32x2_t hi = lds_at<u32x2_t>(base + 8u * e4);
            const uint32_t lo = lds_at<uint32_t>(lbase + 4u * e4);
            return f32x4_t{__uint_as_float(__builtin_amdgcn_perm(hi.x, lo, 0x0504000cu)),
                           __uint_as_float(__builtin_amdgcn_perm(hi.x, lo, 0x0706010cu)),
                           __uint_as_float(__builtin_amdgcn_perm(hi.y, lo, 0x0504020cu)),
                           __uint_as_float(__builtin_amdgcn_perm(hi.y, lo, 0x0706030cu))};
        } else {
            return lds_at<f32x4_t>(base + 16u * e4);
        }
    };

    // (Odd: windows are dword-aligned loads, so the bound is rounded up to
    // whole dwords)
    const int in_bytes = Odd ? (planes * HW * ES + 3) & ~3 : planes * HW * ES;
    const __amdgpu_buffer_rsrc_t xs = uniform_rsrc(xl, in_bytes);
    const __amdgpu_buffer_rsrc_t ls = uniform_rsrc(laml, in_bytes);
    const __amdgpu_buffer_rsrc_t us = uniform_rsrc(ul, in_bytes);
    const __amdgpu_buffer_rsrc_t gs = uniform_rsrc(gyl, in_bytes);
    __amdgpu_buffer_rsrc_t taps[3];
    const __amdgpu_buffer_rsrc_t gws = uniform_rsrc(gwd, gw_bytes);
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        taps[k] = uniform_rsrc(w4 + static_cast<size_t>(k) * HW, w4_bytes - k * HW * ES);
    }
    const int par = (ES == 2 && !Odd) ? ((K * q) & 1) : 0;
    const uint32_t win_b = static_cast<uint32_t>(K * q - par) * ES;
    const uint32_t sel_even = par ? 0x03020c0cu : 0x01000c0cu;
    const uint32_t sel_odd = par ? 0x05040c0cu : 0x03020c0cu;
    const uint32_t tap_b = static_cast<uint32_t>(((dir0 + half) * (planes / cpg) + plane / cpg) * 3 * HW) * ES;
    // the window of this lane on line 0 of its direction's taps, and the
    // bytes of a line: raw taps, or fp32 weights (Pre)
    __amdgpu_buffer_rsrc_t trs[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        if constexpr (Pre)
            trs[k] = uniform_rsrc(wpre + static_cast<size_t>(k) * HW, wpre_bytes - k * HW * 4);
        else
            trs[k] = taps[k];
    }
    const uint32_t t_base = Pre ? static_cast<uint32_t>(((dir0 + half) * (planes / cpg) + plane / cpg) * 3 * HW) * 4u +
                                      static_cast<uint32_t>(K * q) * 4u
                                : tap_b + win_b;
    const uint32_t t_line = static_cast<uint32_t>(L) * (Pre ? 4u : static_cast<uint32_t>(ES));
    // Odd: one resource over all taps; planes 1 and 2 of a tap triple at
    // scalar offsets (plane 1 flips the parity: 4 more bytes when the
    // window starts odd, the other shift)
    const __amdgpu_buffer_rsrc_t tall =
        Odd ? uniform_rsrc(w4, (w4_bytes + 3) & ~3) : taps[0];
    const int so1 = 2 * HW - 2, so2 = 4 * HW;
    const int tap_e = ((dir0 + half) * (planes / cpg) + plane / cpg) * 3 * HW + K * q;   // element of line 0
    const int pix_e = static_cast<int>(pix0) + K * q;
    // segments of a chunked scan; a segment's first line reads no line before it
    const int seg = Chunked ? (NL + k_chunk - 1) / k_chunk : NL;
    const uint32_t line_b = static_cast<uint32_t>(L) * ES;
    const uint32_t plane_base = half ? lay.b : lay.a;
    const uint32_t lplane_base = half ? lay.lb : lay.la;

    // Dropped taps.  bf16: the slot's byte selector decodes a dropped tap (or
    // any tap of a slot past the line end) to -2^127, whose sigmoid is exactly
    // 0 whatever the memory holds, and the values of a slot past the line end
    // to 0.  fp32 (no selector): 1 / (e + inf) = 0.
    constexpr bool kB16 = ES == 2;
    float c0[K], c1[K], c2[K];
    uint32_t st[3][K], sx[K];
    bool valid[K];
    const float inf = __builtin_inff();
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const int p = K * q + j;
        valid[j] = p < L;
        c0[j] = (kB16 || (valid[j] && p > 0)) ? 1.0f : inf;
        c1[j] = (kB16 || valid[j]) ? 1.0f : inf;
        c2[j] = (kB16 || (valid[j] && p < L - 1)) ? 1.0f : inf;
        const uint32_t s_in = (j & 1) ? sel_odd : sel_even;
        st[0][j] = (valid[j] && p > 0) ? s_in : kSelDropped;
        st[1][j] = valid[j] ? s_in : kSelDropped;
        st[2][j] = (valid[j] && p < L - 1) ? s_in : kSelDropped;
        sx[j] = valid[j] ? s_in : kSelZero;
    }
    // s_k = sigmoid(z_k) (0 for dropped taps) and r = 1 / max(sum s, eps)
    auto normalise = [&](const words_t<NW> (&tw)[3], float (&s0)[K], float (&s1)[K], float (&s2)[K],
                         float (&t)[K], float (&r)[K]) {
#pragma unroll
        for (int j = 0; j < K; ++j) {
            s0[j] = window_elem<T, K, NW>(tw[0], j, st[0][j], st[0][j]) * kNegLog2e;
            s1[j] = window_elem<T, K, NW>(tw[1], j, st[1][j], st[1][j]) * kNegLog2e;
            s2[j] = window_elem<T, K, NW>(tw[2], j, st[2][j], st[2][j]) * kNegLog2e;
        }
#pragma unroll
        for (int j = 0; j < K; ++j) {
            s0[j] = __builtin_amdgcn_exp2f(s0[j]);
            s1[j] = __builtin_amdgcn_exp2f(s1[j]);
            s2[j] = __builtin_amdgcn_exp2f(s2[j]);
        }
#pragma unroll
        for (int j = 0; j < K; ++j) {
            s0[j] = __builtin_amdgcn_rcpf(s0[j] + c0[j]);
            s1[j] = __builtin_amdgcn_rcpf(s1[j] + c1[j]);
            s2[j] = __builtin_amdgcn_rcpf(s2[j] + c2[j]);
        }
#pragma unroll
        for (int j = 0; j < K; ++j) {
            t[j] = (s0[j] + s1[j]) + s2[j];
            r[j] = __builtin_amdgcn_rcpf(fmaxf(t[j], eps));
        }
    };

    // Column launch, after each phase: for every pixel pair (r, c), (r, c+1)
    // in row-major order, v = part (the row pair's sum, workspace) + the
    // column pair's sum (LDS, position r of lines c and c+1); out0 = m0 * v
    // and, with Two, out1 = m1 * v.  The global loads of U pairs per lane are
    // issued before any of them is used (these loads, not the arithmetic,
    // set the time of the pass).
    auto column_pass = [&](const float* part, const T* m0, const T* m1, T* out0, T* out1,
                           auto two_tag) {
        constexpr bool kTwo = decltype(two_tag)::value;
        constexpr int U = 24;
        const int W = NL, H = L, npairs = HW / 2;
        const float invW = 1.0f / static_cast<float>(W);
        const f32x2_t* pp = reinterpret_cast<const f32x2_t*>(part + pix0);
        for (int base = 0; base < npairs; base += NT * U) {
            f32x2_t pv[U], a[U], b[U];
#pragma unroll
            for (int k = 0; k < U; ++k) {
                // clamped to the last pair: in bounds, the value is not used
                const int e2 = min(base + NT * k + tid, npairs - 1);
                pv[k] = pp[e2];
                a[k] = load_pair(m0, pix0 + 2 * e2);
                if constexpr (kTwo) b[k] = load_pair(m1, pix0 + 2 * e2);
            }
#pragma unroll
            for (int k = 0; k < U; ++k) {
                const int e2 = base + NT * k + tid;
                if (e2 < npairs) {
                    const int e = 2 * e2;
                    const int r = static_cast<int>((static_cast<float>(e) + 0.5f) * invW);
                    const int c = e - r * W;
                    const uint32_t i0 = c * H + r, i1 = i0 + H;
                    const float v0 = pv[k].x + (get(lay.a + VW * i0, lay.la + i0) + get(lay.b + VW * i0, lay.lb + i0));
                    const float v1 = pv[k].y + (get(lay.a + VW * i1, lay.la + i1) + get(lay.b + VW * i1, lay.lb + i1));
                    store_pair(out0, pix0 + e, a[k].x * v0, a[k].y * v1);
                    if constexpr (kTwo) store_pair(out1, pix0 + e, b[k].x * v0, b[k].y * v1);
                }
            }
        }
    };

    // The same for Odd planes: pixel pairs (e, e+1) of the plane in pixel
    // order, e even, (e+1) on the next row when e ends a row; the row pair's
    // sums at plane stride HWa; m0, m1 and the outputs at any element, read
    // and written as unaligned dwords, except a plane's odd last pixel (read
    // as the high half of the dword before it, written alone).
    auto column_pass_odd = [&](const float* part, const T* m0, const T* m1, T* out0, T* out1,
                               auto two_tag) {
        constexpr bool kTwo = decltype(two_tag)::value;
        constexpr int U = 16;
        const int W = NL, H = L, npairs = (HW + 1) / 2;
        const float invW = 1.0f / static_cast<float>(W);
        const f32x2_t* pp = reinterpret_cast<const f32x2_t*>(part + static_cast<size_t>(plane) * HWa);
        auto load2 = [&](const T* m, int e, bool single) -> f32x2_t {
            const uint32_t w = *reinterpret_cast<const u32_u*>(m + pix0 + e - (single ? 1 : 0));
            const float hi = __uint_as_float(w & 0xffff0000u);
            return f32x2_t{single ? hi : __uint_as_float(w << 16), hi};
        };
        for (int base = 0; base < npairs; base += NT * U) {
            f32x2_t pv[U], a[U], b[U];
#pragma unroll
            for (int k = 0; k < U; ++k) {
                // clamped to the last pair: in bounds, the value is not used
                const int e2 = min(base + NT * k + tid, npairs - 1);
                const bool single = 2 * e2 + 1 == HW;
                pv[k] = pp[e2];
                a[k] = load2(m0, 2 * e2, single);
                if constexpr (kTwo) b[k] = load2(m1, 2 * e2, single);
            }
#pragma unroll
            for (int k = 0; k < U; ++k) {
                const int e2 = base + NT * k + tid;
                if (e2 < npairs) {
                    const int e = 2 * e2;
                    const bool single = e + 1 == HW;
                    const int r = static_cast<int>((static_cast<float>(e) + 0.5f) * invW);
                    const int c = e - r * W;
                    const bool wrap = c + 1 == W;
                    const uint32_t i0 = c * H + r;
                    const uint32_t i1 = wrap ? static_cast<uint32_t>(r + 1) : i0 + H;
                    const float v0 = pv[k].x + (get(lay.a + VW * i0, lay.la + i0) + get(lay.b + VW * i0, lay.lb + i0));
                    const float v1 = pv[k].y + (get(lay.a + VW * i1, lay.la + i1) + get(lay.b + VW * i1, lay.lb + i1));
                    const uint32_t o0 = pack_bf16x2(a[k].x * v0, a[k].y * v1);
                    const uint32_t o1 = kTwo ? pack_bf16x2(b[k].x * v0, b[k].y * v1) : 0u;
                    if (!single) {
                        *reinterpret_cast<u32_u*>(out0 + pix0 + e) = o0;
                        if constexpr (kTwo) *reinterpret_cast<u32_u*>(out1 + pix0 + e) = o1;
                    } else {
                        out0[pix0 + e] = static_cast<T>(o0 & 0xffffu);
                        if constexpr (kTwo) out1[pix0 + e] = static_cast<T>(o1 & 0xffffu);
                    }
                }
            }
        }
    };

    // ------------------------------------------------------------ forward
    {
        const uint32_t lo0 = fwd ? 0u : static_cast<uint32_t>(NL - 1) * line_b;
        const uint32_t dlo = fwd ? line_b : 0u - line_b;
        const uint32_t dto = fwd ? t_line : 0u - t_line;
        uint32_t lo = t_base + (fwd ? 0u : static_cast<uint32_t>(NL - 1) * t_line);
        uint32_t xo = static_cast<uint32_t>(pix0) * ES + win_b + lo0;
        const int i0f = fwd ? 0 : NL - 1;
        const OddStream ot = odd_stream(tap_e + i0f * L, fwd ? L : -L);
        const OddStream ox = odd_stream(pix_e + i0f * L, fwd ? L : -L);
        if constexpr (Odd) {
            lo = ot.off;
            xo = ox.off;
        }
        words_t<TW> tbuf[D][3];
        words_t<NWL> xbuf[D], lbuf[D];
        auto load_line = [&](int d) {
            if constexpr (Odd) {
                const bool od = (d & 1) != 0;
                const uint32_t sh = od ? ot.shE ^ 16u : ot.shE;   // 16 x the window start's parity
                tbuf[d][0] = load_words_so<TW>(tall, lo, 0);
                tbuf[d][1] = load_words_so<TW>(tall, lo + (sh >> 2), so1);
                tbuf[d][2] = load_words_so<TW>(tall, lo, so2);
                xbuf[d] = load_words<NWL>(xs, xo);
                lbuf[d] = load_words<NWL>(ls, xo);
                lo += od ? ot.incO : ot.incE;
                xo += od ? ox.incO : ox.incE;
            } else {
#pragma unroll
                for (int k = 0; k < 3; ++k) tbuf[d][k] = load_words<TW>(trs[k], lo);
                xbuf[d] = load_words<NW>(xs, xo);
                lbuf[d] = load_words<NW>(ls, xo);
                lo += dto;
                xo += dlo;
            }
        };
#pragma unroll
        for (int d = 0; d < D; ++d) {
            load_line(d);
            __builtin_amdgcn_sched_barrier(0);
        }
        const int i0 = fwd ? 0 : NL - 1;
        const int dl = fwd ? L : -L;       // values per line step
        uint32_t aH[K], aL[K];
        int dH[K], dL[K];
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const int v = i0 * L + K * q + j;
            aH[j] = valid[j] ? plane_base + VW * v : dum0 + PairBwdLayout::dum + VW * j;
            aL[j] = valid[j] ? lplane_base + v : dum0 + PairBwdLayout::ldum + j;
            dH[j] = valid[j] ? VW * dl : 0;
            dL[j] = valid[j] ? dl : 0;
        }
        float h[K];
#pragma unroll
        for (int j = 0; j < K; ++j) h[j] = 0.0f;
        // step of the next restart (scan order: lines seg, 2 seg, .. from the
        // top; NL - 1 - (seg - 1), .. from the bottom)
        int next_restart = fwd ? seg : NL - ((NL - 1) / seg) * seg;

        auto step = [&](int s, int d) {
            asm volatile("" : "+v"(tbuf[d][0]), "+v"(tbuf[d][1]), "+v"(tbuf[d][2]));
            asm volatile("" : "+v"(xbuf[d]), "+v"(lbuf[d]));
            // Pre: s0..s2 are the normalised weights and r is 1
            float s0[K], s1[K], s2[K], t[K], r[K], b[K];
            const bool od = (d & 1) != 0;
            {
                const uint32_t sh = od ? ox.shE ^ 16u : ox.shE;
                const words_t<NW> xw = odd_window<Odd, NW, NWL>(xbuf[d], sh);
                const words_t<NW> lw = odd_window<Odd, NW, NWL>(lbuf[d], sh);
#pragma unroll
                for (int j = 0; j < K; ++j)
                    b[j] = window_elem<T, K, NW>(lw, j, sx[j], sx[j]) * window_elem<T, K, NW>(xw, j, sx[j], sx[j]);
            }
            if constexpr (Pre) {
#pragma unroll
                for (int j = 0; j < K; ++j) {
                    s0[j] = __uint_as_float(word<TW>(tbuf[d][0], j));
                    s1[j] = __uint_as_float(word<TW>(tbuf[d][1], j));
                    s2[j] = __uint_as_float(word<TW>(tbuf[d][2], j));
                    t[j] = r[j] = 1.0f;
                }
            } else {
                const uint32_t sh = od ? ot.shE ^ 16u : ot.shE;
                const words_t<NW> tw[3] = {odd_window<Odd, NW, TW>(tbuf[d][0], sh),
                                           odd_window<Odd, NW, TW>(tbuf[d][1], sh ^ 16u),
                                           odd_window<Odd, NW, TW>(tbuf[d][2], sh)};
                normalise(tw, s0, s1, s2, t, r);
            }
#pragma unroll
            for (int j = 0; j < K; ++j)
                asm volatile("" : "+v"(lo), "+v"(xo) : "v"(s0[j]), "v"(s1[j]), "v"(s2[j]), "v"(r[j]), "v"(b[j]));
            load_line(d);
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
                float m = s1[j] * h[j];
                m = fmaf(s0[j], hl, m);
                m = fmaf(s2[j], hr, m);
                hn[j] = Pre ? m + b[j] : fmaf(m, r[j], b[j]);
            }
            // fp32 slots past the line end hold 0 (their windows read the next
            // line or plane; bf16 ones decode to 0 and stay 0; fp32 weights
            // past a line's end are the next line's, so Pre zeroes them too)
#pragma unroll
            for (int j = 0; j < K; ++j) {
                if constexpr (!kB16 || Pre) hn[j] = valid[j] ? hn[j] : 0.0f;
                h[j] = hn[j];
                put(aH[j], aL[j], hn[j]);
                aH[j] += dH[j];
                aL[j] += dL[j];
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
    }
    sync();

    // --------------------------------------------------------- S = h_a + h_b
    // (line-major order is pixel order for the row pair; for the column pair
    // pixel (r, c) is position r of line c)
    if constexpr (!Cols) {
        f32x4_t* sp = reinterpret_cast<f32x4_t*>(s_ws + static_cast<size_t>(plane) * HWa);
        for (int e = tid; e < HWa / 4; e += NT) sp[e] = get4(lay.a, lay.la, e) + get4(lay.b, lay.lb, e);
    } else if constexpr (Odd) {
        column_pass_odd(s_ws, gy, gy, gu, gu, std::false_type{});
    } else {
        column_pass(s_ws, gy, gy, gu, gu, std::false_type{});
    }
    sync();

    // ------------------------------------------------------------ adjoint
    {
        // wavefront 0 walks its lines NL-1 .. 0, wavefront 1 walks 0 .. NL-1
        const int i0 = fwd ? NL - 1 : 0;
        const uint32_t lo0 = static_cast<uint32_t>(i0) * line_b;
        const uint32_t dlo = fwd ? 0u - line_b : line_b;
        const uint32_t dto = fwd ? 0u - t_line : t_line;
        uint32_t lo = t_base + static_cast<uint32_t>(i0) * t_line;
        uint32_t uo = static_cast<uint32_t>(pix0) * ES + win_b + lo0;
        const OddStream ot = odd_stream(tap_e + i0 * L, fwd ? -L : L);
        const OddStream ou = odd_stream(pix_e + i0 * L, fwd ? -L : L);
        if constexpr (Odd) {
            lo = ot.off;
            uo = ou.off;
        }
        words_t<TW> tbuf[D][3];
        words_t<NWL> ubuf[D], gbuf[D];
        auto load_line = [&](int d) {
            if constexpr (Odd) {
                const bool od = (d & 1) != 0;
                const uint32_t sh = od ? ot.shE ^ 16u : ot.shE;
                tbuf[d][0] = load_words_so<TW>(tall, lo, 0);
                tbuf[d][1] = load_words_so<TW>(tall, lo + (sh >> 2), so1);
                tbuf[d][2] = load_words_so<TW>(tall, lo, so2);
                ubuf[d] = load_words<NWL>(us, uo);
                gbuf[d] = load_words<NWL>(gs, uo);
                lo += od ? ot.incO : ot.incE;
                uo += od ? ou.incO : ou.incE;
            } else {
#pragma unroll
                for (int k = 0; k < 3; ++k) tbuf[d][k] = load_words<TW>(trs[k], lo);
                ubuf[d] = load_words<NW>(us, uo);
                gbuf[d] = load_words<NW>(gs, uo);
                lo += dto;
                uo += dlo;
            }
        };
#pragma unroll
        for (int d = 0; d < D; ++d) {
            load_line(d);
            __builtin_amdgcn_sched_barrier(0);
        }
        // read-back of the staging lines: dword f = lane + 64 t of the
        // wavefront's three lines of L ES / 4 dwords, stored at its place on
        // the current line of its direction's tap plane
        constexpr int SL = 64 * K;               // staging line length
        constexpr int NR = (3 * K * GS + 3) / 4; // ceil(3 * SL * GS / 4 / 64)
        constexpr int kLines = 3;
        const int per_line = L * GS / 4;
        // Pre, several planes: the workgroup's planes of a direction each
        // write a share of its three lines, dwords f = share + lane + 64 t,
        // adding that dword of every plane's staging (plane stride pstride)
        constexpr bool summed = CC > 1;
        const int share = summed ? (kLines * per_line + cc - 1) / cc : kLines * per_line;
        const int f0 = summed ? pslot * share : 0;
        // partial-sum planes (Pre) or per-channel planes, and this one's index
        const int out_planes = Pre ? planes / cc : planes;
        const int out_plane = Pre ? static_cast<int>(blockIdx.x) : plane;
        // Odd: the three lines' 3 L elements, element f = lane + 64 t, one a
        // lane per 2-byte store (lines start at any element)
        constexpr int NR16 = Odd ? 3 * K : 1;
        uint32_t rd16[NR16], go16[NR16], gd16[NR16];
        if constexpr (Odd) {
#pragma unroll
            for (int t = 0; t < NR16; ++t) {
                const int f = lane + 64 * t;
                rd16[t] = lay.stage;
                go16[t] = kDrop;
                gd16[t] = 0;
                if (f < 3 * L) {
                    const int k = f / L, m = f - (f / L) * L;
                    const int start = half == 0 ? NL - 1 : 0;
                    rd16[t] = static_cast<uint32_t>(lay.stage + (3 * half + k) * SL * GS + 2 * m);
                    go16[t] = static_cast<uint32_t>(((((dir0 + half) * planes + plane) * 3 + k) * HW + start * L + m) * 2);
                    gd16[t] = half == 0 ? 0u - static_cast<uint32_t>(2 * L) : static_cast<uint32_t>(2 * L);
                }
            }
        }
        uint32_t rd[NR], go[NR], gd[NR];
#pragma unroll
        for (int t = 0; t < NR; ++t) {
            const int f = f0 + lane + 64 * t;
            rd[t] = summed ? stage0 : lay.stage;
            go[t] = kDrop;
            gd[t] = 0;
            if (lane + 64 * t < share && f < kLines * per_line) {
                const int hk = 3 * half + f / per_line;
                const int m = f - (f / per_line) * per_line;
                const int h = hk / 3, k = hk - 3 * h;
                const int start = h == 0 ? NL - 1 : 0;      // first adjoint line of that wavefront
                rd[t] = (summed ? stage0 : static_cast<uint32_t>(lay.stage)) + hk * SL * GS + 4 * m;
                go[t] = static_cast<uint32_t>((((dir0 + h) * out_planes + out_plane) * 3 + k) * HW * GS +
                                              start * L * GS + 4 * m);
                gd[t] = h == 0 ? 0u - static_cast<uint32_t>(L * GS) : static_cast<uint32_t>(L * GS);
            }
        }
        const uint32_t my_stage = lay.stage + 3 * half * SL * GS;
        // K <= 2 on even lines, one plane a workgroup: a lane's K positions of
        // a tap's line are one aligned K GS-byte word of the tap-gradient
        // plane, so the line goes out with one store a lane and tap (taps 1
        // and 2 at scalar offsets of one and two planes) instead of through
        // the staging lines.  Lanes past the line's end store past the buffer
        // (dropped).
        constexpr bool kDirect = !summed && !Odd && K <= 2;
        const uint32_t d_off0 = K * q < L ? static_cast<uint32_t>((((dir0 + half) * out_planes + out_plane) * 3) * HW * GS +
                                                                  i0 * L * GS + K * q * GS)
                                          : 0x80000000u;
        const uint32_t d_step = K * q < L ? (fwd ? 0u - static_cast<uint32_t>(L * GS) : static_cast<uint32_t>(L * GS)) : 0u;
        uint32_t d_off = d_off0;
        // bytes between a triple's tap planes (read through readfirstlane so
        // that the compiler keeps the scalar offsets in scalar registers)
        const int d_tap = __builtin_amdgcn_readfirstlane(HW * GS);
        const uint32_t set_bytes = 6u * SL * GS;    // one staging set of a plane
        // adjoint step of the next restart line: its taps read nothing (tap
        // gradient 0) and the line before it receives no adjoint term from it
        int next_restart = fwd ? (NL - 1) - ((NL - 1) / seg) * seg : seg - 1;
        // LDS: g_i goes to line i (G); h_{i-1} (wavefront 0) or h_{i+1}
        // (wavefront 1) is read one step ahead (P), and P of one step is G of
        // the next
        const int dl = fwd ? -L : L;       // values per step
        uint32_t aGH[K], aGL[K], aPH[K], aPL[K];
        int dH[K], dL[K];
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const int v = i0 * L + K * q + j;
            aGH[j] = valid[j] ? plane_base + VW * v : dum0 + PairBwdLayout::dum + VW * j;
            aGL[j] = valid[j] ? lplane_base + v : dum0 + PairBwdLayout::ldum + j;
            dH[j] = valid[j] ? VW * dl : 0;
            dL[j] = valid[j] ? dl : 0;
            aPH[j] = aGH[j] + dH[j];
            aPL[j] = aGL[j] + dL[j];
        }
        float hp[K], gp[K], w0p[K], w1p[K], w2p[K];
#pragma unroll
        for (int j = 0; j < K; ++j) {
            hp[j] = get(aPH[j], aPL[j]);
            gp[j] = w0p[j] = w1p[j] = w2p[j] = 0.0f;
        }

        auto step = [&](int s, int d) {
            asm volatile("" : "+v"(tbuf[d][0]), "+v"(tbuf[d][1]), "+v"(tbuf[d][2]));
            asm volatile("" : "+v"(ubuf[d]), "+v"(gbuf[d]));
            // Pre: s0..s2 are the normalised weights and r is 1
            float s0[K], s1[K], s2[K], t[K], r[K], ugy[K];
            const bool od = (d & 1) != 0;
            {
                const uint32_t sh = od ? ou.shE ^ 16u : ou.shE;
                const words_t<NW> uw = odd_window<Odd, NW, NWL>(ubuf[d], sh);
                const words_t<NW> gw = odd_window<Odd, NW, NWL>(gbuf[d], sh);
#pragma unroll
                for (int j = 0; j < K; ++j)
                    ugy[j] = window_elem<T, K, NW>(uw, j, sx[j], sx[j]) * window_elem<T, K, NW>(gw, j, sx[j], sx[j]);
            }
            if constexpr (Pre) {
#pragma unroll
                for (int j = 0; j < K; ++j) {
                    s0[j] = __uint_as_float(word<TW>(tbuf[d][0], j));
                    s1[j] = __uint_as_float(word<TW>(tbuf[d][1], j));
                    s2[j] = __uint_as_float(word<TW>(tbuf[d][2], j));
                    t[j] = r[j] = 1.0f;
                }
            } else {
                const uint32_t sh = od ? ot.shE ^ 16u : ot.shE;
                const words_t<NW> tw[3] = {odd_window<Odd, NW, TW>(tbuf[d][0], sh),
                                           odd_window<Odd, NW, TW>(tbuf[d][1], sh ^ 16u),
                                           odd_window<Odd, NW, TW>(tbuf[d][2], sh)};
                normalise(tw, s0, s1, s2, t, r);
            }
#pragma unroll
            for (int j = 0; j < K; ++j)
                asm volatile("" : "+v"(lo), "+v"(uo) : "v"(s0[j]), "v"(s1[j]), "v"(s2[j]), "v"(r[j]), "v"(ugy[j]));
            load_line(d);

            // g_i from the next line's transposed products
            float P0[K], P2[K], g[K];
#pragma unroll
            for (int j = 0; j < K; ++j) {
                P0[j] = w0p[j] * gp[j];
                P2[j] = w2p[j] * gp[j];
                g[j] = fmaf(w1p[j], gp[j], ugy[j]);
            }
            const float P0n = from_next(P0[0]);
            const float P2p = from_prev(P2[K - 1]);
#pragma unroll
            for (int j = 0; j < K; ++j) {
                g[j] += j < K - 1 ? P0[j + 1] : P0n;
                g[j] += j > 0 ? P2[j - 1] : P2p;
                if constexpr (!kB16 || Pre) g[j] = valid[j] ? g[j] : 0.0f;
            }

            // tap gradients of line i
            bool restart = false;
            if constexpr (Chunked) {
                restart = s == next_restart;
                next_restart = restart ? next_restart + seg : next_restart;
#pragma unroll
                for (int j = 0; j < K; ++j) hp[j] = restart ? 0.0f : hp[j];
            }
            const float hl0 = from_prev(hp[K - 1]);
            const float hrK = from_next(hp[0]);
            float gz0[K], gz1[K], gz2[K];
#pragma unroll
            for (int j = 0; j < K; ++j) {
                const float hl = j > 0 ? hp[j - 1] : hl0;
                const float hr = j < K - 1 ? hp[j + 1] : hrK;
                const float e0 = g[j] * hl, e1 = g[j] * hp[j], e2 = g[j] * hr;
                if constexpr (Pre) {
                    // the tap products; the Jacobian comes after the group sum
                    gz0[j] = e0;
                    gz1[j] = e1;
                    gz2[j] = e2;
                    w0p[j] = s0[j];
                    w1p[j] = s1[j];
                    w2p[j] = s2[j];
                    continue;
                }
                const float wn0 = s0[j] * r[j], wn1 = s1[j] * r[j], wn2 = s2[j] * r[j];
                float n0 = e0, n1 = e1, n2 = e2;
                if (t[j] > eps) {
                    const float d01 = e0 - e1, d02 = e0 - e2, d12 = e1 - e2;
                    n0 = fmaf(wn1, d01, wn2 * d02);
                    n1 = fmaf(wn2, d12, -(wn0 * d01));
                    n2 = -fmaf(wn0, d02, wn1 * d12);
                }
                // s (1 - s) is 0 for a dropped tap, so its gradient is 0
                gz0[j] = n0 * (r[j] * fmaf(-s0[j], s0[j], s0[j]));
                gz1[j] = n1 * (r[j] * fmaf(-s1[j], s1[j], s1[j]));
                gz2[j] = n2 * (r[j] * fmaf(-s2[j], s2[j], s2[j]));
                w0p[j] = wn0;
                w1p[j] = wn1;
                w2p[j] = wn2;
            }
            if constexpr (summed) {
                // staging sets alternate by step: a set is rewritten two steps
                // later, after every wavefront has passed the barrier between
                const uint32_t set = static_cast<uint32_t>(s & 1) * set_bytes;
                stage_put<GT, K>(my_stage + set, q, gz0);
                stage_put<GT, K>(my_stage + set + SL * GS, q, gz1);
                stage_put<GT, K>(my_stage + set + 2 * SL * GS, q, gz2);
                sync();
                // this wavefront's share is at most 3 K 64 / CC dwords
                constexpr int NRS = (3 * K + CC - 1) / CC;
                static_assert(NRS <= NR, "a share fits the read-back slots");
#pragma unroll
                for (int t = 0; t < NRS; ++t) {
                    float v[CC];
#pragma unroll
                    for (int c = 0; c < CC; ++c)
                        v[c] = lds_at<float>(rd[t] + set + static_cast<uint32_t>(c * pstride));
                    float acc = 0.0f;
#pragma unroll
                    for (int c = 0; c < CC; ++c) acc += v[c];
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc), gws, go[t], 0, 0);
                    go[t] += gd[t];
                }
            } else if constexpr (kDirect) {
                const float* gzs[3] = {gz0, gz1, gz2};
#pragma unroll
                for (int k = 0; k < 3; ++k) {
                    const float* v = gzs[k];
                    if constexpr (GS == 4 && K == 2)
                        __builtin_amdgcn_raw_buffer_store_b64(
                            u32x2_t{__float_as_uint(v[0]), __float_as_uint(v[1])}, gws, d_off, k * d_tap, 0);
                    else if constexpr (GS == 4)
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[0]), gws, d_off, k * d_tap, 0);
                    else if constexpr (K == 2)
                        __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2(v[0], v[1]), gws, d_off, k * d_tap, 0);
                    else
                        __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(pack_bf16x2(v[0], v[0])), gws,
                                                              d_off, k * d_tap, 0);
                }
                d_off += d_step;
            } else {
                stage_put<GT, K>(my_stage, q, gz0);
                stage_put<GT, K>(my_stage + SL * GS, q, gz1);
                stage_put<GT, K>(my_stage + 2 * SL * GS, q, gz2);
                // the staging lines are written with 16- and 32-bit stores and
                // read back as dwords: keep the compiler from moving the reads
                // above the writes (the LDS then executes them in program order)
                asm volatile("" ::: "memory");
                if constexpr (Odd) {
#pragma unroll
                    for (int t = 0; t < NR16; ++t) {
                        __builtin_amdgcn_raw_buffer_store_b16(lds_at<uint16_t>(rd16[t]), gws, go16[t], 0, 0);
                        go16[t] += gd16[t];
                    }
                } else {
#pragma unroll
                    for (int t = 0; t < NR; ++t) {
                        __builtin_amdgcn_raw_buffer_store_b32(lds_at<uint32_t>(rd[t]), gws, go[t], 0, 0);
                        go[t] += gd[t];
                    }
                }
            }

#pragma unroll
            for (int j = 0; j < K; ++j) {
                gp[j] = restart ? 0.0f : g[j];
                put(aGH[j], aGL[j], g[j]);
                aGH[j] = aPH[j];
                aGL[j] = aPL[j];
                aPH[j] += dH[j];
                aPL[j] += dL[j];
                hp[j] = get(aPH[j], aPL[j]);
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
    }
    sync();

    // --------------------------------------------------------- G = g_a + g_b
    if constexpr (!Cols) {
        f32x4_t* gp4 = reinterpret_cast<f32x4_t*>(g_ws + static_cast<size_t>(plane) * HWa);
        for (int e = tid; e < HWa / 4; e += NT) gp4[e] = get4(lay.a, lay.la, e) + get4(lay.b, lay.lb, e);
    } else if constexpr (Odd) {
        column_pass_odd(g_ws, lam, x, gx, glam, std::true_type{});
    } else {
        column_pass(g_ws, lam, x, gx, glam, std::true_type{});
    }
}

// x, lambda, u, gy of every plane transposed ([H][W] -> [W][H], H and W
// even); one workgroup per (plane, tensor).  The plane is staged in LDS in
// its own layout and element type; global reads, LDS writes and global
// writes move four consecutive elements (H W % 4 == 0), and each thread
// issues up to eight reads before its LDS writes, so the plane's loads
// overlap.
template <typename T>
__global__ void __launch_bounds__(256)
transpose4_kernel(const T* __restrict__ a0, const T* __restrict__ a1, const T* __restrict__ a2,
                  const T* __restrict__ a3, T* __restrict__ t0, T* __restrict__ t1,
                  T* __restrict__ t2, T* __restrict__ t3, int H, int W) {
    extern __shared__ __attribute__((aligned(16))) uint32_t tile_words[];
    T* tile = reinterpret_cast<T*>(tile_words);
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    typedef typename std::conditional<sizeof(T) == 4, u32x4_t, u32x2_t>::type quad_t;
    const int which = blockIdx.y;
    const T* src = which == 0 ? a0 : which == 1 ? a1 : which == 2 ? a2 : a3;
    T* dst = which == 0 ? t0 : which == 1 ? t1 : which == 2 ? t2 : t3;
    const int HW = H * W, nq = HW / 4;
    const size_t base = static_cast<size_t>(blockIdx.x) * HW;
    const quad_t* sq = reinterpret_cast<const quad_t*>(src + base);
    quad_t* dq = reinterpret_cast<quad_t*>(dst + base);
    quad_t* tq = reinterpret_cast<quad_t*>(tile);
    for (int q0 = 0; q0 < nq; q0 += 8 * 256) {
        quad_t v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int t = q0 + 256 * j + static_cast<int>(threadIdx.x);
            if (t < nq) v[j] = sq[t];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int t = q0 + 256 * j + static_cast<int>(threadIdx.x);
            if (t < nq) tq[t] = v[j];
        }
    }
    __syncthreads();
    for (int t = threadIdx.x; t < nq; t += 256) {
        int c = (4 * t) / H, r = 4 * t - c * H;               // output element (c, r), then down the column
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (sizeof(T) == 4) w[i] = __float_as_uint(tile[r * W + c]);
            else w[i] = tile[r * W + c];
            const bool wrap = r + 1 == H;
            r = wrap ? 0 : r + 1;
            c = wrap ? c + 1 : c;
        }
        if constexpr (sizeof(T) == 4) dq[t] = u32x4_t{w[0], w[1], w[2], w[3]};
        else dq[t] = u32x2_t{w[0] | (w[1] << 16), w[2] | (w[3] << 16)};
    }
}

// x, lambda, u, gy of every bf16 plane transposed ([H][W] -> [W][H]) when
// H W is odd, so that planes start at any element; one workgroup per
// (plane, tensor).  The plane is read as the dwords from the even element at
// or below its first, staged in LDS element by element, and written as the
// dwords of the same span, a plane's first or last element alone when its
// dword is shared with the next plane.
__global__ void __launch_bounds__(256)
transpose4_odd_kernel(const uint16_t* __restrict__ a0, const uint16_t* __restrict__ a1,
                      const uint16_t* __restrict__ a2, const uint16_t* __restrict__ a3,
                      uint16_t* __restrict__ t0, uint16_t* __restrict__ t1, uint16_t* __restrict__ t2,
                      uint16_t* __restrict__ t3, int H, int W, int in_bytes) {
    const int which = blockIdx.y;
    const uint16_t* src = which == 0 ? a0 : which == 1 ? a1 : which == 2 ? a2 : a3;
    uint16_t* dst = which == 0 ? t0 : which == 1 ? t1 : which == 2 ? t2 : t3;
    const int HW = H * W;
    const int base = static_cast<int>(blockIdx.x) * HW;
    const int par = base & 1;
    const int nw = (par + HW + 1) / 2;   // dwords of the span
    // (a dword that straddles a buffer's end reads as 0: the bound is
    // rounded up to whole dwords)
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(src), 0, (in_bytes + 3) & ~3, kBufFlags);
    const uint32_t off0 = static_cast<uint32_t>(base - par) * 2u;
    const int tid = static_cast<int>(threadIdx.x);
    for (int q0 = 0; q0 < nw; q0 += 8 * 256) {
        uint32_t v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int t = q0 + 256 * j + tid;
            v[j] = t < nw ? __builtin_amdgcn_raw_buffer_load_b32(rs, off0 + 4u * t, 0, 0) : 0u;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int t = q0 + 256 * j + tid;
            const int g = 2 * t - par;
            if (t < nw) {
                if (g >= 0) lds_at<uint16_t>(2u * g) = static_cast<uint16_t>(v[j]);
                if (g + 1 < HW) lds_at<uint16_t>(2u * (g + 1)) = static_cast<uint16_t>(v[j] >> 16);
            }
        }
    }
    __syncthreads();
    // output element o = c H + r holds input element r W + c
    const float invH = 1.0f / static_cast<float>(H);
    auto in_of = [&](int o) -> uint32_t {
        const int c = static_cast<int>((static_cast<float>(o) + 0.5f) * invH);
        const int r = o - c * H;
        return 2u * static_cast<uint32_t>(r * W + c);
    };
    uint16_t* d0 = dst + (base - par);
    for (int t = tid; t < nw; t += 256) {
        const int o0 = 2 * t - par, o1 = o0 + 1;
        const uint32_t lo = o0 >= 0 ? lds_at<uint16_t>(in_of(o0)) : 0u;
        const uint32_t hi = o1 < HW ? lds_at<uint16_t>(in_of(o1)) : 0u;
        if (o0 >= 0 && o1 < HW)
            *reinterpret_cast<uint32_t*>(d0 + 2 * t) = lo | (hi << 16);
        else if (o0 >= 0)
            d0[2 * t] = static_cast<uint16_t>(lo);
        else
            d0[2 * t + 1] = static_cast<uint16_t>(hi);
    }
}

// Workspace regions (bytes, 256-aligned): x, lambda, u, gy transposed, then
// S and G of the row pair in fp32 (a plane every H W rounded up to 4).
struct PairBwdWs {
    int64_t xt, lt, ut, gt, s, g, bytes;
    PairBwdWs(int64_t planes, int64_t H, int64_t W, int64_t es) {
        auto a256 = [](int64_t v) { return (v + 255) & ~static_cast<int64_t>(255); };
        const int64_t n = planes * H * W;
        const int64_t na = planes * ((H * W + 3) & ~static_cast<int64_t>(3));
        xt = 0;
        lt = a256(xt + n * es);
        ut = a256(lt + n * es);
        gt = a256(ut + n * es);
        s = a256(gt + n * es);
        g = a256(s + na * 4);
        bytes = a256(g + na * 4);
    }
};

// Arguments of one launch of the pair kernel.
template <typename T, typename GT>
struct PassArgs {
    const T *xl, *ll, *ul, *gl;     // line-major inputs of the pair
    const T* w4;
    int w4_bytes;
    GT* gwd;                        // per-channel tap gradients
    int gw_bytes;
    int cpg, k_chunk;
    float eps;
    int64_t planes, NL, L;
    int dir0;
    float *s_ws, *g_ws;
    const T *x, *lam, *gy;          // pixel order (column pair's outputs)
    T *gx, *glam, *gu;
    const float* wpre = nullptr;    // Pre: normalised fp32 weights
    int wpre_bytes = 0;
    int cc = 1;                     // Pre: planes a workgroup
};

template <typename T, typename GT, int K, bool Cols, bool Chunked, bool Pre, int CC, bool Odd>
hipError_t launch_pass_cc(const PassArgs<T, GT>& a, hipStream_t stream) {
    constexpr int D = 4;   // lines prefetched ahead (the steps are long; a deeper unroll outgrows the instruction cache)
    constexpr int cc = CC;
    const size_t lds = cc * static_cast<size_t>(PairBwdLayout(static_cast<int>(a.NL), static_cast<int>(a.L),
                                                              sizeof(T) == 2, sizeof(GT), cc > 1 ? 2 : 1).bytes);
    auto kern = prop2d_backward_pair_kernel<T, GT, K, D, Cols, Chunked, Pre, CC, Odd>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(lds));
        if (e != hipSuccess) return e;
    }
    kern<<<dim3(static_cast<unsigned>(a.planes / cc)), dim3(128 * cc), lds, stream>>>(
        a.xl, a.ll, a.ul, a.gl, a.w4, a.w4_bytes, a.gwd, a.gw_bytes, a.cpg, a.k_chunk, a.eps,
        static_cast<int>(a.planes), static_cast<int>(a.NL), static_cast<int>(a.L), a.dir0, a.s_ws,
        a.g_ws, a.x, a.lam, a.gy, a.gx, a.glam, a.gu, a.wpre, a.wpre_bytes);
    return hipGetLastError();
}

template <typename T, typename GT, int K, bool Cols, bool Chunked, bool Pre, bool Odd>
hipError_t launch_pass(const PassArgs<T, GT>& a, hipStream_t stream) {
    if constexpr (Pre) {
        if (a.cc == 4) return launch_pass_cc<T, GT, K, Cols, Chunked, true, 4, false>(a, stream);
        if (a.cc == 2) return launch_pass_cc<T, GT, K, Cols, Chunked, true, 2, false>(a, stream);
    }
    return launch_pass_cc<T, GT, K, Cols, Chunked, Pre, 1, Odd>(a, stream);
}

// K = ceil(L / 64) positions a lane.  A wavefront per direction needs no
// barrier a step (the directions meet only between passes), and two
// wavefronts a SIMD hide more of each other's latency than the halves of
// one wavefront (K = ceil(L / 32)) saved in idle slots: latent1k 0.480 ms
// against 0.505, 148 x 148 (one plane per CU) 0.42 against 0.58.
template <typename T, typename GT, bool Cols, bool Pre, bool Odd>
hipError_t launch_pass_k(const PassArgs<T, GT>& a, hipStream_t stream) {
    const bool ch = a.k_chunk > 1;
    if (a.L <= 64)
        return ch ? launch_pass<T, GT, 1, Cols, true, Pre, Odd>(a, stream)
                  : launch_pass<T, GT, 1, Cols, false, Pre, Odd>(a, stream);
    if (a.L <= 128)
        return ch ? launch_pass<T, GT, 2, Cols, true, Pre, Odd>(a, stream)
                  : launch_pass<T, GT, 2, Cols, false, Pre, Odd>(a, stream);
    return ch ? launch_pass<T, GT, 3, Cols, true, Pre, Odd>(a, stream)
              : launch_pass<T, GT, 3, Cols, false, Pre, Odd>(a, stream);
}

// gwd_: per-channel tap gradients as GT, or (Pre) the fp32 partial sums of
// the tap products, one plane per cc planes; wpre: the normalised weights.
// Odd: square bf16 planes of odd side (per-channel taps).
template <typename T, typename GT, bool Pre, bool Odd = false>
hipError_t backward_pair_t(const void* x_, const void* lam_, const void* u_, const void* w4_,
                           const void* gy_, float eps, void* gx_, void* glam_, void* gu_, void* gwd_,
                           void* ws_, int64_t planes, int64_t H, int64_t W, const PropOpts& o,
                           hipStream_t stream, const float* wpre = nullptr, int cc = 1) {
    char* ws = static_cast<char*>(ws_);
    const PairBwdWs lay(planes, H, W, sizeof(T));
    T* xt = reinterpret_cast<T*>(ws + lay.xt);
    T* lt = reinterpret_cast<T*>(ws + lay.lt);
    T* ut = reinterpret_cast<T*>(ws + lay.ut);
    T* gt = reinterpret_cast<T*>(ws + lay.gt);
    PassArgs<T, GT> a;
    a.xl = static_cast<const T*>(x_);
    a.ll = static_cast<const T*>(lam_);
    a.ul = static_cast<const T*>(u_);
    a.gl = static_cast<const T*>(gy_);
    a.w4 = static_cast<const T*>(w4_);
    a.w4_bytes = static_cast<int>(12 * (planes / o.cpg) * H * W * sizeof(T));
    a.gwd = static_cast<GT*>(gwd_);
    a.gw_bytes = static_cast<int>(12 * (planes / cc) * H * W * sizeof(GT));
    a.wpre = wpre;
    a.wpre_bytes = static_cast<int>(12 * (planes / o.cpg) * H * W * 4);
    a.cc = cc;
    a.cpg = static_cast<int>(o.cpg);
    a.k_chunk = static_cast<int>(o.k_chunk);
    a.eps = eps;
    a.planes = planes;
    a.NL = H;
    a.L = W;
    a.dir0 = 0;
    a.s_ws = reinterpret_cast<float*>(ws + lay.s);
    a.g_ws = reinterpret_cast<float*>(ws + lay.g);
    a.x = a.xl;
    a.lam = a.ll;
    a.gy = a.gl;
    a.gx = static_cast<T*>(gx_);
    a.glam = static_cast<T*>(glam_);
    a.gu = static_cast<T*>(gu_);

    // row pair on the inputs as they are: taps and gradients of directions 0, 1
    hipError_t e = launch_pass_k<T, GT, false, Pre, Odd>(a, stream);
    if (e != hipSuccess) return e;
    const size_t tlds = static_cast<size_t>(H * W) * sizeof(T);
    if constexpr (Odd) {
        if (tlds > 64 * 1024 &&
            (e = hipFuncSetAttribute(reinterpret_cast<const void*>(transpose4_odd_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(tlds))) != hipSuccess)
            return e;
        transpose4_odd_kernel<<<dim3(static_cast<unsigned>(planes), 4), dim3(256), tlds, stream>>>(
            a.x, a.lam, a.ul, a.gy, xt, lt, ut, gt, static_cast<int>(H), static_cast<int>(W),
            static_cast<int>(planes * H * W * 2));
    } else {
        if (tlds > 64 * 1024 &&
            (e = hipFuncSetAttribute(reinterpret_cast<const void*>(transpose4_kernel<T>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(tlds))) != hipSuccess)
            return e;
        transpose4_kernel<T><<<dim3(static_cast<unsigned>(planes), 4), dim3(256), tlds, stream>>>(
            a.x, a.lam, a.ul, a.gy, xt, lt, ut, gt, static_cast<int>(H), static_cast<int>(W));
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // column pair on the transposed copies: directions 2, 3, then the outputs
    a.xl = xt;
    a.ll = lt;
    a.ul = ut;
    a.gl = gt;
    a.NL = W;
    a.L = H;
    a.dir0 = 2;
    return launch_pass_k<T, GT, true, Pre, Odd>(a, stream);
}

// Normalised weights of every tap group, fp32, in the taps' layout
// ([4][groups][3][NL][L], line-major per direction): one thread per (direction,
// group, position); taps whose source lies off the line get 0.
template <typename T>
__global__ void __launch_bounds__(256)
shared_weights_kernel(const T* __restrict__ w4, float* __restrict__ wn, int64_t tplanes, int H, int W,
                      float eps) {
    const int64_t HW = static_cast<int64_t>(H) * W;
    const int64_t per_dir = tplanes * HW;
    const int64_t total = 4 * per_dir;
    for (int64_t idx = blockIdx.x * 256ll + threadIdx.x; idx < total; idx += static_cast<int64_t>(gridDim.x) * 256) {
        const int dir = static_cast<int>(idx / per_dir);
        const int64_t rem = idx - dir * per_dir;
        const int64_t tp = rem / HW;
        const int64_t t = rem - tp * HW;
        const int L = dir < 2 ? W : H;
        const int p = static_cast<int>(t % L);
        const size_t base = static_cast<size_t>((dir * tplanes + tp) * 3 * HW + t);
        float w0, w1, w2;
        normalize3(load_elem(w4, base), load_elem(w4, base + HW), load_elem(w4, base + 2 * HW), p > 0,
                   p < L - 1, eps, w0, w1, w2);
        wn[base] = w0;
        wn[base + HW] = w1;
        wn[base + 2 * HW] = w2;
    }
}

// Tap gradients of every tap group from the partial sums of the tap
// products (part: [4][groups][nch][3][NL][L], nch partial planes a group,
// added in order), through the normalisation's Jacobian: with s = sigmoid(z),
// T = sum s, r = 1 / max(T, eps), wn = s r and e the summed products,
//   T > eps: gs_m = r sum_{k != m} wn_k (e_m - e_k), else gs_m = r e_m;
//   gz_m = gs_m s_m (1 - s_m); dropped taps have s = 0 and get 0.
template <typename T>
__global__ void __launch_bounds__(256)
shared_tap_grad_kernel(const float* __restrict__ part, const T* __restrict__ w4, T* __restrict__ gw4,
                       int64_t tplanes, int nch, int H, int W, float eps) {
    const int64_t HW = static_cast<int64_t>(H) * W;
    const int64_t per_dir = tplanes * HW;
    const int64_t total = 4 * per_dir;
    for (int64_t idx = blockIdx.x * 256ll + threadIdx.x; idx < total; idx += static_cast<int64_t>(gridDim.x) * 256) {
        const int dir = static_cast<int>(idx / per_dir);
        const int64_t rem = idx - dir * per_dir;
        const int64_t tp = rem / HW;
        const int64_t t = rem - tp * HW;
        const int L = dir < 2 ? W : H;
        const int p = static_cast<int>(t % L);
        const size_t base = static_cast<size_t>((dir * tplanes + tp) * 3 * HW + t);
        const float* pp = part + static_cast<size_t>((dir * tplanes + tp) * nch) * 3 * HW + t;
        float e0 = 0.0f, e1 = 0.0f, e2 = 0.0f;
        for (int j = 0; j < nch; ++j) {
            e0 += pp[0];
            e1 += pp[HW];
            e2 += pp[2 * HW];
            pp += 3 * HW;
        }
        const float s0 = p > 0 ? sigmoid_hw(load_elem(w4, base)) : 0.0f;
        const float s1 = sigmoid_hw(load_elem(w4, base + HW));
        const float s2 = p < L - 1 ? sigmoid_hw(load_elem(w4, base + 2 * HW)) : 0.0f;
        const float tt = (s0 + s1) + s2;
        const float r = __builtin_amdgcn_rcpf(fmaxf(tt, eps));
        const float wn0 = s0 * r, wn1 = s1 * r, wn2 = s2 * r;
        float n0 = e0, n1 = e1, n2 = e2;
        if (tt > eps) {
            const float d01 = e0 - e1, d02 = e0 - e2, d12 = e1 - e2;
            n0 = fmaf(wn1, d01, wn2 * d02);
            n1 = fmaf(wn2, d12, -(wn0 * d01));
            n2 = -fmaf(wn0, d02, wn1 * d12);
        }
        store_elem(gw4, base, n0 * (r * fmaf(-s0, s0, s0)));
        store_elem(gw4, base + HW, n1 * (r * fmaf(-s1, s1, s1)));
        store_elem(gw4, base + 2 * HW, n2 * (r * fmaf(-s2, s2, s2)));
    }
}

// Planes a workgroup for channels that share taps: 4, 2 or 1, a divisor of
// the channels a group whose layouts (two staging sets) fit in LDS together,
// for the row and the column launch.
int shared_planes_per_group(int64_t cpg, int64_t H, int64_t W, bool narrow) {
    for (int cc = 4; cc > 1; cc /= 2) {
        if (cpg % cc != 0) continue;
        const int64_t rows = PairBwdLayout(static_cast<int>(H), static_cast<int>(W), narrow, 4, 2).bytes;
        const int64_t cols = PairBwdLayout(static_cast<int>(W), static_cast<int>(H), narrow, 4, 2).bytes;
        if (cc * rows <= kLdsBytes && cc * cols <= kLdsBytes) return cc;
    }
    return 1;
}

}  // namespace

namespace {

// Even sides up to 160 for bf16 (three slots a lane) and 128 for fp32 (two
// slots) whose layout, for the storage width (narrow: bf16), fp32 staged tap
// gradients (the larger staging) and a wavefront per direction, fits in LDS
// for both the row and the column launch.
bool pair_fits(int64_t planes, int64_t H, int64_t W, bool narrow) {
    const int64_t side = narrow ? 160 : 128;
    if (H < 2 || W < 2 || H > side || W > side) return false;
    // odd sides: square bf16 planes (the kernel's odd form)
    if (((H & 1) || (W & 1)) && !(narrow && H == W && H >= 3)) return false;
    if (PairBwdLayout(static_cast<int>(H), static_cast<int>(W), narrow, 4).bytes > kLdsBytes ||
        PairBwdLayout(static_cast<int>(W), static_cast<int>(H), narrow, 4).bytes > kLdsBytes)
        return false;
    // every stream offset is a 32-bit byte offset into one buffer resource
    return 12 * planes * H * W * 4 <= 0x7fffffff;
}

}  // namespace

// Whether some storage type takes the pair kernel (the narrow bf16 layout is
// the smaller); sizes the workspace.
bool prop2d_backward_pair_shape(int64_t planes, int64_t H, int64_t W) {
    return pair_fits(planes, H, W, true);
}

int64_t prop2d_backward_pair_workspace_bytes(int64_t planes, int64_t H, int64_t W) {
    return PairBwdWs(planes, H, W, 4).bytes;   // fp32 storage needs the most
}

bool prop2d_backward_pair_eligible(int dtype, int64_t planes, int64_t H, int64_t W,
                                   const void* const* ptrs, int nptrs, const void* ws) {
    if (ws == nullptr || !pair_fits(planes, H, W, dtype == 1)) return false;
    // pixel pairs are read and written whole: 8 bytes in fp32, 4 in bf16
    const uintptr_t mask = dtype == 0 ? 7u : 3u;
    for (int i = 0; i < nptrs; ++i)
        if (reinterpret_cast<uintptr_t>(ptrs[i]) & mask) return false;
    return (reinterpret_cast<uintptr_t>(ws) & 15u) == 0;
}

int64_t prop2d_backward_pair_shared_weights_bytes(int64_t planes, int64_t H, int64_t W, int64_t cpg) {
    return (12 * (planes / cpg) * H * W * 4 + 255) & ~static_cast<int64_t>(255);
}

hipError_t launch_prop2d_backward_pair_shared(const void* x, const void* lam, const void* u,
                                              const void* w4, const void* gy, float eps, void* gx,
                                              void* glam, void* gu, void* gw4, float* part, float* wpre,
                                              void* ws, int dtype, int64_t planes, int64_t H,
                                              int64_t W, const PropOpts& o, hipStream_t stream) {
    const int64_t tplanes = planes / o.cpg;
    const int64_t n = 4 * tplanes * H * W;
    const unsigned blocks = static_cast<unsigned>(std::min<int64_t>((n + 255) / 256, 256 * 64));
    const int cc = shared_planes_per_group(o.cpg, H, W, dtype == 1);
    hipError_t e;
    if (dtype == 0) {
        shared_weights_kernel<float><<<dim3(blocks), dim3(256), 0, stream>>>(
            static_cast<const float*>(w4), wpre, tplanes, static_cast<int>(H), static_cast<int>(W), eps);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        e = backward_pair_t<float, float, true>(x, lam, u, w4, gy, eps, gx, glam, gu, part, ws, planes, H, W, o,
                                                stream, wpre, cc);
        if (e != hipSuccess) return e;
        shared_tap_grad_kernel<float><<<dim3(blocks), dim3(256), 0, stream>>>(
            part, static_cast<const float*>(w4), static_cast<float*>(gw4), tplanes,
            static_cast<int>(o.cpg / cc), static_cast<int>(H), static_cast<int>(W), eps);
    } else {
        shared_weights_kernel<uint16_t><<<dim3(blocks), dim3(256), 0, stream>>>(
            static_cast<const uint16_t*>(w4), wpre, tplanes, static_cast<int>(H), static_cast<int>(W), eps);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        e = backward_pair_t<uint16_t, float, true>(x, lam, u, w4, gy, eps, gx, glam, gu, part, ws, planes, H, W,
                                                   o, stream, wpre, cc);
        if (e != hipSuccess) return e;
        shared_tap_grad_kernel<uint16_t><<<dim3(blocks), dim3(256), 0, stream>>>(
            part, static_cast<const uint16_t*>(w4), static_cast<uint16_t*>(gw4), tplanes,
            static_cast<int>(o.cpg / cc), static_cast<int>(H), static_cast<int>(W), eps);
    }
    return hipGetLastError();
}

hipError_t launch_prop2d_backward_pair(const void* x, const void* lam, const void* u,
                                       const void* w4, const void* gy, float eps, void* gx,
                                       void* glam, void* gu, void* gwd, bool gw_fp32, void* ws,
                                       int dtype, int64_t planes, int64_t H, int64_t W,
                                       const PropOpts& o, hipStream_t stream) {
    if (dtype == 0)
        return backward_pair_t<float, float, false>(x, lam, u, w4, gy, eps, gx, glam, gu, gwd, ws, planes, H,
                                                    W, o, stream);
    if (gw_fp32)
        return backward_pair_t<uint16_t, float, false>(x, lam, u, w4, gy, eps, gx, glam, gu, gwd, ws, planes,
                                                       H, W, o, stream);
    if (H & 1)
        return backward_pair_t<uint16_t, uint16_t, false, true>(x, lam, u, w4, gy, eps, gx, glam, gu, gwd, ws,
                                                                planes, H, W, o, stream);
    return backward_pair_t<uint16_t, uint16_t, false>(x, lam, u, w4, gy, eps, gx, glam, gu, gwd, ws, planes,
                                                      H, W, o, stream);
}

}  // namespace gspn
