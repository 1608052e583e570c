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
//      the half.
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
// Sums run in a fixed order (row pair before column pair, first half before
// second), so the result is the same on every run.
#include "gspn_device.h"
#include "gspn_internal.h"
#include "gspn_lane.h"

#include <type_traits>

namespace gspn {
namespace {

using namespace lane;

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
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
    // gsize: bytes of a staged tap gradient
    __host__ __device__ PairBwdLayout(int NL, int L, bool narrow, int gsize) {
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
        bytes = stage + 6 * nh * ((L + nh - 1) / nh) * gsize;   // K = ceil(L / nh) slots a lane
    }
};

// Tap gradients of one adjoint step go out through LDS: each lane puts the
// values of its K slots into a staging line per (half, tap), 32 K elements
// apart so that slots past a line's end land in the padding, and the
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

// Cols = false: the row pair (NL = H, L = W), inputs as they are; writes S and
// G of the pair to s_ws, g_ws ([planes][H][W] fp32).
// Cols = true: the column pair (NL = W, L = H), inputs transposed; adds the
// row pair's S and G and writes gu, gx, glam.
// Taps are read from group plane p / cpg (w4: w4_bytes); the tap gradients
// are written per channel, as GT, to gwd ([4][planes][3][..][..], gw_bytes).
// Chunked: k_chunk > 1.  A wavefront per direction; they meet only between
// passes.
template <typename T, typename GT, int K, int D, bool Cols, bool Chunked>
__global__ void __launch_bounds__(128)
prop2d_backward_pair_kernel(const T* __restrict__ xl, const T* __restrict__ laml,
                            const T* __restrict__ ul, const T* __restrict__ gyl,
                            const T* __restrict__ w4, int w4_bytes, GT* __restrict__ gwd,
                            int gw_bytes, int cpg, int k_chunk,
                            float eps, int planes, int NL, int L, int dir0,
                            float* __restrict__ s_ws, float* __restrict__ g_ws,
                            const T* __restrict__ x, const T* __restrict__ lam,
                            const T* __restrict__ gy, T* __restrict__ gx, T* __restrict__ glam,
                            T* __restrict__ gu) {
    constexpr int ES = sizeof(T);
    constexpr int NW = window_words<T, K>();
    constexpr bool kNarrow = ES == 2;
    constexpr int VW = kNarrow ? 2 : 4;     // bytes of a value in the A / B array
    const int HW = NL * L;
    constexpr int GS = sizeof(GT);
    const PairBwdLayout lay(NL, L, kNarrow, GS);
    constexpr int NT = 128;                 // threads of the workgroup
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int half = tid >> 6;              // the wavefront: its direction
    const int q = lane;
    const bool fwd = half == 0;
    // orders the LDS accesses of the two wavefronts
    auto sync = [&]() { lds_barrier(); };
    const int plane = blockIdx.x;
    const size_t pix0 = static_cast<size_t>(plane) * HW;

    // zero lines (h before a scan's first line) and the dummy words
    if (tid < 8) lds_at<float>(4u * tid) = 0.0f;
    // each wavefront's own dummy words: the values that slots past a line's
    // end leave there (finite, and weighed only by dropped taps) then follow
    // that wavefront's program order, so even the signs of the zero tap
    // gradients they touch are the same from run to run
    const uint32_t dum0 = 16u * half;
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
            typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
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

    const int in_bytes = planes * HW * ES;
    const __amdgpu_buffer_rsrc_t xs = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(xl), 0, in_bytes, kBufFlags);
    const __amdgpu_buffer_rsrc_t ls = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(laml), 0, in_bytes, kBufFlags);
    const __amdgpu_buffer_rsrc_t us = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(ul), 0, in_bytes, kBufFlags);
    const __amdgpu_buffer_rsrc_t gs = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(gyl), 0, in_bytes, kBufFlags);
    __amdgpu_buffer_rsrc_t taps[3];
    const __amdgpu_buffer_rsrc_t gws = __builtin_amdgcn_make_buffer_rsrc(gwd, 0, gw_bytes, kBufFlags);
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        taps[k] = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(w4 + static_cast<size_t>(k) * HW), 0,
                                                    w4_bytes - k * HW * ES, kBufFlags);
    }
    const int par = ES == 2 ? ((K * q) & 1) : 0;
    const uint32_t win_b = static_cast<uint32_t>(K * q - par) * ES;
    const uint32_t sel_even = par ? 0x03020c0cu : 0x01000c0cu;
    const uint32_t sel_odd = par ? 0x05040c0cu : 0x03020c0cu;
    const uint32_t tap_b = static_cast<uint32_t>(((dir0 + half) * (planes / cpg) + plane / cpg) * 3 * HW) * ES;
    // segments of a chunked scan; a segment's first line reads no line before it
    const int seg = Chunked ? (NL + k_chunk - 1) / k_chunk : NL;
    const uint32_t line_b = static_cast<uint32_t>(L) * ES;
    const uint32_t plane_base = half ? lay.b : lay.a;
    const uint32_t lplane_base = half ? lay.lb : lay.la;

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
    // s_k = sigmoid(z_k) (0 for dropped taps) and r = 1 / max(sum s, eps)
    auto normalise = [&](const words_t<NW> (&tw)[3], float (&s0)[K], float (&s1)[K], float (&s2)[K],
                         float (&t)[K], float (&r)[K]) {
#pragma unroll
        for (int j = 0; j < K; ++j) {
            s0[j] = window_elem<T, K, NW>(tw[0], j, sel_even, sel_odd) * kNegLog2e;
            s1[j] = window_elem<T, K, NW>(tw[1], j, sel_even, sel_odd) * kNegLog2e;
            s2[j] = window_elem<T, K, NW>(tw[2], j, sel_even, sel_odd) * kNegLog2e;
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

    // ------------------------------------------------------------ forward
    {
        const uint32_t lo0 = fwd ? 0u : static_cast<uint32_t>(NL - 1) * line_b;
        const uint32_t dlo = fwd ? line_b : 0u - line_b;
        uint32_t lo = tap_b + win_b + lo0;
        uint32_t xo = static_cast<uint32_t>(pix0) * ES + win_b + lo0;
        words_t<NW> tbuf[D][3], xbuf[D], lbuf[D];
        auto load_line = [&](int d) {
#pragma unroll
            for (int k = 0; k < 3; ++k) tbuf[d][k] = load_words<NW>(taps[k], lo);
            xbuf[d] = load_words<NW>(xs, xo);
            lbuf[d] = load_words<NW>(ls, xo);
            lo += dlo;
            xo += dlo;
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
            float s0[K], s1[K], s2[K], t[K], r[K], b[K];
#pragma unroll
            for (int j = 0; j < K; ++j)
                b[j] = window_elem<T, K, NW>(lbuf[d], j, sel_even, sel_odd) *
                       window_elem<T, K, NW>(xbuf[d], j, sel_even, sel_odd);
            normalise(tbuf[d], s0, s1, s2, t, r);
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
                hn[j] = fmaf(m, r[j], b[j]);
            }
#pragma unroll
            for (int j = 0; j < K; ++j) {
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
        f32x4_t* sp = reinterpret_cast<f32x4_t*>(s_ws + pix0);
        for (int e = tid; e < HW / 4; e += NT) sp[e] = get4(lay.a, lay.la, e) + get4(lay.b, lay.lb, e);
    } else {
        column_pass(s_ws, gy, gy, gu, gu, std::false_type{});
    }
    sync();

    // ------------------------------------------------------------ adjoint
    {
        // lanes 0-31 walk their lines NL-1 .. 0, lanes 32-63 walk 0 .. NL-1
        const int i0 = fwd ? NL - 1 : 0;
        const uint32_t lo0 = static_cast<uint32_t>(i0) * line_b;
        const uint32_t dlo = fwd ? 0u - line_b : line_b;
        uint32_t lo = tap_b + win_b + lo0;
        uint32_t uo = static_cast<uint32_t>(pix0) * ES + win_b + lo0;
        words_t<NW> tbuf[D][3], ubuf[D], gbuf[D];
        auto load_line = [&](int d) {
#pragma unroll
            for (int k = 0; k < 3; ++k) tbuf[d][k] = load_words<NW>(taps[k], lo);
            ubuf[d] = load_words<NW>(us, uo);
            gbuf[d] = load_words<NW>(gs, uo);
            lo += dlo;
            uo += dlo;
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
        uint32_t rd[NR], go[NR], gd[NR];
#pragma unroll
        for (int t = 0; t < NR; ++t) {
            const int f = lane + 64 * t;
            rd[t] = lay.stage;
            go[t] = kDrop;
            gd[t] = 0;
            if (f < kLines * per_line) {
                const int hk = 3 * half + f / per_line;
                const int m = f - (f / per_line) * per_line;
                const int h = hk / 3, k = hk - 3 * h;
                const int start = h == 0 ? NL - 1 : 0;      // first adjoint line of that half
                rd[t] = lay.stage + hk * SL * GS + 4 * m;
                go[t] = static_cast<uint32_t>((((dir0 + h) * planes + plane) * 3 + k) * HW * GS +
                                              start * L * GS + 4 * m);
                gd[t] = h == 0 ? 0u - static_cast<uint32_t>(L * GS) : static_cast<uint32_t>(L * GS);
            }
        }
        const uint32_t my_stage = lay.stage + 3 * half * SL * GS;
        // adjoint step of the next restart line: its taps read nothing (tap
        // gradient 0) and the line before it receives no adjoint term from it
        int next_restart = fwd ? (NL - 1) - ((NL - 1) / seg) * seg : seg - 1;
        // LDS: g_i goes to line i (G); h_{i-1} (lanes 0-31) or h_{i+1}
        // (32-63) is read one step ahead (P), and P of one step is G of the next
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
            float s0[K], s1[K], s2[K], t[K], r[K], ugy[K];
#pragma unroll
            for (int j = 0; j < K; ++j)
                ugy[j] = window_elem<T, K, NW>(ubuf[d], j, sel_even, sel_odd) *
                         window_elem<T, K, NW>(gbuf[d], j, sel_even, sel_odd);
            normalise(tbuf[d], s0, s1, s2, t, r);
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
            stage_put<GT, K>(my_stage, q, gz0);
            stage_put<GT, K>(my_stage + SL * GS, q, gz1);
            stage_put<GT, K>(my_stage + 2 * SL * GS, q, gz2);
            // the staging lines are written with 16- and 32-bit stores and read
            // back as dwords: keep the compiler from moving the reads above
            // the writes (the LDS then executes them in program order)
            asm volatile("" ::: "memory");
#pragma unroll
            for (int t = 0; t < NR; ++t) {
                __builtin_amdgcn_raw_buffer_store_b32(lds_at<uint32_t>(rd[t]), gws, go[t], 0, 0);
                go[t] += gd[t];
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
        f32x4_t* gp4 = reinterpret_cast<f32x4_t*>(g_ws + pix0);
        for (int e = tid; e < HW / 4; e += NT) gp4[e] = get4(lay.a, lay.la, e) + get4(lay.b, lay.lb, e);
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

// Workspace regions (bytes, 256-aligned): x, lambda, u, gy transposed, then
// S and G of the row pair in fp32.
struct PairBwdWs {
    int64_t xt, lt, ut, gt, s, g, bytes;
    PairBwdWs(int64_t planes, int64_t H, int64_t W, int64_t es) {
        auto a256 = [](int64_t v) { return (v + 255) & ~static_cast<int64_t>(255); };
        const int64_t n = planes * H * W;
        xt = 0;
        lt = a256(xt + n * es);
        ut = a256(lt + n * es);
        gt = a256(ut + n * es);
        s = a256(gt + n * es);
        g = a256(s + n * 4);
        bytes = a256(g + n * 4);
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
};

template <typename T, typename GT, int K, bool Cols, bool Chunked>
hipError_t launch_pass(const PassArgs<T, GT>& a, hipStream_t stream) {
    constexpr int D = 4;   // lines prefetched ahead (the steps are long; a deeper unroll outgrows the instruction cache)
    const size_t lds = PairBwdLayout(static_cast<int>(a.NL), static_cast<int>(a.L), sizeof(T) == 2,
                                     sizeof(GT)).bytes;
    auto kern = prop2d_backward_pair_kernel<T, GT, K, D, Cols, Chunked>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(lds));
        if (e != hipSuccess) return e;
    }
    kern<<<dim3(static_cast<unsigned>(a.planes)), dim3(128), lds, stream>>>(
        a.xl, a.ll, a.ul, a.gl, a.w4, a.w4_bytes, a.gwd, a.gw_bytes, a.cpg, a.k_chunk, a.eps,
        static_cast<int>(a.planes), static_cast<int>(a.NL), static_cast<int>(a.L), a.dir0, a.s_ws,
        a.g_ws, a.x, a.lam, a.gy, a.gx, a.glam, a.gu);
    return hipGetLastError();
}

// K = ceil(L / 64) positions a lane.  A wavefront per direction needs no
// barrier a step (the directions meet only between passes), and two
// wavefronts a SIMD hide more of each other's latency than the halves of
// one wavefront (K = ceil(L / 32)) saved in idle slots: latent1k 0.480 ms
// against 0.505, 148 x 148 (one plane per CU) 0.42 against 0.58.
template <typename T, typename GT, bool Cols>
hipError_t launch_pass_k(const PassArgs<T, GT>& a, hipStream_t stream) {
    const bool ch = a.k_chunk > 1;
    if (a.L <= 64)
        return ch ? launch_pass<T, GT, 1, Cols, true>(a, stream) : launch_pass<T, GT, 1, Cols, false>(a, stream);
    if (a.L <= 128)
        return ch ? launch_pass<T, GT, 2, Cols, true>(a, stream) : launch_pass<T, GT, 2, Cols, false>(a, stream);
    return ch ? launch_pass<T, GT, 3, Cols, true>(a, stream) : launch_pass<T, GT, 3, Cols, false>(a, stream);
}

template <typename T, typename GT>
hipError_t backward_pair_t(const void* x_, const void* lam_, const void* u_, const void* w4_,
                           const void* gy_, float eps, void* gx_, void* glam_, void* gu_, void* gwd_,
                           void* ws_, int64_t planes, int64_t H, int64_t W, const PropOpts& o,
                           hipStream_t stream) {
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
    a.gw_bytes = static_cast<int>(12 * planes * H * W * sizeof(GT));
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
    hipError_t e = launch_pass_k<T, GT, false>(a, stream);
    if (e != hipSuccess) return e;
    const size_t tlds = static_cast<size_t>(H * W) * sizeof(T);
    if (tlds > 64 * 1024 &&
        (e = hipFuncSetAttribute(reinterpret_cast<const void*>(transpose4_kernel<T>),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(tlds))) != hipSuccess)
        return e;
    transpose4_kernel<T><<<dim3(static_cast<unsigned>(planes), 4), dim3(256), tlds, stream>>>(
        a.x, a.lam, a.ul, a.gy, xt, lt, ut, gt, static_cast<int>(H), static_cast<int>(W));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // column pair on the transposed copies: directions 2, 3, then the outputs
    a.xl = xt;
    a.ll = lt;
    a.ul = ut;
    a.gl = gt;
    a.NL = W;
    a.L = H;
    a.dir0 = 2;
    return launch_pass_k<T, GT, true>(a, stream);
}

}  // namespace

namespace {

// Even sides up to 160 for bf16 (three slots a lane) and 128 for fp32 (two
// slots) whose layout, for the storage width (narrow: bf16), fp32 staged tap
// gradients (the larger staging) and a wavefront per direction, fits in LDS
// for both the row and the column launch.
bool pair_fits(int64_t planes, int64_t H, int64_t W, bool narrow) {
    const int64_t side = narrow ? 160 : 128;
    if (H < 2 || W < 2 || H > side || W > side || (H & 1) || (W & 1)) return false;
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

hipError_t launch_prop2d_backward_pair(const void* x, const void* lam, const void* u,
                                       const void* w4, const void* gy, float eps, void* gx,
                                       void* glam, void* gu, void* gwd, bool gw_fp32, void* ws,
                                       int dtype, int64_t planes, int64_t H, int64_t W,
                                       const PropOpts& o, hipStream_t stream) {
    if (dtype == 0)
        return backward_pair_t<float, float>(x, lam, u, w4, gy, eps, gx, glam, gu, gwd, ws, planes, H, W,
                                             o, stream);
    if (gw_fp32)
        return backward_pair_t<uint16_t, float>(x, lam, u, w4, gy, eps, gx, glam, gu, gwd, ws, planes, H,
                                                W, o, stream);
    return backward_pair_t<uint16_t, uint16_t>(x, lam, u, w4, gy, eps, gx, glam, gu, gwd, ws, planes, H,
                                               W, o, stream);
}

}  // namespace gspn
