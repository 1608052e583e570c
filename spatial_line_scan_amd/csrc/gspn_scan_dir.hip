// One-direction scan (gspn_scan_dir) for lines up to 256 (gfx950): one
// wavefront per (b, c) plane, no barrier.
//
// Operator: "Scaling Parallel Sequence Models to Foundation-Scale Vision
// Encoders", §3 line-scan recurrence (standard GSPN form) and §4.3
// stream-based concurrency (directions run as separate passes); reading
// notes, method / overall framework (the top-down scan and the fused
// normalisation: sigmoid, local sum, clamp, divide).
//
// Work split.  The wavefront walks the NL lines of its direction in scan
// order; lane q holds positions Kq .. Kq+K-1 of the current line (K = 1..4
// for lines up to 64, 128, 192, 256) and the three-tap neighbour exchange is
// one whole-wavefront DPP shift each way (lanes 0 and 63 receive 0, which
// only dropped taps weigh).  The taps (line-major for every direction)
// stream one element a slot, several lines ahead, as raw words widened where
// they are used.
//
// Row directions (top-down, bottom-up) read x, lambda, u (and y) of their
// slots with the taps and write y at each step: no LDS, so every plane of a
// large launch is resident at once.  Column directions would gather along
// columns that way; they stage b = lambda x one strip of 128-byte row lines
// at a time in LDS, transposed, scan the strip's columns there (h replaces b)
// and write the strip's y rows.
//
// Taps: raw logits are normalised in registers (sigmoid; taps whose source
// lies outside the line dropped; sum clamped below by eps; divide);
// normalised taps are used as given, those outside the line weighing 0
// whatever their value.
#include "gspn_device.h"
#include "gspn_internal.h"
#include "gspn_lane.h"

#include <type_traits>

namespace gspn {
namespace {

using namespace lane;

constexpr int kPad = 16;   // bytes: the dummy word (and alignment) before the plane

template <typename V> using lds_t = __attribute__((address_space(3))) V;

template <typename V>
__device__ __forceinline__ lds_t<V>& lds_ref(uint32_t byte_off) {
    // the kernel's only LDS is its dynamic array, which starts at address 0
    return *reinterpret_cast<lds_t<V>*>(static_cast<uintptr_t>(byte_off));
}

__device__ __forceinline__ void lds_order() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
}

// Raw bits of one tap element and their fp32 value.  The bits keep the
// storage width, so that widening happens where they are used, not where
// they are loaded.
template <typename T> using tap_bits_t = std::conditional_t<sizeof(T) == 4, uint32_t, uint16_t>;
template <typename T>
__device__ __forceinline__ tap_bits_t<T> load_tap_bits(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
    if constexpr (sizeof(T) == 4) return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
    else return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}
template <typename T>
__device__ __forceinline__ float tap_value(tap_bits_t<T> bits) {
    if constexpr (sizeof(T) == 4) return __uint_as_float(bits);
    else return __uint_as_float(static_cast<uint32_t>(bits) << 16);
}

// ------------------------------------------------ whole-plane vector I/O
// V consecutive elements at element e (a multiple of V) of a plane's buffer,
// as fp32; past the buffer's end they read 0 (the buffer's range check).
template <typename T, int V>
__device__ __forceinline__ void load_vec(__amdgpu_buffer_rsrc_t r, int e, float (&v)[V]) {
    constexpr int NB = V * static_cast<int>(sizeof(T));
    const uint32_t off = static_cast<uint32_t>(e) * sizeof(T);
    if constexpr (NB == 2) {
        v[0] = __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0)) << 16);
    } else {
        const words_t<NB / 4> wv = load_words<NB / 4>(r, off);
#pragma unroll
        for (int i = 0; i < NB / 4; ++i) {
            const uint32_t wd = word<NB / 4>(wv, i);
            if constexpr (sizeof(T) == 4) {
                v[i] = __uint_as_float(wd);
            } else {
                v[2 * i] = __uint_as_float(wd << 16);
                v[2 * i + 1] = __uint_as_float(wd & 0xffff0000u);
            }
        }
    }
}

// Stores V fp32 values as T at element e; stores past the end are dropped.
template <typename T, int V>
__device__ __forceinline__ void store_vec(__amdgpu_buffer_rsrc_t r, int e, const float (&v)[V]) {
    constexpr int NB = V * static_cast<int>(sizeof(T));
    const uint32_t off = static_cast<uint32_t>(e) * sizeof(T);
    if constexpr (NB == 2) {
        __builtin_amdgcn_raw_buffer_store_b16(bf16_rne(v[0]), r, off, 0, 0);
    } else {
        uint32_t wd[NB / 4];
#pragma unroll
        for (int i = 0; i < NB / 4; ++i)
            wd[i] = sizeof(T) == 4 ? __float_as_uint(v[i])
                                   : static_cast<uint32_t>(bf16_rne(v[2 * i])) |
                                         (static_cast<uint32_t>(bf16_rne(v[2 * i + 1])) << 16);
        if constexpr (NB == 4) {
            __builtin_amdgcn_raw_buffer_store_b32(wd[0], r, off, 0, 0);
        } else if constexpr (NB == 8) {
            const words_t<2> q = {wd[0], wd[1]};
            __builtin_amdgcn_raw_buffer_store_b64(q, r, off, 0, 0);
        } else {
            const words_t<4> q = {wd[0], wd[1], wd[2], wd[3]};
            __builtin_amdgcn_raw_buffer_store_b128(q, r, off, 0, 0);
        }
    }
}

// ------------------------------------------------ streaming forms (no LDS)
// A plane's lambda x need not sit in LDS when every lane reads its own
// slots' x, lambda and u and writes its own y: then a plane costs registers
// only, and every plane of a launch the size of latent1k is resident at
// once (the LDS form above holds seven 74 x 74 planes a CU).
//
// Row directions (top-down, bottom-up): the line is a row; lane q reads x,
// lambda, u (and y) of positions Kq .. Kq+K-1 of the row along with its
// taps, D rows ahead, and writes y of the row at its step.  Vec: the K
// elements of a lane are one aligned window (K divides the row and windows
// start on dwords), one load per tensor and row; else one load per slot.
//

template <typename T, int K>
__device__ __forceinline__ void tap_weights(const tap_bits_t<T> (&tb)[3][K], const float (&keep)[3][K],
                                            float eps, bool raw, float (&w0)[K], float (&w1)[K],
                                            float (&w2)[K]) {
    if (raw) {
        float r[K];
#pragma unroll
        for (int j = 0; j < K; ++j) {
            // a dropped tap's sigmoid is 0: exp2 of +inf
            const float z0 = keep[0][j] != 0.0f ? tap_value<T>(tb[0][j]) * kNegLog2e : __builtin_inff();
            const float z1 = keep[1][j] != 0.0f ? tap_value<T>(tb[1][j]) * kNegLog2e : __builtin_inff();
            const float z2 = keep[2][j] != 0.0f ? tap_value<T>(tb[2][j]) * kNegLog2e : __builtin_inff();
            w0[j] = __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(z0) + 1.0f);
            w1[j] = __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(z1) + 1.0f);
            w2[j] = __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(z2) + 1.0f);
            r[j] = __builtin_amdgcn_rcpf(fmaxf((w0[j] + w1[j]) + w2[j], eps));
        }
#pragma unroll
        for (int j = 0; j < K; ++j) {
            w0[j] *= r[j];
            w1[j] *= r[j];
            w2[j] *= r[j];
        }
    } else {
        // given weights; out-of-line taps weigh 0 whatever their value
#pragma unroll
        for (int j = 0; j < K; ++j) {
            w0[j] = keep[0][j] != 0.0f ? tap_value<T>(tb[0][j]) : 0.0f;
            w1[j] = keep[1][j] != 0.0f ? tap_value<T>(tb[1][j]) : 0.0f;
            w2[j] = keep[2][j] != 0.0f ? tap_value<T>(tb[2][j]) : 0.0f;
        }
    }
}

// Element e of a window of raw words as fp32.
template <typename T, int NW>
__device__ __forceinline__ float win_elem(const words_t<NW>& w, int e) {
    if constexpr (sizeof(T) == 4) {
        return __uint_as_float(word<NW>(w, e));
    } else {
        const uint32_t d = word<NW>(w, e >> 1);
        return __uint_as_float((e & 1) ? (d & 0xffff0000u) : (d << 16));
    }
}

// Packs fp32 values 2i, 2i+1 (bf16) or i (fp32) of v into dword i.
template <typename T, int N>
__device__ __forceinline__ uint32_t pack_word(const float (&v)[N], int i) {
    if constexpr (sizeof(T) == 4) return __float_as_uint(v[i]);
    else return static_cast<uint32_t>(bf16_rne(v[2 * i])) | (static_cast<uint32_t>(bf16_rne(v[2 * i + 1])) << 16);
}

template <typename T, int K, int D, bool Vec, bool Acc>
__global__ void __launch_bounds__(64)
scan_rows_kernel(const T* __restrict__ x, const T* __restrict__ lam, const T* __restrict__ u,
                 const T* __restrict__ w, int raw_i, float eps, T* __restrict__ y, int H, int W, int dir) {
    constexpr int ES = sizeof(T);
    static_assert(!Vec || (K * ES) % 4 == 0, "a window of whole dwords");
    constexpr int NWV = Vec ? (K * ES) / 4 : 1;       // dwords of a lane's window
    const bool raw = raw_i != 0;
    const int lane = threadIdx.x;
    const int HW = H * W;
    const size_t plane = blockIdx.x;
    const bool fwd = dir == 0;
    const int NL = H, L = W;
    auto rsrc = [&](const T* base, int n) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(base), 0, n * ES, kBufFlags);
    };
    const __amdgpu_buffer_rsrc_t xr = rsrc(x + plane * HW, HW), lr = rsrc(lam + plane * HW, HW),
                                 ur = rsrc(u + plane * HW, HW), yr = rsrc(y + plane * HW, HW),
                                 wr = rsrc(w + plane * 3 * static_cast<size_t>(HW), 3 * HW);
    bool valid[K];
    uint32_t voff[K];
    float keep[3][K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const int p = K * lane + j;
        valid[j] = p < L;
        voff[j] = static_cast<uint32_t>((valid[j] ? p : L - 1) * ES);
        keep[0][j] = (valid[j] && p > 0) ? 1.0f : 0.0f;
        keep[1][j] = valid[j] ? 1.0f : 0.0f;
        keep[2][j] = (valid[j] && p < L - 1) ? 1.0f : 0.0f;
    }
    // Vec: the lane's window (lanes past the row's end read the row's last
    // window; their values are not used)
    const uint32_t vwin = static_cast<uint32_t>((K * lane < L ? K * lane : L - K) * ES);
    tap_bits_t<T> tb[D][3][K];
    words_t<NWV> xw[D], lw[D], uw[D], yw[D];
    tap_bits_t<T> xe[D][K], le[D][K], ue[D][K], ye[D][K];
    const int line0 = fwd ? 0 : NL - 1;
    const int dline = fwd ? 1 : -1;
    auto load_line = [&](int d, int ln) {
        const int lc = ln < 0 ? 0 : (ln >= NL ? NL - 1 : ln);
        const int so = lc * L * ES;
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const int sk = (k * NL + lc) * L * ES;
#pragma unroll
            for (int j = 0; j < K; ++j) tb[d][k][j] = load_tap_bits<T>(wr, voff[j], sk);
        }
        if constexpr (Vec) {
            xw[d] = load_words_so<NWV>(xr, vwin, so);
            lw[d] = load_words_so<NWV>(lr, vwin, so);
            uw[d] = load_words_so<NWV>(ur, vwin, so);
            if constexpr (Acc) yw[d] = load_words_so<NWV>(yr, vwin, so);
        } else {
#pragma unroll
            for (int j = 0; j < K; ++j) {
                xe[d][j] = load_tap_bits<T>(xr, voff[j], so);
                le[d][j] = load_tap_bits<T>(lr, voff[j], so);
                ue[d][j] = load_tap_bits<T>(ur, voff[j], so);
                if constexpr (Acc) ye[d][j] = load_tap_bits<T>(yr, voff[j], so);
            }
        }
    };
#pragma unroll
    for (int d = 0; d < D; ++d) load_line(d, line0 + d * dline);

    float h[K];
#pragma unroll
    for (int j = 0; j < K; ++j) h[j] = 0.0f;

    auto step = [&](int s, int d) {
        const int ln = line0 + s * dline;
        float w0[K], w1[K], w2[K], b[K], uu[K], yo[K];
        tap_weights<T, K>(tb[d], keep, eps, raw, w0, w1, w2);
#pragma unroll
        for (int j = 0; j < K; ++j) {
            if constexpr (Vec) {
                b[j] = win_elem<T, NWV>(lw[d], j) * win_elem<T, NWV>(xw[d], j);
                uu[j] = win_elem<T, NWV>(uw[d], j);
                yo[j] = Acc ? win_elem<T, NWV>(yw[d], j) : 0.0f;
            } else {
                b[j] = tap_value<T>(le[d][j]) * tap_value<T>(xe[d][j]);
                uu[j] = tap_value<T>(ue[d][j]);
                yo[j] = Acc ? tap_value<T>(ye[d][j]) : 0.0f;
            }
        }
        load_line(d, ln + D * dline);
        const float hl0 = from_prev(h[K - 1]);
        const float hrK = from_next(h[0]);
        float hn[K], o[K];
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const float hl = j > 0 ? h[j - 1] : hl0;
            const float hr = j < K - 1 ? h[j + 1] : hrK;
            hn[j] = s == 0 ? b[j] : fmaf(w2[j], hr, fmaf(w0[j], hl, fmaf(w1[j], h[j], b[j])));
            hn[j] = valid[j] ? hn[j] : 0.0f;
            o[j] = Acc ? yo[j] + uu[j] * hn[j] : uu[j] * hn[j];
        }
#pragma unroll
        for (int j = 0; j < K; ++j) h[j] = hn[j];
        const int so = ln * L * ES;
        if constexpr (Vec) {
            if (valid[0]) {
                if constexpr (NWV == 1) {
                    __builtin_amdgcn_raw_buffer_store_b32(pack_word<T, K>(o, 0), yr, vwin, so, 0);
                } else if constexpr (NWV == 2) {
                    const words_t<2> v2 = {pack_word<T, K>(o, 0), pack_word<T, K>(o, 1)};
                    __builtin_amdgcn_raw_buffer_store_b64(v2, yr, vwin, so, 0);
                } else if constexpr (NWV == 3) {
                    const words_t<3> v3 = {pack_word<T, K>(o, 0), pack_word<T, K>(o, 1), pack_word<T, K>(o, 2)};
                    __builtin_amdgcn_raw_buffer_store_b96(v3, yr, vwin, so, 0);
                } else {
                    const words_t<4> v4 = {pack_word<T, K>(o, 0), pack_word<T, K>(o, 1), pack_word<T, K>(o, 2),
                                           pack_word<T, K>(o, 3)};
                    __builtin_amdgcn_raw_buffer_store_b128(v4, yr, vwin, so, 0);
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < K; ++j) {
                if (valid[j]) {
                    if constexpr (ES == 4)
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o[j]), yr, voff[j], so, 0);
                    else
                        __builtin_amdgcn_raw_buffer_store_b16(bf16_rne(o[j]), yr, voff[j], so, 0);
                }
            }
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

template <typename T, int K, int D, bool Vec>
hipError_t launch_rows(const void* x, const void* lam, const void* u, const void* w, int raw, float eps,
                       void* y, int accumulate, int64_t planes, int64_t H, int64_t W, int dir,
                       hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(planes)), block(64);
    if (accumulate)
        scan_rows_kernel<T, K, D, Vec, true><<<grid, block, 0, stream>>>(
            static_cast<const T*>(x), static_cast<const T*>(lam), static_cast<const T*>(u),
            static_cast<const T*>(w), raw, eps, static_cast<T*>(y), static_cast<int>(H), static_cast<int>(W), dir);
    else
        scan_rows_kernel<T, K, D, Vec, false><<<grid, block, 0, stream>>>(
            static_cast<const T*>(x), static_cast<const T*>(lam), static_cast<const T*>(u),
            static_cast<const T*>(w), raw, eps, static_cast<T*>(y), static_cast<int>(H), static_cast<int>(W), dir);
    return hipGetLastError();
}

// Row directions: K = ceil(W / 64) slots a lane; lines in flight sized so
// that a lane's loads in flight stay within the 63 its counter tracks.
template <typename T>
hipError_t launch_rows_t(const void* x, const void* lam, const void* u, const void* w, int raw, float eps,
                         void* y, int accumulate, int64_t planes, int64_t H, int64_t W, int dir,
                         hipStream_t stream) {
    constexpr int ES = sizeof(T);
    const int K = W <= 64 ? 1 : (W <= 128 ? 2 : (W <= 192 ? 3 : 4));
    const uintptr_t any = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(lam) |
                          reinterpret_cast<uintptr_t>(u) | reinterpret_cast<uintptr_t>(y);
    // whole-window loads: K divides the row, windows of whole dwords
    const bool vec = W % K == 0 && (K * ES) % 4 == 0 && (any & 3) == 0;
#define GSPN_ROWS(KK, DV, DE)                                                                            \
    if constexpr ((KK * ES) % 4 == 0) {                                                                  \
        if (vec) return launch_rows<T, KK, DV, true>(x, lam, u, w, raw, eps, y, accumulate, planes, H, W, dir, stream); \
    }                                                                                                    \
    return launch_rows<T, KK, DE, false>(x, lam, u, w, raw, eps, y, accumulate, planes, H, W, dir, stream)
    if (K == 1) { GSPN_ROWS(1, 8, 8); }
    if (K == 2) { GSPN_ROWS(2, 6, 4); }
    if (K == 3) { GSPN_ROWS(3, 4, 3); }
    GSPN_ROWS(4, 3, 2);
#undef GSPN_ROWS
}

// ------------------------------------------------ column strips
// Column directions stage lambda x one strip of columns at a time: SC
// columns (one 128-byte line of a row: 64 bf16 or 32 fp32), transposed, in
// an fp32 LDS buffer with column cc at float cc P and row r at + r (P odd,
// at least H: the fill's stores and the scan's reads spread over the banks).
template <typename T> constexpr int strip_cols() { return 128 / static_cast<int>(sizeof(T)); }

// b = lambda x of rows 0..H-1, columns c0 .. c0+SC-1 of the plane into the
// strip buffer; a lane moves V elements of a row (V divides W and c0), U
// loads a tensor in flight.  Columns past the row and rows past the plane
// read what the buffer holds there (0 past its end) and are not used.
template <typename T, int V>
__device__ __forceinline__ void strip_fill(__amdgpu_buffer_rsrc_t xr, __amdgpu_buffer_rsrc_t lr, int H, int W,
                                           int c0, int P) {
    constexpr int SC = strip_cols<T>();
    constexpr int CPR = SC / V;            // chunks a row
    constexpr int RPI = 64 / CPR;          // rows a load instruction
    constexpr int U = 32 / V < 16 ? 32 / V : 16;   // 32 elements a tensor in flight, 16 loads at most
    const int lane = threadIdx.x;
    const int ch = lane % CPR, rr = lane / CPR;
    for (int r0 = 0; r0 < H; r0 += RPI * U) {
        float xv[U][V], lv[U][V];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int e = (r0 + RPI * k + rr) * W + c0 + ch * V;
            load_vec<T, V>(xr, e, xv[k]);
            load_vec<T, V>(lr, e, lv[k]);
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int r = r0 + RPI * k + rr;
            if (r < H) {
#pragma unroll
                for (int i = 0; i < V; ++i)
                    lds_ref<float>(kPad + 4u * ((ch * V + i) * P + r)) = lv[k][i] * xv[k][i];
            }
        }
    }
}

// y = u h (or y += u h) of the strip's first ncols columns (a multiple of V).
template <typename T, int V>
__device__ __forceinline__ void strip_emit(__amdgpu_buffer_rsrc_t ur, __amdgpu_buffer_rsrc_t yr, int H, int W,
                                           int c0, int ncols, int P, bool accumulate) {
    constexpr int SC = strip_cols<T>();
    constexpr int CPR = SC / V;
    constexpr int RPI = 64 / CPR;
    constexpr int U = 32 / V < 16 ? 32 / V : 16;
    const int lane = threadIdx.x;
    const int ch = lane % CPR, rr = lane / CPR;
    const bool in_strip = ch * V < ncols;
    for (int r0 = 0; r0 < H; r0 += RPI * U) {
        float uv[U][V], yv[U][V];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int e = (r0 + RPI * k + rr) * W + c0 + ch * V;
            load_vec<T, V>(ur, e, uv[k]);
            if (accumulate) {
                load_vec<T, V>(yr, e, yv[k]);
            } else {
#pragma unroll
                for (int i = 0; i < V; ++i) yv[k][i] = 0.0f;
            }
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int r = r0 + RPI * k + rr;
            if (r < H && in_strip) {
                float o[V];
#pragma unroll
                for (int i = 0; i < V; ++i) {
                    const float t = uv[k][i] * lds_ref<float>(kPad + 4u * ((ch * V + i) * P + r));
                    o[i] = accumulate ? yv[k][i] + t : t;
                }
                store_vec<T, V>(yr, r * W + c0 + ch * V, o);
            }
        }
    }
}

// T: float or bf16 bits (uint16_t).  K: rows a lane (H up to 64 K).  D: lines
// of taps in flight.  RAW: taps are logits to normalise.  Fwd: left-right.
template <typename T, int K, int D, bool RAW, bool Fwd>
__global__ void __launch_bounds__(64)
scan_cols_kernel(const T* __restrict__ x, const T* __restrict__ lam, const T* __restrict__ u,
                 const T* __restrict__ w, float eps, T* __restrict__ y, int accumulate, int H, int W, int vec) {
    constexpr int ES = sizeof(T);
    constexpr int SC = strip_cols<T>();
    static_assert(SC % D == 0, "strips hold whole rounds of the tap ring");
    const int lane = threadIdx.x;
    const int HW = H * W;
    const size_t plane = blockIdx.x;
    const int NL = W, L = H;               // lines are columns, positions rows
    const int P = H | 1;                   // strip buffer pitch (floats), odd
    auto rsrc = [&](const T* base, int n) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(base), 0, n * ES, kBufFlags);
    };
    const __amdgpu_buffer_rsrc_t xr = rsrc(x + plane * HW, HW), lr = rsrc(lam + plane * HW, HW),
                                 ur = rsrc(u + plane * HW, HW), yr = rsrc(y + plane * HW, HW),
                                 wr = rsrc(w + plane * 3 * static_cast<size_t>(HW), 3 * HW);
    if (lane == 0) lds_ref<float>(0) = 0.0f;   // the dummy word of slots past a line's end

    bool valid[K];
    uint32_t voff[K];
    float keep[3][K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const int p = K * lane + j;
        valid[j] = p < L;
        voff[j] = static_cast<uint32_t>((valid[j] ? p : L - 1) * ES);
        keep[0][j] = (valid[j] && p > 0) ? 1.0f : 0.0f;
        keep[1][j] = valid[j] ? 1.0f : 0.0f;
        keep[2][j] = (valid[j] && p < L - 1) ? 1.0f : 0.0f;
    }
    // taps of step s: line (column) Fwd ? s : W - 1 - s, clamped into the plane
    tap_bits_t<T> tb[D][3][K];
    auto load_taps = [&](int d, int st) {
        int c = Fwd ? st : NL - 1 - st;
        c = c < 0 ? 0 : (c >= NL ? NL - 1 : c);
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const int sk = (k * NL + c) * L * ES;
#pragma unroll
            for (int j = 0; j < K; ++j) tb[d][k][j] = load_tap_bits<T>(wr, voff[j], sk);
        }
    };
#pragma unroll
    for (int d = 0; d < D; ++d) load_taps(d, d);

    float h[K], bv[K];
    uint32_t aS[K];
#pragma unroll
    for (int j = 0; j < K; ++j) h[j] = 0.0f;
    const int dS = Fwd ? 4 * P : -4 * P;   // LDS step from one column to the next scanned

    auto step = [&](int st, int d) {
        float w0[K], w1[K], w2[K];
        tap_weights<T, K>(tb[d], keep, eps, RAW, w0, w1, w2);
        load_taps(d, st + D);
        const float hl0 = from_prev(h[K - 1]);
        const float hrK = from_next(h[0]);
        float hn[K];
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const float hl = j > 0 ? h[j - 1] : hl0;
            const float hr = j < K - 1 ? h[j + 1] : hrK;
            // the first line has no line before it: h = lambda x
            hn[j] = st == 0 ? bv[j] : fmaf(w2[j], hr, fmaf(w0[j], hl, fmaf(w1[j], h[j], bv[j])));
            hn[j] = valid[j] ? hn[j] : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < K; ++j) {
            h[j] = hn[j];
            lds_ref<float>(aS[j]) = hn[j];
            aS[j] += valid[j] ? dS : 0;
            bv[j] = lds_ref<float>(aS[j]);   // the next column's b (read after this write)
        }
    };

    // strips in scan order, aligned to the scan's first column: full ones,
    // then a partial one
    const int nstrips = (NL + SC - 1) / SC;
    for (int ks = 0; ks < nstrips; ++ks) {
        const int s_begin = ks * SC;
        const int s_end = min(s_begin + SC, NL);
        const int ncols = s_end - s_begin;
        const int c0 = Fwd ? s_begin : NL - s_end;           // the strip's leftmost column
        if (vec == 1) strip_fill<T, 1>(xr, lr, H, W, c0, P);
        else if (vec == 2) strip_fill<T, 2>(xr, lr, H, W, c0, P);
        else if (sizeof(T) == 4 || vec == 4) strip_fill<T, 4>(xr, lr, H, W, c0, P);
        else strip_fill<T, 16 / ES>(xr, lr, H, W, c0, P);
        lds_order();
        const int cc0 = Fwd ? 0 : ncols - 1;                  // the strip column scanned first
#pragma unroll
        for (int j = 0; j < K; ++j) {
            aS[j] = valid[j] ? static_cast<uint32_t>(kPad + 4 * (cc0 * P + K * lane + j)) : 0u;
            bv[j] = lds_ref<float>(aS[j]);
        }
        int s0 = s_begin;
        for (; s0 + D <= s_end; s0 += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) step(s0 + d, d);
        }
#pragma unroll
        for (int d = 0; d < D; ++d)
            if (s0 + d < s_end) step(s0 + d, d);
        lds_order();
        const bool acc = accumulate != 0;
        if (vec == 1) strip_emit<T, 1>(ur, yr, H, W, c0, ncols, P, acc);
        else if (vec == 2) strip_emit<T, 2>(ur, yr, H, W, c0, ncols, P, acc);
        else if (sizeof(T) == 4 || vec == 4) strip_emit<T, 4>(ur, yr, H, W, c0, ncols, P, acc);
        else strip_emit<T, 16 / ES>(ur, yr, H, W, c0, ncols, P, acc);
        lds_order();
    }
}

size_t cols_lds_bytes(int64_t H, int64_t es) {
    return kPad + static_cast<size_t>(128 / es) * static_cast<size_t>(H | 1) * 4;
}

template <typename T, int K, bool RAW>
hipError_t launch_cols_k(const void* x, const void* lam, const void* u, const void* w, float eps,
                         void* y, int accumulate, int64_t planes, int64_t H, int64_t W, int dir,
                         hipStream_t stream) {
    // loads in flight (3 K D) stay within the 63 the wave's counter tracks
    constexpr int D = K <= 2 ? 8 : 4;
    const size_t lds = cols_lds_bytes(H, sizeof(T));
    // widest vector (up to 16 bytes) that divides the row and on which every
    // plane of x, lambda, u and y starts
    int vec = 16 / static_cast<int>(sizeof(T));
    const uintptr_t any = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(lam) |
                          reinterpret_cast<uintptr_t>(u) | reinterpret_cast<uintptr_t>(y);
    while (vec > 1 && (W % vec != 0 || (H * W) % vec != 0 || any % (vec * sizeof(T)) != 0)) vec /= 2;
    auto go = [&](auto kern) {
        if (lds > 64 * 1024) {
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
            if (e != hipSuccess) return e;
        }
        kern<<<dim3(static_cast<unsigned>(planes)), dim3(64), lds, stream>>>(
            static_cast<const T*>(x), static_cast<const T*>(lam), static_cast<const T*>(u),
            static_cast<const T*>(w), eps, static_cast<T*>(y), accumulate, static_cast<int>(H),
            static_cast<int>(W), vec);
        return hipGetLastError();
    };
    return dir == 2 ? go(scan_cols_kernel<T, K, D, RAW, true>) : go(scan_cols_kernel<T, K, D, RAW, false>);
}

template <typename T, bool RAW>
hipError_t launch_cols_t(const void* x, const void* lam, const void* u, const void* w, float eps,
                         void* y, int accumulate, int64_t planes, int64_t H, int64_t W, int dir,
                         hipStream_t stream) {
    if (H <= 64) return launch_cols_k<T, 1, RAW>(x, lam, u, w, eps, y, accumulate, planes, H, W, dir, stream);
    if (H <= 128) return launch_cols_k<T, 2, RAW>(x, lam, u, w, eps, y, accumulate, planes, H, W, dir, stream);
    if (H <= 192) return launch_cols_k<T, 3, RAW>(x, lam, u, w, eps, y, accumulate, planes, H, W, dir, stream);
    return launch_cols_k<T, 4, RAW>(x, lam, u, w, eps, y, accumulate, planes, H, W, dir, stream);
}

}  // namespace

bool scan_dir_fast_eligible(int64_t H, int64_t W, int dir) {
    // lines up to 256; the column form's strip buffer fits in LDS for any
    // such column
    return (dir < 2 ? W : H) <= 256;
}

hipError_t launch_scan_dir_fast(const void* x, const void* lam, const void* u, const void* w,
                                int w_is_raw, float eps, void* y, int accumulate, int dtype,
                                int64_t planes, int64_t H, int64_t W, int dir, hipStream_t stream) {
    if (dir < 2)
        return dtype == 0 ? launch_rows_t<float>(x, lam, u, w, w_is_raw, eps, y, accumulate, planes, H, W, dir, stream)
                          : launch_rows_t<uint16_t>(x, lam, u, w, w_is_raw, eps, y, accumulate, planes, H, W, dir,
                                                    stream);
    if (dtype == 0)
        return w_is_raw ? launch_cols_t<float, true>(x, lam, u, w, eps, y, accumulate, planes, H, W, dir, stream)
                        : launch_cols_t<float, false>(x, lam, u, w, eps, y, accumulate, planes, H, W, dir, stream);
    return w_is_raw ? launch_cols_t<uint16_t, true>(x, lam, u, w, eps, y, accumulate, planes, H, W, dir, stream)
                    : launch_cols_t<uint16_t, false>(x, lam, u, w, eps, y, accumulate, planes, H, W, dir, stream);
}

}  // namespace gspn
