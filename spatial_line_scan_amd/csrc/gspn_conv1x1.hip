// 1x1 convolutions of the latent sublayer on the matrix cores (gfx950, bf16
// storage, fp32 accumulation).  P_down (tokens to latent, inner dimension C)
// has a kernel of its own, described above pdown_kernel; the rest:
//
// "Scaling Parallel Sequence Models to Foundation-Scale Vision Encoders",
// §5.1 (propagation in a compressed latent); reading notes, key design 1: the
// propagation parameters (lambda, u, the raw taps) are per-position 1x1
// convolutions of the latent z, and P_up maps the scanned latent back to the
// token channels.  Each is a product out = Wm in with a short inner dimension
// K = Cc (the latent channels): Wm is [M][K] row-major, in is a batch of
// planar latents [B][K][N = H W].  Their time is the writing of the output,
// so the kernel is built around stores:
//   - a workgroup takes one batch entry and 128 consecutive positions; the
//     latent block [K][128] is staged once in LDS;
//   - each of the four wavefronts takes one 32-row weight tile per pass (128
//     output rows a pass, the next pass's weights loaded ahead) against all
//     four 32-position tiles (v_mfma_f32_32x32x16_bf16; the weights come from
//     L2, the position operands stay in registers);
//   - a pass is staged in LDS as bf16 and written back in long contiguous
//     runs whose row (or token) is uniform across a wavefront.
// Two output forms:
//   kRowMajor   out[seg][b][m][p]   (p = position in the input's order):
//               lambda, u and the row scans' taps from z; the column scans'
//               taps, which the scan kernels read column-major, from the
//               transposed latent zt (transpose_plane_kernel);
//   kTokenMajor y[b][p][m]          (P_up, to the token layout).
// Every output element is one fp32 dot product of length K rounded once to
// bf16 (round to nearest even), in a fixed order, so repeated calls are
// bitwise equal.
#include "gspn_device.h"
#include "gspn_internal.h"
#include "gspn_lane.h"

namespace gspn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

enum { kRowMajor = 0, kTokenMajor = 1 };

constexpr int kMaxK = 64;
constexpr int kP = 128;                 // positions per workgroup
constexpr int kPT = kP / 32;            // position tiles
constexpr int kMC = 128;                // output rows per pass: one 32-row tile per wavefront
// LDS pitches in halves: the +8 keeps rows 16-byte aligned and puts the two
// lane halves of an operand read (8 k rows apart) on other banks.
constexpr int kPitchIn = kP + 8;
constexpr int kPitchOut = kP + 8;       // [kMC rows][kP] or [kP tokens][kMC]
constexpr int kMaxSide = 96;            // transpose_plane_kernel's LDS plane

size_t lds_bytes(int K) {
    return static_cast<size_t>((K + 15) & ~15) * kPitchIn * 2 + static_cast<size_t>(kMC) * kPitchOut * 2;
}

// Workgroup barrier that orders LDS only: the staged blocks are exchanged
// through LDS, and the global stores of one pass stay in flight while the
// next pass computes (a full __syncthreads would wait for them).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Work item of a block: blocks are dealt to the XCDs in turn, so block i
// takes item (i % 8) per + i / 8 and each XCD gets a run of consecutive
// items (neighbouring position runs, whose output rows share cache lines,
// meet in one L2).  Returns -1 for the few blocks past the last item.
__device__ __forceinline__ int xcd_item(int total) {
    const int id = blockIdx.x;
    const int per = (total + 7) / 8;
    const int item = (id & 7) * per + (id >> 3);
    return item < total ? item : -1;
}

// Output segments of the row-major form: rows [start[s], start[s + 1]) of Wm
// go to base[s] + b bstride[s] + (m - start[s]) N.
struct Segs {
    int start[5];
    uint16_t* base[4];
    int64_t bstride[4];
};

template <int Mode>
__global__ void __launch_bounds__(256)
conv1x1_kernel(const uint16_t* __restrict__ in, int in_bytes, const uint16_t* __restrict__ wm,
               int M, int K, int N, int tiles, int items, Segs segs, uint16_t* __restrict__ yt) {
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    const int item = xcd_item(items);
    if (item < 0) return;                       // whole block: no barrier is left half-reached
    const int b = item / tiles;
    const int o0 = (item - b * tiles) * kP;     // positions o0 .. o0 + Pe - 1
    const int Pe = N - o0 < kP ? N - o0 : kP;   // a multiple of 4 (N % 4 == 0)
    const int tid = threadIdx.x;
    const int Kp = (K + 15) & ~15;
    uint16_t* stage_in = lds;
    uint16_t* stage_out = lds + static_cast<size_t>(Kp) * kPitchIn;

    // ---- stage in[b][0..K)[o0 ..] into LDS [k][p], zero past K and Pe; the
    // loads of a batch are issued before its LDS writes
    {
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(in), 0, in_bytes, lane::kBufFlags);
        constexpr int C8 = kP / 8;             // 16-byte chunks of a k row
        const int total = Kp * C8;
        for (int f0 = 0; f0 < total; f0 += 4 * 256) {
            u32x4_t v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int f = f0 + 256 * j + tid;
                const int k = f / C8, c = f % C8;
                v[j] = u32x4_t{0u, 0u, 0u, 0u};
                // a chunk that runs past Pe picks up the next row's values:
                // those positions' outputs are never written
                if (f < total && k < K && 8 * c < Pe) {
                    const int64_t e = static_cast<int64_t>(b * K + k) * N + o0 + 8 * c;
                    v[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, static_cast<uint32_t>(2 * e), 0, 0);
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int f = f0 + 256 * j + tid;
                if (f < total)
                    *reinterpret_cast<u32x4_t*>(&stage_in[(f / C8) * kPitchIn + 8 * (f % C8)]) = v[j];
            }
        }
    }
    lds_barrier();

    const int l = tid & 63;
    const int wave = tid >> 6;
    const int q = l & 31, hk = l >> 5;
    const int ks = Kp / 16;

    // position operands: position 32 pt + q, k = 16 s + 8 hk .. + 7
    bf16x8_t pos_op[kPT][kMaxK / 16];
#pragma unroll
    for (int pt = 0; pt < kPT; ++pt) {
#pragma unroll
        for (int s = 0; s < kMaxK / 16; ++s) {
            if (s < ks) {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    pos_op[pt][s][i] = __builtin_bit_cast(
                        __bf16, stage_in[(16 * s + 8 * hk + i) * kPitchIn + 32 * pt + q]);
            }
        }
    }

    // weight operand of this wavefront's tile in the pass at row mc0: row
    // mc0 + 32 wave + q, k = 16 s + 8 hk .. + 7 (zero past M or K)
    auto load_w = [&](int mc0, u32x4_t* w) {
        const int mw = mc0 + 32 * wave + q;
#pragma unroll
        for (int s = 0; s < kMaxK / 16; ++s) {
            w[s] = u32x4_t{0u, 0u, 0u, 0u};
            const int k = 16 * s + 8 * hk;
            if (s < ks && mw < M && k < K)
                w[s] = *reinterpret_cast<const u32x4_t*>(wm + static_cast<int64_t>(mw) * K + k);
        }
    };
    u32x4_t wcur[kMaxK / 16], wnext[kMaxK / 16];
    load_w(0, wcur);

    for (int mc0 = 0; mc0 < M; mc0 += kMC) {
        load_w(mc0 + kMC, wnext);
        if (mc0 + 32 * wave < M) {
#pragma unroll
            for (int pt = 0; pt < kPT; ++pt) {
                if (32 * pt >= Pe) break;
                f32x16_t acc = {};
#pragma unroll
                for (int s = 0; s < kMaxK / 16; ++s) {
                    if (s < ks) {
                        const bf16x8_t wop = __builtin_bit_cast(bf16x8_t, wcur[s]);
                        if constexpr (Mode == kTokenMajor)
                            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wop, pos_op[pt][s], acc, 0, 0, 0);
                        else
                            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pos_op[pt][s], wop, acc, 0, 0, 0);
                    }
                }
                // D row 8 g + 4 hk + r, column q: four consecutive D rows per
                // lane and g, contiguous in the staged block
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const u32x2_t v = {lane::pack_bf16x2(acc[4 * g], acc[4 * g + 1]),
                                       lane::pack_bf16x2(acc[4 * g + 2], acc[4 * g + 3])};
                    const int drow = 8 * g + 4 * hk;
                    if constexpr (Mode == kTokenMajor)
                        *reinterpret_cast<u32x2_t*>(&stage_out[(32 * pt + q) * kPitchOut + 32 * wave + drow]) = v;
                    else
                        *reinterpret_cast<u32x2_t*>(&stage_out[(32 * wave + q) * kPitchOut + 32 * pt + drow]) = v;
                }
            }
        }
#pragma unroll
        for (int s = 0; s < kMaxK / 16; ++s) wcur[s] = wnext[s];
        lds_barrier();

        // ---- write the staged block in long contiguous runs; the row (or
        // token) of each store is wave-uniform, so its address is scalar work
        const int rows = M - mc0 < kMC ? M - mc0 : kMC;
        if constexpr (Mode == kTokenMajor) {
            // four tokens per wavefront and step, 16 lanes a token: 16 bytes a
            // lane (M % 8 == 0), else 8 bytes a lane in two halves (M % 4 == 0)
            const int tl = l >> 4, c = l & 15;
            for (int t4 = 4 * wave; t4 < Pe; t4 += 16) {
                const int tt = t4 + tl;
                uint16_t* row = yt + (static_cast<int64_t>(b) * N + o0 + tt) * M + mc0;
                if (M % 8 == 0) {
                    if (tt < Pe && 8 * c < rows)
                        *reinterpret_cast<u32x4_t*>(row + 8 * c) =
                            *reinterpret_cast<const u32x4_t*>(&stage_out[tt * kPitchOut + 8 * c]);
                } else {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int cc = c + 16 * h;
                        if (tt < Pe && 4 * cc < rows)
                            *reinterpret_cast<u32x2_t*>(row + 4 * cc) =
                                *reinterpret_cast<const u32x2_t*>(&stage_out[tt * kPitchOut + 4 * cc]);
                    }
                }
            }
        } else {
            // two rows per wavefront and step, 32 lanes a row, 8 bytes a lane
            const int half = l >> 5, c = l & 31;
            for (int r2 = 2 * wave; r2 < rows; r2 += 8) {
                const int r = r2 + half;
                const int m = mc0 + r;
                const int sg = (m >= segs.start[1]) + (m >= segs.start[2]) + (m >= segs.start[3]);
                if (r < rows && 4 * c < Pe) {
                    uint16_t* dst = segs.base[sg] + b * segs.bstride[sg] +
                                    static_cast<int64_t>(m - segs.start[sg]) * N + o0 + 4 * c;
                    *reinterpret_cast<u32x2_t*>(dst) =
                        *reinterpret_cast<const u32x2_t*>(&stage_out[r * kPitchOut + 4 * c]);
                }
            }
        }
        lds_barrier();
    }
}

// zt[p][x H + y] = z[p][y W + x] for every plane p of H x W <= 96 x 96
// (H W % 4 == 0): the plane is staged whole in LDS; reads and writes are
// contiguous 8-byte accesses.
__global__ void __launch_bounds__(256)
transpose_plane_kernel(const uint16_t* __restrict__ z, uint16_t* __restrict__ zt, int H, int W) {
    __shared__ __attribute__((aligned(16))) uint16_t pl[kMaxSide * kMaxSide];
    const int N = H * W;
    const int units = N / 4;
    const size_t base = static_cast<size_t>(blockIdx.x) * N;
    const u32x2_t* src = reinterpret_cast<const u32x2_t*>(z + base);
    for (int f0 = 0; f0 < units; f0 += 8 * 256) {
        u32x2_t v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int f = f0 + 256 * j + threadIdx.x;
            if (f < units) v[j] = src[f];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int f = f0 + 256 * j + threadIdx.x;
            if (f < units) *reinterpret_cast<u32x2_t*>(&pl[4 * f]) = v[j];
        }
    }
    lds_barrier();
    u32x2_t* dst = reinterpret_cast<u32x2_t*>(zt + base);
    for (int f = threadIdx.x; f < units; f += 256) {
        int x = (4 * f) / H, y = 4 * f - x * H;
        uint32_t v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = pl[y * W + x];
            const bool wrap = y + 1 == H;
            y = wrap ? 0 : y + 1;
            x = wrap ? x + 1 : x;
        }
        dst[f] = u32x2_t{v[0] | (v[1] << 16), v[2] | (v[3] << 16)};
    }
}

// P_down: z[b][ch][n] = sum_c p_down[ch][c] x[b][n][c] for the tokens of the
// whole batch, t = b N + n (token-major input, C channels contiguous; planar
// latent output).  Its time is the reading of the tokens (404 MB at the 1K
// shape against 22 MB written and about 26 GFLOP), so the kernel is built
// to read them as a plain copy would:
//   - a workgroup of 8 wavefronts takes 32-token tiles blockIdx.x,
//     blockIdx.x + gridDim.x, ...; a tile is one contiguous block of 64 C
//     bytes, which the workgroup reads with consecutive 16-byte loads (a
//     tile ahead, into registers) and writes into LDS, token rows padded to
//     2 C + 16 bytes;
//   - wavefront w multiplies channels C w / 8 .. C (w + 1) / 8 of the tile: in
//     k-step s (KS = C / 128 of them, v_mfma_f32_32x32x16_bf16) lane (q, h)
//     reads channels C w / 8 + 16 s + 8 h .. + 7 of token q from LDS, and its
//     p_down operands, the same channels of latent channel 32 nt + q, stay in
//     registers;
//   - each wavefront's 32 x Cc partial sums go to LDS, and the workgroup adds
//     the 8 partials of each output in wavefront order and writes four
//     consecutive tokens of a channel a thread (8-byte stores; N % 4 == 0, so
//     they never straddle two images).
// Every output is one fp32 sum in a fixed order, rounded once to bf16, so
// repeated calls are bitwise equal.
constexpr int kDownWaves = 8;
constexpr int kDownPitch = 36;          // floats a channel row of a partial (32 tokens + pad)

template <int NT, int KS>
__global__ void __launch_bounds__(64 * kDownWaves)
pdown_kernel(const uint16_t* __restrict__ x, int x_bytes, const uint16_t* __restrict__ pd,
             uint16_t* __restrict__ z, int N, int tokens, int tiles) {
    extern __shared__ __attribute__((aligned(16))) u32x4_t lds4[];
    constexpr int C = 128 * KS;
    constexpr int CC = 32 * NT;
    constexpr int ROW = C / 8 + 1;                 // 16-byte units a padded token row
    constexpr int UNITS = 32 * C / 8;              // 16-byte units of a tile
    constexpr int PER = (UNITS + 64 * kDownWaves - 1) / (64 * kDownWaves);   // a thread's loads
    constexpr int PW = CC * kDownPitch;            // floats of one wavefront's partial
    u32x4_t* tile_lds = lds4;                      // [32][ROW]
    float* part = reinterpret_cast<float*>(lds4 + 32 * ROW);   // [8 waves][CC][kDownPitch]
    const int tid = threadIdx.x;
    const int l = tid & 63, w = tid >> 6;
    const int q = l & 31, hk = l >> 5;
    const int u0 = 2 * KS * w + hk;                // 16-byte unit of this lane's k-step 0 in a row

    // p_down operands of this wavefront: latent channel 32 nt + q, k-step s
    u32x4_t bw[NT][KS];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int s4 = 0; s4 < KS; ++s4)
            bw[nt][s4] = *reinterpret_cast<const u32x4_t*>(pd + static_cast<int64_t>(32 * nt + q) * C + 8 * (u0 + 2 * s4));

    const __amdgpu_buffer_rsrc_t xs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), 0, x_bytes, lane::kBufFlags);
    // unit f = tid + 512 k of tile t; tiles past the last read past the buffer
    // (which ends below 2^31 bytes): zeros, never used
    u32x4_t tv[PER];
    auto issue = [&](int t) {
        const uint32_t base = t < tiles ? static_cast<uint32_t>(t) * (64u * C) : 0x80000000u;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int f = tid + 64 * kDownWaves * k;
            tv[k] = (UNITS % (64 * kDownWaves) == 0 || f < UNITS)
                        ? __builtin_amdgcn_raw_buffer_load_b128(xs, base + 16u * static_cast<uint32_t>(f), 0, 0)
                        : u32x4_t{0u, 0u, 0u, 0u};
        }
    };
    const int G = static_cast<int>(gridDim.x);
    int t = static_cast<int>(blockIdx.x);
    issue(t);
    for (; t < tiles; t += G) {
        // every thread has read the previous tile's operands and partials
        __syncthreads();
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int f = tid + 64 * kDownWaves * k;
            if (UNITS % (64 * kDownWaves) == 0 || f < UNITS) tile_lds[(f / (C / 8)) * ROW + f % (C / 8)] = tv[k];
        }
        issue(t + G);
        __syncthreads();
        f32x16_t acc[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x16_t{};
#pragma unroll
        for (int s4 = 0; s4 < KS; ++s4) {
            const u32x4_t a = tile_lds[q * ROW + u0 + 2 * s4];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                                  __builtin_bit_cast(bf16x8_t, bw[nt][s4]),
                                                                  acc[nt], 0, 0, 0);
        }
        // D row 8 g + 4 hk + r (token), column q (latent channel 32 nt + q)
        float* mine = part + w * PW;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *reinterpret_cast<f32x4_t*>(mine + (32 * nt + q) * kDownPitch + 8 * g + 4 * hk) =
                    f32x4_t{acc[nt][4 * g], acc[nt][4 * g + 1], acc[nt][4 * g + 2], acc[nt][4 * g + 3]};
        __syncthreads();
        // outputs: channel ch = i / 8, tokens 4 (i % 8) .. + 3 of the tile
        for (int i = tid; i < CC * 8; i += 64 * kDownWaves) {
            const int ch = i >> 3, j = i & 7;
            f32x4_t v = *reinterpret_cast<const f32x4_t*>(part + ch * kDownPitch + 4 * j);
#pragma unroll
            for (int ww = 1; ww < kDownWaves; ++ww)
                v += *reinterpret_cast<const f32x4_t*>(part + ww * PW + ch * kDownPitch + 4 * j);
            const int tk = 32 * t + 4 * j;
            if (tk < tokens) {
                const int b = tk / N, n = tk - b * N;
                *reinterpret_cast<u32x2_t*>(z + (static_cast<int64_t>(b) * CC + ch) * N + n) =
                    u32x2_t{lane::pack_bf16x2(v[0], v[1]), lane::pack_bf16x2(v[2], v[3])};
            }
        }
    }
}

// LDS of the P_down kernel: the padded tile and the wavefronts' partials.
size_t pdown_lds_bytes(int64_t C, int64_t Cc) {
    return static_cast<size_t>(32 * (C / 8 + 1)) * 16 + static_cast<size_t>(kDownWaves) * Cc * kDownPitch * 4;
}

template <int Mode>
hipError_t launch(const void* in, int64_t B, int64_t K, int64_t N, const void* wm, int64_t M,
                  const Segs& segs, void* yt, hipStream_t stream) {
    const int64_t tiles = (N + kP - 1) / kP;
    const int64_t items = B * tiles;
    const size_t lds = lds_bytes(static_cast<int>(K));
    auto kern = conv1x1_kernel<Mode>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(lds));
        if (e != hipSuccess) return e;
    }
    kern<<<dim3(static_cast<unsigned>((items + 7) / 8 * 8)), dim3(256), lds, stream>>>(
        static_cast<const uint16_t*>(in), static_cast<int>(B * K * N * 2),
        static_cast<const uint16_t*>(wm), static_cast<int>(M), static_cast<int>(K),
        static_cast<int>(N), static_cast<int>(tiles), static_cast<int>(items), segs,
        static_cast<uint16_t*>(yt));
    return hipGetLastError();
}

Segs make_segs(int n, const int64_t* start, void* const* base, const int64_t* bstride) {
    Segs s;
    for (int i = 0; i < 5; ++i) s.start[i] = i < n ? static_cast<int>(start[i]) : 0x7fffffff;
    for (int i = 0; i < 4; ++i) {
        s.base[i] = i < n ? static_cast<uint16_t*>(base[i]) : nullptr;
        s.bstride[i] = i < n ? bstride[i] : 0;
    }
    return s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// P_down instances: k-steps a lane KS = C / 128 up to 10 (C up to 1280), Cc
// of 64 (two 32-channel tiles) or 32
constexpr int kMaxDownKS = 10;

template <int NT, int KS = 1, typename Go>
hipError_t dispatch_down_ks(Go& go, int ks) {
    if constexpr (KS > kMaxDownKS) {
        return hipErrorInvalidValue;
    } else {
        if (ks == KS) return go(pdown_kernel<NT, KS>);
        return dispatch_down_ks<NT, KS + 1>(go, ks);
    }
}

template <typename Go>
hipError_t dispatch_down(Go& go, bool two, int ks) {
    return two ? dispatch_down_ks<2>(go, ks) : dispatch_down_ks<1>(go, ks);
}

}  // namespace

bool conv1x1_eligible(int dtype, int64_t B, int64_t K, int64_t H, int64_t W, int64_t C) {
    const int64_t N = H * W;
    return dtype == 1 && K >= 8 && K <= kMaxK && K % 8 == 0 && N % 4 == 0 && H <= kMaxSide &&
           W <= kMaxSide && C % 4 == 0 && B * ((N + kP - 1) / kP) + 8 <= 0x7fffffff &&
           B * K * N * 2 <= 0x7fffffff && B * N * C <= (1ll << 40);
}

hipError_t launch_conv1x1_params(const void* z, void* zt, const void* w_param, int64_t B,
                                 int64_t Cc, int64_t G, int64_t H, int64_t W, void* lam, void* u,
                                 void* const* taps4, hipStream_t stream) {
    if (!aligned16(w_param) || !aligned16(z) || !aligned16(zt)) return hipErrorInvalidValue;
    const int64_t N = H * W;
    const int64_t tg = 3 * G;
    // lambda, u and the row scans' taps: rows 0 .. 2 Cc + 6 G of w_param on z
    {
        const int64_t start[5] = {0, Cc, 2 * Cc, 2 * Cc + tg, 2 * Cc + 2 * tg};
        void* const base[4] = {lam, u, taps4[0], taps4[1]};
        const int64_t bs[4] = {Cc * N, Cc * N, tg * N, tg * N};
        hipError_t e = launch<kRowMajor>(z, B, Cc, N, w_param, 2 * Cc + 2 * tg,
                                         make_segs(4, start, base, bs), nullptr, stream);
        if (e != hipSuccess) return e;
    }
    // the column scans' taps: the same product on the transposed latent, so
    // they come out column-major
    transpose_plane_kernel<<<dim3(static_cast<unsigned>(B * Cc)), dim3(256), 0, stream>>>(
        static_cast<const uint16_t*>(z), static_cast<uint16_t*>(zt), static_cast<int>(H),
        static_cast<int>(W));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const uint16_t* wcol = static_cast<const uint16_t*>(w_param) + (2 * Cc + 2 * tg) * Cc;
    const int64_t start[5] = {0, tg, 2 * tg, 0, 0};
    void* const base[4] = {taps4[2], taps4[3], nullptr, nullptr};
    const int64_t bs[4] = {tg * N, tg * N, 0, 0};
    return launch<kRowMajor>(zt, B, Cc, N, wcol, 2 * tg, make_segs(2, start, base, bs), nullptr,
                             stream);
}

bool conv1x1_down_eligible(int dtype, int64_t B, int64_t Cc, int64_t H, int64_t W, int64_t C) {
    const int64_t N = H * W;
    return dtype == 1 && (Cc == 32 || Cc == 64) && C % 128 == 0 && C >= 128 && C <= 128 * kMaxDownKS &&
           N % 4 == 0 && B * N * C * 2 + 64 <= 0x7fffffff &&
           static_cast<int64_t>(pdown_lds_bytes(C, Cc)) <= kLdsBytes;
}

hipError_t launch_conv1x1_down(const void* x_tok, const void* p_down, int64_t B, int64_t C,
                               int64_t Cc, int64_t H, int64_t W, void* z, hipStream_t stream) {
    if (!aligned16(p_down) || !aligned16(x_tok) || !aligned16(z)) return hipErrorInvalidValue;
    const int64_t N = H * W;
    const int64_t tokens = B * N;
    const int64_t tiles = (tokens + 31) / 32;
    const size_t lds = pdown_lds_bytes(C, Cc);
    int cus = 1;
    hipError_t e = device_cu_count(&cus);
    if (e != hipSuccess) return e;
    const int64_t grid = tiles < cus ? tiles : cus;
    auto go = [&](auto kern) -> hipError_t {
        if (lds > 64 * 1024) {
            const hipError_t fe = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                      hipFuncAttributeMaxDynamicSharedMemorySize,
                                                      static_cast<int>(lds));
            if (fe != hipSuccess) return fe;
        }
        kern<<<dim3(static_cast<unsigned>(grid)), dim3(64 * kDownWaves), lds, stream>>>(
            static_cast<const uint16_t*>(x_tok), static_cast<int>(tokens * C * 2),
            static_cast<const uint16_t*>(p_down), static_cast<uint16_t*>(z), static_cast<int>(N),
            static_cast<int>(tokens), static_cast<int>(tiles));
        return hipGetLastError();
    };
    return dispatch_down(go, Cc == 64, static_cast<int>(C / 128));
}

hipError_t launch_conv1x1_up(const void* yc, const void* p_up, int64_t B, int64_t Cc, int64_t C,
                             int64_t H, int64_t W, void* y_tok, hipStream_t stream) {
    if (!aligned16(p_up) || !aligned16(yc) || !aligned16(y_tok)) return hipErrorInvalidValue;
    const int64_t none[5] = {0, 0, 0, 0, 0};
    void* const nb[4] = {nullptr, nullptr, nullptr, nullptr};
    return launch<kTokenMajor>(yc, B, Cc, H * W, p_up, C, make_segs(0, none, nb, none), y_tok,
                               stream);
}

}  // namespace gspn
