// Latent-space propagation sublayer around the four-direction scan (gfx950).
//
// "Scaling Parallel Sequence Models to Foundation-Scale Vision Encoders",
// §5.1 (a more efficient ViT block: propagation in a compressed latent); the
// reading notes, key design 1: a per-position 1x1 convolution P_down maps the
// C token channels to Cc latent channels, the propagation parameters (lambda,
// u and the raw taps) are per-position 1x1 convolutions of the latent, the
// four-direction scan runs on the Cc channels, and P_up maps back to C.
//
// Data flow (one call, all on one stream; bf16 or fp32 storage, fp32
// accumulation everywhere):
//   tokens x [B][N = H W][C]
//     --GEMM (P_down)-->          z [B][Cc][H][W]          (latent planes)
//     --transpose each plane-->   zt [B][Cc][W][H]         (column-major copy)
//     --GEMM (lambda rows)-->     lambda [B][Cc][H][W]
//     --GEMM (u rows)-->          u [B][Cc][H][W]
//     --GEMM (tap rows, TD, BU from z; LR, RL from zt)--> taps [4][B][G][3][..]
//        (the column scans' tap planes come out column-major, as the scan
//        kernels read them, because their GEMM reads the transposed latent)
//     --four-direction scan-->    yc [B][Cc][H][W]
//     --GEMM (P_up)-->            tokens y [B][N][C]
// The 1x1 convolutions are plain GEMMs: in bf16 they run on this library's
// matrix-core kernels where the shape fits them (gspn_conv1x1.hip), else in
// hipBLASLt; the scan and the transposes are this library's kernels.  Every
// intermediate lives in the caller's workspace.
#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

#include "gspn_device.h"
#include "gspn_internal.h"

namespace gspn {
namespace {

constexpr int kTile = 64;
constexpr int64_t kBlasWorkspace = 32ll << 20;   // hipBLASLt scratch inside the workspace
constexpr int64_t kAlign = 256;

int64_t align_up(int64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Plane transpose [H][W] -> [W][H] through a 64 x 64 LDS tile; block
// (plane, tile) = blockIdx.x, one plane's tiles consecutive.
template <typename T>
__global__ void __launch_bounds__(256)
transpose_planes_kernel(const T* __restrict__ src, T* __restrict__ dst, int H, int W,
                        int tiles_w, int tiles_per_plane) {
    __shared__ float tile[kTile][kTile + 1];
    const size_t plane = blockIdx.x / tiles_per_plane;
    const int t = blockIdx.x - static_cast<int>(plane) * tiles_per_plane;
    const int r0 = (t / tiles_w) * kTile;
    const int c0 = (t % tiles_w) * kTile;
    const size_t npix = static_cast<size_t>(H) * W;
    const T* s = src + plane * npix;
    T* d = dst + plane * npix;
    for (int e = threadIdx.x; e < kTile * kTile; e += 256) {
        const int i = e / kTile, j = e % kTile;          // coalesced along the source row
        const int r = r0 + i, c = c0 + j;
        if (r < H && c < W) tile[i][j] = load_elem(s, static_cast<size_t>(r) * W + c);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < kTile * kTile; e += 256) {
        const int j = e / kTile, i = e % kTile;          // coalesced along the destination row
        const int r = r0 + i, c = c0 + j;
        if (r < H && c < W) store_elem(d, static_cast<size_t>(c) * H + r, tile[i][j]);
    }
}

// ------------------------------------------------------------------ hipBLASLt

// One strided-batched product D = op(A) op(B), column-major, D m x n.
struct GemmShape {
    hipblasOperation_t ta, tb;
    int64_t m, n, k, lda, ldb, ldd, sa, sb, sd;
    int batch;
    auto key(int dt) const {
        return std::make_tuple(dt, static_cast<int>(ta), static_cast<int>(tb), m, n, k, lda, ldb,
                               ldd, sa, sb, sd, batch);
    }
};

std::mutex g_mu;
std::map<int, hipblasLtHandle_t> g_handles;
std::map<std::tuple<int, int, int, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t,
                    int64_t, int64_t, int>,
         hipblasLtMatmulAlgo_t>
    g_algos;

hipError_t blas_error(hipblasStatus_t s) {
    return s == HIPBLAS_STATUS_SUCCESS ? hipSuccess : hipErrorUnknown;
}

// Layout descriptor of a rows x cols column-major operand with batch strides.
hipblasStatus_t make_layout(hipblasLtMatrixLayout_t* l, hipDataType dt, int64_t rows,
                            int64_t cols, int64_t ld, int batch, int64_t stride) {
    hipblasStatus_t s = hipblasLtMatrixLayoutCreate(l, dt, rows, cols, ld);
    if (s != HIPBLAS_STATUS_SUCCESS) return s;
    int32_t b = batch;
    s = hipblasLtMatrixLayoutSetAttribute(*l, HIPBLASLT_MATRIX_LAYOUT_BATCH_COUNT, &b, sizeof(b));
    if (s != HIPBLAS_STATUS_SUCCESS) return s;
    return hipblasLtMatrixLayoutSetAttribute(*l, HIPBLASLT_MATRIX_LAYOUT_STRIDED_BATCH_OFFSET,
                                             &stride, sizeof(stride));
}

hipError_t gemm(int dtype, const GemmShape& g, const void* A, const void* B, void* D, void* ws,
                hipStream_t stream) {
    int dev = 0;
    hipError_t he = hipGetDevice(&dev);
    if (he != hipSuccess) return he;
    const hipDataType dt = dtype == 0 ? HIP_R_32F : HIP_R_16BF;
    hipblasLtHandle_t h;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        auto it = g_handles.find(dev);
        if (it == g_handles.end()) {
            hipblasLtHandle_t nh;
            hipblasStatus_t s = hipblasLtCreate(&nh);
            if (s != HIPBLAS_STATUS_SUCCESS) return blas_error(s);
            it = g_handles.emplace(dev, nh).first;
        }
        h = it->second;
    }
    hipblasLtMatmulDesc_t desc = nullptr;
    hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, ld = nullptr;
    hipblasLtMatmulPreference_t pref = nullptr;
    hipblasStatus_t s = hipblasLtMatmulDescCreate(&desc, HIPBLAS_COMPUTE_32F, HIP_R_32F);
    auto cleanup = [&]() {
        if (pref) hipblasLtMatmulPreferenceDestroy(pref);
        if (la) hipblasLtMatrixLayoutDestroy(la);
        if (lb) hipblasLtMatrixLayoutDestroy(lb);
        if (ld) hipblasLtMatrixLayoutDestroy(ld);
        if (desc) hipblasLtMatmulDescDestroy(desc);
    };
    const int32_t ta = g.ta, tb = g.tb;
    if (s == HIPBLAS_STATUS_SUCCESS)
        s = hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof(ta));
    if (s == HIPBLAS_STATUS_SUCCESS)
        s = hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof(tb));
    const bool na = g.ta == HIPBLAS_OP_N, nb = g.tb == HIPBLAS_OP_N;
    if (s == HIPBLAS_STATUS_SUCCESS)
        s = make_layout(&la, dt, na ? g.m : g.k, na ? g.k : g.m, g.lda, g.batch, g.sa);
    if (s == HIPBLAS_STATUS_SUCCESS)
        s = make_layout(&lb, dt, nb ? g.k : g.n, nb ? g.n : g.k, g.ldb, g.batch, g.sb);
    if (s == HIPBLAS_STATUS_SUCCESS) s = make_layout(&ld, dt, g.m, g.n, g.ldd, g.batch, g.sd);
    if (s != HIPBLAS_STATUS_SUCCESS) {
        cleanup();
        return blas_error(s);
    }
    // One algorithm per shape: the heuristic's first candidate that reports
    // success and fits the workspace.  The heuristic is a function of the
    // device, the shape and the library version, so every process runs the
    // same kernel for a shape and results repeat bitwise; nothing is timed and
    // nothing waits on the stream.  The choice is remembered per shape.
    const float one = 1.0f, zero = 0.0f;
    hipblasLtMatmulAlgo_t algo;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        auto it = g_algos.find(g.key(dtype));
        if (it == g_algos.end()) {
            s = hipblasLtMatmulPreferenceCreate(&pref);
            const uint64_t wsb = kBlasWorkspace;
            if (s == HIPBLAS_STATUS_SUCCESS)
                s = hipblasLtMatmulPreferenceSetAttribute(
                    pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsb, sizeof(wsb));
            constexpr int kCandidates = 8;
            hipblasLtMatmulHeuristicResult_t res[kCandidates];
            int found = 0;
            if (s == HIPBLAS_STATUS_SUCCESS)
                s = hipblasLtMatmulAlgoGetHeuristic(h, desc, la, lb, ld, ld, pref, kCandidates,
                                                    res, &found);
            if (s != HIPBLAS_STATUS_SUCCESS) {
                cleanup();
                return blas_error(s);
            }
            int pick = -1;
            for (int a = 0; a < found && pick < 0; ++a)
                if (res[a].state == HIPBLAS_STATUS_SUCCESS &&
                    res[a].workspaceSize <= static_cast<size_t>(kBlasWorkspace))
                    pick = a;
            if (pick < 0) {
                cleanup();
                return hipErrorNotSupported;
            }
            it = g_algos.emplace(g.key(dtype), res[pick].algo).first;
        }
        algo = it->second;
    }
    s = hipblasLtMatmul(h, desc, &one, A, la, B, lb, &zero, D, ld, D, ld, &algo, ws,
                        static_cast<size_t>(kBlasWorkspace), stream);
    cleanup();
    return blas_error(s);
}

// Bytes of the prepared-weight scratch the scan uses when its tap groups
// share a normalisation (bf16 square planes with even sides up to 80, one
// segment a scan; sized here whatever the segment count), else 0.
int64_t shared_prep_bytes(int dtype, int64_t B, int64_t Cc, int64_t G, int64_t H, int64_t W) {
    PropOpts o;
    o.cpg = Cc / G;
    const void* a = reinterpret_cast<const void*>(uintptr_t{256});
    if (!prop2d_quad_shared_eligible(dtype, B * Cc, H, W, o, a, a, a, a, a)) return 0;
    return prop2d_quad_shared_workspace_bytes(B * Cc, H, o.cpg);
}

struct SublayerLayout {
    int64_t z, zt, lam, u, taps, yc, prep, blas, total;
    SublayerLayout(int dtype, int64_t B, int64_t Cc, int64_t G, int64_t H, int64_t W) {
        const int64_t N = H * W;
        const int64_t es = dtype == 0 ? 4 : 2;
        const int64_t plane = align_up(B * Cc * N * es);
        z = 0;
        zt = z + plane;
        lam = zt + plane;
        u = lam + plane;
        taps = u + plane;
        yc = taps + align_up(12 * B * G * N * es);
        prep = yc + plane;
        blas = prep + align_up(shared_prep_bytes(dtype, B, Cc, G, H, W));
        total = blas + kBlasWorkspace;
    }
};

}  // namespace

int64_t latent_sublayer_workspace_bytes(int dtype, int64_t B, int64_t Cc, int64_t G, int64_t H,
                                        int64_t W) {
    return SublayerLayout(dtype, B, Cc, G, H, W).total;
}

hipError_t launch_latent_sublayer(const void* x_tok, const void* p_down, const void* w_param,
                                  const void* p_up, int64_t G, int64_t k_chunk, float eps,
                                  void* y_tok, void* ws, int dtype, int64_t B, int64_t C,
                                  int64_t Cc, int64_t H, int64_t W, hipStream_t stream) {
    const int64_t N = H * W;
    const int64_t es = dtype == 0 ? 4 : 2;
    const SublayerLayout lay(dtype, B, Cc, G, H, W);
    char* base = static_cast<char*>(ws);
    void* z = base + lay.z;
    void* zt = base + lay.zt;
    void* lam = base + lay.lam;
    void* u = base + lay.u;
    char* taps = base + lay.taps;
    void* yc = base + lay.yc;
    void* bws = base + lay.blas;
    const char* wp = static_cast<const char*>(w_param);
    const int bt = static_cast<int>(B);
    hipError_t e;

    // z[b] (Cc x N, row-major) = P_down x[b]^T, i.e. z[b]^T = x[b] P_down^T with
    // x[b] the N x C token matrix: on the matrix cores where the shape fits
    // the token-streaming kernel, else in hipBLASLt
    if (conv1x1_down_eligible(dtype, B, Cc, H, W, C))
        e = launch_conv1x1_down(x_tok, p_down, B, C, Cc, H, W, z, stream);
    else
        e = gemm(dtype, {HIPBLAS_OP_T, HIPBLAS_OP_N, N, Cc, C, C, C, N, N * C, 0, Cc * N, bt}, x_tok,
                 p_down, z, bws, stream);
    if (e != hipSuccess) return e;
    PropOpts opts;
    opts.cpg = Cc / G;
    opts.k_chunk = k_chunk;
    // the scan: shared tap groups are normalised once into the prep region
    auto scan = [&]() {
        if (lay.blas > lay.prep &&
            prop2d_quad_shared_eligible(dtype, B * Cc, H, W, opts, z, lam, u, taps, yc))
            return launch_prop2d_quad_shared(z, lam, u, taps, eps, yc, B * Cc, H, opts,
                                             base + lay.prep, stream);
        return launch_prop2d(z, lam, u, taps, eps, yc, dtype, B * Cc, H, W, opts, stream);
    };
    if (conv1x1_eligible(dtype, B, Cc, H, W, C)) {
        // the parameter convolutions and P_up on the matrix cores: one launch
        // writes lambda, u and the row scans' taps from z, one the column
        // scans' taps from the transposed latent zt
        void* taps4[4];
        for (int d = 0; d < 4; ++d) taps4[d] = taps + d * B * 3 * G * N * es;
        e = launch_conv1x1_params(z, zt, w_param, B, Cc, G, H, W, lam, u, taps4, stream);
        if (e != hipSuccess) return e;
        e = scan();
        if (e != hipSuccess) return e;
        return launch_conv1x1_up(yc, p_up, B, Cc, C, H, W, y_tok, stream);
    }
    // column-major copy of every latent plane, for the column scans' taps
    {
        const int tiles_w = static_cast<int>((W + kTile - 1) / kTile);
        const int tiles = tiles_w * static_cast<int>((H + kTile - 1) / kTile);
        const int64_t blocks = B * Cc * tiles;
        if (dtype == 0)
            transpose_planes_kernel<float><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream>>>(
                static_cast<const float*>(z), static_cast<float*>(zt), static_cast<int>(H),
                static_cast<int>(W), tiles_w, tiles);
        else
            transpose_planes_kernel<uint16_t><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream>>>(
                static_cast<const uint16_t*>(z), static_cast<uint16_t*>(zt), static_cast<int>(H),
                static_cast<int>(W), tiles_w, tiles);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // parameter rows r0 .. r0 + rows - 1 of w_param applied to a latent:
    // out[b] (rows x N, row-major) = Wp[r0:] src[b]
    auto params = [&](int64_t r0, int64_t rows, const void* src, void* out, int64_t out_stride) {
        return gemm(dtype, {HIPBLAS_OP_N, HIPBLAS_OP_N, N, rows, Cc, N, Cc, N, Cc * N, 0, out_stride, bt},
                    src, wp + r0 * Cc * es, out, bws, stream);
    };
    if ((e = params(0, Cc, z, lam, Cc * N)) != hipSuccess) return e;
    if ((e = params(Cc, Cc, z, u, Cc * N)) != hipSuccess) return e;
    for (int d = 0; d < 4; ++d) {
        // the column scans read their taps column-major: take them from zt
        e = params(2 * Cc + 3 * G * d, 3 * G, d < 2 ? z : zt, taps + d * B * 3 * G * N * es,
                   3 * G * N);
        if (e != hipSuccess) return e;
    }
    e = scan();
    if (e != hipSuccess) return e;
    // y[b] (N x C, row-major) = yc[b]^T P_up^T: column-major y^T = P_up yc[b]
    return gemm(dtype, {HIPBLAS_OP_T, HIPBLAS_OP_T, C, N, Cc, Cc, N, C, 0, Cc * N, N * C, bt}, p_up,
                yc, y_tok, bws, stream);
}

}  // namespace gspn
