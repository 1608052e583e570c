/*
 * gspn.h - C ABI of the MI355X (gfx950) GSPN line-scan propagation library.
 *
 * The operator is the 2D line-scan propagation of GSPN as used inside the
 * C-GSPN latent sublayer ("Scaling Parallel Sequence Models to
 * Foundation-Scale Vision Encoders": §3 "Background: 2D Spatial
 * Propagation", §4 "A Fast GSPN Kernel", §5.1 "Latent-space 2D
 * propagation" and "Fused CUDA normalization"; reading notes of the same
 * paper, method / overall framework and key designs 1-2).
 *
 * For every (b, c) plane of a B x C x H x W feature map and for each of the
 * four scan directions d (top-down TD, bottom-up BU, left-right LR,
 * right-left RL) the lines of the plane are visited in order and
 *
 *     h_first = lambda * x                       (state before the first line is 0)
 *     h_i[p]  = sum_k wn_k(i, p) * h_{i-1}[p + k - 1] + lambda_i[p] * x_i[p]
 *     out_d   = u * h
 *
 * with the three taps k = 0, 1, 2 of destination position p made
 * row-stochastic from raw logits w~ by the fused normalisation
 *
 *     s_k = sigmoid(w~_k) if p + k - 1 lies on the line, else 0
 *     S   = max(s_0 + s_1 + s_2, eps)
 *     wn_k = s_k / S.
 *
 * gspn_prop2d_4dir returns y = sum_d u * h_d.  Readings taken where the pages
 * are silent: zero initial state; tap offsets are absolute (not mirrored for
 * BU or RL); out-of-line taps are dropped from numerator and sum; the clamp
 * bounds the sum below by eps; lambda and u are shared by the directions;
 * the directional outputs are summed.
 *
 * ------------------------------------------------------------------------
 * Layouts (all row-major, innermost index last, densely packed):
 *   x, lambda, u, y        [B][C][H][W]
 *   taps of one direction  [B][C][3][NL][L], indexed by (line i, position p)
 *                          of that direction:
 *                            TD, BU: line = row,    NL = H, L = W
 *                            LR, RL: line = column, NL = W, L = H
 *                          i.e. the LR/RL tap planes are stored transposed
 *                          relative to the pixel grid, so that every line's
 *                          taps are contiguous in memory.
 *   taps of all directions [4][B][C][3][..][..] in the order TD, BU, LR, RL.
 * Element types: every tensor of one call has the same type (GSPN_FP32 or
 * GSPN_BF16); arithmetic is fp32; bf16 results are rounded to nearest even.
 *
 * Ownership: every pointer is a device pointer owned by the caller; the
 * library keeps no pointer after a call returns and allocates no device
 * memory at call time (its one static device buffer, 64 MiB per GPU, exists
 * from library load and serves gspn_prop2d_4dir_ex_backward_noalloc only).
 * Work is enqueued on `stream` (a hipStream_t; NULL = the null
 * stream) and the call returns without synchronising.
 *
 * Errors: every argument is validated on the host before anything is
 * enqueued; on any error the call returns a non-zero gspn_status, enqueues
 * nothing and leaves every output untouched.  GSPN_ERR_HIP reports a failed
 * launch.  The library never prints, aborts or throws, and may be called
 * from several host threads.  Its only global state is remembered results
 * of one-time queries (device attributes, the static scratch buffer's
 * address, the sublayer's hipBLASLt handle and algorithm per shape) and the
 * static scratch buffer's contents; none of it changes a result.  Non-finite inputs propagate by IEEE
 * rules; the results of a plane holding a non-finite input are unspecified
 * but confined to that plane.
 * ------------------------------------------------------------------------
 */
#ifndef GSPN_H
#define GSPN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GSPN_ABI_VERSION 7

/* Longest line (H or W) any entry point accepts. */
#define GSPN_MAX_LINE 8192

typedef enum {
    GSPN_OK = 0,
    GSPN_ERR_NULL = 1,   /* a required pointer is NULL                          */
    GSPN_ERR_SHAPE = 2,  /* a size < 1, a line > GSPN_MAX_LINE, an element count
                            >= 2^31, or a plane too large for the entry point  */
    GSPN_ERR_DTYPE = 3,  /* unknown element type                                */
    GSPN_ERR_DIR = 4,    /* unknown direction (or GSPN_ALL4 where one is needed)*/
    GSPN_ERR_ALIGN = 5,  /* a pointer is not aligned to its element size        */
    GSPN_ERR_ALIAS = 6,  /* an output overlaps an input                         */
    GSPN_ERR_VALUE = 7,  /* eps is not finite and > 0, or a flag is not 0/1     */
    GSPN_ERR_HIP = 8,    /* the HIP runtime reported an error                   */
    GSPN_ERR_SCRATCH = 9 /* the problem needs more than the static scratch
                            buffer (gspn_prop2d_4dir_ex_backward_noalloc)      */
} gspn_status;

typedef enum { GSPN_FP32 = 0, GSPN_BF16 = 1 } gspn_dtype;

typedef enum { GSPN_TD = 0, GSPN_BU = 1, GSPN_LR = 2, GSPN_RL = 3, GSPN_ALL4 = 4 } gspn_dir;

/* GSPN_ABI_VERSION of the built library. */
int gspn_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char* gspn_status_str(int status);

/*
 * Row-stochastic normalisation of raw taps (sigmoid -> neighbourhood sum ->
 * clamp -> divide; paper §5.1 "Fused CUDA normalization", reading notes,
 * normalisation formula).
 *   w_raw, w_norm : taps of direction `dir` ([B][C][3][NL][L]), or of all four
 *                   directions ([4][B][C][3][..][..]) when dir == GSPN_ALL4.
 *   Every position is written, the first line of each scan included.
 *   w_norm must not overlap w_raw.
 */
int gspn_normalize_weights(const void* w_raw, void* w_norm, int dtype,
                           int64_t B, int64_t C, int64_t H, int64_t W,
                           int dir, float eps, void* stream);

/*
 * One scan direction (paper §3 line-scan recurrence; §4.1 single-kernel
 * design: every line step of the scan runs inside one launch).
 *   x, lam, u, y : [B][C][H][W];  w : taps of direction `dir`.
 *   w_is_raw = 1 : w holds logits, normalised on the fly (fused);
 *   w_is_raw = 0 : w holds final weights, used as given (a tap whose source
 *                  lies outside the line contributes nothing).
 *   accumulate = 0 : y = u * h;   accumulate = 1 : y = y + u * h.
 *   y must not overlap x, lam, u or w.
 */
int gspn_scan_dir(const void* x, const void* lam, const void* u, const void* w,
                  int w_is_raw, float eps, void* y, int accumulate, int dtype,
                  int64_t B, int64_t C, int64_t H, int64_t W, int dir,
                  void* stream);

/*
 * All four directions with fused normalisation, in one launch:
 *   y = u * (h_TD + h_BU + h_LR + h_RL)
 * (the latent propagation y_c = Prop2D(x_c; u, lambda, w) of reading notes
 * key design 1, run on whatever channel count the caller passes, e.g. the
 * compressed latent C_c).
 *   x, lam, u, y : [B][C][H][W];  w_raw4 : [4][B][C][3][..][..] logits.
 *   y must not overlap any input.  The result is bitwise reproducible
 *   from run to run.
 *   bf16 planes whose fp32 direction sum does not fit on chip (H W above
 *   40960 - 2 max(H, W) pixels, about 200 x 200) return GSPN_ERR_SHAPE here:
 *   gspn_prop2d_4dir_ex_ws with groups = C takes them, keeping the sum in its
 *   workspace (fp32 output is its own accumulator and has no such limit).
 */
int gspn_prop2d_4dir(const void* x, const void* lam, const void* u,
                     const void* w_raw4, float eps, void* y, int dtype,
                     int64_t B, int64_t C, int64_t H, int64_t W, void* stream);

/*
 * gspn_prop2d_4dir with two options of the operator:
 *   groups  : taps shared by channel groups (paper §4.2 channel-shared
 *             weights; §6.2 shares them across channels in every module).
 *             The C channels form `groups` contiguous groups of C / groups
 *             channels; channel c reads the taps of group c / (C / groups).
 *             w_raw4 is [4][B][groups][3][..][..].  groups = C is
 *             gspn_prop2d_4dir; groups = 1 shares one set of taps per image.
 *             Must divide C (else GSPN_ERR_SHAPE).
 *   k_chunk : chunked (local) scan (paper §4.1: the grid is indexed by
 *             (chunk, b, c)).  Each direction's NL lines are cut into
 *             k_chunk segments of ceil(NL / k_chunk) lines (the last may be
 *             shorter), the same segments for both scan orders of an axis;
 *             each segment is scanned on its own and its first line in scan
 *             order is lambda * x.  k_chunk = 1 is the global scan; values at
 *             or above a scan's line count give single-line segments.  Must
 *             be >= 1 (else GSPN_ERR_VALUE).
 * Other arguments, layouts, errors and determinism as gspn_prop2d_4dir.
 */
int gspn_prop2d_4dir_ex(const void* x, const void* lam, const void* u,
                        const void* w_raw4, int64_t groups, int64_t k_chunk,
                        float eps, void* y, int dtype, int64_t B, int64_t C,
                        int64_t H, int64_t W, void* stream);

/*
 * gspn_prop2d_4dir_ex with a workspace that lets channels sharing taps share
 * their normalisation (paper §4.2, channel-shared weights): where the
 * workspace is used, a first kernel normalises each group's taps once into
 * it (fp32 weights, the fused sigmoid / sum / clamp / divide with the same
 * arithmetic) and the scan reads them, instead of every channel normalising
 * its group's taps again.  Results agree with gspn_prop2d_4dir_ex within
 * rounding (the weight is formed as s_k * (1 / S) before the products, not
 * after); each path is deterministic.
 *   workspace : at least gspn_prop2d_4dir_ex_workspace(...) bytes, 16-byte
 *               aligned, not overlapping any argument; contents on return
 *               unspecified.  When that size is 0 the workspace is not used
 *               (may be NULL) and the call is gspn_prop2d_4dir_ex.  bf16
 *               planes too large for gspn_prop2d_4dir_ex (see
 *               gspn_prop2d_4dir) keep their fp32 direction sum here, 4 bytes
 *               per pixel-channel (any groups and k_chunk), and are accepted
 *               only by this call.
 * Other arguments, layouts and errors as gspn_prop2d_4dir_ex, plus
 * GSPN_ERR_SHAPE for a workspace smaller than needed.
 */
int gspn_prop2d_4dir_ex_ws(const void* x, const void* lam, const void* u, const void* w_raw4,
                           int64_t groups, int64_t k_chunk, float eps, void* y, void* workspace,
                           int64_t workspace_bytes, int dtype, int64_t B, int64_t C, int64_t H,
                           int64_t W, void* stream);

/* Workspace bytes gspn_prop2d_4dir_ex_ws uses for these sizes: 0 where it
 * runs as gspn_prop2d_4dir_ex (today: all but bf16 square planes with even
 * sides up to 80, one segment a scan and at least 2 channels a group, and
 * bf16 planes whose direction sum does not fit on chip), or -1 if the sizes
 * are not accepted. */
int64_t gspn_prop2d_4dir_ex_workspace(int dtype, int64_t B, int64_t C, int64_t groups, int64_t H,
                                      int64_t W);

/*
 * Gradient of gspn_prop2d_4dir (the pages report backward kernels, paper text
 * §6.1, without describing them; this is the exact derivative of the
 * operator above).  Given gy = dL/dy:
 *   gx = lambda * G,  glam = x * G,  gu = gy * sum_d h_d,  G = sum_d g_d,
 * where g_d is the adjoint of direction d, run in reverse scan order with
 * the transposed tridiagonal tap map:
 *   g_last = u * gy,   g_i[p] = u * gy + sum_k wn_k(i+1, p-k+1) g_{i+1}[p-k+1];
 * and gw4 (layout of w_raw4) is the gradient with respect to the logits:
 *   gwn_k(i, p) = g_i[p] h_{i-1}[p+k-1]  (0 on the first line of the scan
 *                 and for out-of-line taps),
 *   T = sum of the in-line sigmoids s_k;
 *   T > eps : gs_m = (gwn_m - sum_k gwn_k wn_k) / T,  else gs_m = gwn_m / eps
 *   gz_m = gs_m s_m (1 - s_m).
 *   x, lam, u, gy, gx, glam, gu : [B][C][H][W];  w_raw4, gw4 : [4][B][C][3][..][..].
 *   workspace : scratch of at least
 *               gspn_prop2d_4dir_backward_workspace(B, C, H, W) bytes, 4-byte
 *               aligned (16-byte alignment lets the fast kernels run);
 *               contents on return are unspecified.  Sizes are for fp32
 *               storage.  Planes with even H and W up to 160 need it for
 *               transposed copies of x, lam, u, gy and two fp32 partial sums
 *               per pixel-channel, and so do bf16 planes with H = W odd, up to
 *               159.  Another plane with an odd side whose sides, padded to
 *               even, are at most 160 (fp32, or H != W) also holds padded
 *               copies of the inputs, outputs, taps and tap gradients there,
 *               and is run as the padded plane (the padding is exact: the
 *               added row and column start at 0 and no real position reads
 *               them); the size covers that for every odd side.  Other
 *               planes need three fp32 planes per (b, c) once those no longer
 *               fit in LDS (above about 115 x 115); below that the size is 0
 *               and NULL is allowed.
 *   Outputs must not overlap inputs, each other or the workspace.  Lines up
 *   to 5851 (H and W).  bf16 gradients are rounded to nearest even.  The
 *   result is bitwise reproducible from run to run.
 */
int gspn_prop2d_4dir_backward(const void* x, const void* lam, const void* u,
                              const void* w_raw4, const void* gy, float eps, void* gx,
                              void* glam, void* gu, void* gw4, void* workspace,
                              int64_t workspace_bytes, int dtype, int64_t B, int64_t C,
                              int64_t H, int64_t W, void* stream);

/* Workspace bytes gspn_prop2d_4dir_backward needs for these sizes (0 if
 * none), or -1 if it does not accept them. */
int64_t gspn_prop2d_4dir_backward_workspace(int64_t B, int64_t C, int64_t H, int64_t W);

/*
 * Gradient of gspn_prop2d_4dir_ex (tap groups and chunked scans): the exact
 * derivative of that operator, with the formulas of gspn_prop2d_4dir_backward
 * and two changes that follow from the forward:
 *   - the first line of each segment (in its scan order) reads no line before
 *     it, so its taps get gradient 0 and the line before it receives no
 *     adjoint term from it;
 *   - channel c reads the taps of group c / (C / groups), so the gradient of
 *     a group's taps is the sum over its channels, taken in channel order.
 *   groups, k_chunk : as gspn_prop2d_4dir_ex (groups must divide C, else
 *               GSPN_ERR_SHAPE; k_chunk >= 1, else GSPN_ERR_VALUE).
 *   w_raw4, gw4 : [4][B][groups][3][..][..] (gw4 has the layout of w_raw4).
 *   workspace : at least gspn_prop2d_4dir_ex_backward_workspace(B, C, groups,
 *               H, W) bytes, 4-byte aligned (16 for the fast kernels).  On top
 *               of what gspn_prop2d_4dir_backward needs, channels that share
 *               taps (groups < C) keep fp32 tap gradients or partial sums of
 *               tap products there (48 bytes per pixel-channel) and their
 *               group's normalised taps (48 bytes per pixel-group).  Shared
 *               taps with an odd side run padded as above, except a chunked
 *               scan whose k_chunk divides an odd side, which runs that plane
 *               unpadded.
 * Other arguments, layouts, errors and determinism as
 * gspn_prop2d_4dir_backward, which is this call with groups = C, k_chunk = 1.
 */
int gspn_prop2d_4dir_ex_backward(const void* x, const void* lam, const void* u,
                                 const void* w_raw4, int64_t groups, int64_t k_chunk,
                                 const void* gy, float eps, void* gx, void* glam, void* gu,
                                 void* gw4, void* workspace, int64_t workspace_bytes, int dtype,
                                 int64_t B, int64_t C, int64_t H, int64_t W, void* stream);

/* Workspace bytes gspn_prop2d_4dir_ex_backward needs for these sizes (0 if
 * none), or -1 if it does not accept them. */
int64_t gspn_prop2d_4dir_ex_backward_workspace(int64_t B, int64_t C, int64_t groups, int64_t H,
                                               int64_t W);

/*
 * gspn_prop2d_4dir_ex_backward for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, results, layouts and errors, minus the
 * workspace: the kernels use the library's static device buffer instead
 * (gspn_noalloc_scratch_bytes() = 64 MiB on each GPU, held from library load
 * until the process ends).  A problem whose workspace
 * (gspn_prop2d_4dir_ex_backward_workspace) exceeds that returns
 * GSPN_ERR_SCRATCH and enqueues nothing.  The call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine); its first call on a
 * device looks up that device's buffer address once.
 * Every call on one GPU shares that GPU's buffer: calls whose work overlaps
 * in time on one GPU (two streams, or two host threads without ordering)
 * race and give undefined results; calls ordered on one stream are safe.
 * The buffer keeps the last call's contents; nothing reads them before
 * writing them.
 */
int gspn_prop2d_4dir_ex_backward_noalloc(const void* x, const void* lam, const void* u,
                                         const void* w_raw4, int64_t groups, int64_t k_chunk,
                                         const void* gy, float eps, void* gx, void* glam,
                                         void* gu, void* gw4, int dtype, int64_t B, int64_t C,
                                         int64_t H, int64_t W, void* stream);

/* Size of the static scratch buffer (bytes per GPU). */
int64_t gspn_noalloc_scratch_bytes(void);

/*
 * Latent-space propagation sublayer (paper §5.1, a more efficient ViT block:
 * propagation in a compressed latent; reading notes, key design 1): the
 * four-direction propagation wrapped in its 1x1 projections.
 *   z      = P_down x            per token: Cc latent channels from C
 *   lambda = W_lambda z,  u = W_u z,  w_raw = W_taps z   (1x1 convolutions
 *            of the latent: the propagation parameters are per-position)
 *   y_c    = gspn_prop2d_4dir_ex(z, lambda, u, w_raw, groups, k_chunk)
 *   y      = P_up y_c            per token: C channels from Cc
 *   x_tok, y_tok : [B][H*W][C] tokens (row-major grid, channels last).
 *   p_down  : [Cc][C];   p_up : [C][Cc];
 *   w_param : [2 Cc + 12 groups][Cc], rows lambda (Cc), u (Cc), then the raw
 *             taps in [direction TD, BU, LR, RL][group][tap k] order.
 *   workspace : at least gspn_latent_sublayer_workspace(...) bytes; holds the
 *             latent, its parameters, the scan output and the GEMM library's
 *             scratch; contents on return are unspecified.
 *   All pointers 16-byte aligned; y_tok and workspace must not overlap any
 *   input or each other.  The projections accumulate in fp32; bf16 storage
 *   rounds every intermediate to bf16.  In bf16 they run on this library's
 *   matrix-core kernels where the shape fits them (P_down: Cc of 32 or 64
 *   and C a multiple of 128 up to 1280; the parameter convolutions and
 *   P_up: Cc a multiple of 8 up to 64, sides up to 96; H W a multiple of 4),
 *   else in hipBLASLt.  Per shape the hipBLASLt algorithm is the library
 *   heuristic's first candidate that succeeds and fits the scratch: nothing
 *   is timed, the call never waits on the stream, and every process runs
 *   the same kernels, so results repeat bitwise.  The first hipBLASLt call
 *   on a device creates that device's handle, and the first call for a
 *   shape queries the heuristic; both are remembered for the process (so
 *   make those first calls outside stream capture).  Errors as gspn_prop2d_4dir_ex, plus
 *   GSPN_ERR_SHAPE for a workspace that is too small or C outside
 *   [1, 65536].
 */
int gspn_latent_sublayer(const void* x_tok, const void* p_down, const void* w_param,
                         const void* p_up, int64_t groups, int64_t k_chunk, float eps,
                         void* y_tok, void* workspace, int64_t workspace_bytes, int dtype,
                         int64_t B, int64_t C, int64_t Cc, int64_t H, int64_t W, void* stream);

/* Workspace bytes gspn_latent_sublayer needs, or -1 if it does not accept
 * these sizes. */
int64_t gspn_latent_sublayer_workspace(int dtype, int64_t B, int64_t C, int64_t Cc,
                                       int64_t groups, int64_t H, int64_t W);

#ifdef __cplusplus
}
#endif

#endif /* GSPN_H */
