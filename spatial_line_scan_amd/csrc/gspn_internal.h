// Internal interface between the C-ABI host layer (gspn_host.cpp) and the
// gfx950 kernels (gspn_kernels.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gspn {

// LDS a single workgroup may address on gfx950 (160 KiB per CU).
constexpr int64_t kLdsBytes = 160 * 1024;
// Plane count up to which a launch of one wavefront a plane leaves SIMDs idle
// enough that a wavefront a direction finishes sooner (MI355X: 256 CUs;
// 74 x 74: 512 planes 0.035 ms against 0.042, 1024 planes 0.056 against
// 0.047).
constexpr int64_t kFewPlanes = 512;

// Options of the four-direction propagation: channels per tap group (taps
// are [4][planes / cpg][3][..][..]; tap plane of plane p is p / cpg) and the
// number of segments each scan is cut into.
struct PropOpts {
    int64_t cpg = 1;
    int64_t k_chunk = 1;
};

// Launchers.  Arguments are already validated; each enqueues work on
// `stream` and returns the launch status.
hipError_t launch_normalize(const void* w_raw, void* w_norm, int dtype, int64_t planes,
                            int64_t H, int64_t W, int dir0, int ndir, float eps,
                            hipStream_t stream);

hipError_t launch_scan_dir(const void* x, const void* lam, const void* u, const void* w,
                           int w_is_raw, float eps, void* y, int accumulate, int dtype,
                           int64_t planes, int64_t H, int64_t W, int dir, hipStream_t stream);

hipError_t launch_prop2d(const void* x, const void* lam, const void* u, const void* w4,
                         float eps, void* y, int dtype, int64_t planes, int64_t H, int64_t W,
                         const PropOpts& opts, hipStream_t stream);

// Fast path of gspn_scan_dir: one wavefront per plane, lambda x and the
// hidden state in LDS (gspn_scan_dir.hip).
bool scan_dir_fast_eligible(int64_t H, int64_t W, int dir);
hipError_t launch_scan_dir_fast(const void* x, const void* lam, const void* u, const void* w,
                                int w_is_raw, float eps, void* y, int accumulate, int dtype,
                                int64_t planes, int64_t H, int64_t W, int dir, hipStream_t stream);

// Fast path of gspn_prop2d_4dir: two wavefronts per plane (gspn_prop2d_pair.hip).
bool prop2d_pair_eligible(int dtype, int64_t planes, int64_t H, int64_t W, const void* x,
                          const void* lam, const void* u, const void* w4, const void* y);
hipError_t launch_prop2d_pair(const void* x, const void* lam, const void* u, const void* w4,
                              float eps, void* y, int dtype, int64_t planes, int64_t H, int64_t W,
                              const PropOpts& opts, hipStream_t stream);

// Large fp32 planes (sides up to 256, multiples of 4): one launch, one
// wavefront a plane, a pass per direction with y as the accumulator
// (gspn_prop2d_wide.hip).
bool prop2d_wide_eligible(int dtype, int64_t planes, int64_t H, int64_t W, const void* x,
                          const void* lam, const void* u, const void* w4, const void* y);
hipError_t launch_prop2d_wide(const void* x, const void* lam, const void* u, const void* w4,
                              float eps, void* y, int64_t planes, int64_t H, int64_t W,
                              const PropOpts& opts, hipStream_t stream);
// The same for bf16 planes with sides 196..256 (multiples of 4), the
// direction sum in acc (fp32, one plane per (b, c)).
bool prop2d_wide_bf16_eligible(int64_t planes, int64_t H, int64_t W, const void* x, const void* lam,
                               const void* u, const void* w4, const void* y, const void* acc);
hipError_t launch_prop2d_wide_bf16(const void* x, const void* lam, const void* u, const void* w4,
                                   float eps, void* y, int64_t planes, int64_t H, int64_t W,
                                   const PropOpts& opts, float* acc, hipStream_t stream);

// Fast path for bf16 planes: one wavefront per plane, rows then columns,
// lambda x and the direction sum on chip (gspn_prop2d_phase.hip).
bool prop2d_phase_eligible(int dtype, int64_t planes, int64_t H, int64_t W, const void* x,
                           const void* lam, const void* u, const void* w4, const void* y);
hipError_t launch_prop2d_phase(const void* x, const void* lam, const void* u, const void* w4,
                               float eps, void* y, int dtype, int64_t planes, int64_t H, int64_t W,
                               const PropOpts& opts, hipStream_t stream);

// Fast path for square bf16 planes with even sides up to 80: one wavefront
// per plane scans all four directions at once (gspn_prop2d_quad.hip).
bool prop2d_duo_eligible(int dtype, int64_t planes, int64_t H, int64_t W, const PropOpts& o,
                         const void* x, const void* lam, const void* u, const void* w4,
                         const void* y);
hipError_t launch_prop2d_duo(const void* x, const void* lam, const void* u, const void* w4,
                             float eps, void* y, int64_t planes, int64_t L, const PropOpts& o,
                             hipStream_t stream);
bool prop2d_quad_eligible(int dtype, int64_t planes, int64_t H, int64_t W, const PropOpts& o,
                          const void* x, const void* lam, const void* u, const void* w4,
                          const void* y);
hipError_t launch_prop2d_quad(const void* x, const void* lam, const void* u, const void* w4,
                              float eps, void* y, int64_t planes, int64_t L, const PropOpts& o,
                              hipStream_t stream);
// Taps shared by cpg >= 2 channels: normalised once per tap plane into ws
// (fp32, prop2d_quad_shared_workspace_bytes), then the scan reads them.
int64_t prop2d_quad_shared_workspace_bytes(int64_t planes, int64_t L, int64_t cpg);
bool prop2d_quad_shared_eligible(int dtype, int64_t planes, int64_t H, int64_t W, const PropOpts& o,
                                 const void* x, const void* lam, const void* u, const void* w4,
                                 const void* y);
hipError_t launch_prop2d_quad_shared(const void* x, const void* lam, const void* u, const void* w4,
                                     float eps, void* y, int64_t planes, int64_t L,
                                     const PropOpts& o, void* ws, hipStream_t stream);

// Gradient of gspn_prop2d_4dir_ex (gspn_backward.hip): taps of plane p read
// from group plane p / cpg, scans cut into k_chunk segments.  ws holds
// prop2d_backward_workspace_bytes(planes, H, W, cpg) bytes (NULL when that
// is 0).
hipError_t launch_prop2d_backward(const void* x, const void* lam, const void* u, const void* w4,
                                  const void* gy, float eps, void* gx, void* glam, void* gu,
                                  void* gw4, void* ws, int dtype, int64_t planes, int64_t H,
                                  int64_t W, const PropOpts& opts, hipStream_t stream);
int64_t prop2d_backward_workspace_bytes(int64_t planes, int64_t H, int64_t W, int64_t cpg);

// Fast path of the gradient for planes of even sides up to 96: one wavefront
// per plane and direction pair (gspn_backward_pair.hip).  Needs a workspace of
// prop2d_backward_pair_workspace_bytes bytes, 16-byte aligned.
bool prop2d_backward_pair_shape(int64_t planes, int64_t H, int64_t W);
int64_t prop2d_backward_pair_workspace_bytes(int64_t planes, int64_t H, int64_t W);
bool prop2d_backward_pair_eligible(int dtype, int64_t planes, int64_t H, int64_t W,
                                   const void* const* ptrs, int nptrs, const void* ws);
// gwd receives the per-channel tap gradients: gw4 itself (storage type), or
// with gw_fp32 an fp32 buffer [4][planes][3][H W] for channels sharing taps.
hipError_t launch_prop2d_backward_pair(const void* x, const void* lam, const void* u,
                                       const void* w4, const void* gy, float eps, void* gx,
                                       void* glam, void* gu, void* gwd, bool gw_fp32, void* ws,
                                       int dtype, int64_t planes, int64_t H, int64_t W,
                                       const PropOpts& opts, hipStream_t stream);
// Channels sharing taps (cpg > 1) on the pair kernel: the taps are
// normalised once per group into wpre (prop2d_backward_pair_shared_weights_bytes
// bytes), the pair kernel sums its planes' tap products on chip into part
// (up to 12 planes H W fp32) and a last kernel applies the normalisation's
// Jacobian per group into gw4 (storage type).  ws as for the pair kernel.
int64_t prop2d_backward_pair_shared_weights_bytes(int64_t planes, int64_t H, int64_t W, int64_t cpg);
hipError_t launch_prop2d_backward_pair_shared(const void* x, const void* lam, const void* u,
                                              const void* w4, const void* gy, float eps, void* gx,
                                              void* glam, void* gu, void* gw4, float* part, float* wpre,
                                              void* ws, int dtype, int64_t planes, int64_t H,
                                              int64_t W, const PropOpts& opts, hipStream_t stream);
// Longest line the backward's LDS lines allow.
int64_t prop2d_backward_max_line();

// Gradient for large fp32 planes (sides up to 256, multiples of 4): one
// wavefront per plane, h kept in ws (prop2d_backward_wide_workspace_bytes,
// 16-byte aligned; ws_bytes is what is available there), gx and gu used as
// the accumulators (gspn_backward_wide.hip).  gwd as for the pair kernel.
int64_t prop2d_backward_wide_workspace_bytes(int64_t planes, int64_t H, int64_t W);
bool prop2d_backward_wide_eligible(int dtype, int64_t planes, int64_t H, int64_t W,
                                   const void* const* ptrs, int nptrs, const void* ws,
                                   int64_t ws_bytes);
hipError_t launch_prop2d_backward_wide(const void* x, const void* lam, const void* u, const void* w4,
                                       const void* gy, float eps, void* gx, void* glam, void* gu,
                                       void* gwd, void* ws, int64_t planes, int64_t H, int64_t W,
                                       const PropOpts& opts, hipStream_t stream);

// Latent propagation sublayer (gspn_sublayer.hip): hipBLASLt 1x1 projections
// around launch_prop2d.  ws holds latent_sublayer_workspace_bytes bytes.
hipError_t launch_latent_sublayer(const void* x_tok, const void* p_down, const void* w_param,
                                  const void* p_up, int64_t G, int64_t k_chunk, float eps,
                                  void* y_tok, void* ws, int dtype, int64_t B, int64_t C,
                                  int64_t Cc, int64_t H, int64_t W, hipStream_t stream);
int64_t latent_sublayer_workspace_bytes(int dtype, int64_t B, int64_t Cc, int64_t G, int64_t H,
                                        int64_t W);

// Matrix-core 1x1 convolutions of the latent sublayer (bf16 storage).
// conv1x1_eligible: shapes the kernels take (K = Cc a multiple of 8 up to
// 64, H W a multiple of 4, H and W at most 96, C a multiple of 4).
bool conv1x1_eligible(int dtype, int64_t B, int64_t K, int64_t H, int64_t W, int64_t C);
// lambda, u ([B][Cc][H W]) and the four directions' raw taps (taps4[d]:
// [B][G][3][..], row-major for TD and BU, column-major for LR and RL) from
// the latent z [B][Cc][H W] and w_param [2 Cc + 12 G][Cc]; zt receives the
// transposed latent ([B][Cc][W][H]).
hipError_t launch_conv1x1_params(const void* z, void* zt, const void* w_param, int64_t B,
                                 int64_t Cc, int64_t G, int64_t H, int64_t W, void* lam, void* u,
                                 void* const* taps4, hipStream_t stream);
// z [B][Cc][H W] = P_down applied to the tokens x_tok [B][H W][C] (bf16, Cc
// of 32 or 64, C a multiple of 128 up to 1280, H W a multiple of 4).
bool conv1x1_down_eligible(int dtype, int64_t B, int64_t Cc, int64_t H, int64_t W, int64_t C);
hipError_t launch_conv1x1_down(const void* x_tok, const void* p_down, int64_t B, int64_t C,
                               int64_t Cc, int64_t H, int64_t W, void* z, hipStream_t stream);
// CUs of the current device (queried once per device).
hipError_t device_cu_count(int* out);
// y_tok [B][H W][C] = P_up applied to the planar latent yc [B][Cc][H W].
hipError_t launch_conv1x1_up(const void* yc, const void* p_up, int64_t B, int64_t Cc, int64_t C,
                             int64_t H, int64_t W, void* y_tok, hipStream_t stream);

// The library's static device scratch (gspn_noalloc.hip): its size, and its
// address on the current device (looked up once per device).
int64_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void** out);

// Largest plane (H * W pixels) gspn_prop2d_4dir accepts for an element type.
int64_t prop2d_max_plane(int dtype, int64_t H, int64_t W);

// bf16 planes above that size: the bytes of an fp32 accumulator plane per
// (b, c) (0 for planes that need none), and the four-direction forward that
// keeps the direction sum there.
int64_t prop2d_global_acc_bytes(int dtype, int64_t planes, int64_t H, int64_t W);
hipError_t launch_prop2d_global_acc(const void* x, const void* lam, const void* u, const void* w4,
                                    float eps, void* y, int64_t planes, int64_t H, int64_t W,
                                    const PropOpts& o, float* acc, hipStream_t stream);

}  // namespace gspn
