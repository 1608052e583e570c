// C-ABI entry points of libgspn: argument validation and dispatch.
//
// Every check runs on the host before anything touches the device, so a bad
// call returns its status with nothing enqueued and every output untouched.
#include "gspn.h"
#include "gspn_internal.h"

#include <algorithm>
#include <cmath>
#include <cstdint>

namespace {

constexpr int64_t kMaxElems = (int64_t{1} << 31) - 1;
// token channels of the latent sublayer (1x1 projections C <-> Cc)
constexpr int64_t kMaxTokenChannels = int64_t{1} << 16;

int64_t elem_size(int dtype) { return dtype == GSPN_FP32 ? 4 : 2; }

bool valid_dtype(int dtype) { return dtype == GSPN_FP32 || dtype == GSPN_BF16; }

// Sizes of a B x C x H x W problem whose largest tensor holds `mult` values
// per pixel-channel.
int check_dims(int64_t B, int64_t C, int64_t H, int64_t W, int64_t mult) {
    if (B < 1 || C < 1 || H < 1 || W < 1) return GSPN_ERR_SHAPE;
    if (H > GSPN_MAX_LINE || W > GSPN_MAX_LINE) return GSPN_ERR_SHAPE;
    if (B > kMaxElems || C > kMaxElems) return GSPN_ERR_SHAPE;
    const int64_t plane = H * W;  // <= 2^26
    if (B * C > kMaxElems / plane) return GSPN_ERR_SHAPE;
    if (B * C * plane > kMaxElems / mult) return GSPN_ERR_SHAPE;
    return GSPN_OK;
}

bool valid_eps(float eps) { return std::isfinite(eps) && eps > 0.0f; }

// Natural alignment of the element type.
bool aligned(const void* p, int dtype) {
    return (reinterpret_cast<uintptr_t>(p) & static_cast<uintptr_t>(elem_size(dtype) - 1)) == 0;
}

bool overlap(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + static_cast<uintptr_t>(bbytes) && b0 < a0 + static_cast<uintptr_t>(abytes);
}

int launch_status(hipError_t e) { return e == hipSuccess ? GSPN_OK : GSPN_ERR_HIP; }

// Workspace the grouped forward uses to normalise each group's taps once
// (0: the taps are normalised by every channel as it scans).
int64_t shared_workspace(int dtype, int64_t B, int64_t C, int64_t groups, int64_t H, int64_t W) {
    // bf16 planes whose direction sum leaves LDS: an fp32 accumulator plane
    // per (b, c)
    if (int64_t acc = gspn::prop2d_global_acc_bytes(dtype, B * C, H, W)) return acc;
    gspn::PropOpts o;
    o.cpg = C / groups;
    // the eligibility test reads only alignment from these
    const void* a = reinterpret_cast<const void*>(uintptr_t{256});
    if (!gspn::prop2d_quad_shared_eligible(dtype, B * C, H, W, o, a, a, a, a, a)) return 0;
    return gspn::prop2d_quad_shared_workspace_bytes(B * C, H, o.cpg);
}

// Shared by gspn_prop2d_4dir_ex and gspn_prop2d_4dir_ex_ws (with_ws).
int ex_forward(const void* x, const void* lam, const void* u, const void* w_raw4, int64_t groups,
               int64_t k_chunk, float eps, void* y, void* workspace, int64_t workspace_bytes,
               bool with_ws, int dtype, int64_t B, int64_t C, int64_t H, int64_t W, void* stream) {
    if (!valid_dtype(dtype)) return GSPN_ERR_DTYPE;
    if (int s = check_dims(B, C, H, W, 12)) return s;
    // bf16 planes above the LDS direction sum need the workspace's accumulator
    const bool global_acc = H * W > gspn::prop2d_max_plane(dtype, H, W);
    if (global_acc && !with_ws) return GSPN_ERR_SHAPE;
    if (groups < 1 || groups > C || C % groups != 0) return GSPN_ERR_SHAPE;
    if (k_chunk < 1) return GSPN_ERR_VALUE;
    if (!valid_eps(eps)) return GSPN_ERR_VALUE;
    if (!x || !lam || !u || !w_raw4 || !y) return GSPN_ERR_NULL;
    if (!aligned(x, dtype) || !aligned(lam, dtype) || !aligned(u, dtype) ||
        !aligned(w_raw4, dtype) || !aligned(y, dtype))
        return GSPN_ERR_ALIGN;
    const int64_t n = B * C * H * W * elem_size(dtype);
    const int64_t taps = 12 * B * groups * H * W * elem_size(dtype);
    if (overlap(y, n, x, n) || overlap(y, n, lam, n) || overlap(y, n, u, n) ||
        overlap(y, n, w_raw4, taps))
        return GSPN_ERR_ALIAS;
    gspn::PropOpts opts;
    opts.cpg = C / groups;
    // any count at or above a scan's line count cuts it into single lines
    opts.k_chunk = std::min<int64_t>(k_chunk, std::max(H, W));
    const int64_t need = with_ws ? shared_workspace(dtype, B, C, groups, H, W) : 0;
    if (need > 0) {
        if (!workspace) return GSPN_ERR_NULL;
        if (workspace_bytes < need) return GSPN_ERR_SHAPE;
        if (reinterpret_cast<uintptr_t>(workspace) & 15u) return GSPN_ERR_ALIGN;
        if (overlap(workspace, need, x, n) || overlap(workspace, need, lam, n) ||
            overlap(workspace, need, u, n) || overlap(workspace, need, w_raw4, taps) ||
            overlap(workspace, need, y, n))
            return GSPN_ERR_ALIAS;
        if (global_acc) {
            float* acc = static_cast<float*>(workspace);
            const hipStream_t st = static_cast<hipStream_t>(stream);
            if (gspn::prop2d_wide_bf16_eligible(B * C, H, W, x, lam, u, w_raw4, y, acc))
                return launch_status(gspn::launch_prop2d_wide_bf16(x, lam, u, w_raw4, eps, y, B * C, H, W, opts,
                                                                   acc, st));
            return launch_status(gspn::launch_prop2d_global_acc(x, lam, u, w_raw4, eps, y, B * C, H, W, opts,
                                                                acc, st));
        }
        // buffers the fast kernels cannot address (2-byte aligned) take the
        // path that normalises per channel
        if (gspn::prop2d_quad_shared_eligible(dtype, B * C, H, W, opts, x, lam, u, w_raw4, y))
            return launch_status(gspn::launch_prop2d_quad_shared(x, lam, u, w_raw4, eps, y, B * C,
                                                                 H, opts, workspace,
                                                                 static_cast<hipStream_t>(stream)));
    } else if (with_ws && workspace_bytes < 0) {
        return GSPN_ERR_SHAPE;
    }
    return launch_status(gspn::launch_prop2d(x, lam, u, w_raw4, eps, y, dtype, B * C, H, W, opts,
                                             static_cast<hipStream_t>(stream)));
}

// Shared by gspn_prop2d_4dir_ex_backward (caller's workspace) and its
// _noalloc variant (scratch: the library's static buffer, looked up after
// validation).
int ex_backward(const void* x, const void* lam, const void* u, const void* w_raw4,
                int64_t groups, int64_t k_chunk, const void* gy, float eps, void* gx,
                void* glam, void* gu, void* gw4, void* workspace, int64_t workspace_bytes,
                bool scratch, int dtype, int64_t B, int64_t C, int64_t H, int64_t W,
                void* stream) {
    if (!valid_dtype(dtype)) return GSPN_ERR_DTYPE;
    if (int s = check_dims(B, C, H, W, 12)) return s;
    if (H > gspn::prop2d_backward_max_line() || W > gspn::prop2d_backward_max_line())
        return GSPN_ERR_SHAPE;
    if (groups < 1 || groups > C || C % groups != 0) return GSPN_ERR_SHAPE;
    if (k_chunk < 1) return GSPN_ERR_VALUE;
    if (!valid_eps(eps)) return GSPN_ERR_VALUE;
    if (!x || !lam || !u || !w_raw4 || !gy || !gx || !glam || !gu || !gw4) return GSPN_ERR_NULL;
    const int64_t need = gspn::prop2d_backward_workspace_bytes(B * C, H, W, C / groups);
    if (scratch) {
        if (need > gspn::noalloc_scratch_bytes()) return GSPN_ERR_SCRATCH;
    } else {
        if (need > 0 && !workspace) return GSPN_ERR_NULL;
        if (workspace_bytes < 0 || (need > 0 && workspace_bytes < need)) return GSPN_ERR_SHAPE;
    }
    const void* ptrs[] = {x, lam, u, w_raw4, gy, gx, glam, gu, gw4};
    for (const void* p : ptrs)
        if (!aligned(p, dtype)) return GSPN_ERR_ALIGN;
    if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) & 3u)) return GSPN_ERR_ALIGN;
    const int64_t n = B * C * H * W * elem_size(dtype);
    const int64_t taps = 12 * B * groups * H * W * elem_size(dtype);
    const void* ins[] = {x, lam, u, w_raw4, gy};
    const int64_t in_bytes[] = {n, n, n, taps, n};
    void* outs[] = {gx, glam, gu, gw4};
    const int64_t out_bytes[] = {n, n, n, taps};
    // the static scratch buffer cannot overlap a caller's buffer: only a
    // caller's workspace is checked
    const bool check_ws = !scratch && need > 0;
    for (int o = 0; o < 4; ++o) {
        for (int i = 0; i < 5; ++i)
            if (overlap(outs[o], out_bytes[o], ins[i], in_bytes[i])) return GSPN_ERR_ALIAS;
        for (int o2 = 0; o2 < o; ++o2)
            if (overlap(outs[o], out_bytes[o], outs[o2], out_bytes[o2])) return GSPN_ERR_ALIAS;
        if (check_ws && overlap(outs[o], out_bytes[o], workspace, need)) return GSPN_ERR_ALIAS;
    }
    if (check_ws)
        for (int i = 0; i < 5; ++i)
            if (overlap(workspace, need, ins[i], in_bytes[i])) return GSPN_ERR_ALIAS;
    if (scratch && need > 0 && gspn::noalloc_scratch(&workspace) != hipSuccess)
        return GSPN_ERR_HIP;
    gspn::PropOpts opts;
    opts.cpg = C / groups;
    opts.k_chunk = std::min<int64_t>(k_chunk, std::max(H, W));
    return launch_status(gspn::launch_prop2d_backward(
        x, lam, u, w_raw4, gy, eps, gx, glam, gu, gw4, need > 0 ? workspace : nullptr, dtype,
        B * C, H, W, opts, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int gspn_abi_version(void) { return GSPN_ABI_VERSION; }

const char* gspn_status_str(int status) {
    switch (status) {
        case GSPN_OK: return "GSPN_OK";
        case GSPN_ERR_NULL: return "GSPN_ERR_NULL: a required pointer is NULL";
        case GSPN_ERR_SHAPE: return "GSPN_ERR_SHAPE: unsupported sizes";
        case GSPN_ERR_DTYPE: return "GSPN_ERR_DTYPE: unknown element type";
        case GSPN_ERR_DIR: return "GSPN_ERR_DIR: unknown direction";
        case GSPN_ERR_ALIGN: return "GSPN_ERR_ALIGN: pointer not aligned to its element size";
        case GSPN_ERR_ALIAS: return "GSPN_ERR_ALIAS: output overlaps an input";
        case GSPN_ERR_VALUE: return "GSPN_ERR_VALUE: eps must be finite and > 0, flags 0 or 1";
        case GSPN_ERR_HIP: return "GSPN_ERR_HIP: HIP runtime error";
        case GSPN_ERR_SCRATCH:
            return "GSPN_ERR_SCRATCH: the problem needs more scratch than the library's static buffer";
        default: return "GSPN: unknown status";
    }
}

int gspn_normalize_weights(const void* w_raw, void* w_norm, int dtype, int64_t B, int64_t C,
                           int64_t H, int64_t W, int dir, float eps, void* stream) {
    if (!valid_dtype(dtype)) return GSPN_ERR_DTYPE;
    if (dir < GSPN_TD || dir > GSPN_ALL4) return GSPN_ERR_DIR;
    const int ndir = dir == GSPN_ALL4 ? 4 : 1;
    if (int s = check_dims(B, C, H, W, 3 * ndir)) return s;
    if (!valid_eps(eps)) return GSPN_ERR_VALUE;
    if (!w_raw || !w_norm) return GSPN_ERR_NULL;
    if (!aligned(w_raw, dtype) || !aligned(w_norm, dtype)) return GSPN_ERR_ALIGN;
    const int64_t bytes = B * C * H * W * 3 * ndir * elem_size(dtype);
    if (overlap(w_raw, bytes, w_norm, bytes)) return GSPN_ERR_ALIAS;
    return launch_status(gspn::launch_normalize(w_raw, w_norm, dtype, B * C, H, W,
                                                dir == GSPN_ALL4 ? 0 : dir, ndir, eps,
                                                static_cast<hipStream_t>(stream)));
}

int gspn_scan_dir(const void* x, const void* lam, const void* u, const void* w, int w_is_raw,
                  float eps, void* y, int accumulate, int dtype, int64_t B, int64_t C,
                  int64_t H, int64_t W, int dir, void* stream) {
    if (!valid_dtype(dtype)) return GSPN_ERR_DTYPE;
    if (dir < GSPN_TD || dir > GSPN_RL) return GSPN_ERR_DIR;
    if (int s = check_dims(B, C, H, W, 3)) return s;
    if ((w_is_raw != 0 && w_is_raw != 1) || (accumulate != 0 && accumulate != 1))
        return GSPN_ERR_VALUE;
    if (w_is_raw && !valid_eps(eps)) return GSPN_ERR_VALUE;
    if (!x || !lam || !u || !w || !y) return GSPN_ERR_NULL;
    if (!aligned(x, dtype) || !aligned(lam, dtype) || !aligned(u, dtype) || !aligned(w, dtype) ||
        !aligned(y, dtype))
        return GSPN_ERR_ALIGN;
    const int64_t n = B * C * H * W * elem_size(dtype);
    if (overlap(y, n, x, n) || overlap(y, n, lam, n) || overlap(y, n, u, n) ||
        overlap(y, n, w, 3 * n))
        return GSPN_ERR_ALIAS;
    return launch_status(gspn::launch_scan_dir(x, lam, u, w, w_is_raw, eps, y, accumulate, dtype,
                                               B * C, H, W, dir,
                                               static_cast<hipStream_t>(stream)));
}

int gspn_prop2d_4dir(const void* x, const void* lam, const void* u, const void* w_raw4,
                     float eps, void* y, int dtype, int64_t B, int64_t C, int64_t H, int64_t W,
                     void* stream) {
    return gspn_prop2d_4dir_ex(x, lam, u, w_raw4, C, 1, eps, y, dtype, B, C, H, W, stream);
}

int gspn_prop2d_4dir_ex(const void* x, const void* lam, const void* u, const void* w_raw4,
                        int64_t groups, int64_t k_chunk, float eps, void* y, int dtype,
                        int64_t B, int64_t C, int64_t H, int64_t W, void* stream) {
    return ex_forward(x, lam, u, w_raw4, groups, k_chunk, eps, y, nullptr, 0, false, dtype, B, C, H,
                      W, stream);
}

int gspn_prop2d_4dir_ex_ws(const void* x, const void* lam, const void* u, const void* w_raw4,
                           int64_t groups, int64_t k_chunk, float eps, void* y, void* workspace,
                           int64_t workspace_bytes, int dtype, int64_t B, int64_t C, int64_t H,
                           int64_t W, void* stream) {
    return ex_forward(x, lam, u, w_raw4, groups, k_chunk, eps, y, workspace, workspace_bytes, true,
                      dtype, B, C, H, W, stream);
}

int64_t gspn_prop2d_4dir_ex_workspace(int dtype, int64_t B, int64_t C, int64_t groups, int64_t H,
                                      int64_t W) {
    if (!valid_dtype(dtype) || check_dims(B, C, H, W, 12) != GSPN_OK) return -1;
    if (groups < 1 || groups > C || C % groups != 0) return -1;
    return shared_workspace(dtype, B, C, groups, H, W);
}

int64_t gspn_prop2d_4dir_ex_backward_workspace(int64_t B, int64_t C, int64_t groups, int64_t H,
                                               int64_t W) {
    if (check_dims(B, C, H, W, 12) != GSPN_OK) return -1;
    if (H > gspn::prop2d_backward_max_line() || W > gspn::prop2d_backward_max_line()) return -1;
    if (groups < 1 || groups > C || C % groups != 0) return -1;
    return gspn::prop2d_backward_workspace_bytes(B * C, H, W, C / groups);
}

int64_t gspn_prop2d_4dir_backward_workspace(int64_t B, int64_t C, int64_t H, int64_t W) {
    return gspn_prop2d_4dir_ex_backward_workspace(B, C, C, H, W);
}

int gspn_prop2d_4dir_ex_backward(const void* x, const void* lam, const void* u,
                                 const void* w_raw4, int64_t groups, int64_t k_chunk,
                                 const void* gy, float eps, void* gx, void* glam, void* gu,
                                 void* gw4, void* workspace, int64_t workspace_bytes, int dtype,
                                 int64_t B, int64_t C, int64_t H, int64_t W, void* stream) {
    return ex_backward(x, lam, u, w_raw4, groups, k_chunk, gy, eps, gx, glam, gu, gw4, workspace,
                       workspace_bytes, false, dtype, B, C, H, W, stream);
}

int gspn_prop2d_4dir_ex_backward_noalloc(const void* x, const void* lam, const void* u,
                                         const void* w_raw4, int64_t groups, int64_t k_chunk,
                                         const void* gy, float eps, void* gx, void* glam,
                                         void* gu, void* gw4, int dtype, int64_t B, int64_t C,
                                         int64_t H, int64_t W, void* stream) {
    return ex_backward(x, lam, u, w_raw4, groups, k_chunk, gy, eps, gx, glam, gu, gw4, nullptr, 0,
                       true, dtype, B, C, H, W, stream);
}

int64_t gspn_noalloc_scratch_bytes(void) { return gspn::noalloc_scratch_bytes(); }

int gspn_prop2d_4dir_backward(const void* x, const void* lam, const void* u,
                              const void* w_raw4, const void* gy, float eps, void* gx,
                              void* glam, void* gu, void* gw4, void* workspace,
                              int64_t workspace_bytes, int dtype, int64_t B, int64_t C,
                              int64_t H, int64_t W, void* stream) {
    return gspn_prop2d_4dir_ex_backward(x, lam, u, w_raw4, C, 1, gy, eps, gx, glam, gu, gw4,
                                        workspace, workspace_bytes, dtype, B, C, H, W, stream);
}

int64_t gspn_latent_sublayer_workspace(int dtype, int64_t B, int64_t C, int64_t Cc,
                                       int64_t groups, int64_t H, int64_t W) {
    if (!valid_dtype(dtype)) return -1;
    if (check_dims(B, Cc, H, W, 12) != GSPN_OK || C < 1 || C > kMaxTokenChannels) return -1;
    if (groups < 1 || groups > Cc || Cc % groups != 0) return -1;
    return gspn::latent_sublayer_workspace_bytes(dtype, B, Cc, groups, H, W);
}

int gspn_latent_sublayer(const void* x_tok, const void* p_down, const void* w_param,
                         const void* p_up, int64_t groups, int64_t k_chunk, float eps,
                         void* y_tok, void* workspace, int64_t workspace_bytes, int dtype,
                         int64_t B, int64_t C, int64_t Cc, int64_t H, int64_t W, void* stream) {
    if (!valid_dtype(dtype)) return GSPN_ERR_DTYPE;
    if (int s = check_dims(B, Cc, H, W, 12)) return s;
    if (C < 1 || C > kMaxTokenChannels) return GSPN_ERR_SHAPE;
    if (H * W > gspn::prop2d_max_plane(dtype, H, W)) return GSPN_ERR_SHAPE;
    if (groups < 1 || groups > Cc || Cc % groups != 0) return GSPN_ERR_SHAPE;
    if (k_chunk < 1) return GSPN_ERR_VALUE;
    if (!valid_eps(eps)) return GSPN_ERR_VALUE;
    if (!x_tok || !p_down || !w_param || !p_up || !y_tok || !workspace) return GSPN_ERR_NULL;
    const int64_t need = gspn::latent_sublayer_workspace_bytes(dtype, B, Cc, groups, H, W);
    if (workspace_bytes < need) return GSPN_ERR_SHAPE;
    const void* ptrs[] = {x_tok, p_down, w_param, p_up, y_tok, workspace};
    for (const void* p : ptrs)
        if (reinterpret_cast<uintptr_t>(p) & 15u) return GSPN_ERR_ALIGN;
    const int64_t es = elem_size(dtype);
    const int64_t tok = B * H * W * C * es;
    const void* ins[] = {x_tok, p_down, w_param, p_up};
    const int64_t in_bytes[] = {tok, Cc * C * es, (2 * Cc + 12 * groups) * Cc * es, C * Cc * es};
    for (int i = 0; i < 4; ++i)
        if (overlap(y_tok, tok, ins[i], in_bytes[i]) || overlap(workspace, need, ins[i], in_bytes[i]))
            return GSPN_ERR_ALIAS;
    if (overlap(y_tok, tok, workspace, need)) return GSPN_ERR_ALIAS;
    return launch_status(gspn::launch_latent_sublayer(
        x_tok, p_down, w_param, p_up, groups, std::min<int64_t>(k_chunk, std::max(H, W)), eps,
        y_tok, workspace, dtype, B, C, Cc, H, W, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
