// Sanitizer driver for the C-ABI host layer (spatial_line_scan_amd/csrc/
// gspn_host.cpp): built host-only under AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_sanitizers.py, with the kernel
// launchers replaced by stubs that only count calls.  Every entry point is
// called with valid arguments (the stub must be reached exactly once) and
// with each kind of invalid argument (nothing may be launched): null and
// misaligned pointers, overlapping buffers, zero, negative and huge sizes
// whose products overflow 64 bits, bad element types, directions, flags and
// eps values.  Pointers are fake addresses that nothing dereferences.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <limits>

#include "gspn.h"
#include "gspn_internal.h"

namespace gspn {
static int g_launches = 0;
hipError_t launch_normalize(const void*, void*, int, int64_t, int64_t, int64_t, int, int, float,
                            hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_scan_dir(const void*, const void*, const void*, const void*, int, float, void*,
                           int, int, int64_t, int64_t, int64_t, int, hipStream_t) {
    ++g_launches; return hipSuccess;
}
hipError_t launch_prop2d(const void*, const void*, const void*, const void*, float, void*, int,
                         int64_t, int64_t, int64_t, const PropOpts&, hipStream_t) {
    ++g_launches; return hipSuccess;
}
hipError_t launch_prop2d_backward(const void*, const void*, const void*, const void*, const void*,
                                  float, void*, void*, void*, void*, void*, int, int64_t, int64_t,
                                  int64_t, const PropOpts&, hipStream_t) {
    ++g_launches; return hipSuccess;
}
hipError_t launch_prop2d_quad_shared(const void*, const void*, const void*, const void*, float, void*,
                                     int64_t, int64_t, const PropOpts&, void*, hipStream_t) {
    ++g_launches; return hipSuccess;
}
int64_t prop2d_quad_shared_workspace_bytes(int64_t planes, int64_t L, int64_t cpg) {
    return 4 * (planes / cpg) * L * 16 * 16 * 4;
}
bool prop2d_quad_shared_eligible(int dtype, int64_t, int64_t H, int64_t W, const PropOpts& o, const void*,
                                 const void*, const void*, const void*, const void*) {
    return dtype == 1 && H == W && H % 2 == 0 && H <= 80 && o.cpg >= 2 && o.k_chunk == 1;
}
hipError_t launch_latent_sublayer(const void*, const void*, const void*, const void*, int64_t,
                                  int64_t, float, void*, void*, int, int64_t, int64_t, int64_t,
                                  int64_t, int64_t, hipStream_t) {
    ++g_launches; return hipSuccess;
}
// size queries: the forms the kernels' own give (within the bounds the host
// layer checks first)
int64_t prop2d_max_plane(int dtype, int64_t, int64_t) { return dtype == 0 ? (int64_t{1} << 62) : 40000; }
int64_t prop2d_global_acc_bytes(int dtype, int64_t planes, int64_t H, int64_t W) {
    return (dtype == 1 && H * W > 40000) ? ((planes * H * W * 4 + 255) & ~int64_t{255}) : 0;
}
hipError_t launch_prop2d_global_acc(const void*, const void*, const void*, const void*, float, void*, int64_t,
                                    int64_t, int64_t, const PropOpts&, float*, hipStream_t) {
    ++g_launches; return hipSuccess;
}
bool prop2d_wide_bf16_eligible(int64_t, int64_t H, int64_t W, const void*, const void*, const void*,
                               const void*, const void*, const void*) {
    return H % 4 == 0 && W % 4 == 0 && H > 192 && W > 192 && H <= 256 && W <= 256;
}
hipError_t launch_prop2d_wide_bf16(const void*, const void*, const void*, const void*, float, void*, int64_t,
                                   int64_t, int64_t, const PropOpts&, float*, hipStream_t) {
    ++g_launches; return hipSuccess;
}
int64_t prop2d_backward_max_line() { return 8192; }
int64_t prop2d_backward_workspace_bytes(int64_t planes, int64_t H, int64_t W, int64_t cpg) {
    return 24 * planes * H * W + (cpg > 1 ? 48 * planes * H * W : 0);
}
int64_t latent_sublayer_workspace_bytes(int, int64_t B, int64_t Cc, int64_t G, int64_t H, int64_t W) {
    return 8 * B * (Cc + G) * H * W + (int64_t{32} << 20);
}
int64_t noalloc_scratch_bytes() { return int64_t{64} << 20; }
hipError_t noalloc_scratch(void** out) { *out = reinterpret_cast<void*>(uintptr_t{0x100000000}); return hipSuccess; }
}  // namespace gspn

namespace {
int fails = 0;
const void* P(int i) { return reinterpret_cast<const void*>(uintptr_t{0x7f0000000000} + uintptr_t(i) * 0x10000000000); }
void* M(int i) { return const_cast<void*>(P(i)); }

void expect(int got, int want, int launches, const char* what) {
    const int before = gspn::g_launches;
    (void)before;
    if (got != want) {
        std::fprintf(stderr, "%s: status %d, expected %d\n", what, got, want);
        ++fails;
    }
    static int last = 0;
    if (gspn::g_launches - last != launches) {
        std::fprintf(stderr, "%s: %d launches, expected %d\n", what, gspn::g_launches - last, launches);
        ++fails;
    }
    last = gspn::g_launches;
}
}  // namespace

int main() {
    const int64_t big = std::numeric_limits<int64_t>::max();
    const float nan = std::nanf(""), inf = std::numeric_limits<float>::infinity();
    // gspn_prop2d_4dir
    expect(gspn_prop2d_4dir(P(0), P(1), P(2), P(3), 1e-6f, M(5), 0, 2, 3, 5, 7, nullptr), GSPN_OK, 1, "prop ok");
    expect(gspn_prop2d_4dir(P(0), P(1), P(2), P(3), 1e-6f, M(5), 1, 2, 3, 5, 7, nullptr), GSPN_OK, 1, "prop bf16 ok");
    expect(gspn_prop2d_4dir(nullptr, P(1), P(2), P(3), 1e-6f, M(5), 0, 2, 3, 5, 7, nullptr), GSPN_ERR_NULL, 0, "prop null");
    expect(gspn_prop2d_4dir(P(0), P(1), P(2), P(3), 1e-6f, M(0), 0, 2, 3, 5, 7, nullptr), GSPN_ERR_ALIAS, 0, "prop alias");
    expect(gspn_prop2d_4dir(P(0), P(1), P(2), P(3), nan, M(5), 0, 2, 3, 5, 7, nullptr), GSPN_ERR_VALUE, 0, "prop nan eps");
    expect(gspn_prop2d_4dir(P(0), P(1), P(2), P(3), inf, M(5), 0, 2, 3, 5, 7, nullptr), GSPN_ERR_VALUE, 0, "prop inf eps");
    expect(gspn_prop2d_4dir(P(0), P(1), P(2), P(3), -1.0f, M(5), 0, 2, 3, 5, 7, nullptr), GSPN_ERR_VALUE, 0, "prop neg eps");
    expect(gspn_prop2d_4dir(P(0), P(1), P(2), P(3), 1e-6f, M(5), 7, 2, 3, 5, 7, nullptr), GSPN_ERR_DTYPE, 0, "prop dtype");
    const int64_t dims[][4] = {{0, 3, 5, 7}, {-1, 3, 5, 7}, {2, 3, 5, 9000}, {big, big, big, big},
                               {big, 2, 1, 1}, {1 << 20, 1 << 20, 1 << 20, 1 << 20}, {3, big / 2, 2, 2}};
    for (const auto& d : dims)
        expect(gspn_prop2d_4dir(P(0), P(1), P(2), P(3), 1e-6f, M(5), 0, d[0], d[1], d[2], d[3], nullptr),
               GSPN_ERR_SHAPE, 0, "prop dims");
    const void* odd = reinterpret_cast<const void*>(uintptr_t{0x7f0000000002});
    expect(gspn_prop2d_4dir(odd, P(1), P(2), P(3), 1e-6f, M(5), 0, 2, 3, 5, 7, nullptr), GSPN_ERR_ALIGN, 0, "prop align");
    // gspn_prop2d_4dir_ex
    expect(gspn_prop2d_4dir_ex(P(0), P(1), P(2), P(3), 1, 3, 1e-6f, M(5), 0, 2, 3, 5, 7, nullptr), GSPN_OK, 1, "ex ok");
    expect(gspn_prop2d_4dir_ex(P(0), P(1), P(2), P(3), 2, 1, 1e-6f, M(5), 0, 2, 3, 5, 7, nullptr), GSPN_ERR_SHAPE, 0, "ex groups");
    expect(gspn_prop2d_4dir_ex(P(0), P(1), P(2), P(3), big, 1, 1e-6f, M(5), 0, 2, 3, 5, 7, nullptr), GSPN_ERR_SHAPE, 0, "ex big groups");
    expect(gspn_prop2d_4dir_ex(P(0), P(1), P(2), P(3), 3, 0, 1e-6f, M(5), 0, 2, 3, 5, 7, nullptr), GSPN_ERR_VALUE, 0, "ex chunk");
    expect(gspn_prop2d_4dir_ex(P(0), P(1), P(2), P(3), 3, big, 1e-6f, M(5), 0, 2, 3, 5, 7, nullptr), GSPN_OK, 1, "ex huge chunk");
    // gspn_prop2d_4dir_ex_ws: workspace used (bf16, square even side, shared taps) or not
    const int64_t wse = gspn_prop2d_4dir_ex_workspace(1, 2, 4, 1, 6, 6);
    if (wse <= 0) ++fails;
    if (gspn_prop2d_4dir_ex_workspace(0, 2, 4, 1, 6, 6) != 0) ++fails;
    if (gspn_prop2d_4dir_ex_workspace(1, 2, 4, 3, 6, 6) != -1) ++fails;
    expect(gspn_prop2d_4dir_ex_ws(P(0), P(1), P(2), P(3), 1, 1, 1e-6f, M(5), M(6), wse, 1, 2, 4, 6, 6, nullptr),
           GSPN_OK, 1, "ex_ws ok");
    expect(gspn_prop2d_4dir_ex_ws(P(0), P(1), P(2), P(3), 1, 1, 1e-6f, M(5), M(6), wse - 1, 1, 2, 4, 6, 6,
                                  nullptr), GSPN_ERR_SHAPE, 0, "ex_ws small");
    expect(gspn_prop2d_4dir_ex_ws(P(0), P(1), P(2), P(3), 1, 1, 1e-6f, M(5), nullptr, wse, 1, 2, 4, 6, 6,
                                  nullptr), GSPN_ERR_NULL, 0, "ex_ws null");
    expect(gspn_prop2d_4dir_ex_ws(P(0), P(1), P(2), P(3), 1, 1, 1e-6f, M(5), M(3), wse, 1, 2, 4, 6, 6,
                                  nullptr), GSPN_ERR_ALIAS, 0, "ex_ws alias");
    expect(gspn_prop2d_4dir_ex_ws(P(0), P(1), P(2), P(3), 1, 1, 1e-6f, M(5), nullptr, 0, 0, 2, 4, 6, 6,
                                  nullptr), GSPN_OK, 1, "ex_ws unused");
    // bf16 planes beyond the on-chip sum: only with the workspace's accumulator
    const int64_t wacc = gspn_prop2d_4dir_ex_workspace(1, 2, 4, 4, 256, 256);
    if (wacc != 8 * 256 * 256 * 4) ++fails;
    expect(gspn_prop2d_4dir(P(0), P(1), P(2), P(3), 1e-6f, M(5), 1, 2, 4, 256, 256, nullptr), GSPN_ERR_SHAPE, 0,
           "prop bf16 beyond LDS");
    expect(gspn_prop2d_4dir_ex_ws(P(0), P(1), P(2), P(3), 4, 1, 1e-6f, M(5), M(6), wacc, 1, 2, 4, 256, 256,
                                  nullptr), GSPN_OK, 1, "ex_ws bf16 beyond LDS");
    expect(gspn_prop2d_4dir_ex_ws(P(0), P(1), P(2), P(3), 2, 3, 1e-6f, M(5), M(6), wacc, 1, 2, 4, 203, 201,
                                  nullptr), GSPN_OK, 1, "ex_ws bf16 beyond LDS, general");
    expect(gspn_prop2d_4dir_ex_ws(P(0), P(1), P(2), P(3), 4, 1, 1e-6f, M(5), M(6), wacc - 1, 1, 2, 4, 256, 256,
                                  nullptr), GSPN_ERR_SHAPE, 0, "ex_ws bf16 beyond LDS, small");
    expect(gspn_prop2d_4dir_ex_ws(P(0), P(1), P(2), P(3), 4, 1, 1e-6f, M(5), nullptr, wacc, 1, 2, 4, 256, 256,
                                  nullptr), GSPN_ERR_NULL, 0, "ex_ws bf16 beyond LDS, null");
    // gspn_scan_dir and gspn_normalize_weights
    for (int dir = 0; dir < 4; ++dir)
        expect(gspn_scan_dir(P(0), P(1), P(2), P(3), 1, 1e-6f, M(5), 1, 0, 2, 3, 5, 7, dir, nullptr), GSPN_OK, 1, "scan ok");
    expect(gspn_scan_dir(P(0), P(1), P(2), P(3), 1, 1e-6f, M(5), 2, 0, 2, 3, 5, 7, 0, nullptr), GSPN_ERR_VALUE, 0, "scan flag");
    expect(gspn_scan_dir(P(0), P(1), P(2), P(3), 1, 1e-6f, M(5), 0, 0, 2, 3, 5, 7, 4, nullptr), GSPN_ERR_DIR, 0, "scan all4");
    expect(gspn_scan_dir(P(0), P(1), P(2), P(3), 1, 1e-6f, M(5), 0, 0, 2, 3, 5, 7, -1, nullptr), GSPN_ERR_DIR, 0, "scan dir");
    expect(gspn_normalize_weights(P(0), M(1), 0, 2, 3, 5, 7, 4, 1e-6f, nullptr), GSPN_OK, 1, "norm ok");
    expect(gspn_normalize_weights(P(0), M(1), 0, 2, 3, 5, 7, 9, 1e-6f, nullptr), GSPN_ERR_DIR, 0, "norm dir");
    expect(gspn_normalize_weights(P(0), M(0), 0, 2, 3, 5, 7, 4, 1e-6f, nullptr), GSPN_ERR_ALIAS, 0, "norm alias");
    // gradients, with a caller workspace and with the static scratch
    const int64_t need = gspn_prop2d_4dir_ex_backward_workspace(2, 3, 1, 5, 7);
    expect(gspn_prop2d_4dir_ex_backward(P(0), P(1), P(2), P(3), 1, 2, P(4), 1e-6f, M(5), M(6), M(7), M(8),
                                        M(9), need, 0, 2, 3, 5, 7, nullptr), GSPN_OK, 1, "exb ok");
    expect(gspn_prop2d_4dir_ex_backward(P(0), P(1), P(2), P(3), 1, 2, P(4), 1e-6f, M(5), M(6), M(7), M(8),
                                        M(9), need - 1, 0, 2, 3, 5, 7, nullptr), GSPN_ERR_SHAPE, 0, "exb small ws");
    expect(gspn_prop2d_4dir_ex_backward(P(0), P(1), P(2), P(3), 1, 2, P(4), 1e-6f, M(5), M(6), M(7), M(8),
                                        M(0), need, 0, 2, 3, 5, 7, nullptr), GSPN_ERR_ALIAS, 0, "exb ws alias");
    expect(gspn_prop2d_4dir_ex_backward_noalloc(P(0), P(1), P(2), P(3), 1, 2, P(4), 1e-6f, M(5), M(6), M(7),
                                                M(8), 0, 2, 3, 5, 7, nullptr), GSPN_OK, 1, "noalloc ok");
    expect(gspn_prop2d_4dir_ex_backward_noalloc(P(0), P(1), P(2), P(3), 64, 1, P(4), 1e-6f, M(5), M(6), M(7),
                                                M(8), 1, 32, 64, 74, 74, nullptr), GSPN_ERR_SCRATCH, 0, "noalloc big");
    const int64_t needb = gspn_prop2d_4dir_backward_workspace(2, 3, 5, 7);
    expect(gspn_prop2d_4dir_backward(P(0), P(1), P(2), P(3), P(4), 1e-6f, M(5), M(6), M(7), M(8), M(9), needb,
                                     0, 2, 3, 5, 7, nullptr), GSPN_OK, 1, "bwd ok");
    expect(gspn_prop2d_4dir_backward(P(0), P(1), P(2), P(3), P(4), 1e-6f, M(5), M(6), M(6), M(8), M(9), needb,
                                     0, 2, 3, 5, 7, nullptr), GSPN_ERR_ALIAS, 0, "bwd out alias");
    for (const auto& d : dims)
        (void)gspn_prop2d_4dir_ex_backward_workspace(d[0], d[1], 1, d[2], d[3]);
    // sublayer
    const int64_t wsl = gspn_latent_sublayer_workspace(1, 2, 96, 16, 4, 6, 8);
    expect(gspn_latent_sublayer(P(0), P(1), P(2), P(3), 4, 1, 1e-6f, M(5), M(6), wsl, 1, 2, 96, 16, 6, 8,
                                nullptr), GSPN_OK, 1, "sublayer ok");
    expect(gspn_latent_sublayer(P(0), P(1), P(2), P(3), 4, 1, 1e-6f, M(5), M(6), wsl - 16, 1, 2, 96, 16, 6,
                                8, nullptr), GSPN_ERR_SHAPE, 0, "sublayer small ws");
    for (const auto& d : dims)
        (void)gspn_latent_sublayer_workspace(1, d[0], d[1], d[2], 1, d[3], d[3]);
    for (int s = -2; s < 12; ++s)
        if (!gspn_status_str(s)) ++fails;
    if (fails) {
        std::fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    std::printf("host driver: ok\n");
    return 0;
}
