"""The C ABI: the library loads on any host, exports what include/gspn.h
declares, and rejects every bad argument on the host before touching a device.

No test here launches a kernel: each call has exactly one thing wrong, and
validation returns before any HIP call.  Pointers are fake addresses that are
never dereferenced.
"""
import ctypes
import os
import re

import pytest

from spatial_line_scan_amd import gspn

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "gspn.h")

OK, NULL, SHAPE, DTYPE, DIR, ALIGN, ALIAS, VALUE, HIP, SCRATCH = range(10)
A = 0x7F0000000000          # fake 16-byte-aligned device addresses, far apart
STEP = 0x10000000000


def P(i):
    return ctypes.c_void_p(A + i * STEP)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(gspn.library_path()):
        pytest.skip("libgspn.so not built")
    return gspn.lib()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|int64_t|const char\*)\s+(gspn_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(L):
    syms = declared_symbols()
    assert set(syms) >= {"gspn_abi_version", "gspn_status_str", "gspn_normalize_weights",
                         "gspn_scan_dir", "gspn_prop2d_4dir",
                         "gspn_prop2d_4dir_backward", "gspn_prop2d_4dir_backward_workspace",
                         "gspn_prop2d_4dir_ex", "gspn_latent_sublayer",
                         "gspn_latent_sublayer_workspace", "gspn_prop2d_4dir_ex_backward",
                         "gspn_prop2d_4dir_ex_backward_workspace",
                         "gspn_prop2d_4dir_ex_backward_noalloc", "gspn_noalloc_scratch_bytes"}
    for s in syms:
        assert hasattr(L, s), s


def test_version_and_status_strings(L):
    assert L.gspn_abi_version() == 7
    for s in range(10):
        assert L.gspn_status_str(s).decode().startswith("GSPN")
    assert "scratch" in L.gspn_status_str(SCRATCH).decode()
    assert L.gspn_status_str(12345)


def prop(L, x=None, lam=None, u=None, w=None, eps=1e-6, y=None, dt=0, B=2, C=3, H=5, W=7):
    return L.gspn_prop2d_4dir(x or P(0), lam or P(1), u or P(2), w or P(3), eps, y or P(5), dt,
                              B, C, H, W, None)


def scan(L, w_is_raw=1, eps=1e-6, acc=0, dt=0, B=2, C=3, H=5, W=7, d=0, x=None, y=None):
    return L.gspn_scan_dir(x or P(0), P(1), P(2), P(3), w_is_raw, eps, y or P(5), acc, dt, B, C,
                           H, W, d, None)


def norm(L, dt=0, B=2, C=3, H=5, W=7, d=4, eps=1e-6, src=None, dst=None):
    return L.gspn_normalize_weights(src or P(3), dst or P(6), dt, B, C, H, W, d, eps, None)


def test_dtype_and_direction(L):
    assert prop(L, dt=2) == DTYPE
    assert scan(L, dt=-1) == DTYPE
    assert norm(L, dt=7) == DTYPE
    assert scan(L, d=4) == DIR           # scan needs a single direction
    assert scan(L, d=-1) == DIR
    assert norm(L, d=5) == DIR


@pytest.mark.parametrize("dims", [(0, 3, 5, 7), (2, 0, 5, 7), (2, 3, 0, 7), (2, 3, 5, 0),
                                  (-1, 3, 5, 7), (1, 1, 8193, 4), (1, 1, 4, 8193),
                                  (1 << 20, 1 << 20, 2, 2), (1, 1 << 18, 64, 64)])
def test_bad_sizes(L, dims):
    B, C, H, W = dims
    assert prop(L, B=B, C=C, H=H, W=W) == SHAPE
    assert scan(L, B=B, C=C, H=H, W=W) == SHAPE
    assert norm(L, B=B, C=C, H=H, W=W) == SHAPE


def test_element_count_limit_counts_all_taps(L):
    # 12 taps per pixel-channel must stay below 2^31 elements
    assert prop(L, B=1, C=2048, H=512, W=512) == SHAPE      # 12 * 2^29 > 2^31
    assert norm(L, B=1, C=4096, H=256, W=256, d=4) == SHAPE  # 12 * 2^28 > 2^31
    # 12 * 2^26 = 805M < 2^31 is accepted: this call is rejected only by its
    # overlapping (fake) pointers
    assert norm(L, B=1, C=1024, H=256, W=256, d=4, dst=ctypes.c_void_p(A + 3 * STEP + 16)) == ALIAS


def test_bf16_plane_limit(L):
    # the plain call has no room for a bf16 plane whose fp32 direction sum
    # leaves LDS (above 160 KiB / 4 - 2 max(H, W) pixels); the workspace call
    # takes it with an fp32 accumulator plane per (b, c)
    assert prop(L, dt=1, B=1, C=1, H=256, W=256) == SHAPE
    assert L.gspn_prop2d_4dir_ex_workspace(1, 1, 2, 2, 200, 200) == 0       # fits: 40000 <= 40560
    need = L.gspn_prop2d_4dir_ex_workspace(1, 1, 2, 2, 202, 202)           # 40804 > 40556
    assert need == (2 * 202 * 202 * 4 + 255) // 256 * 256
    big = L.gspn_prop2d_4dir_ex_workspace(1, 3, 4, 2, 256, 256)             # any grouping
    assert big == 12 * 256 * 256 * 4
    assert L.gspn_prop2d_4dir_ex_workspace(0, 1, 2, 2, 256, 256) == 0       # fp32: y accumulates

    def exw(ws=P(6), nb=big, dt=1):
        return L.gspn_prop2d_4dir_ex_ws(P(0), P(1), P(2), P(3), 2, 1, 1e-6, P(5), ws, nb, dt, 3, 4,
                                        256, 256, None)
    assert exw(nb=big - 1) == SHAPE
    assert exw(ws=None) == NULL
    assert exw(ws=ctypes.c_void_p(A + 6 * STEP + 8)) == ALIGN
    assert exw(ws=P(5)) == ALIAS


@pytest.mark.parametrize("eps", [0.0, -1e-6, float("nan"), float("inf")])
def test_bad_eps(L, eps):
    assert prop(L, eps=eps) == VALUE
    assert scan(L, eps=eps) == VALUE
    assert norm(L, eps=eps) == VALUE


def test_eps_ignored_for_normalised_taps(L):
    # with w_is_raw = 0 eps is unused; the call fails later, on the alias check
    assert scan(L, w_is_raw=0, eps=float("nan"), y=P(0)) == ALIAS


def test_bad_flags(L):
    assert scan(L, w_is_raw=2) == VALUE
    assert scan(L, acc=-1) == VALUE


def test_null_pointers(L):
    null = ctypes.c_void_p(0)
    for i in range(5):
        args = [P(0), P(1), P(2), P(3), P(5)]
        args[i] = null
        assert L.gspn_prop2d_4dir(args[0], args[1], args[2], args[3], 1e-6, args[4], 0, 2, 3, 5, 7,
                                  None) == NULL
        assert L.gspn_scan_dir(args[0], args[1], args[2], args[3], 1, 1e-6, args[4], 0, 0, 2, 3, 5,
                               7, 0, None) == NULL
    assert L.gspn_normalize_weights(null, P(6), 0, 2, 3, 5, 7, 4, 1e-6, None) == NULL
    assert L.gspn_normalize_weights(P(3), null, 0, 2, 3, 5, 7, 4, 1e-6, None) == NULL


def test_misaligned(L):
    bad = ctypes.c_void_p(A + 2)           # fp32 needs 4-byte alignment
    assert prop(L, x=bad) == ALIGN
    assert prop(L, y=ctypes.c_void_p(A + 5 * STEP + 1)) == ALIGN
    assert scan(L, x=bad) == ALIGN
    assert norm(L, src=bad) == ALIGN
    odd = ctypes.c_void_p(A + 1)           # bf16 needs 2-byte alignment
    assert prop(L, x=odd, dt=1) == ALIGN
    # 8-byte offsets are fine for both types: rejected later by the alias check
    assert prop(L, x=ctypes.c_void_p(A + 5 * STEP + 8), dt=1) == ALIAS


def test_aliasing(L):
    assert prop(L, y=P(0)) == ALIAS
    assert prop(L, y=ctypes.c_void_p(A + 3 * STEP + 16)) == ALIAS          # inside w4
    n = 2 * 3 * 5 * 7 * 4
    assert prop(L, y=ctypes.c_void_p(A + 3 * STEP + 12 * n - 16)) == ALIAS  # tail of w4
    assert scan(L, y=P(0)) == ALIAS
    assert norm(L, dst=P(3)) == ALIAS


# Backward workspace layout (fp32-sized regions, each rounded up to 256 bytes):
# the pair kernel's transposed x, lambda, u, gy and two fp32 sums; with shared
# taps first the per-channel fp32 tap gradients or partial sums and the
# group's normalised taps; planes with an odd side add padded copies of the
# seven planes per pixel-channel and of the taps and tap gradients.
def r256(v):
    return (v + 255) // 256 * 256


def pair_ws(planes, H, W):
    return 6 * r256(planes * H * W * 4)


def group_ws(planes, H, W, cpg):
    return r256(12 * planes * H * W * 4) + r256(12 * (planes // cpg) * H * W * 4) if cpg > 1 else 0


def padded_ws(planes, H, W, cpg=1):
    Hp, Wp = H + H % 2, W + W % 2
    return (group_ws(planes, Hp, Wp, cpg) + pair_ws(planes, Hp, Wp) + 7 * r256(planes * Hp * Wp * 4) +
            2 * r256(12 * (planes // cpg) * Hp * Wp * 4))


# the argument checks below run on a 3 x 170 plane: too long a line for the
# pair kernel, padded or not, and small enough for LDS, so no workspace
def bwd(L, ptrs=None, eps=1e-6, ws=None, ws_bytes=0, dt=0, B=2, C=3, H=3, W=170):
    p = list(ptrs) if ptrs else [P(i) for i in range(9)]
    return L.gspn_prop2d_4dir_backward(p[0], p[1], p[2], p[3], p[4], eps, p[5], p[6], p[7], p[8],
                                       ws, ws_bytes, dt, B, C, H, W, None)


def test_backward_workspace_query(L):
    # even sides up to 160 (the pair kernel's bf16 limit): transposed x,
    # lambda, u, gy and two fp32 planes per pixel-channel, sized for fp32
    # storage
    n = 32 * 64 * 74 * 74
    assert L.gspn_prop2d_4dir_backward_workspace(32, 64, 74, 74) == 6 * 4 * n
    assert L.gspn_prop2d_4dir_backward_workspace(1, 1, 2, 96) == 6 * 768    # 256-byte regions
    assert L.gspn_prop2d_4dir_backward_workspace(2, 3, 120, 120) == 6 * 4 * 2 * 3 * 120 * 120
    assert L.gspn_prop2d_4dir_backward_workspace(1, 1, 148, 148) == 6 * ((148 * 148 * 4 + 255) // 256 * 256)
    # odd sides: the padded plane's workspace plus the padded copies
    assert L.gspn_prop2d_4dir_backward_workspace(2, 3, 5, 7) == padded_ws(6, 5, 7)
    assert L.gspn_prop2d_4dir_backward_workspace(1, 1, 115, 115) == padded_ws(1, 115, 115)
    assert L.gspn_prop2d_4dir_backward_workspace(2, 3, 121, 121) == padded_ws(6, 121, 121)
    assert L.gspn_prop2d_4dir_backward_workspace(4, 64, 147, 147) == padded_ws(256, 147, 147)
    assert L.gspn_prop2d_4dir_backward_workspace(1, 1, 159, 2) == padded_ws(1, 159, 2)
    # otherwise 7 LDS lines plus three fp32 planes fit in 160 KiB up to about 115 x 115
    assert L.gspn_prop2d_4dir_backward_workspace(2, 3, 3, 170) == 0
    assert L.gspn_prop2d_4dir_backward_workspace(1, 1, 161, 2) == 0
    assert L.gspn_prop2d_4dir_backward_workspace(2, 3, 170, 170) == 2 * 3 * 3 * 170 * 170 * 4
    assert L.gspn_prop2d_4dir_backward_workspace(1, 1, 5852, 2) == -1      # line too long
    assert L.gspn_prop2d_4dir_backward_workspace(0, 1, 4, 4) == -1
    assert L.gspn_prop2d_4dir_backward_workspace(1, 1 << 18, 64, 64) == -1


def test_backward_rejects_bad_arguments(L):
    assert bwd(L, dt=2) == DTYPE
    assert bwd(L, B=0) == SHAPE
    assert bwd(L, H=5852, W=2) == SHAPE
    assert bwd(L, eps=0.0) == VALUE
    assert bwd(L, eps=float("nan")) == VALUE
    null = ctypes.c_void_p(0)
    for i in range(9):
        ptrs = [P(j) for j in range(9)]
        ptrs[i] = null
        assert bwd(L, ptrs) == NULL
    ptrs = [P(j) for j in range(9)]
    ptrs[0] = ctypes.c_void_p(A + 2)
    assert bwd(L, ptrs) == ALIGN
    assert bwd(L, H=5, W=7) == NULL                          # padded odd planes need a workspace
    ptrs = [P(j) for j in range(9)]
    ptrs[8] = ctypes.c_void_p(A + 8 * STEP + 1)
    assert bwd(L, ptrs, dt=1) == ALIGN


def test_backward_aliasing(L):
    for o in range(5, 9):
        for other in range(9):
            if other == o:
                continue
            ptrs = [P(j) for j in range(9)]
            ptrs[o] = P(other)
            assert bwd(L, ptrs) == ALIAS, (o, other)
    ptrs = [P(j) for j in range(9)]
    ptrs[5] = ctypes.c_void_p(A + 3 * STEP + 16)            # gx inside w4
    assert bwd(L, ptrs) == ALIAS


def test_backward_workspace_checks(L):
    need = 2 * 3 * 3 * 170 * 170 * 4
    assert bwd(L, H=170, W=170) == NULL                      # workspace needed, none given
    assert bwd(L, H=6, W=8) == NULL                          # the even-sided path needs one too
    assert bwd(L, ws=P(10), ws_bytes=need - 4, H=170, W=170) == SHAPE
    assert bwd(L, ws=ctypes.c_void_p(A + 10 * STEP + 2), ws_bytes=need, H=170, W=170) == ALIGN
    assert bwd(L, ws=P(0), ws_bytes=need, H=170, W=170) == ALIAS        # over x
    assert bwd(L, ws=P(7), ws_bytes=need, H=170, W=170) == ALIAS        # over gu
    assert bwd(L, ws_bytes=-1) == SHAPE


def exb(L, groups=3, k=1, ws=None, ws_bytes=0, dt=0, B=2, C=3, H=3, W=170, ptrs=None):
    p = list(ptrs) if ptrs else [P(i) for i in range(9)]
    return L.gspn_prop2d_4dir_ex_backward(p[0], p[1], p[2], p[3], groups, k, p[4], 1e-6, p[5], p[6],
                                          p[7], p[8], ws, ws_bytes, dt, B, C, H, W, None)


def test_ex_backward_workspace_query(L):
    # shared taps add 48 bytes of fp32 tap gradients (or partial sums of tap
    # products) per pixel-channel and 48 bytes of normalised weights per
    # pixel-group, each region rounded up to 256 bytes
    assert L.gspn_prop2d_4dir_ex_backward_workspace(2, 3, 3, 3, 170) == 0
    assert L.gspn_prop2d_4dir_ex_backward_workspace(2, 3, 1, 3, 170) == group_ws(6, 3, 170, 3)
    assert L.gspn_prop2d_4dir_ex_backward_workspace(2, 3, 3, 5, 7) == padded_ws(6, 5, 7)
    assert L.gspn_prop2d_4dir_ex_backward_workspace(2, 3, 1, 5, 7) == padded_ws(6, 5, 7, 3)
    n = 32 * 64 * 74 * 74
    assert L.gspn_prop2d_4dir_ex_backward_workspace(32, 64, 64, 74, 74) == 6 * 4 * n
    assert L.gspn_prop2d_4dir_ex_backward_workspace(32, 64, 1, 74, 74) == 6 * 4 * n + 48 * n + r256(48 * n // 64)
    assert L.gspn_prop2d_4dir_ex_backward_workspace(2, 3, 2, 5, 7) == -1       # 2 does not divide 3
    assert L.gspn_prop2d_4dir_ex_backward_workspace(2, 3, 0, 5, 7) == -1


def test_ex_backward_rejects_bad_arguments(L):
    assert exb(L, groups=2) == SHAPE
    assert exb(L, groups=0) == SHAPE
    assert exb(L, k=0) == VALUE
    assert exb(L, dt=2) == DTYPE
    assert exb(L, groups=1) == NULL                          # shared taps need a workspace
    need = L.gspn_prop2d_4dir_ex_backward_workspace(2, 3, 1, 3, 170)
    assert exb(L, groups=1, ws=P(10), ws_bytes=need - 4) == SHAPE
    assert exb(L, groups=1, ws=P(0), ws_bytes=need) == ALIAS      # over x
    ptrs = [P(j) for j in range(9)]
    ptrs[8] = P(3)
    assert exb(L, ptrs=ptrs) == ALIAS                        # gw4 over w_raw4
    ptrs = [P(j) for j in range(9)]
    ptrs[8] = ctypes.c_void_p(A + 3 * STEP + 12 * 2 * 1 * 510 * 4 - 4)
    assert exb(L, groups=1, ptrs=ptrs, ws=P(10), ws_bytes=need) == ALIAS   # last word of 1-group taps


def exb_noalloc(L, groups=3, k=1, dt=0, B=2, C=3, H=3, W=170, ptrs=None):
    p = list(ptrs) if ptrs else [P(i) for i in range(9)]
    return L.gspn_prop2d_4dir_ex_backward_noalloc(p[0], p[1], p[2], p[3], groups, k, p[4], 1e-6,
                                                  p[5], p[6], p[7], p[8], dt, B, C, H, W, None)


def test_noalloc_scratch_limit(L):
    # the static scratch is 64 MiB per GPU; a problem whose workspace exceeds
    # it is rejected before anything is enqueued, one that fits is not
    # rejected for its size (not called here: it would launch)
    cap = L.gspn_noalloc_scratch_bytes()
    assert cap == 64 << 20
    assert L.gspn_prop2d_4dir_ex_backward_workspace(32, 64, 64, 74, 74) > cap   # latent1k batch
    assert exb_noalloc(L, B=32, C=64, groups=64, H=74, W=74) == SCRATCH
    assert exb_noalloc(L, B=32, C=64, groups=1, H=74, W=74) == SCRATCH
    assert L.gspn_prop2d_4dir_ex_backward_workspace(2, 64, 64, 74, 74) <= cap


def test_noalloc_rejects_bad_arguments(L):
    # same validation as gspn_prop2d_4dir_ex_backward, minus the workspace
    assert exb_noalloc(L, groups=2) == SHAPE
    assert exb_noalloc(L, k=0) == VALUE
    assert exb_noalloc(L, dt=2) == DTYPE
    assert exb_noalloc(L, B=0) == SHAPE
    ptrs = [P(j) for j in range(9)]
    ptrs[2] = None
    assert exb_noalloc(L, ptrs=ptrs) == NULL
    ptrs = [P(j) for j in range(9)]
    ptrs[6] = ctypes.c_void_p(A + 6 * STEP + 2)
    assert exb_noalloc(L, ptrs=ptrs) == ALIGN
    ptrs = [P(j) for j in range(9)]
    ptrs[8] = P(3)
    assert exb_noalloc(L, ptrs=ptrs) == ALIAS                # gw4 over w_raw4
    ptrs = [P(j) for j in range(9)]
    ptrs[5] = P(4)
    assert exb_noalloc(L, ptrs=ptrs) == ALIAS                # gx over gy


def test_ex_ws_workspace_query_and_rejections(L):
    # bf16 square planes with even sides up to 80 and shared taps use the
    # workspace (48 floats a lane-step are the most a direction keeps); other
    # sizes run as gspn_prop2d_4dir_ex and need none
    need = L.gspn_prop2d_4dir_ex_workspace(1, 32, 64, 1, 74, 74)
    assert need == 4 * 32 * 74 * 16 * 16 * 4
    assert L.gspn_prop2d_4dir_ex_workspace(1, 32, 64, 64, 74, 74) == 0      # no sharing
    assert L.gspn_prop2d_4dir_ex_workspace(0, 32, 64, 1, 74, 74) == 0       # fp32
    assert L.gspn_prop2d_4dir_ex_workspace(1, 4, 64, 1, 148, 148) == 0      # beyond 80
    assert L.gspn_prop2d_4dir_ex_workspace(1, 2, 3, 2, 6, 6) == -1          # 2 does not divide 3
    assert L.gspn_prop2d_4dir_ex_workspace(7, 2, 3, 1, 6, 6) == -1
    n6 = L.gspn_prop2d_4dir_ex_workspace(1, 2, 4, 1, 6, 6)
    assert n6 > 0

    def exw(ws=P(6), nb=n6, groups=1, dt=1, H=6, W=6, ptrs=None):
        p = list(ptrs) if ptrs else [P(i) for i in range(6)]
        return L.gspn_prop2d_4dir_ex_ws(p[0], p[1], p[2], p[3], groups, 1, 1e-6, p[5], ws, nb, dt, 2, 4,
                                        H, W, None)
    assert exw(nb=n6 - 1) == SHAPE
    assert exw(ws=None) == NULL
    assert exw(ws=ctypes.c_void_p(A + 6 * STEP + 8)) == ALIGN
    assert exw(ws=P(0)) == ALIAS
    assert exw(ws=P(5)) == ALIAS
    assert exw(groups=3) == SHAPE
    assert exw(dt=9) == DTYPE


def ex(L, groups=3, k=1, eps=1e-6, dt=0, B=2, C=3, H=5, W=7, y=None):
    return L.gspn_prop2d_4dir_ex(P(0), P(1), P(2), P(3), groups, k, eps, y or P(5), dt, B, C, H, W,
                                 None)


def test_ex_rejects_bad_groups_and_chunks(L):
    assert ex(L, groups=2) == SHAPE          # 2 does not divide 3
    assert ex(L, groups=0) == SHAPE
    assert ex(L, groups=6) == SHAPE
    assert ex(L, groups=-3) == SHAPE
    assert ex(L, k=0) == VALUE
    assert ex(L, k=-2) == VALUE
    assert ex(L, dt=2) == DTYPE
    assert ex(L, eps=0.0) == VALUE
    assert ex(L, B=0) == SHAPE


def test_ex_alias_extent_follows_groups(L):
    # groups = 1: the taps take 12 * B * H * W elements and an output starting
    # on their last element is an alias; with groups = C the tap tensor is
    # three times larger and the address just past the grouped one is inside
    taps = 12 * 2 * 1 * 5 * 7 * 4
    assert ex(L, groups=1, y=ctypes.c_void_p(A + 3 * STEP + taps - 4)) == ALIAS
    assert ex(L, groups=3, y=ctypes.c_void_p(A + 3 * STEP + taps)) == ALIAS
    assert ex(L, y=P(0)) == ALIAS


def sub(L, ptrs=None, groups=4, k=1, eps=1e-6, ws_bytes=None, dt=0, B=2, C=12, Cc=4, H=5, W=7):
    p = list(ptrs) if ptrs else [P(i) for i in range(6)]
    if ws_bytes is None:
        ws_bytes = L.gspn_latent_sublayer_workspace(dt, B, C, Cc, groups, H, W)
    return L.gspn_latent_sublayer(p[0], p[1], p[2], p[3], groups, k, eps, p[4], p[5], ws_bytes, dt,
                                  B, C, Cc, H, W, None)


def test_sublayer_workspace_query(L):
    n = L.gspn_latent_sublayer_workspace(1, 32, 1152, 64, 64, 74, 74)
    plane = 32 * 64 * 74 * 74 * 2
    assert n >= (5 + 12) * plane and n <= (5 + 12) * plane + (64 << 20)
    assert L.gspn_latent_sublayer_workspace(1, 32, 1152, 64, 1, 74, 74) < n
    assert L.gspn_latent_sublayer_workspace(2, 1, 8, 4, 4, 5, 5) == -1
    assert L.gspn_latent_sublayer_workspace(0, 1, 8, 4, 3, 5, 5) == -1      # 3 does not divide 4
    assert L.gspn_latent_sublayer_workspace(0, 1, 1 << 17, 4, 4, 5, 5) == -1


def test_sublayer_rejects_bad_arguments(L):
    assert sub(L, dt=2) == DTYPE
    assert sub(L, groups=3) == SHAPE
    assert sub(L, C=0) == SHAPE
    assert sub(L, k=0) == VALUE
    assert sub(L, eps=float("inf")) == VALUE
    need = L.gspn_latent_sublayer_workspace(0, 2, 12, 4, 4, 5, 7)
    assert sub(L, ws_bytes=need - 1) == SHAPE
    for i in range(6):
        ptrs = [P(j) for j in range(6)]
        ptrs[i] = ctypes.c_void_p(0)
        assert sub(L, ptrs) == NULL
        ptrs[i] = ctypes.c_void_p(A + i * STEP + 8)        # 16-byte alignment required
        assert sub(L, ptrs) == ALIGN
    ptrs = [P(j) for j in range(6)]
    ptrs[4] = P(0)                                          # output over the tokens
    assert sub(L, ptrs) == ALIAS
    ptrs = [P(j) for j in range(6)]
    ptrs[5] = P(2)                                          # workspace over w_param
    assert sub(L, ptrs) == ALIAS
    ptrs = [P(j) for j in range(6)]
    ptrs[4] = P(5)                                          # output over the workspace
    assert sub(L, ptrs) == ALIAS
