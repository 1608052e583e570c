"""GPU parity: every entry point of libgspn against the fp64 oracle.

All calls go through the C ABI (spatial_line_scan_amd.gspn).  Inputs are the
seeded N(0, 1) draws of spatial_line_scan_amd.inputs, rounded to the storage
type; the oracle sees exactly the same values.  Tolerances: oracle/tolerance.py.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from spatial_line_scan_amd import gspn, inputs
from spatial_line_scan_amd.workloads import WORKLOADS
from oracle.tolerance import RTOL, assert_close

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _np(t):
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def _problem(B, C, H, W, seed, dtype, device=DEV):
    return inputs.problem_torch(B, C, H, W, seed, dtype, device)


# ------------------------------------------------------------------ prop2d

@pytest.mark.parametrize("name", ["tiny", "base378"])
def test_prop2d_small_workloads_all_seeds(name):
    wl = WORKLOADS[name]
    for seed in wl.seeds:
        say("prop2d", name, "seed", seed)
        p = _problem(wl.B, wl.C, wl.H, wl.W, seed, wl.dtype)
        y = gspn.prop2d_4dir(p["x"], p["lam"], p["u"], p["w"])
        torch.cuda.synchronize()
        r = oracle.prop2d(p["x"], p["lam"], p["u"], p["w"])
        assert_close(_np(y), r, RTOL[wl.dtype], "%s seed %d" % (name, seed))


# Forward dispatch.  bf16: square planes with even sides up to 80 take the
# four-directions-a-wavefront kernel (K = 1..5 positions a lane in 16-lane
# rows), except that sides 66..80 with at most 512 planes, even sides
# 82..150 and odd sides 97..149 take the kernel with the row and column
# scans in different wavefronts; other planes with sides up to 160 take the
# rows-then-columns phase kernel.
# fp32: planes up to 96 the two-wavefront pair kernel, planes with sides up
# to 256 that are multiples of 4 the one-launch-per-direction kernel (y
# accumulates; columns in strips of 32).  The rest take the general kernel.
EDGE_SHAPES = [(1, 1), (1, 2), (2, 1), (2, 2), (3, 5), (5, 3), (1, 74), (74, 1), (63, 64), (64, 65),
               (65, 63), (74, 74), (127, 33), (13, 148), (148, 148), (256, 7),
               (98, 98), (128, 128), (130, 160), (160, 2), (2, 160), (158, 126), (96, 128), (162, 40),
               (27, 27), (37, 37), (75, 75), (147, 147), (147, 146), (33, 147)]
# fp32 only: the one-launch-per-direction kernel (bf16 planes this large are
# rejected: no bf16 kernel holds their direction sum)
WIDE_SHAPES = [(100, 100), (4, 256), (256, 4), (200, 100), (100, 196), (148, 152), (256, 256),
               (252, 68), (120, 120)]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("H,W", EDGE_SHAPES)
def test_prop2d_edge_shapes(H, W, dtype):
    say("prop2d edge", H, W, dtype)
    B, C = 2, 3
    p = _problem(B, C, H, W, 11 + H + 3 * W, dtype)
    y = gspn.prop2d_4dir(p["x"], p["lam"], p["u"], p["w"])
    torch.cuda.synchronize()
    r = oracle.prop2d(p["x"], p["lam"], p["u"], p["w"])
    assert_close(_np(y), r, RTOL[dtype], "%dx%d %s" % (H, W, dtype))


def _sampled_planes(B, C, k=6):
    planes = {(0, 0), (B - 1, C - 1), (0, C - 1), (B - 1, 0)}
    rng = np.random.default_rng(B * 1000 + C)
    while len(planes) < min(k, B * C):
        planes.add((int(rng.integers(B)), int(rng.integers(C))))
    return sorted(planes)


# bf16 planes that the one-wavefront form of the phase kernel takes (LDS for
# four planes a CU, a plane for every SIMD: 1024 planes here) with K = 1 .. 5
# positions a lane; fewer planes take its two-wavefront form
ONE_WAVE_SHAPES = [(16, 16), (64, 64), (30, 66), (74, 74), (20, 120), (8, 150)]


@pytest.mark.parametrize("H,W", ONE_WAVE_SHAPES)
def test_prop2d_phase_one_wave_form(H, W):
    say("prop2d one-wave", H, W)
    p = _problem(8, 128, H, W, 77 + H + 5 * W, "bf16")
    y = gspn.prop2d_4dir(p["x"], p["lam"], p["u"], p["w"])
    torch.cuda.synchronize()
    assert_close(_np(y), oracle.prop2d(p["x"], p["lam"], p["u"], p["w"]), RTOL["bf16"],
                 "%dx%d bf16, 1024 planes" % (H, W))


# square bf16 planes with even sides up to 80 take the kernel that scans the
# four directions at once (16 lanes a direction, K = 1 .. 5 positions a lane);
# sides cover every K and every value of (L - 1) mod K it is built for.  Sides
# above 64 take it only with more than 512 planes.
QUAD_SIDES = [2, 4, 6, 14, 16, 18, 30, 32, 34, 36, 38, 46, 48, 50, 52, 62, 64, 66, 68, 70, 72, 74,
              76, 78, 80]


@pytest.mark.parametrize("L", QUAD_SIDES)
def test_prop2d_quad_sides(L):
    say("prop2d quad", L)
    B, C = (3, 5) if L <= 64 else (6, 90)
    p = _problem(B, C, L, L, 101 + L, "bf16")
    y = gspn.prop2d_4dir(p["x"], p["lam"], p["u"], p["w"])
    torch.cuda.synchronize()
    assert_close(_np(y), oracle.prop2d(p["x"], p["lam"], p["u"], p["w"]), RTOL["bf16"],
                 "%dx%d bf16" % (L, L))


# square bf16 planes with even sides 66..80 and at most 512 planes, and sides
# 82..150, take the kernel that runs the row and the column scans in different
# wavefronts: a wavefront a direction (64 lanes, K = 2 up to 128, 3 up to 150)
# at 66..80 and 98..150, two wavefronts a plane (32 lanes a direction, K = 3)
# at 82..96; the sides cover every (L - 1) mod K an even side has.  Odd sides
# 97..149 take its wavefront-a-direction form (every (L - 1) mod K an odd
# side has; planes start at even and odd elements, the middle row and column
# are met by both scans of a pair).
DUO_SIDES = [66, 68, 70, 74, 80, 82, 84, 86, 90, 94, 96, 98, 100, 112, 126, 128, 130, 132, 134, 136,
             138, 148, 150, 97, 99, 101, 115, 127, 129, 131, 133, 147, 149]


@pytest.mark.parametrize("L", DUO_SIDES)
def test_prop2d_duo_sides(L):
    say("prop2d duo", L)
    p = _problem(2, 5, L, L, 301 + L, "bf16")
    y = gspn.prop2d_4dir(p["x"], p["lam"], p["u"], p["w"])
    torch.cuda.synchronize()
    assert_close(_np(y), oracle.prop2d(p["x"], p["lam"], p["u"], p["w"]), RTOL["bf16"],
                 "%dx%d bf16" % (L, L))


@pytest.mark.parametrize("L,B,C", [(147, 4, 71), (99, 3, 101)])
def test_prop2d_duo_odd_many_planes(L, B, C):
    # more planes than the CUs hold at once, an odd count: planes at every
    # element parity, the last one ending inside a dword of the tensor
    say("prop2d duo odd planes", L, B, C)
    p = _problem(B, C, L, L, 5 + L, "bf16")
    y = gspn.prop2d_4dir(p["x"], p["lam"], p["u"], p["w"])
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all())
    for (b, c) in _sampled_planes(B, C, k=8):
        sl = lambda t: t[b:b + 1, c:c + 1]
        r = oracle.prop2d(sl(p["x"]), sl(p["lam"]), sl(p["u"]), p["w"][:, b:b + 1, c:c + 1])
        assert_close(_np(sl(y)), r, RTOL["bf16"], "%dx%d plane (%d,%d)" % (L, L, b, c))


def test_prop2d_duo_and_quad_agree_bitwise():
    # both kernels add each pixel's four directional terms in step order (the
    # terms of a step's meeting pixels after the scan), so the plane a small
    # launch computes with a wavefront a direction equals the one a full
    # launch computes with one wavefront a plane
    say("prop2d duo vs quad 74x74")
    p = _problem(8, 80, 74, 74, 77, "bf16")            # 640 planes: the quad kernel
    y_all = gspn.prop2d_4dir(p["x"], p["lam"], p["u"], p["w"])
    sl = lambda t: t[1:2].contiguous()                   # 80 planes: the duo kernel
    y_one = gspn.prop2d_4dir(sl(p["x"]), sl(p["lam"]), sl(p["u"]), p["w"][:, 1:2].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(y_all[1:2], y_one)


# Plane counts above what the CUs hold at once (LDS allows four 74 x 74
# planes a CU) run in several rounds of workgroups; the oracle checks sampled
# planes of every round.
PERSISTENT_CASES = [(16, 19, 1000), (34, 5, 1000), (50, 3, 700), (64, 2, 650), (74, 3, 370), (80, 2, 410)]


@pytest.mark.parametrize("L,B,C", PERSISTENT_CASES)
def test_prop2d_quad_planes_beyond_one_round(L, B, C):
    say("prop2d quad rounds", L, B, C)
    p = _problem(B, C, L, L, 7 + L, "bf16")
    y = gspn.prop2d_4dir(p["x"], p["lam"], p["u"], p["w"])
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all())
    for (b, c) in _sampled_planes(B, C, k=10):
        sl = lambda t: t[b:b + 1, c:c + 1]
        r = oracle.prop2d(sl(p["x"]), sl(p["lam"]), sl(p["u"]), p["w"][:, b:b + 1, c:c + 1])
        assert_close(_np(sl(y)), r, RTOL["bf16"], "%dx%d plane (%d,%d)" % (L, L, b, c))


@pytest.mark.parametrize("L,B,C", [(74, 3, 370), (80, 2, 410), (34, 5, 1000), (74, 2, 1100)])
def test_prop2d_quad_persistent_grid_matches_single_rounds(L, B, C):
    # A launch of more planes than the CUs keep resident walks the planes
    # with a resident-sized grid (a workgroup takes planes blockIdx.x,
    # blockIdx.x + gridDim.x, ..., the next one's inputs loading while it
    # finishes the current one).  Every plane of it must equal the same plane
    # from a launch of one image (C planes, one round: the same kernel, or
    # the wavefront-a-direction kernel, which sums in the same order).
    say("prop2d persistent vs single rounds", L, B, C)
    p = _problem(B, C, L, L, 11 + L + C, "bf16")
    y = gspn.prop2d_4dir(p["x"], p["lam"], p["u"], p["w"])
    parts = []
    for b in range(B):
        sl = lambda t: t[b:b + 1].contiguous()
        parts.append(gspn.prop2d_4dir(sl(p["x"]), sl(p["lam"]), sl(p["u"]), p["w"][:, b:b + 1].contiguous()))
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), torch.cat(parts).view(torch.int16))


@pytest.mark.parametrize("H,W", WIDE_SHAPES)
def test_prop2d_wide_fp32_shapes(H, W):
    say("prop2d wide", H, W)
    p = _problem(2, 3, H, W, 31 + H + 7 * W, "fp32")
    y = gspn.prop2d_4dir(p["x"], p["lam"], p["u"], p["w"])
    torch.cuda.synchronize()
    assert_close(_np(y), oracle.prop2d(p["x"], p["lam"], p["u"], p["w"]), RTOL["fp32"],
                 "%dx%d fp32" % (H, W))


@pytest.mark.parametrize("name", ["latent1k", "latent2k", "wide256"])
def test_prop2d_full_size_sampled_planes(name):
    """Full-size launch; the oracle recomputes a sample of whole planes."""
    wl = WORKLOADS[name]
    for seed in wl.seeds:
        say("prop2d full size", name, "seed", seed)
        p = _problem(wl.B, wl.C, wl.H, wl.W, seed, wl.dtype)
        y = gspn.prop2d_4dir(p["x"], p["lam"], p["u"], p["w"])
        torch.cuda.synchronize()
        assert bool(torch.isfinite(y).all())
        for (b, c) in _sampled_planes(wl.B, wl.C):
            sl = lambda t: t[b:b + 1, c:c + 1]
            r = oracle.prop2d(sl(p["x"]), sl(p["lam"]), sl(p["u"]), p["w"][:, b:b + 1, c:c + 1])
            assert_close(_np(sl(y)), r, RTOL[wl.dtype], "%s plane (%d,%d)" % (name, b, c))
        del p, y
        torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["latent1k", "base378", "latent2k"])
def test_prop2d_deterministic(name):
    wl = WORKLOADS[name]
    say("determinism", name)
    p = _problem(wl.B, wl.C, wl.H, wl.W, 0, wl.dtype)
    y1 = gspn.prop2d_4dir(p["x"], p["lam"], p["u"], p["w"])
    y2 = gspn.prop2d_4dir(p["x"], p["lam"], p["u"], p["w"])
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16) if y1.dtype == torch.bfloat16 else y1.view(torch.int32),
                       y2.view(torch.int16) if y2.dtype == torch.bfloat16 else y2.view(torch.int32))


def test_prop2d_clamp_and_saturated_logits():
    """Logits deep in the clamp (-20) and underflowing sigmoids (-800, +800)."""
    say("prop2d clamp")
    B, C, H, W = 1, 4, 9, 11
    p = _problem(B, C, H, W, 3, "fp32")
    w = p["w"].clone().view(4, B, C, 3, H * W)
    w[:, :, 0] = -20.0
    w[:, :, 1, :, :3] = -800.0
    w[:, :, 2, :, 5:9] = 800.0
    w[:, :, 3] = torch.where(torch.arange(3 * H * W, device=DEV).view(3, H * W) % 2 == 0, -800.0, 2.0)
    y = gspn.prop2d_4dir(p["x"], p["lam"], p["u"], w)
    torch.cuda.synchronize()
    r = oracle.prop2d(p["x"], p["lam"], p["u"], w)
    assert_close(_np(y), r, RTOL["fp32"], "clamp")


def test_prop2d_writes_into_given_output_and_rejects_big_bf16_planes():
    say("prop2d out / limits")
    p = _problem(1, 2, 6, 6, 0, "bf16")
    out = torch.full((1, 2, 6, 6), 7.0, dtype=torch.bfloat16, device=DEV)
    y = gspn.prop2d_4dir(p["x"], p["lam"], p["u"], p["w"], out=out)
    torch.cuda.synchronize()
    assert y.data_ptr() == out.data_ptr()
    r = oracle.prop2d(p["x"], p["lam"], p["u"], p["w"])
    assert_close(_np(out), r, RTOL["bf16"])
    big = torch.zeros((1, 1, 256, 256), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        gspn.prop2d_4dir(big, big.clone(), big.clone(), torch.zeros(12 * 256 * 256, dtype=torch.bfloat16,
                                                                  device=DEV))


# ------------------------------------------------------------------ scan_dir

# One wavefront a plane, lines up to 256 (K = 1 .. 4 positions a lane).
# Rows (top-down, bottom-up) stream, with whole-window loads where K divides
# the row and windows are whole dwords (74, 70, 200; fp32 also 27, 129).
# Columns stage lambda x one strip of 64 (bf16) or 32 (fp32) columns at a
# time in LDS, transposed (one strip at 16, 27, 33; a partial last strip at
# 70, 74, 129, 193, 200, 210; bf16 odd W moves one element a lane, W a
# multiple of 4 or 8 wider vectors).  Longer lines take the general kernel:
# (1, 300) rows.
SCAN_DIR_SHAPES = [(1, 1), (7, 1), (1, 9), (2, 2), (16, 16), (27, 27), (33, 70), (74, 74), (65, 129),
                   (129, 65), (190, 200), (256, 40), (3, 193), (1, 300), (210, 210), (128, 34),
                   (64, 48)]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("H,W", SCAN_DIR_SHAPES)
def test_scan_dir_raw_and_normalised(H, W, dtype):
    B, C = 2, 3
    p = _problem(B, C, H, W, 5 + H * W, dtype)
    w4 = p["w"].view(4, B, C, 3, H * W)
    for d in range(4):
        say("scan_dir", d, H, W, dtype)
        y = gspn.scan_dir(p["x"], p["lam"], p["u"], w4[d].contiguous(), d)
        torch.cuda.synchronize()
        r = oracle.scan_dir(p["x"], p["lam"], p["u"], w4[d], d, w_is_raw=True)
        assert_close(_np(y), r, RTOL[dtype], "raw dir %d" % d)
        # pre-normalised arbitrary weights (not row-stochastic), in-range magnitudes
        wn = (0.5 * torch.tanh(w4[d].float())).to(w4.dtype).contiguous()
        y = gspn.scan_dir(p["x"], p["lam"], p["u"], wn, d, w_is_raw=False)
        torch.cuda.synchronize()
        r = oracle.scan_dir(p["x"], p["lam"], p["u"], wn, d, w_is_raw=False)
        assert_close(_np(y), r, RTOL[dtype], "normalised dir %d" % d)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_scan_dir_latent1k_sampled_planes(dtype):
    """B=32, C=64, 74x74 (the latent1k shape): every direction, raw and
    pre-normalised taps, and an accumulated four-direction sum, checked on
    sampled planes."""
    B, C, H, W = 32, 64, 74, 74
    p = _problem(B, C, H, W, 4242, dtype)
    w4 = p["w"].view(4, B, C, 3, H * W)
    planes = _sampled_planes(B, C)
    acc = torch.zeros_like(p["x"])
    for d in range(4):
        wd = w4[d].contiguous()
        wn = (0.5 * torch.tanh(wd.float())).to(wd.dtype).contiguous()
        say("scan_dir latent1k", d, dtype)
        y_raw = gspn.scan_dir(p["x"], p["lam"], p["u"], wd, d)
        y_nrm = gspn.scan_dir(p["x"], p["lam"], p["u"], wn, d, w_is_raw=False)
        gspn.scan_dir(p["x"], p["lam"], p["u"], wd, d, out=acc, accumulate=True)
        torch.cuda.synchronize()
        for b, c in planes:
            sl = (slice(b, b + 1), slice(c, c + 1))
            args = [p[k][sl] for k in ("x", "lam", "u")]
            r = oracle.scan_dir(*args, wd[sl], d, w_is_raw=True)
            assert_close(_np(y_raw[sl]), r, RTOL[dtype], "raw dir %d plane %d,%d" % (d, b, c))
            r = oracle.scan_dir(*args, wn[sl], d, w_is_raw=False)
            assert_close(_np(y_nrm[sl]), r, RTOL[dtype], "normalised dir %d plane %d,%d" % (d, b, c))
    if dtype == "fp32":
        for b, c in planes:
            sl = (slice(b, b + 1), slice(c, c + 1))
            r = oracle.prop2d(*[p[k][sl] for k in ("x", "lam", "u")],
                              w4[:, b:b + 1, c:c + 1].contiguous())
            assert_close(_np(acc[sl]), r, RTOL[dtype], "accumulated plane %d,%d" % (b, c))


def test_scan_dir_accumulate_sums_to_prop2d():
    """Four accumulated fp32 scans equal the fused four-direction launch."""
    say("scan_dir accumulate")
    B, C, H, W = 2, 5, 19, 23
    p = _problem(B, C, H, W, 9, "fp32")
    w4 = p["w"].view(4, B, C, 3, H * W)
    y = torch.zeros_like(p["x"])
    for d in range(4):
        gspn.scan_dir(p["x"], p["lam"], p["u"], w4[d].contiguous(), d, out=y, accumulate=True)
    torch.cuda.synchronize()
    r = oracle.prop2d(p["x"], p["lam"], p["u"], p["w"])
    assert_close(_np(y), r, RTOL["fp32"])


# ------------------------------------------------------------------ normalize

@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("H,W", [(1, 1), (1, 5), (6, 1), (9, 13), (74, 74)])
def test_normalize_weights(H, W, dtype):
    say("normalize", H, W, dtype)
    B, C = 2, 3
    p = _problem(B, C, H, W, 21, dtype)
    w = p["w"].clone()
    w.view(-1)[:7] = torch.tensor([-20.0, -800.0, 800.0, 0.0, 3.5, -3.5, 1.0], dtype=w.dtype)
    wn = gspn.normalize_weights(w, gspn.ALL4, B, C, H, W)
    torch.cuda.synchronize()
    w64 = w.view(4, B * C, 3, H * W).to("cpu", torch.float32).numpy()
    for d in range(4):
        NL, L = oracle.line_geometry(d, H, W)
        r = oracle.normalize(w64[d].reshape(B * C, 3, NL, L), NL, L)
        g = _np(wn.view(4, B * C, 3, H * W)[d]).reshape(r.shape)
        # weights lie in [0, 1]: compare absolutely at the storage precision
        tol = 2e-6 if dtype == "fp32" else 8e-3
        assert np.max(np.abs(g - r)) <= tol, "dir %d" % d
        one = wn.view(4, B * C, 3, H * W)[d].float().reshape(B * C, 3, NL, L)
        assert torch.all(one[:, 0, :, 0] == 0) and torch.all(one[:, 2, :, L - 1] == 0)
    # single-direction call equals the matching block of the ALL4 call
    w_lr = w.view(4, -1)[2].contiguous()
    wn_lr = gspn.normalize_weights(w_lr, gspn.LR, B, C, H, W)
    torch.cuda.synchronize()
    assert torch.equal(wn_lr, wn.view(4, -1)[2])
