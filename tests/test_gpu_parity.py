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


# bf16 planes with even sides up to 160 take the one-wavefront phase kernel
# (K = 1..5 positions a lane: sides up to 32, 64, 96, 128, 160); fp32 ones up
# to 96 the two-wavefront kernel, and fp32 ones with sides up to 256 that are
# multiples of 4 the one-launch-per-direction kernel (y accumulates; K = 1..4
# positions a lane over 64 lanes; columns in strips of 16); the rest the
# general kernel.
EDGE_SHAPES = [(1, 1), (1, 2), (2, 1), (2, 2), (3, 5), (5, 3), (1, 74), (74, 1), (63, 64), (64, 65),
               (65, 63), (74, 74), (127, 33), (13, 148), (148, 148), (256, 7),
               (98, 98), (128, 128), (130, 160), (160, 2), (2, 160), (158, 126), (96, 128), (162, 40)]
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

@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("H,W", [(1, 1), (7, 1), (1, 9), (16, 16), (27, 27), (33, 70), (74, 74)])
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
