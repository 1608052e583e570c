"""GPU parity of gspn_prop2d_4dir_ex (tap groups, chunked scans) against the
fp64 oracle's prop2d_ex, through the C ABI.

Inputs are the seeded N(0, 1) draws of spatial_line_scan_amd.inputs (grouped
taps are the "w" stream drawn at the grouped shape), rounded to the storage
type; tolerances are oracle/tolerance.py's (fp32 1e-5, bf16 2e-2).  Shapes
cover both kernels: planes up to 96 x 96 (even for bf16) take the
two-wavefront kernel, the others the general one.
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


def _problem(B, C, H, W, G, seed, dtype):
    shp = (B, C, H, W)
    return {"x": inputs.draw_torch(seed, "x", shp, dtype, DEV),
            "lam": inputs.draw_torch(seed, "lam", shp, dtype, DEV),
            "u": inputs.draw_torch(seed, "u", shp, dtype, DEV),
            "w": inputs.draw_torch(seed, "w", (4, B, G, 3, H * W), dtype, DEV)}


def _run_check(p, G, k, dtype, what):
    y = gspn.prop2d_4dir_ex(p["x"], p["lam"], p["u"], p["w"], G, k)
    torch.cuda.synchronize()
    r = oracle.prop2d_ex(p["x"], p["lam"], p["u"], p["w"], G, k)
    assert_close(_np(y), r, RTOL[dtype], what)
    return y


SHAPES = [(1, 1), (3, 5), (16, 16), (27, 27), (33, 70), (74, 74), (96, 96), (97, 40), (130, 20),
          (148, 100), (200, 36)]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("H,W", SHAPES)
@pytest.mark.parametrize("G,k", [(1, 1), (2, 1), (4, 3), (1, 2), (2, 5), (4, 200)])
def test_ex_groups_and_chunks(H, W, G, k, dtype):
    say("ex", H, W, "G", G, "k", k, dtype)
    p = _problem(2, 4, H, W, G, 7 + H + W + 10 * k + G, dtype)
    _run_check(p, G, k, dtype, "%dx%d G=%d k=%d %s" % (H, W, G, k, dtype))


@pytest.mark.parametrize("H,W", [(7, 9), (10, 4), (75, 73)])
@pytest.mark.parametrize("k", [2, 3, 4, 7])
def test_ex_ragged_segments(H, W, k):
    say("ex ragged", H, W, k)
    p = _problem(1, 3, H, W, 3, 40 + k, "fp32")
    _run_check(p, 3, k, "fp32", "%dx%d k=%d" % (H, W, k))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_ex_default_options_bitwise_equal_prop2d(dtype):
    say("ex == prop2d", dtype)
    p = inputs.problem_torch(2, 8, 74, 74, 1, dtype, DEV)
    a = gspn.prop2d_4dir(p["x"], p["lam"], p["u"], p["w"])
    b = gspn.prop2d_4dir_ex(p["x"], p["lam"], p["u"], p["w"], 8, 1)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("G,k", [(1, 1), (1, 4), (64, 4)])
def test_ex_latent1k_sampled_planes(G, k):
    """Full latent1k launch (B=32, C=64, 74 x 74, bf16); the oracle recomputes
    sampled planes with their group's taps."""
    wl = WORKLOADS["latent1k"]
    say("ex latent1k G", G, "k", k)
    p = _problem(wl.B, wl.C, wl.H, wl.W, G, 0, wl.dtype)
    y = gspn.prop2d_4dir_ex(p["x"], p["lam"], p["u"], p["w"], G, k)
    y2 = gspn.prop2d_4dir_ex(p["x"], p["lam"], p["u"], p["w"], G, k)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))   # run-to-run bitwise
    cpg = wl.C // G
    rng = np.random.default_rng(G * 100 + k)
    planes = {(0, 0), (wl.B - 1, wl.C - 1)}
    while len(planes) < 6:
        planes.add((int(rng.integers(wl.B)), int(rng.integers(wl.C))))
    w = p["w"].view(4, wl.B, G, 3, -1)
    for (b, c) in sorted(planes):
        sl = lambda t: t[b:b + 1, c:c + 1]
        g = c // cpg
        r = oracle.prop2d_ex(sl(p["x"]), sl(p["lam"]), sl(p["u"]), w[:, b:b + 1, g:g + 1], 1, k)
        assert_close(_np(sl(y)), r, RTOL[wl.dtype], "plane (%d,%d)" % (b, c))
