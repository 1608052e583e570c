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


# bf16 planes whose fp32 direction sum does not fit in LDS (above about
# 40,500 pixels) run with an fp32 accumulator plane per (b, c) in the
# workspace (gspn_prop2d_4dir_ex_ws; the binding allocates it): sides
# 196..256 that are multiples of 4 in the one-wavefront-a-plane kernel
# (202 x 202 is not: the general kernel), the rest in the general kernel;
# the plain call refuses them
@pytest.mark.parametrize("H,W", [(204, 204), (256, 256), (244, 200), (202, 202), (203, 201),
                                 (256, 170)])
@pytest.mark.parametrize("G,k", [(3, 1), (1, 4)])
def test_ex_bf16_planes_beyond_lds(H, W, G, k):
    say("ex bf16 beyond LDS", H, W, G, k)
    p = _problem(1, 3, H, W, G, 17 + H + W + k, "bf16")
    assert gspn.prop2d_4dir_ex_workspace_bytes(torch.bfloat16, 1, 3, G, H, W) == 3 * H * W * 4 + (-(3 * H * W * 4)) % 256
    y = _run_check(p, G, k, "bf16", "%dx%d bf16 G=%d k=%d" % (H, W, G, k))
    y2 = gspn.prop2d_4dir_ex(p["x"], p["lam"], p["u"], p["w"], G, k)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    if G == 3 and k == 1:
        with pytest.raises(Exception):
            gspn.prop2d_4dir(p["x"], p["lam"], p["u"], p["w"])


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


# gspn_prop2d_4dir_ex_ws: bf16 square planes with even sides up to 80, one
# segment a scan and at least 2 channels a group normalise each group's taps
# once into the workspace; the sides cover every K (positions a lane) and
# every (L - 1) mod K of the scan kernel
SHARED_SIDES = [2, 4, 14, 16, 18, 30, 32, 34, 36, 46, 48, 50, 52, 62, 64, 66, 68, 70, 72, 74, 80]


@pytest.mark.parametrize("L", SHARED_SIDES)
@pytest.mark.parametrize("B,C,G", [(2, 4, 1), (1, 8, 4)])
def test_ex_shared_weights_sides(L, B, C, G):
    say("ex shared", L, "B", B, "C", C, "G", G)
    assert gspn.prop2d_4dir_ex_workspace_bytes(torch.bfloat16, B, C, G, L, L) > 0
    p = _problem(B, C, L, L, G, 500 + L + G, "bf16")
    _run_check(p, G, 1, "bf16", "shared %dx%d G=%d" % (L, L, G))


@pytest.mark.parametrize("L", [16, 50, 74])
def test_ex_shared_weights_xcd_plane_order(L):
    # planes a multiple of 8 groups: workgroups take planes in the order that
    # keeps each tap group on one XCD; every plane is checked
    say("ex shared xcd order", L)
    B, C, G = 4, 16, 2
    p = _problem(B, C, L, L, G, 700 + L, "bf16")
    _run_check(p, G, 1, "bf16", "shared xcd order %dx%d" % (L, L))


@pytest.mark.parametrize("L", [16, 74])
def test_ex_shared_weights_deterministic_and_close_to_per_channel(L):
    say("ex shared vs per-channel", L)
    B, C, G = 4, 16, 1
    p = _problem(B, C, L, L, G, 900 + L, "bf16")
    args = (p["x"], p["lam"], p["u"], p["w"], G, 1)
    y1 = gspn.prop2d_4dir_ex(*args)
    y2 = gspn.prop2d_4dir_ex(*args)
    y_pc = gspn.prop2d_4dir_ex(*args, workspace=None)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    # the two paths round the weights differently; both are within the bf16
    # tolerance of the oracle, and of each other
    assert_close(_np(y1), _np(y_pc), RTOL["bf16"], "shared vs per-channel %dx%d" % (L, L))
    r = oracle.prop2d_ex(p["x"], p["lam"], p["u"], p["w"], G, 1)
    assert_close(_np(y1), r, RTOL["bf16"], "shared %dx%d" % (L, L))


def test_ex_shared_weights_clamp_and_saturation():
    # logits near -20 (every sigmoid tiny: the clamp at eps acts), at +-800
    # (saturated) and a large eps, through the prepared-weight kernel
    say("ex shared clamp")
    B, C, G, L = 2, 8, 2, 74
    p = _problem(B, C, L, L, G, 1234, "bf16")
    w = p["w"].float().reshape(4, B, G, 3, L * L)
    w[:, 0] = -20.0 + 0.3 * w[:, 0]
    w[0, 1, :, :, : L * L // 3] = -800.0
    w[1, 1, :, 2, L * L // 2:] = 800.0
    p["w"] = w.to(torch.bfloat16).reshape(p["w"].shape).contiguous()
    for eps in (1e-6, 1e-3):
        y = gspn.prop2d_4dir_ex(p["x"], p["lam"], p["u"], p["w"], G, 1, eps)
        torch.cuda.synchronize()
        r = oracle.prop2d_ex(p["x"], p["lam"], p["u"], p["w"], G, 1, eps)
        assert_close(_np(y), r, RTOL["bf16"], "shared clamp eps %g" % eps)


def test_ex_shared_weights_misaligned_buffers_fall_back():
    # 2-byte aligned tensors cannot take the fast kernels: the call still
    # succeeds with the workspace and matches the oracle
    say("ex shared misaligned")
    B, C, G, L = 1, 4, 1, 16
    p = _problem(B, C, L, L, G, 77, "bf16")

    def shifted(t):
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
        v = buf[1:].view(t.shape)
        v.copy_(t)
        return v
    q = {k: shifted(v) for k, v in p.items()}
    assert q["x"].data_ptr() % 4 == 2
    _run_check(q, G, 1, "bf16", "misaligned shared")
