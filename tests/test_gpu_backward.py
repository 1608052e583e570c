"""GPU parity of the gradient entry point (gspn_prop2d_4dir_backward) against
the fp64 oracle's prop2d_backward, through the C ABI.

Inputs are the seeded N(0, 1) draws of spatial_line_scan_amd.inputs (the
upstream gradient gy is its own stream), rounded to the storage type; the
oracle sees exactly the same values.  Each of the four gradients is compared
with oracle/tolerance.py's rule (relative to max(|r|, rms(r)) elementwise and
normwise; GRAD_RTOL: fp32 1e-5 for gx, glambda, gu and 2e-5 for the tap
gradient, a product of two scanned values; bf16 2e-2).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from spatial_line_scan_amd import gspn, inputs
from spatial_line_scan_amd.workloads import WORKLOADS
from oracle.tolerance import GRAD_RTOL, assert_close

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
NAMES = ("gx", "glam", "gu", "gw4")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _np(t):
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def _problem(B, C, H, W, seed, dtype):
    p = inputs.problem_torch(B, C, H, W, seed, dtype, DEV)
    p["gy"] = inputs.draw_torch(seed, "gy", (B, C, H, W), dtype, DEV)
    return p


def _check(got, ref, dtype, what):
    for name, g, r in zip(NAMES, got, ref):
        assert_close(_np(g).reshape(-1), np.asarray(r).reshape(-1), GRAD_RTOL[dtype][name],
                     "%s %s" % (what, name))


def _run(p, eps=1e-6):
    g = gspn.prop2d_4dir_backward(p["x"], p["lam"], p["u"], p["w"], p["gy"], eps)
    torch.cuda.synchronize()
    return g


def _oracle(p, eps=1e-6):
    return oracle.prop2d_backward(p["x"], p["lam"], p["u"], p["w"], p["gy"], eps)


@pytest.mark.parametrize("name", ["tiny", "base378"])
def test_backward_small_workloads(name):
    wl = WORKLOADS[name]
    for seed in wl.seeds[:2]:
        say("backward", name, "seed", seed)
        p = _problem(wl.B, wl.C, wl.H, wl.W, seed, wl.dtype)
        _check(_run(p), _oracle(p), wl.dtype, "%s seed %d" % (name, seed))


# Even sides take the one-wavefront-per-direction-pair kernel up to 160 in
# bf16 and 128 in fp32 (its lines cover 1 to 5 positions per lane; the two
# launches of a plane can differ), and so do square bf16 planes of odd side
# 3..159 (its odd form: 1, 2 or 3 positions a lane; planes start at even
# and odd elements); other odd shapes that fit it padded run padded; fp32
# planes whose sums leave LDS (above about 13K pixels) with sides up to 256,
# multiples of 4, the wide kernel ((120, 120) and (148, 148) in fp32); the
# rest the general kernel.
BWD_SHAPES = [(1, 1), (1, 2), (2, 1), (3, 5), (5, 3), (1, 74), (74, 1), (63, 64), (74, 74),
              (127, 33), (13, 148), (120, 120), (148, 148), (300, 5), (5, 300),
              (2, 2), (2, 96), (96, 2), (32, 34), (34, 32), (64, 66), (96, 96), (30, 66), (8, 74),
              (98, 98), (128, 128), (130, 160), (160, 2), (2, 160), (158, 126), (96, 128), (162, 40),
              (27, 27), (37, 37), (147, 147), (3, 3), (5, 5), (63, 63), (65, 65), (97, 97),
              (127, 127), (129, 129), (159, 159)]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("H,W", BWD_SHAPES)
def test_backward_edge_shapes(H, W, dtype):
    say("backward edge", H, W, dtype)
    p = _problem(2, 3, H, W, 21 + H + 5 * W, dtype)
    _check(_run(p), _oracle(p), dtype, "%dx%d %s" % (H, W, dtype))


@pytest.mark.parametrize("L,B,C", [(147, 4, 33), (65, 3, 67)])
def test_backward_odd_many_planes(L, B, C):
    # the odd form over more planes than the CUs hold at once, an odd count
    # (planes at both element parities); the oracle recomputes sampled planes
    say("backward odd planes", L, B, C)
    p = _problem(B, C, L, L, 9 + L, "bf16")
    got = _run(p)
    for t in got:
        assert bool(torch.isfinite(t).all())
    w = p["w"].view(4, B, C, 3, -1)
    gw = got[3].view(4, B, C, 3, -1)
    for (b, c) in [(0, 0), (0, 1), (B - 1, C - 1), (1, C // 2), (B - 1, 0)]:
        sl = lambda t: t[b:b + 1, c:c + 1]
        ref = oracle.prop2d_backward(sl(p["x"]), sl(p["lam"]), sl(p["u"]), w[:, b:b + 1, c:c + 1],
                                     sl(p["gy"]))
        mine = (sl(got[0]), sl(got[1]), sl(got[2]), gw[:, b:b + 1, c:c + 1])
        _check(mine, ref, "bf16", "%dx%d plane (%d,%d)" % (L, L, b, c))


# fp32 only: the one-wavefront-per-plane kernel for planes whose sums leave
# LDS (K = 2, 3, 4 positions a lane; strips of 32 columns with a partial last
# one; row and column lines of different lengths)
WIDE_BWD_SHAPES = [(116, 116), (120, 124), (148, 152), (200, 100), (100, 200), (252, 68),
                   (68, 252), (124, 256), (256, 256)]


@pytest.mark.parametrize("H,W", WIDE_BWD_SHAPES)
def test_backward_wide_fp32_shapes(H, W):
    say("backward wide", H, W)
    p = _problem(1, 2, H, W, 61 + H + 3 * W, "fp32")
    _check(_run(p), _oracle(p), "fp32", "%dx%d fp32" % (H, W))


def test_backward_wide256_sampled_planes():
    """Full wide256 launch (fp32, 1024 planes of 256 x 256); the oracle
    recomputes a sample of whole planes."""
    wl = WORKLOADS["wide256"]
    say("backward wide256")
    p = _problem(wl.B, wl.C, wl.H, wl.W, 0, wl.dtype)
    got = _run(p)
    for t in got:
        assert bool(torch.isfinite(t).all())
    w = p["w"].view(4, wl.B, wl.C, 3, -1)
    gw = got[3].view(4, wl.B, wl.C, 3, -1)
    for c in (0, 517, wl.C - 1):
        sl = lambda t: t[0:1, c:c + 1]
        ref = oracle.prop2d_backward(sl(p["x"]), sl(p["lam"]), sl(p["u"]), w[:, 0:1, c:c + 1],
                                     sl(p["gy"]))
        mine = (sl(got[0]), sl(got[1]), sl(got[2]), gw[:, 0:1, c:c + 1])
        _check(mine, ref, wl.dtype, "wide256 plane %d" % c)


def test_backward_latent1k_sampled_planes():
    """Full latent1k launch (bf16, 32 x 64 planes of 74 x 74); the oracle
    recomputes a sample of whole planes."""
    wl = WORKLOADS["latent1k"]
    say("backward latent1k")
    p = _problem(wl.B, wl.C, wl.H, wl.W, 0, wl.dtype)
    got = _run(p)
    for t in got:
        assert bool(torch.isfinite(t).all())
    w = p["w"].view(4, wl.B, wl.C, 3, -1)
    gw = got[3].view(4, wl.B, wl.C, 3, -1)
    rng = np.random.default_rng(7)
    planes = {(0, 0), (wl.B - 1, wl.C - 1)}
    while len(planes) < 6:
        planes.add((int(rng.integers(wl.B)), int(rng.integers(wl.C))))
    for (b, c) in sorted(planes):
        sl = lambda t: t[b:b + 1, c:c + 1]
        ref = oracle.prop2d_backward(sl(p["x"]), sl(p["lam"]), sl(p["u"]), w[:, b:b + 1, c:c + 1],
                                     sl(p["gy"]))
        mine = (sl(got[0]), sl(got[1]), sl(got[2]), gw[:, b:b + 1, c:c + 1])
        _check(mine, ref, wl.dtype, "latent1k plane (%d,%d)" % (b, c))


@pytest.mark.parametrize("H,W,dtype", [(74, 74, "bf16"), (148, 148, "fp32")])
def test_backward_deterministic(H, W, dtype):
    say("backward determinism", H, W, dtype)
    p = _problem(4, 16, H, W, 2, dtype)
    a = _run(p)
    b = _run(p)
    iv = torch.int16 if dtype == "bf16" else torch.int32
    for x, y in zip(a, b):
        assert torch.equal(x.view(iv), y.view(iv))


@pytest.mark.parametrize("H,W", [(9, 11), (10, 12)])
def test_backward_clamp_and_saturated_logits(H, W):
    say("backward clamp", H, W)
    B, C = 1, 4
    p = _problem(B, C, H, W, 3, "fp32")
    w = p["w"].clone().view(4, B, C, 3, H * W)
    w[:, :, 0] = -20.0 + 0.3 * w[:, :, 0]
    w[:, :, 1, :, :3] = -800.0
    w[:, :, 2, :, 5:9] = 800.0
    p["w"] = w.contiguous()
    _check(_run(p), _oracle(p), "fp32", "clamp")


def test_backward_caller_workspace_and_eps():
    """A caller-provided (oversized) workspace and a non-default eps."""
    say("backward workspace")
    B, C, H, W = 1, 2, 170, 90
    p = _problem(B, C, H, W, 4, "fp32")
    need = gspn.prop2d_4dir_backward_workspace_bytes(B, C, H, W)
    assert need == B * C * 3 * H * W * 4
    ws = torch.full((need // 4 + 1000,), float("nan"), device=DEV)
    got = gspn.prop2d_4dir_backward(p["x"], p["lam"], p["u"], p["w"], p["gy"], 1e-3, workspace=ws)
    torch.cuda.synchronize()
    _check(got, _oracle(p, 1e-3), "fp32", "workspace")


def test_autograd_function_matches_entry_point():
    say("backward autograd")
    p = _problem(2, 3, 10, 12, 5, "fp32")
    leaves = [p[k].clone().requires_grad_(True) for k in ("x", "lam", "u", "w")]
    y = gspn.Prop2d4Dir.apply(*leaves)
    y.backward(p["gy"])
    direct = _run(p)
    for leaf, g in zip(leaves, direct):
        assert torch.equal(leaf.grad.view(-1), g.view(-1))
