"""GPU parity of the gradient of the extended operator
(gspn_prop2d_4dir_ex_backward: tap groups, chunked scans) against the fp64
oracle's prop2d_ex_backward, through the C ABI.

Inputs are the seeded N(0, 1) draws of spatial_line_scan_amd.inputs (grouped
taps are the "w" stream drawn at the grouped shape, gy its own stream),
rounded to the storage type; the oracle sees exactly the same values.  Each
gradient is compared with oracle/tolerance.py's GRAD_RTOL rule; a grouped tap
gradient is a sum over the channels of its group, which that rule's rms floor
covers.  Shapes cover the three kernels: even sides up to 160 (bf16) or 128
(fp32) take the one-wavefront-per-direction-pair kernel, fp32 planes above
about 13K pixels with sides multiples of 4 up to 256 the one-wavefront-per-
plane kernel, the rest the general one.
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


def _problem(B, C, H, W, G, seed, dtype):
    shp = (B, C, H, W)
    return {"x": inputs.draw_torch(seed, "x", shp, dtype, DEV),
            "lam": inputs.draw_torch(seed, "lam", shp, dtype, DEV),
            "u": inputs.draw_torch(seed, "u", shp, dtype, DEV),
            "w": inputs.draw_torch(seed, "w", (4, B, G, 3, H * W), dtype, DEV),
            "gy": inputs.draw_torch(seed, "gy", shp, dtype, DEV)}


def _run(p, G, k, eps=1e-6, workspace=None):
    g = gspn.prop2d_4dir_ex_backward(p["x"], p["lam"], p["u"], p["w"], p["gy"], G, k, eps,
                                     workspace=workspace)
    torch.cuda.synchronize()
    return g


def _oracle(p, G, k, eps=1e-6):
    return oracle.prop2d_ex_backward(p["x"], p["lam"], p["u"], p["w"], p["gy"], G, k, eps)


def _check(got, ref, dtype, what):
    for name, g, r in zip(NAMES, got, ref):
        assert_close(_np(g).reshape(-1), np.asarray(r).reshape(-1), GRAD_RTOL[dtype][name],
                     "%s %s" % (what, name))


SHAPES = [(1, 1), (3, 5), (2, 96), (16, 16), (27, 27), (32, 34), (74, 74), (96, 96), (97, 40),
          (130, 20), (148, 148), (200, 100), (65, 65)]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("H,W", SHAPES)
@pytest.mark.parametrize("G,k", [(1, 1), (2, 1), (4, 3), (1, 2), (2, 5), (4, 200)])
def test_ex_backward_groups_and_chunks(H, W, G, k, dtype):
    say("ex backward", H, W, "G", G, "k", k, dtype)
    p = _problem(2, 4, H, W, G, 11 + H + W + 10 * k + G, dtype)
    _check(_run(p, G, k), _oracle(p, G, k), dtype, "%dx%d G=%d k=%d %s" % (H, W, G, k, dtype))


@pytest.mark.parametrize("H,W", [(7, 9), (10, 4), (74, 72), (75, 73)])
@pytest.mark.parametrize("k", [2, 3, 4, 7])
def test_ex_backward_ragged_segments(H, W, k):
    say("ex backward ragged", H, W, k)
    p = _problem(1, 3, H, W, 3, 50 + k, "fp32")
    _check(_run(p, 3, k), _oracle(p, 3, k), "fp32", "%dx%d k=%d" % (H, W, k))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_ex_backward_default_options_bitwise_equal_backward(dtype):
    say("ex backward == backward", dtype)
    p = _problem(2, 8, 74, 74, 8, 1, dtype)
    a = gspn.prop2d_4dir_backward(p["x"], p["lam"], p["u"], p["w"], p["gy"])
    b = _run(p, 8, 1)
    iv = torch.int16 if dtype == "bf16" else torch.int32
    for s, t in zip(a, b):
        assert torch.equal(s.view(iv), t.view(iv))


def test_ex_backward_latent1k_sampled_planes():
    """Full latent1k launch (bf16, 32 x 64 planes of 74 x 74) with all 64
    channels sharing one tap set and four-segment scans; the oracle recomputes
    the gradients of a sample of batch entries (the tap gradient of one entry
    needs all its channels)."""
    wl = WORKLOADS["latent1k"]
    say("ex backward latent1k")
    G, k = 1, 4
    p = _problem(wl.B, wl.C, wl.H, wl.W, G, 0, wl.dtype)
    got = _run(p, G, k)
    for t in got:
        assert bool(torch.isfinite(t).all())
    gw = got[3].view(4, wl.B, G, 3, -1)
    w = p["w"].view(4, wl.B, G, 3, -1)
    for b in (0, wl.B - 1, 13):
        sl = lambda t: t[b:b + 1]
        ref = oracle.prop2d_ex_backward(sl(p["x"]), sl(p["lam"]), sl(p["u"]), w[:, b:b + 1],
                                        sl(p["gy"]), G, k)
        mine = (sl(got[0]), sl(got[1]), sl(got[2]), gw[:, b:b + 1])
        _check(mine, ref, wl.dtype, "latent1k batch %d" % b)


@pytest.mark.parametrize("H,W,dtype,G,k", [(74, 74, "bf16", 1, 4), (74, 74, "fp32", 2, 3),
                                           (130, 20, "bf16", 2, 2)])
def test_ex_backward_deterministic(H, W, dtype, G, k):
    say("ex backward determinism", H, W, dtype, G, k)
    p = _problem(4, 16, H, W, G, 2, dtype)
    a = _run(p, G, k)
    b = _run(p, G, k)
    iv = torch.int16 if dtype == "bf16" else torch.int32
    for x, y in zip(a, b):
        assert torch.equal(x.view(iv), y.view(iv))


def test_ex_backward_caller_workspace_and_eps():
    """A caller-provided (oversized, NaN-filled) workspace and a non-default
    eps, on a plane the general kernel takes with its tap gradients reduced
    across the group."""
    say("ex backward workspace")
    B, C, G, H, W = 1, 4, 2, 170, 90
    p = _problem(B, C, H, W, G, 4, "fp32")
    need = gspn.prop2d_4dir_ex_backward_workspace_bytes(B, C, G, H, W)
    ws = torch.full((need // 4 + 1000,), float("nan"), device=DEV)
    _check(_run(p, G, 3, 1e-3, workspace=ws), _oracle(p, G, 3, 1e-3), "fp32", "workspace")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_ex_autograd_function_matches_entry_point(dtype):
    say("ex autograd", dtype)
    G, k = 2, 3
    p = _problem(2, 4, 10, 12, G, 6, dtype)
    leaves = [p[n].clone().requires_grad_(True) for n in ("x", "lam", "u", "w")]
    y = gspn.Prop2d4DirEx.apply(*leaves, G, k)
    y.backward(p["gy"])
    direct = _run(p, G, k)
    iv = torch.int16 if dtype == "bf16" else torch.int32
    for leaf, g in zip(leaves, direct):
        assert torch.equal(leaf.grad.reshape(-1).view(iv), g.reshape(-1).view(iv))
