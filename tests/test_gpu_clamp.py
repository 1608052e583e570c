"""GPU parity of the normalisation's edge branches on every kernel the
dispatch can take, forward and backward, against the fp64 oracle.

The fused normalisation (paper text §5.1, "Fused CUDA normalization":
sigmoid, local sum, clamp, divide; the reading notes' normalisation formula)
has branches that N(0, 1) logits never reach:
  - the clamp S = max(sum of sigmoids, eps) with the sum below eps: logits
    near -20 with eps = 1e-6, or near -8 with eps = 1e-3, where the sum
    straddles the threshold;
  - sigmoids that saturate to exactly 0 or 1: logits at -800 and +800;
  - pixels whose three taps all vanish (every tap at -800: the sum is 0 and
    the clamp alone keeps the division finite).
`_edge_logits` writes these patterns into the taps channel by channel
(channel c mod 4 selects the pattern), so every plane count and kernel form
below sees all of them.  The oracle sees the same (storage-rounded) values.

Also here: non-finite values in one plane must not reach another plane
(every kernel's slots past a line's end, and its look-ahead loads, read
memory of the neighbouring plane).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from spatial_line_scan_amd import gspn, inputs
from oracle.tolerance import GRAD_RTOL, RTOL, assert_close

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
NAMES = ("gx", "glam", "gu", "gw4")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _np(t):
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def _edge_logits(w, B, C, H, W, mode):
    """Taps [4][B][C][3][H W] (any layout of the last axis) with per-channel
    edge patterns.  mode "deep": clamp at eps = 1e-6 and saturation;
    mode "eps": sums near eps = 1e-3."""
    G = w.numel() // (4 * B * 3 * H * W)
    v = w.view(4, B, G, 3, H * W).clone()
    n = H * W
    for c in range(min(G, 4)):
        sl = slice(c, G, 4)
        if mode == "deep":
            if c == 0:    # every sum far below 1e-6: the clamped branch
                v[:, :, sl] = -20.0 + 0.3 * v[:, :, sl]
            elif c == 1:  # saturated-to-zero left taps on the first quarter
                v[:, :, sl, 0, : max(1, n // 4)] = -800.0
            elif c == 2:  # saturated-to-one right taps on a middle band
                v[:, :, sl, 2, n // 3: max(n // 3 + 1, n // 2)] = 800.0
            else:         # alternating: pixels whose three taps all vanish
                idx = torch.arange(3 * n, device=w.device).view(3, n)
                v[:, :, sl] = torch.where(idx % 2 == 0, torch.full_like(v[:, :, sl], -800.0),
                                          torch.full_like(v[:, :, sl], 2.0))
        else:
            if c % 2 == 0:  # sums of three sigmoids near 1e-3: both sides of the clamp
                v[:, :, sl] = -8.0 + 0.7 * v[:, :, sl]
    return v.view(w.shape).contiguous()


def _problem(B, C, H, W, seed, dtype, mode, G=None):
    p = inputs.problem_torch(B, C, H, W, seed, dtype, DEV)
    if G is not None and G != C:
        p["w"] = inputs.draw_torch(seed, "w", (4, B, G, 3, H, W), dtype, DEV).view(-1)
    p["w"] = _edge_logits(p["w"], B, C, H, W, mode)
    p["gy"] = inputs.draw_torch(seed, "gy", (B, C, H, W), dtype, DEV)
    return p


EPS = {"deep": 1e-6, "eps": 1e-3}

# (H, W, dtype, B, C): the kernel each shape takes in the forward dispatch
#   74 x 74 bf16, 1024 planes       four-direction-at-once kernel
#   30 x 66 bf16, 1024 planes       phase kernel, one wavefront a plane
#   148 x 148, 40 x 30 bf16, few     phase kernel, two wavefronts a plane
#   74 x 74, 9 x 11 fp32             two-wavefront fp32 kernel
#   120 x 120, 256 x 252 fp32        wide fp32 kernel (y accumulates)
#   27 x 27, 37 x 35 bf16            phase kernel, odd sides
#   74 x 74, 90 x 90 bf16, few       row and column scans in different wavefronts
#   147 x 147, 99 x 99 bf16          the same, odd form (K = 3, 2)
FWD_CASES = [(74, 74, "bf16", 8, 128), (30, 66, "bf16", 8, 128), (148, 148, "bf16", 1, 8),
             (40, 30, "bf16", 2, 4), (74, 74, "fp32", 1, 8), (9, 11, "fp32", 1, 4),
             (120, 120, "fp32", 1, 4), (256, 252, "fp32", 1, 4), (27, 27, "bf16", 2, 4),
             (37, 35, "bf16", 1, 4), (74, 74, "bf16", 2, 4), (90, 90, "bf16", 1, 4),
             (147, 147, "bf16", 1, 5), (99, 99, "bf16", 1, 5)]


def _sampled(B, C):
    planes = {(0, 0), (0, 1), (0, 2), (0, 3), (B - 1, C - 1)}
    return sorted(planes)


@pytest.mark.parametrize("mode", ["deep", "eps"])
@pytest.mark.parametrize("H,W,dtype,B,C", FWD_CASES)
def test_forward_edge_logits(H, W, dtype, B, C, mode):
    say("forward edge logits", H, W, dtype, B, C, mode)
    p = _problem(B, C, H, W, 13 + H, dtype, mode)
    eps = EPS[mode]
    y = gspn.prop2d_4dir(p["x"], p["lam"], p["u"], p["w"], eps)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all())
    w = p["w"].view(4, B, C, 3, -1)
    for (b, c) in _sampled(B, C):
        sl = lambda t: t[b:b + 1, c:c + 1]
        r = oracle.prop2d(sl(p["x"]), sl(p["lam"]), sl(p["u"]), w[:, b:b + 1, c:c + 1], eps)
        assert_close(_np(sl(y)), r, RTOL[dtype], "%dx%d %s plane (%d,%d) %s" % (H, W, dtype, b, c, mode))


# grouped taps and chunked scans: G = 1 (all channels share the pattern of
# their one tap set), k_chunk = 4
@pytest.mark.parametrize("mode", ["deep", "eps"])
@pytest.mark.parametrize("G,k", [(1, 1), (8, 4)])
def test_forward_edge_logits_groups_chunks(G, k, mode):
    B, C, H, W = 2, 8, 74, 74
    say("forward edge logits ex", G, k, mode)
    p = _problem(B, C, H, W, 29, "bf16", mode, G=G)
    eps = EPS[mode]
    y = gspn.prop2d_4dir_ex(p["x"], p["lam"], p["u"], p["w"], G, k, eps)
    torch.cuda.synchronize()
    r = oracle.prop2d_ex(p["x"], p["lam"], p["u"], p["w"], G, k, eps)
    assert_close(_np(y), r, RTOL["bf16"], "G=%d k=%d %s" % (G, k, mode))


# backward: 74 x 74 (bf16 and fp32) the pair kernel, 148 x 152 fp32 the wide
# kernel, 27 x 27, 65 x 65 and 147 x 147 bf16 the pair kernel's odd form,
# 9 x 11 fp32 the pair kernel on the padded plane
BWD_CASES = [(74, 74, "bf16", 2, 4), (74, 74, "fp32", 1, 4), (148, 152, "fp32", 1, 4),
             (27, 27, "bf16", 1, 4), (9, 11, "fp32", 1, 4), (65, 65, "bf16", 1, 5),
             (147, 147, "bf16", 1, 5)]


@pytest.mark.parametrize("mode", ["deep", "eps"])
@pytest.mark.parametrize("H,W,dtype,B,C", BWD_CASES)
def test_backward_edge_logits(H, W, dtype, B, C, mode):
    say("backward edge logits", H, W, dtype, B, C, mode)
    p = _problem(B, C, H, W, 17 + W, dtype, mode)
    eps = EPS[mode]
    got = gspn.prop2d_4dir_backward(p["x"], p["lam"], p["u"], p["w"], p["gy"], eps)
    torch.cuda.synchronize()
    ref = oracle.prop2d_backward(p["x"], p["lam"], p["u"], p["w"], p["gy"], eps)
    for name, g, r in zip(NAMES, got, ref):
        assert_close(_np(g).reshape(-1), np.asarray(r).reshape(-1), GRAD_RTOL[dtype][name],
                     "%dx%d %s %s %s" % (H, W, dtype, name, mode))


@pytest.mark.parametrize("mode", ["deep", "eps"])
def test_backward_edge_logits_groups_chunks(mode):
    B, C, H, W, G, k = 2, 8, 74, 74, 1, 4
    say("backward edge logits ex", mode)
    p = _problem(B, C, H, W, 31, "bf16", mode, G=G)
    eps = EPS[mode]
    got = gspn.prop2d_4dir_ex_backward(p["x"], p["lam"], p["u"], p["w"], p["gy"], G, k, eps)
    torch.cuda.synchronize()
    ref = oracle.prop2d_ex_backward(p["x"], p["lam"], p["u"], p["w"], p["gy"], G, k, eps)
    for name, g, r in zip(NAMES, got, ref):
        assert_close(_np(g).reshape(-1), np.asarray(r).reshape(-1), GRAD_RTOL["bf16"][name],
                     "G=%d k=%d %s %s" % (G, k, name, mode))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("mode", ["deep", "eps"])
def test_scan_dir_edge_logits_and_accumulate(dtype, mode):
    """Each direction alone, raw taps, accumulated into one output."""
    B, C, H, W = 1, 4, 20, 26
    say("scan_dir edge logits", dtype, mode)
    p = _problem(B, C, H, W, 37, dtype, mode)
    eps = EPS[mode]
    w4 = p["w"].view(4, B, C, 3, H * W)
    y = torch.zeros_like(p["x"])
    for d in range(4):
        gspn.scan_dir(p["x"], p["lam"], p["u"], w4[d].contiguous(), d, out=y, accumulate=True, eps=eps)
    torch.cuda.synchronize()
    # the bf16 output is rounded after every accumulation; the oracle's sum of
    # per-direction results is rounded once, so compare against the rounded
    # running sum
    r = np.zeros(p["x"].shape)
    for d in range(4):
        r = r + oracle.scan_dir(p["x"], p["lam"], p["u"], w4[d], d, w_is_raw=True, eps=eps)
        if dtype == "bf16":
            r = _np(torch.from_numpy(r).to(torch.bfloat16))
    assert_close(_np(y), r, RTOL[dtype], "scan_dir accumulate %s %s" % (dtype, mode))


# A non-finite value in plane p + 1 (its first row of x and lambda, and its
# taps) must leave plane p exactly as the oracle computes it.
CONFINE_CASES = [(74, 74, "bf16", 8, 128), (30, 66, "bf16", 8, 128), (40, 30, "bf16", 1, 4),
                 (74, 74, "fp32", 1, 4), (120, 120, "fp32", 1, 4), (27, 27, "bf16", 1, 4),
                 (74, 74, "bf16", 1, 4), (90, 90, "bf16", 1, 4), (147, 147, "bf16", 1, 4),
                 (99, 99, "bf16", 1, 4)]


@pytest.mark.parametrize("H,W,dtype,B,C", CONFINE_CASES)
def test_nonfinite_values_stay_in_their_plane(H, W, dtype, B, C):
    say("confinement", H, W, dtype, B, C)
    p = inputs.problem_torch(B, C, H, W, 41, dtype, DEV)
    x, lam = p["x"].clone(), p["lam"].clone()
    # first and last rows of plane (0, 1); its taps' first and last lines
    x[0, 1, 0, :] = float("inf")
    x[0, 1, H - 1, :] = float("inf")
    lam[0, 1, 0, :] = float("nan")
    lam[0, 1, H - 1, :] = float("nan")
    w = p["w"].clone().view(4, B, C, 3, H * W)
    w[:, 0, 1, :, :W] = float("nan")
    w[:, 0, 1, :, -W:] = float("nan")
    w[2:, 0, 1, :, :H] = float("nan")
    w[2:, 0, 1, :, -H:] = float("nan")
    w = w.view(-1).contiguous()
    y = gspn.prop2d_4dir(x, lam, p["u"], w)
    torch.cuda.synchronize()
    w5 = w.view(4, B, C, 3, -1)
    sl = lambda t: t[0:1, 0:1]
    r = oracle.prop2d(sl(x), sl(lam), sl(p["u"]), w5[:, 0:1, 0:1])
    assert_close(_np(sl(y)), r, RTOL[dtype], "plane (0,0) beside a non-finite plane")
    if C > 2:
        sl2 = lambda t: t[0:1, 2:3]
        r2 = oracle.prop2d(sl2(x), sl2(lam), sl2(p["u"]), w5[:, 0:1, 2:3])
        assert_close(_np(sl2(y)), r2, RTOL[dtype], "plane (0,2) after a non-finite plane")


# (bf16 147 x 147 and 27 x 27: the pair kernel's odd form, whose windows and
# transposes read dwords that a plane shares with its neighbours)
@pytest.mark.parametrize("dtype,L", [("fp32", 74), ("bf16", 74), ("bf16", 147), ("bf16", 27)])
def test_backward_nonfinite_values_stay_in_their_plane(dtype, L):
    B, C, H, W = 1, 4, L, L
    say("backward confinement", dtype, L)
    p = inputs.problem_torch(B, C, H, W, 43, dtype, DEV)
    gy = inputs.draw_torch(43, "gy", (B, C, H, W), dtype, DEV)
    x, lam, u = p["x"].clone(), p["lam"].clone(), p["u"].clone()
    for t in (x, lam, u):
        t[0, 1, 0, :] = float("nan")
        t[0, 1, H - 1, :] = float("inf")
    gy = gy.clone()
    gy[0, 1, 0, :] = float("nan")
    gy[0, 1, H - 1, :] = float("nan")
    w = p["w"].clone().view(4, B, C, 3, H * W)
    w[:, 0, 1, :, :W] = float("nan")
    w[:, 0, 1, :, -W:] = float("nan")
    w = w.view(-1).contiguous()
    got = gspn.prop2d_4dir_backward(x, lam, u, w, gy)
    torch.cuda.synchronize()
    w5 = w.view(4, B, C, 3, -1)
    gw5 = got[3].view(4, B, C, 3, -1)
    for c in (0, 2):
        sl = lambda t: t[0:1, c:c + 1]
        ref = oracle.prop2d_backward(sl(x), sl(lam), sl(u), w5[:, 0:1, c:c + 1], sl(gy))
        mine = (sl(got[0]), sl(got[1]), sl(got[2]), gw5[:, 0:1, c:c + 1])
        for name, g, r in zip(NAMES, mine, ref):
            assert_close(_np(g).reshape(-1), np.asarray(r).reshape(-1), GRAD_RTOL[dtype][name],
                         "plane (0,%d) %s beside a non-finite plane" % (c, name))
