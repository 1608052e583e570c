"""GPU parity of gspn_latent_sublayer against the oracle's latent_sublayer
(fp64 matmuls around prop2d_ex), through the C ABI.

Inputs: tokens N(0, 1) and weights N(0, 1) / sqrt(fan-in), from
spatial_line_scan_amd.inputs, in the storage type.  The layer stores its
intermediates (latent, parameters, scan output) in the storage type, and the
oracle rounds them at the same points (storage=dtype).  Agreement:
oracle/tolerance.py's compare_scaled (fp32 1e-5, bf16 2e-2), whose
elementwise floor is the output projection's componentwise magnitude
|y_c^T| |P_up^T|.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from spatial_line_scan_amd import gspn, inputs
from oracle.tolerance import RTOL, compare_scaled

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _np(t):
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def _run(B, C, Cc, G, H, W, k, dtype, seed, batches=None):
    p = inputs.sublayer_problem_torch(B, C, Cc, G, H, W, seed, dtype, DEV)
    y = gspn.latent_sublayer(p["x_tok"], p["p_down"], p["w_param"], p["p_up"], H, W, G, k)
    torch.cuda.synchronize()
    sel = slice(None) if batches is None else batches
    r, scale = oracle.latent_sublayer(p["x_tok"][sel], p["p_down"], p["w_param"], p["p_up"], H, W,
                                      G, k, storage=dtype, with_scale=True)
    ok, msg = compare_scaled(_np(y[sel]), r, scale, RTOL[dtype])
    assert ok, "sublayer B%d C%d Cc%d G%d %dx%d k%d %s: %s" % (B, C, Cc, G, H, W, k, dtype, msg)
    return p, y


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("B,C,Cc,G,H,W,k", [
    (2, 24, 8, 8, 10, 10, 1), (2, 24, 8, 1, 10, 12, 1), (1, 40, 8, 2, 9, 14, 3),
    (3, 16, 4, 4, 27, 27, 1), (2, 64, 16, 16, 74, 74, 1), (1, 32, 8, 1, 100, 36, 2),
    # matrix-core path edges: C % 8 == 4 (8-byte token stores), Cc = 24 (a
    # zero-padded 16-k step), a rectangular plane through the transpose, the
    # largest side it takes (96), and a shape just past it (97: hipBLASLt)
    (1, 20, 8, 2, 10, 12, 1), (2, 36, 24, 3, 12, 20, 2), (1, 64, 64, 1, 96, 96, 1),
    (1, 24, 8, 8, 4, 97, 1)])
def test_sublayer_small(B, C, Cc, G, H, W, k, dtype):
    say("sublayer", B, C, Cc, G, H, W, k, dtype)
    _run(B, C, Cc, G, H, W, k, dtype, 5 + B + C + G + k)


# The matrix-core P_down (bf16, Cc of 32 or 64, C a multiple of 128 up to
# 1280): one to ten k-steps a lane (C / 128), 32-token tiles that span
# two or more images (H W not a multiple of 32, and below 32), a ragged last
# tile, and a batch of fewer tiles than CUs
@pytest.mark.parametrize("B,C,Cc,G,H,W", [
    (3, 128, 32, 32, 10, 10), (2, 256, 64, 4, 9, 12), (5, 384, 64, 64, 6, 6),
    (2, 640, 32, 1, 12, 12), (3, 1280, 64, 2, 4, 4), (1, 896, 32, 8, 14, 10),
    (2, 1536, 64, 64, 6, 6)])   # C past the matrix-core form: hipBLASLt
def test_sublayer_matrix_core_p_down(B, C, Cc, G, H, W):
    say("sublayer p_down", B, C, Cc, G, H, W)
    _run(B, C, Cc, G, H, W, 1, "bf16", 40 + B + C + G)


@pytest.mark.parametrize("G", [64, 1])
def test_sublayer_latent1k_sampled_batches(G):
    """The pages' 1K sublayer shape: B=32 images of 74 x 74 tokens, C=1152
    compressed to Cc=64 (s = 18), bf16; the oracle recomputes two images."""
    say("sublayer latent1k G", G)
    p, y = _run(32, 1152, 64, G, 74, 74, 1, "bf16", 0, batches=[0, 31])
    y2 = gspn.latent_sublayer(p["x_tok"], p["p_down"], p["w_param"], p["p_up"], 74, 74, G, 1)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))   # run-to-run bitwise
