"""Agreement test between a GPU result and the fp64 oracle (test infrastructure).

Pass iff both hold, with r the oracle and g the GPU output widened to fp64:
  elementwise  |g - r| <= rtol * max(|r|, rms(r))   (rms over the whole output)
  normwise     ||g - r||_2 <= rtol * ||r||_2
fp32 storage: rtol 1e-5; bf16 storage (fp32 arithmetic): rtol 2e-2.

Gradients (backward of the four-direction propagation; the pages give no
tolerance for them): gx, glambda and gu are a sum of adjoint or forward scans
and keep the output's rtol.  The tap gradient is a product of an adjoint value
and a forward value, g_i[p] * h_{i-1}[p+k-1], each carrying a scan's rounding
error of the size the output's rtol allows, so its relative error is the sum
of the two: 2e-5 for fp32 storage.  bf16 storage keeps 2e-2 (its 2^-9 output
rounding is far below it).

Latent sublayer (1x1 projections around the propagation): its output is a
matrix product y = P_up y_c, and an element of y can be far smaller than the
terms it sums.  The textbook componentwise bound of a product is relative to
|P_up| |y_c|, so the elementwise floor there is max(|P_up| |y_c|, rms(r))
(compare_scaled) with the same rtol; the normwise condition is unchanged.
With bf16 storage the GPU and the oracle accumulate each stored intermediate
in different precisions before rounding it, so a few of its elements land one
bf16 step apart; the componentwise floor is what such steps are measured
against.
"""
import numpy as np

RTOL = {"fp32": 1e-5, "bf16": 2e-2}
GRAD_RTOL = {"fp32": {"gx": 1e-5, "glam": 1e-5, "gu": 1e-5, "gw4": 2e-5},
             "bf16": {"gx": 2e-2, "glam": 2e-2, "gu": 2e-2, "gw4": 2e-2}}


def compare(g, r, rtol):
    g = np.asarray(g, dtype=np.float64).reshape(-1)
    r = np.asarray(r, dtype=np.float64).reshape(-1)
    if r.size == 0:
        return True, "empty"
    err = np.abs(g - r)
    rms = float(np.sqrt(np.mean(r * r)))
    floor = np.maximum(np.abs(r), rms)
    worst = float(np.max(err / np.where(floor > 0, floor, 1.0)))
    nr = float(np.linalg.norm(r))
    normwise = float(np.linalg.norm(g - r)) / (nr if nr > 0 else 1.0)
    ok = bool(np.all(np.isfinite(g))) and worst <= rtol and normwise <= rtol
    return ok, "worst elementwise %.3e, normwise %.3e (rtol %.1e)" % (worst, normwise, rtol)


def assert_close(g, r, rtol, what=""):
    ok, msg = compare(g, r, rtol)
    assert ok, (what + ": " if what else "") + msg


def compare_scaled(g, r, scale, rtol):
    """compare() with the elementwise floor max(scale, rms(r)), where `scale`
    holds the componentwise magnitudes of the terms summed into r."""
    g = np.asarray(g, dtype=np.float64).reshape(-1)
    r = np.asarray(r, dtype=np.float64).reshape(-1)
    scale = np.abs(np.asarray(scale, dtype=np.float64).reshape(-1))
    if r.size == 0:
        return True, "empty"
    err = np.abs(g - r)
    rms = float(np.sqrt(np.mean(r * r)))
    floor = np.maximum(scale, rms)
    worst = float(np.max(err / np.where(floor > 0, floor, 1.0)))
    nr = float(np.linalg.norm(r))
    normwise = float(np.linalg.norm(g - r)) / (nr if nr > 0 else 1.0)
    ok = bool(np.all(np.isfinite(g))) and worst <= rtol and normwise <= rtol
    return ok, "worst componentwise %.3e, normwise %.3e (rtol %.1e)" % (worst, normwise, rtol)
