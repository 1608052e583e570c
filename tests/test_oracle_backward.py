"""Pins of the oracle's gradient (oracle.prop2d_backward), CPU only.

The backward is not described on the pages (the paper text, §6.1, reports
that forward and backward kernels exist); the oracle computes the exact
derivative of the forward definition.  It is pinned here by things that do
not share its formula:
  - central finite differences of the forward oracle, along random
    directions and element by element on tiny grids;
  - the adjoint identities of a map that is linear in x, in lambda and in u
    (for fixed other inputs): <gy, y> = <gx, x> = <glambda, lambda> = <gu, u>;
  - the clamp branch (all logits near -20, neighbourhood sum below eps),
    where the normalised taps scale as sigmoid / eps.
"""
import numpy as np
import pytest

import oracle

EPS = 1e-6


def _problem(B, C, H, W, seed, scale_w=1.0, shift_w=0.0):
    rng = np.random.default_rng(seed)
    x, lam, u, gy = (rng.standard_normal((B, C, H, W)) for _ in range(4))
    w4 = shift_w + scale_w * rng.standard_normal((4, B, C, 3, H * W))
    return x, lam, u, w4, gy


def _loss(gy, x, lam, u, w4):
    return float(np.sum(gy * oracle.prop2d(x, lam, u, w4, EPS)))


@pytest.mark.parametrize("H,W", [(2, 2), (3, 5), (4, 3), (1, 4), (5, 1), (1, 1)])
@pytest.mark.parametrize("seed", [0, 1])
def test_backward_matches_directional_finite_differences(H, W, seed):
    x, lam, u, w4, gy = _problem(1, 2, H, W, seed)
    grads = oracle.prop2d_backward(x, lam, u, w4, gy, EPS)
    rng = np.random.default_rng(100 + seed)
    args = [x, lam, u, w4]
    for idx, g in enumerate(grads):
        v = rng.standard_normal(args[idx].shape)
        e = 1e-6
        ap = list(args)
        am = list(args)
        ap[idx] = args[idx] + e * v
        am[idx] = args[idx] - e * v
        fd = (_loss(gy, *ap) - _loss(gy, *am)) / (2 * e)
        an = float(np.sum(g * v))
        scale = max(1.0, abs(fd), abs(an))
        assert abs(fd - an) <= 1e-6 * scale, (idx, fd, an)


@pytest.mark.parametrize("H,W", [(2, 2), (1, 3), (3, 2)])
def test_backward_matches_elementwise_finite_differences(H, W):
    x, lam, u, w4, gy = _problem(1, 1, H, W, 7)
    grads = oracle.prop2d_backward(x, lam, u, w4, gy, EPS)
    args = [x, lam, u, w4]
    e = 1e-6
    for idx, g in enumerate(grads):
        flat = args[idx].reshape(-1)
        for j in range(flat.size):
            ap = [a.copy() for a in args]
            am = [a.copy() for a in args]
            ap[idx].reshape(-1)[j] += e
            am[idx].reshape(-1)[j] -= e
            fd = (_loss(gy, *ap) - _loss(gy, *am)) / (2 * e)
            an = float(g.reshape(-1)[j])
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (idx, j, fd, an)


@pytest.mark.parametrize("H,W", [(3, 4), (5, 2), (6, 6)])
def test_backward_adjoint_identities(H, W):
    """y is linear in x, in lambda and in u separately, so the gradient of
    <gy, y> with respect to each, paired with that input, gives <gy, y> back."""
    x, lam, u, w4, gy = _problem(2, 2, H, W, 3)
    gx, glam, gu, _ = oracle.prop2d_backward(x, lam, u, w4, gy, EPS)
    ref = _loss(gy, x, lam, u, w4)
    for g, a in ((gx, x), (glam, lam), (gu, u)):
        got = float(np.sum(g * a))
        assert abs(got - ref) <= 1e-12 * max(1.0, abs(ref)), (got, ref)


def test_backward_clamp_branch():
    """Logits near -20: the neighbourhood sum (~6e-9) is below eps, the
    normalised taps are sigmoid / eps and their gradient follows that branch."""
    x, lam, u, w4, gy = _problem(1, 1, 3, 4, 11, scale_w=0.3, shift_w=-20.0)
    grads = oracle.prop2d_backward(x, lam, u, w4, gy, EPS)
    rng = np.random.default_rng(5)
    v = rng.standard_normal(w4.shape)
    e = 1e-5
    fd = (_loss(gy, x, lam, u, w4 + e * v) - _loss(gy, x, lam, u, w4 - e * v)) / (2 * e)
    an = float(np.sum(grads[3] * v))
    assert an != 0.0
    assert abs(fd - an) <= 1e-6 * max(1e-12, abs(fd)), (fd, an)


def test_backward_first_line_and_dropped_taps_have_zero_gradient():
    x, lam, u, w4, gy = _problem(1, 1, 4, 5, 2)
    gw4 = oracle.prop2d_backward(x, lam, u, w4, gy, EPS)[3].reshape(4, 3, -1)
    H, W = 4, 5
    for d in range(4):
        NL, L = oracle.line_geometry(d, H, W)
        t = gw4[d].reshape(3, NL, L)
        first = 0 if d in (oracle.TD, oracle.LR) else NL - 1
        assert np.all(t[:, first, :] == 0.0)
        assert np.all(t[0, :, 0] == 0.0) and np.all(t[2, :, L - 1] == 0.0)
