"""Pins of the oracle's gradient of the extended operator (tap groups and
chunked scans), oracle.prop2d_ex_backward.

The gradient is the exact derivative of oracle.prop2d_ex, so it is pinned
against that forward by central finite differences (any dropped or misplaced
term of the adjoint, the restart handling or the group reduction changes the
directional derivative), by the per-channel operator it reduces to, by the
identity between shared taps and taps replicated per channel, and by the
closed form of one-line segments.  Everything runs on the CPU in fp64.
"""
import numpy as np
import pytest

import oracle


def _problem(B, C, H, W, G, seed):
    rng = np.random.default_rng(seed)
    x, lam, u, gy = (rng.standard_normal((B, C, H, W)) for _ in range(4))
    w = rng.standard_normal((4, B, G, 3, H * W))
    return x, lam, u, w, gy


def test_ex_backward_reduces_to_per_channel_backward():
    x, lam, u, w, gy = _problem(2, 3, 5, 6, 3, 1)
    ref = oracle.prop2d_backward(x, lam, u, w, gy)
    got = oracle.prop2d_ex_backward(x, lam, u, w, gy, 3, 1)
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("G,k", [(1, 1), (2, 2), (4, 3), (1, 4), (2, 7)])
def test_ex_backward_matches_finite_differences(G, k):
    """<grad, v> equals the central difference of <gy, prop2d_ex> along a
    random direction v, for each of x, lambda, u and the grouped taps."""
    B, C, H, W = 2, 4, 5, 6
    x, lam, u, w, gy = _problem(B, C, H, W, G, 10 * G + k)
    grads = oracle.prop2d_ex_backward(x, lam, u, w, gy, G, k)
    rng = np.random.default_rng(99 + G + k)
    h = 1e-5
    args = [x, lam, u, w]
    for slot in range(4):
        v = rng.standard_normal(args[slot].shape)
        plus = list(args)
        minus = list(args)
        plus[slot] = args[slot] + h * v
        minus[slot] = args[slot] - h * v
        fp = float(np.sum(gy * oracle.prop2d_ex(*plus, G, k)))
        fm = float(np.sum(gy * oracle.prop2d_ex(*minus, G, k)))
        fd = (fp - fm) / (2 * h)
        an = float(np.sum(grads[slot] * v))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (slot, fd, an)


@pytest.mark.parametrize("G,k", [(1, 1), (2, 3)])
def test_ex_backward_shared_taps_sum_the_replicated_gradients(G, k):
    """Taps shared by a channel group act like per-channel copies: the group's
    tap gradient is the sum of the copies' gradients, the rest is equal."""
    B, C, H, W = 2, 4, 4, 7
    x, lam, u, w, gy = _problem(B, C, H, W, G, 5 + G)
    cpg = C // G
    w_exp = np.repeat(w, cpg, axis=2)              # [4][B][C][3][HW], channel c <- group c // cpg
    got = oracle.prop2d_ex_backward(x, lam, u, w, gy, G, k)
    per = oracle.prop2d_ex_backward(x, lam, u, w_exp, gy, C, k)
    for a, b in zip(got[:3], per[:3]):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
    summed = per[3].reshape(4, B, G, cpg, 3, H * W).sum(axis=3)
    np.testing.assert_allclose(got[3], summed, rtol=1e-12, atol=1e-12)


def test_ex_backward_one_line_segments_closed_form():
    """With every line its own segment, h = lambda x in each direction, so
    y = 4 u lambda x: gx = 4 lambda u gy, glambda = 4 x u gy, gu = 4 lambda x
    gy, and no tap is ever read (gradient 0)."""
    B, C, H, W = 1, 2, 5, 4
    x, lam, u, w, gy = _problem(B, C, H, W, 2, 3)
    gx, glam, gu, gw = oracle.prop2d_ex_backward(x, lam, u, w, gy, 2, max(H, W))
    np.testing.assert_allclose(gx, 4 * lam * u * gy, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(glam, 4 * x * u * gy, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(gu, 4 * lam * x * gy, rtol=1e-13, atol=1e-13)
    assert np.all(gw == 0.0)


def test_ex_backward_rejects_bad_groups_and_chunks():
    x, lam, u, w, gy = _problem(1, 4, 3, 3, 4, 0)
    with pytest.raises(ValueError):
        oracle.prop2d_ex_backward(x, lam, u, w[:, :, :3], gy, 3, 1)
    with pytest.raises(ValueError):
        oracle.prop2d_ex_backward(x, lam, u, w, gy, 4, 0)
