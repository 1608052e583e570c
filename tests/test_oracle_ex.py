"""Pins of the extended oracle (oracle.prop2d_ex): taps shared by channel
groups and chunked scans, CPU only.

Readings (paper text §4.1, the grid indexed by (chunk, b, c); §4.2 and §6.2,
propagation weights shared across channels):
  - groups are contiguous: channel c of C reads the taps of group c // (C // G);
  - a chunked scan cuts each direction's lines into k_chunk segments of
    ceil(NL / k_chunk) lines, the same segments for both scan orders of an
    axis, and restarts every segment from lambda * x.
Each pin reduces the extended operator to the pinned per-channel oracle
(oracle.prop2d / oracle.scan_dir) by a construction that does not share the
extended function's code: expanding grouped taps to every channel, and
running the global scan on each segment cut out of the grid.
"""
import math

import numpy as np
import pytest

import oracle

EPS = 1e-6
RT = 1e-13


def _problem(B, C, H, W, G, seed):
    rng = np.random.default_rng(seed)
    x, lam, u = (rng.standard_normal((B, C, H, W)) for _ in range(3))
    wg = rng.standard_normal((4, B, G, 3, H * W))
    return x, lam, u, wg


def _expand(wg, C):
    """Per-channel taps [4][B][C][3][HW] from grouped ones (contiguous groups)."""
    G = wg.shape[2]
    return np.repeat(wg, C // G, axis=2)


def _close(a, b, rtol=RT):
    scale = max(1.0, float(np.max(np.abs(b))))
    assert np.max(np.abs(a - b)) <= rtol * scale, float(np.max(np.abs(a - b)))


@pytest.mark.parametrize("H,W", [(1, 1), (3, 5), (6, 4)])
def test_ex_reduces_to_prop2d(H, W):
    x, lam, u, w = _problem(2, 3, H, W, 3, 0)
    _close(oracle.prop2d_ex(x, lam, u, w, groups=3, k_chunk=1, eps=EPS),
           oracle.prop2d(x, lam, u, w, EPS))


@pytest.mark.parametrize("C,G", [(6, 1), (6, 2), (6, 3), (4, 4), (5, 1)])
def test_grouped_taps_equal_expanded_per_channel_taps(C, G):
    x, lam, u, wg = _problem(2, C, 5, 4, G, 1)
    _close(oracle.prop2d_ex(x, lam, u, wg, groups=G, eps=EPS),
           oracle.prop2d(x, lam, u, _expand(wg, C), EPS))


def test_groups_are_contiguous_channel_blocks():
    """Channels with equal x, lambda, u agree exactly when in one group."""
    B, C, G, H, W = 1, 4, 2, 4, 5
    x, lam, u, wg = _problem(B, C, H, W, G, 2)
    for a in (x, lam, u):
        a[:, :] = a[:, :1]
    y = oracle.prop2d_ex(x, lam, u, wg, groups=G, eps=EPS)
    assert np.array_equal(y[0, 0], y[0, 1]) and np.array_equal(y[0, 2], y[0, 3])
    assert not np.allclose(y[0, 0], y[0, 2])


def _segments(NL, k):
    Lc = math.ceil(NL / k)
    return [(a, min(NL, a + Lc)) for a in range(0, NL, Lc)]


def _chunked_by_cropping(x, lam, u, w, k):
    """Sum over directions and segments of the global scan of each segment
    cut out of the grid (rows for TD/BU, columns for LR/RL)."""
    B, C, H, W = x.shape
    y = np.zeros_like(x)
    w = w.reshape(4, B, C, 3, -1)
    for d in range(4):
        NL, L = oracle.line_geometry(d, H, W)
        wd = w[d].reshape(B, C, 3, NL, L)
        for a, b in _segments(NL, k):
            if d in (oracle.TD, oracle.BU):
                sl = (slice(None), slice(None), slice(a, b), slice(None))
            else:
                sl = (slice(None), slice(None), slice(None), slice(a, b))
            y[sl] += oracle.scan_dir(x[sl], lam[sl], u[sl], np.ascontiguousarray(wd[:, :, :, a:b]),
                                     d, True, EPS)
    return y


@pytest.mark.parametrize("H,W,k", [(8, 6, 2), (7, 9, 2), (7, 9, 3), (10, 4, 4), (5, 5, 5),
                                   (9, 7, 4), (6, 11, 5)])
def test_chunked_scan_equals_global_scans_of_segments(H, W, k):
    x, lam, u, w = _problem(1, 2, H, W, 2, 3 + k)
    _close(oracle.prop2d_ex(x, lam, u, w, groups=2, k_chunk=k, eps=EPS),
           _chunked_by_cropping(x, lam, u, w, k))


def test_grouped_and_chunked_together():
    x, lam, u, wg = _problem(2, 4, 7, 6, 2, 9)
    _close(oracle.prop2d_ex(x, lam, u, wg, groups=2, k_chunk=3, eps=EPS),
           _chunked_by_cropping(x, lam, u, _expand(wg, 4), 3))


@pytest.mark.parametrize("k", [6, 7, 1000])
def test_one_line_segments_reduce_to_4_u_lambda_x(k):
    """k_chunk >= every line count: each line restarts, y = 4 u lambda x."""
    x, lam, u, w = _problem(1, 2, 6, 4, 1, 4)
    y = oracle.prop2d_ex(x, lam, u, w, groups=1, k_chunk=k, eps=EPS)
    _close(y, 4 * u * lam * x)


def test_bad_groups_and_chunks_rejected():
    x, lam, u, w = _problem(1, 4, 3, 3, 3, 0)
    with pytest.raises(ValueError):
        oracle.prop2d_ex(x, lam, u, w, groups=3)
    x, lam, u, w = _problem(1, 4, 3, 3, 2, 0)
    with pytest.raises(ValueError):
        oracle.prop2d_ex(x, lam, u, w, groups=2, k_chunk=0)
