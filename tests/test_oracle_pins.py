"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

None of these checks re-types the oracle's own loops: they use hand-derived
closed forms (tests/golden), an explicit dense linear map assembled from
matrix products, textbook reductions (running sums), invariants of a
row-stochastic recurrence, and symmetries between the scan directions.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import TD, BU, LR, RL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def _rand(*shape, rng=RNG):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- normalisation

def test_normalize_closed_forms():
    spec = json.load(open(os.path.join(GOLDEN, "normalize_closed_forms.json")))
    eps = spec["eps"]
    for case in spec["cases"]:
        L, p = case["L"], case["p"]
        raw = np.zeros((3, 1, L))
        raw[:, 0, p] = case["raw"]
        got = oracle.normalize(raw, 1, L, eps)[:, 0, p]
        assert np.all(np.isfinite(got)), case["name"]
        np.testing.assert_allclose(got, case["expect"], rtol=1e-14, atol=1e-300, err_msg=case["name"])


@pytest.mark.parametrize("NL,L", [(1, 1), (3, 1), (4, 2), (5, 7), (2, 64)])
def test_normalize_invariants(NL, L):
    raw = 3.0 * _rand(2, 3, NL, L)
    w = oracle.normalize(raw, NL, L, 1e-6)
    assert np.all(w >= 0.0)
    # dropped taps are exactly zero
    assert np.all(w[:, 0, :, 0] == 0.0)
    assert np.all(w[:, 2, :, L - 1] == 0.0)
    # in-grid taps sum to one (the clamp is inactive for these logits)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    # ratios of kept taps are ratios of sigmoids
    if L >= 3:
        sig = 1.0 / (1.0 + np.exp(-raw[:, :, :, 1:-1]))
        np.testing.assert_allclose(w[:, 0, :, 1:-1] / w[:, 2, :, 1:-1], sig[:, 0] / sig[:, 2], rtol=1e-13)


# ---------------------------------------------------------- dense linear map

def _line_pixel(dir, i, p):
    return (i, p) if dir in (TD, BU) else (p, i)


def _dense_map(lam, u, taps, dir, H, W):
    """G with vec(u*h) = G vec(x) for one plane, built from explicit products.

    taps: [3][NL][L] pre-normalised (any values).  Line matrices M_i are L x L
    tridiagonal with M_i[p, p+k-1] = taps[k, i, p]; the scan visits lines in
    `order`; T(s, t) = M_{order[s]} ... M_{order[t+1]} for t <= s; then
    G[(line order[s]), (line order[t])] = U_s T(s, t) Lambda_t.
    """
    NL, L = oracle.line_geometry(dir, H, W)
    order = list(range(NL)) if dir in (TD, LR) else list(range(NL - 1, -1, -1))
    M = []
    for i in range(NL):
        m = np.zeros((L, L))
        for p in range(L):
            for k in range(3):
                q = p + k - 1
                if 0 <= q < L:
                    m[p, q] = taps[k, i, p]
        M.append(m)
    idx = lambda i, p: _line_pixel(dir, i, p)[0] * W + _line_pixel(dir, i, p)[1]
    G = np.zeros((H * W, H * W))
    for s in range(NL):
        T = np.eye(L)
        for t in range(s, -1, -1):
            i_s, i_t = order[s], order[t]
            Us = np.diag([u.flat[idx(i_s, p)] for p in range(L)])
            Lt = np.diag([lam.flat[idx(i_t, p)] for p in range(L)])
            blk = Us @ T @ Lt
            for p in range(L):
                for q in range(L):
                    G[idx(i_s, p), idx(i_t, q)] = blk[p, q]
            if t > 0:
                T = T @ M[order[t]]
    return G


@pytest.mark.parametrize("H,W", [(1, 1), (1, 4), (4, 1), (2, 3), (3, 5), (5, 2), (8, 8)])
@pytest.mark.parametrize("dir", [TD, BU, LR, RL])
def test_scan_matches_dense_map(H, W, dir):
    rng = np.random.default_rng(100 * H + 10 * W + dir)
    x, lam, u = (rng.standard_normal((1, 1, H, W)) for _ in range(3))
    taps = rng.standard_normal((1, 1, 3, H * W))          # arbitrary pre-normalised taps
    NL, L = oracle.line_geometry(dir, H, W)
    G = _dense_map(lam[0, 0], u[0, 0], taps[0, 0].reshape(3, NL, L), dir, H, W)
    got = oracle.scan_dir(x, lam, u, taps, dir, w_is_raw=False)
    np.testing.assert_allclose(got.reshape(-1), G @ x.reshape(-1), rtol=1e-12, atol=1e-12)
    # impulse responses are the columns of G
    for j in (0, H * W - 1, (H * W) // 2):
        e = np.zeros((1, 1, H, W))
        e.flat[j] = 1.0
        col = oracle.scan_dir(e, lam, u, taps, dir, w_is_raw=False).reshape(-1)
        np.testing.assert_allclose(col, G[:, j], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("H,W", [(2, 2), (3, 4), (5, 3)])
def test_raw_scan_uses_normalised_taps(H, W):
    """A raw-tap scan equals the pre-normalised scan fed the normalised taps."""
    rng = np.random.default_rng(7)
    x, lam, u = (rng.standard_normal((2, 1, H, W)) for _ in range(3))
    raw = rng.standard_normal((2, 1, 3, H * W))
    for dir in (TD, BU, LR, RL):
        NL, L = oracle.line_geometry(dir, H, W)
        wn = oracle.normalize(raw.reshape(2, 3, NL, L), NL, L).reshape(raw.shape)
        a = oracle.scan_dir(x, lam, u, raw, dir, w_is_raw=True)
        b = oracle.scan_dir(x, lam, u, wn, dir, w_is_raw=False)
        np.testing.assert_allclose(a, b, rtol=1e-14, atol=1e-15)


# --------------------------------------------------------- worked example

def test_worked_2x2():
    spec = json.load(open(os.path.join(GOLDEN, "worked_2x2.json")))
    x = np.array(spec["x"]).reshape(1, 1, 2, 2)
    one = np.ones_like(x)
    w4 = np.zeros((4, 1, 1, 3, 4))
    y = oracle.prop2d(x, one, one, w4)
    np.testing.assert_allclose(y[0, 0], spec["y"], rtol=1e-15)
    # the general closed form for random a, b, c, d
    a, b, c, d = RNG.standard_normal(4)
    x = np.array([[a, b], [c, d]]).reshape(1, 1, 2, 2)
    y = oracle.prop2d(x, one, one, w4)[0, 0]
    expect = [[4 * a + (b + c) / 2 + d, 4 * b + a / 2 + c + d / 2],
              [4 * c + a / 2 + b + d / 2, 4 * d + a + (b + c) / 2]]
    np.testing.assert_allclose(y, expect, rtol=1e-14, atol=1e-14)


# ------------------------------------------------- textbook reductions

@pytest.mark.parametrize("dir", [TD, BU, LR, RL])
def test_single_position_lines_are_running_sums(dir):
    """Lines of length one keep only the centre tap (weight 1): h is a cumsum."""
    H, W = (7, 1) if dir in (TD, BU) else (1, 7)
    x, lam, u = (RNG.standard_normal((1, 2, H, W)) for _ in range(3))
    raw = 4.0 * RNG.standard_normal((1, 2, 3, H * W))
    got = oracle.scan_dir(x, lam, u, raw, dir, w_is_raw=True)
    bx = (lam * x).reshape(1, 2, -1)
    if dir in (BU, RL):
        h = np.cumsum(bx[..., ::-1], axis=-1)[..., ::-1]
    else:
        h = np.cumsum(bx, axis=-1)
    np.testing.assert_allclose(got.reshape(1, 2, -1), u.reshape(1, 2, -1) * h, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("dir", [TD, BU, LR, RL])
def test_identity_and_shift_taps(dir):
    H, W = 5, 6
    NL, L = oracle.line_geometry(dir, H, W)
    x, lam = (RNG.standard_normal((1, 1, H, W)) for _ in range(2))
    u = np.ones((1, 1, H, W))
    # line-major views of b = lam * x
    bx = (lam * x)[0, 0]
    bl = bx if dir in (TD, BU) else bx.T                       # [NL][L]
    order = list(range(NL)) if dir in (TD, LR) else list(range(NL - 1, -1, -1))
    bs = bl[order]                                              # lines in scan order
    # identity taps (0, 1, 0): per-position running sums along the scan
    ident = np.zeros((1, 1, 3, NL, L))
    ident[:, :, 1] = 1.0
    got = oracle.scan_dir(x, lam, u, ident.reshape(1, 1, 3, -1), dir, w_is_raw=False)[0, 0]
    gl = (got if dir in (TD, BU) else got.T)[order]
    np.testing.assert_allclose(gl, np.cumsum(bs, axis=0), rtol=1e-13, atol=1e-13)
    # shift taps (1, 0, 0): h_s[p] = h_{s-1}[p-1] + b_s[p]  ->  diagonal sums
    shift = np.zeros((1, 1, 3, NL, L))
    shift[:, :, 0] = 1.0
    got = oracle.scan_dir(x, lam, u, shift.reshape(1, 1, 3, -1), dir, w_is_raw=False)[0, 0]
    gl = (got if dir in (TD, BU) else got.T)[order]
    expect = np.zeros_like(bs)
    for s in range(NL):
        for p in range(L):
            expect[s, p] = sum(bs[s - t, p - t] for t in range(min(s, p) + 1))
    np.testing.assert_allclose(gl, expect, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------ invariants

@pytest.mark.parametrize("dir", [TD, BU, LR, RL])
@pytest.mark.parametrize("H,W", [(6, 9), (9, 6), (1, 5), (5, 1)])
def test_row_stochastic_constant_propagates(dir, H, W):
    """lambda = 1 on the first line only, x = c there, u = 1: y == c everywhere."""
    NL, L = oracle.line_geometry(dir, H, W)
    first = 0 if dir in (TD, LR) else NL - 1
    lam = np.zeros((1, 1, H, W))
    x = RNG.standard_normal((1, 1, H, W))
    cval = 0.7318
    if dir in (TD, BU):
        lam[0, 0, first, :] = 1.0
        x[0, 0, first, :] = cval
    else:
        lam[0, 0, :, first] = 1.0
        x[0, 0, :, first] = cval
    raw = 3.0 * RNG.standard_normal((1, 1, 3, H * W))
    y = oracle.scan_dir(x, lam, np.ones_like(x), raw, dir, w_is_raw=True)
    np.testing.assert_allclose(y, cval, rtol=0, atol=1e-12)
    # maximum principle with a random first line
    if dir in (TD, BU):
        x[0, 0, first, :] = RNG.standard_normal(W)
        lo, hi = x[0, 0, first, :].min(), x[0, 0, first, :].max()
    else:
        x[0, 0, :, first] = RNG.standard_normal(H)
        lo, hi = x[0, 0, :, first].min(), x[0, 0, :, first].max()
    y = oracle.scan_dir(x, lam, np.ones_like(x), raw, dir, w_is_raw=True)
    assert y.min() >= lo - 1e-12 and y.max() <= hi + 1e-12


# ------------------------------------------------------ symmetries

def _flip_lines(taps, NL, L):
    """Reverse the line index of a [.., 3, NL*L] tap array; positions kept."""
    t = taps.reshape(taps.shape[:-1] + (NL, L))
    return t[..., ::-1, :].reshape(taps.shape).copy()


@pytest.mark.parametrize("H,W", [(4, 7), (7, 4), (3, 3)])
def test_direction_symmetries(H, W):
    x, lam, u = (RNG.standard_normal((2, 2, H, W)) for _ in range(3))
    raw = RNG.standard_normal((2, 2, 3, H * W))
    fh = lambda a: a[..., ::-1, :].copy()
    fw = lambda a: a[..., :, ::-1].copy()
    tr = lambda a: np.swapaxes(a, -1, -2).copy()
    # BU = flipH o TD o flipH, taps' line index reversed, positions unchanged
    bu = oracle.scan_dir(x, lam, u, raw, BU)
    td_f = oracle.scan_dir(fh(x), fh(lam), fh(u), _flip_lines(raw, H, W), TD)
    np.testing.assert_allclose(bu, fh(td_f), rtol=1e-13, atol=1e-13)
    # LR on the grid = TD on the transposed grid with the same (line-major) taps
    lr = oracle.scan_dir(x, lam, u, raw, LR)
    td_t = oracle.scan_dir(tr(x), tr(lam), tr(u), raw, TD)
    np.testing.assert_allclose(lr, tr(td_t), rtol=1e-13, atol=1e-13)
    # RL = flipW o LR o flipW, taps' line index (the column) reversed
    rl = oracle.scan_dir(x, lam, u, raw, RL)
    lr_f = oracle.scan_dir(fw(x), fw(lam), fw(u), _flip_lines(raw, W, H), LR)
    np.testing.assert_allclose(rl, fw(lr_f), rtol=1e-13, atol=1e-13)


def test_linearity_in_x():
    H, W = 5, 8
    x1, x2, lam, u = (RNG.standard_normal((1, 3, H, W)) for _ in range(4))
    w4 = RNG.standard_normal((4, 1, 3, 3, H * W))
    a, b = 0.37, -2.5
    y = oracle.prop2d(a * x1 + b * x2, lam, u, w4)
    y1 = oracle.prop2d(x1, lam, u, w4)
    y2 = oracle.prop2d(x2, lam, u, w4)
    np.testing.assert_allclose(y, a * y1 + b * y2, rtol=1e-12, atol=1e-12)


def test_prop2d_is_sum_of_directions():
    H, W = 6, 5
    x, lam, u = (RNG.standard_normal((2, 3, H, W)) for _ in range(3))
    w4 = RNG.standard_normal((4, 2, 3, 3, H * W))
    y = oracle.prop2d(x, lam, u, w4)
    s = sum(oracle.scan_dir(x, lam, u, w4[d], d) for d in range(4))
    np.testing.assert_allclose(y, s, rtol=1e-14, atol=1e-14)


def test_planes_are_independent():
    """Each (b, c) plane depends only on its own inputs."""
    H, W = 4, 6
    x, lam, u = (RNG.standard_normal((2, 3, H, W)) for _ in range(3))
    w4 = RNG.standard_normal((4, 2, 3, 3, H * W))
    y = oracle.prop2d(x, lam, u, w4)
    y11 = oracle.prop2d(x[1:2, 1:2], lam[1:2, 1:2], u[1:2, 1:2], w4[:, 1:2, 1:2])
    np.testing.assert_array_equal(y[1:2, 1:2], y11)
