"""Pins of the latent sublayer oracle (oracle.latent_sublayer), CPU only.

The sublayer is a composition of 1x1 projections (plain fp64 matmuls) with
the pinned propagation oracle; these pins check the composition's wiring by
properties the definition fixes:
  - transposing the token grid and swapping the row scans with the column
    scans (TD <-> LR, BU <-> RL in the parameter rows) transposes the output
    (this pins the column-major tap planes of LR / RL);
  - with every scan cut into single lines (k_chunk >= H, W) each direction
    returns lambda * z, so y = p_up (4 u lambda z) per token;
  - linearity in p_up;
  - storage rounding: exact on values the storage type holds, round to
    nearest even on halfway cases, and within half an ulp otherwise.
"""
import numpy as np
import pytest

import oracle


def _weights(B, C, Cc, G, H, W, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, H * W, C))
    pd = rng.standard_normal((Cc, C)) / np.sqrt(C)
    wp = rng.standard_normal((2 * Cc + 12 * G, Cc)) / np.sqrt(Cc)
    pu = rng.standard_normal((C, Cc)) / np.sqrt(Cc)
    return x, pd, wp, pu


@pytest.mark.parametrize("G,k", [(1, 1), (2, 1), (2, 3)])
def test_sublayer_transpose_symmetry(G, k):
    B, C, Cc, H, W = 2, 6, 4, 5, 7
    x, pd, wp, pu = _weights(B, C, Cc, G, H, W, 1)
    y = oracle.latent_sublayer(x, pd, wp, pu, H, W, G, k)
    xt = x.reshape(B, H, W, C).transpose(0, 2, 1, 3).reshape(B, W * H, C)
    taps = wp[2 * Cc:].reshape(4, G, 3, Cc)
    wpt = np.concatenate([wp[:2 * Cc], taps[[2, 3, 0, 1]].reshape(12 * G, Cc)])
    yt = oracle.latent_sublayer(xt, pd, wpt, pu, W, H, G, k)
    back = yt.reshape(B, W, H, C).transpose(0, 2, 1, 3).reshape(B, H * W, C)
    assert np.max(np.abs(back - y)) <= 1e-12 * max(1.0, np.max(np.abs(y)))


def test_sublayer_single_line_segments_closed_form():
    B, C, Cc, G, H, W = 2, 5, 3, 3, 4, 6
    x, pd, wp, pu = _weights(B, C, Cc, G, H, W, 2)
    y = oracle.latent_sublayer(x, pd, wp, pu, H, W, G, k_chunk=6)
    z = np.einsum("ck,bnk->bcn", pd, x)
    lam = np.einsum("jc,bcn->bjn", wp[:Cc], z)
    u = np.einsum("jc,bcn->bjn", wp[Cc:2 * Cc], z)
    ref = np.einsum("oc,bcn->bno", pu, 4 * u * lam * z)
    assert np.max(np.abs(ref - y)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_sublayer_linear_in_p_up():
    B, C, Cc, G, H, W = 1, 4, 2, 1, 3, 3
    x, pd, wp, pu = _weights(B, C, Cc, G, H, W, 3)
    a = oracle.latent_sublayer(x, pd, wp, pu, H, W, G)
    b = oracle.latent_sublayer(x, pd, wp, 2.5 * pu, H, W, G)
    assert np.allclose(b, 2.5 * a, rtol=1e-13, atol=0)


SUBLAYER_MUTANTS = [
    ("LR / RL tap planes left row-major", "if d in (LR, RL):", "if d in ():"),
    ("tap rows read group-major", "taps = par[:, 2 * Cc:].reshape(B, 4, G, 3, H, W)",
     "taps = par[:, 2 * Cc:].reshape(B, G, 4, 3, H, W).transpose(0, 2, 1, 3, 4, 5)"),
    ("u taken from the lambda rows", "u = par[:, Cc:2 * Cc]", "u = par[:, :Cc]"),
    ("output projected with reordered latent channels", "y = np.matmul(yt, p_up.T)",
     "y = np.matmul(yt, p_up[:, ::-1].T)"),
]


@pytest.mark.parametrize("name,old,new", SUBLAYER_MUTANTS, ids=[m[0] for m in SUBLAYER_MUTANTS])
def test_sublayer_pins_reject_mutant(monkeypatch, name, old, new):
    import inspect
    src = inspect.getsource(oracle.latent_sublayer)
    assert src.count(old) == 1, old
    ns = dict(vars(oracle))
    exec(src.replace(old, new), ns)
    monkeypatch.setattr(oracle, "latent_sublayer", ns["latent_sublayer"])
    failed = 0
    for check in (lambda: test_sublayer_transpose_symmetry(2, 3),
                  test_sublayer_single_line_segments_closed_form, test_sublayer_linear_in_p_up):
        try:
            check()
        except AssertionError:
            failed += 1
    assert failed > 0, name


def test_storage_rounding():
    to = oracle._to_storage
    # bf16 keeps 8 significand bits: 1 + 2^-8 is a halfway case between 1 and
    # 1 + 2^-7 and rounds to the even one (1); 1 + 3 * 2^-8 rounds up to 1 + 2^-6
    a = np.array([1.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -2.5, 0.0, 1 + 2.0 ** -7])
    assert np.array_equal(to(a, "bf16"), [1.0, 1.0, 1 + 2.0 ** -6, -2.5, 0.0, 1 + 2.0 ** -7])
    rng = np.random.default_rng(0)
    v = rng.standard_normal(10000)
    r = to(v, "bf16")
    # half an ulp of an 8-bit significand: at most 2^-8 relative (plus the
    # first rounding to fp32)
    assert np.all(np.abs(r - v) <= (2.0 ** -8 + 2.0 ** -24) * np.abs(v))
    assert np.max(np.abs(r - v) / np.abs(v)) > 2.0 ** -9      # not a finer type
    assert np.array_equal(to(r, "bf16"), r)
    f = to(v, "fp32")
    assert np.array_equal(f, v.astype(np.float32).astype(np.float64))
    assert to(v, None) is v
