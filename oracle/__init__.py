"""fp64 CPU oracle for the GSPN four-direction line-scan propagation.

TEST INFRASTRUCTURE ONLY.  The tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the product library
(``spatial_line_scan_amd``) never imports it and shares no code with it.

The arithmetic lives in ``gspn_oracle.c`` (plain C, compiled with gcc); this
module only marshals numpy arrays into it.  Every input is widened exactly to
float64 (fp32 and bf16 values are exactly representable), so the oracle sees
the same numbers the GPU path sees.

Functions
---------
normalize(w_raw, NL, L, eps)              -> normalised taps (one direction)
scan_dir(x, lam, u, w, dir, w_is_raw, eps) -> u * h for one direction
prop2d(x, lam, u, w4, eps)                -> sum over the four directions
prop2d_backward(x, lam, u, w4, gy, eps)   -> (gx, glam, gu, gw4), the gradient
                                             of <gy, prop2d(x, lam, u, w4)>
prop2d_ex(x, lam, u, w4g, groups, k_chunk, eps)
                                          -> prop2d with taps shared by groups of
                                             channels and/or chunked scans
latent_sublayer(x_tok, p_down, w_param, p_up, H, W, groups, k_chunk, eps)
                                          -> the latent propagation sublayer:
                                             1x1 projections around prop2d_ex

Layouts follow the C file's header: x, lam, u: [B][C][H][W]; the taps of one
direction: [B][C][3][NL][L] indexed by (line, position) of that direction
(TD/BU: NL=H, L=W; LR/RL: NL=W, L=H); w4: [4][B][C][3][..][..]; grouped
taps w4g: [4][B][G][3][..][..].

Parity unpinned: none.  Each function is pinned: tests/test_oracle_pins.py,
tests/test_oracle_backward.py, tests/test_oracle_ex.py.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

TD, BU, LR, RL = 0, 1, 2, 3

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gspn_oracle.c")
_LIB = os.path.join(_HERE, "libgspn_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile gspn_oracle.c with gcc into oracle/libgspn_oracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load(path: str | None = None):
    """Load the compiled oracle (building it first), or a given build of it."""
    global _lib
    if path is not None or _lib is None:
        if path is None:
            path = build()
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        L = ctypes.c_long
        lib.gspn_oracle_normalize.argtypes = [dp, dp, L, L, L, ctypes.c_double]
        lib.gspn_oracle_normalize.restype = None
        lib.gspn_oracle_scan_dir.argtypes = [dp, dp, dp, dp, ctypes.c_int, ctypes.c_double,
                                             dp, L, L, L, L, ctypes.c_int]
        lib.gspn_oracle_scan_dir.restype = ctypes.c_int
        lib.gspn_oracle_prop2d.argtypes = [dp, dp, dp, dp, ctypes.c_double, dp, L, L, L, L]
        lib.gspn_oracle_prop2d.restype = ctypes.c_int
        if hasattr(lib, "gspn_oracle_prop2d_backward"):
            lib.gspn_oracle_prop2d_backward.argtypes = [dp, dp, dp, dp, dp, ctypes.c_double,
                                                        dp, dp, dp, dp, L, L, L, L]
            lib.gspn_oracle_prop2d_backward.restype = ctypes.c_int
        if hasattr(lib, "gspn_oracle_prop2d_ex"):
            lib.gspn_oracle_prop2d_ex.argtypes = [dp, dp, dp, dp, L, L, ctypes.c_double, dp,
                                                  L, L, L, L]
            lib.gspn_oracle_prop2d_ex.restype = ctypes.c_int
        if hasattr(lib, "gspn_oracle_prop2d_ex_backward"):
            lib.gspn_oracle_prop2d_ex_backward.argtypes = [dp, dp, dp, dp, dp, L, L, ctypes.c_double,
                                                           dp, dp, dp, dp, L, L, L, L]
            lib.gspn_oracle_prop2d_ex_backward.restype = ctypes.c_int
        _lib = lib
    return _lib


def use_library(path: str | None):
    """Point this module at another build of gspn_oracle.c (None: the default).

    Used by the mutation tests, which compile deliberately broken copies of
    the oracle and check that the pins reject them.
    """
    global _lib
    _lib = None
    if path is not None:
        _load(path)


def _f64(a) -> np.ndarray:
    """Exact widening to a contiguous float64 numpy array (torch tensors too)."""
    if hasattr(a, "detach"):  # torch tensor: go through fp32 (exact for bf16/fp32)
        import torch
        a = a.detach().to("cpu", torch.float32).numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def line_geometry(dir: int, H: int, W: int):
    """(number of lines, line length) for a direction."""
    return (H, W) if dir in (TD, BU) else (W, H)


def normalize(w_raw, NL: int, L: int, eps: float = 1e-6) -> np.ndarray:
    """Row-stochastic normalisation of taps laid out [..][3][NL][L]."""
    w = _f64(w_raw)
    assert w.size % (3 * NL * L) == 0
    out = np.empty_like(w)
    _load().gspn_oracle_normalize(_ptr(w), _ptr(out), w.size // (3 * NL * L), NL, L, float(eps))
    return out


def scan_dir(x, lam, u, w, dir: int, w_is_raw: bool = True, eps: float = 1e-6) -> np.ndarray:
    """u * h for one direction; x, lam, u: [B][C][H][W], w: [B][C][3][NL][L]."""
    x, lam, u, w = _f64(x), _f64(lam), _f64(u), _f64(w)
    B, C, H, W = x.shape
    assert lam.shape == x.shape and u.shape == x.shape and w.size == 3 * x.size
    out = np.empty_like(x)
    rc = _load().gspn_oracle_scan_dir(_ptr(x), _ptr(lam), _ptr(u), _ptr(w), int(bool(w_is_raw)),
                                      float(eps), _ptr(out), B, C, H, W, int(dir))
    if rc != 0:
        raise MemoryError("oracle scan could not allocate scratch")
    return out


def prop2d(x, lam, u, w4, eps: float = 1e-6) -> np.ndarray:
    """y = sum over TD, BU, LR, RL of u * h_d with normalised taps."""
    x, lam, u, w4 = _f64(x), _f64(lam), _f64(u), _f64(w4)
    B, C, H, W = x.shape
    assert w4.size == 12 * x.size
    y = np.empty_like(x)
    rc = _load().gspn_oracle_prop2d(_ptr(x), _ptr(lam), _ptr(u), _ptr(w4), float(eps), _ptr(y),
                                    B, C, H, W)
    if rc != 0:
        raise MemoryError("oracle propagation could not allocate scratch")
    return y


def prop2d_backward(x, lam, u, w4, gy, eps: float = 1e-6):
    """Gradient of <gy, prop2d(x, lam, u, w4)> with respect to x, lam, u and w4."""
    x, lam, u, w4, gy = _f64(x), _f64(lam), _f64(u), _f64(w4), _f64(gy)
    B, C, H, W = x.shape
    assert w4.size == 12 * x.size and gy.shape == x.shape
    gx, glam, gu = np.empty_like(x), np.empty_like(x), np.empty_like(x)
    gw4 = np.empty_like(w4)
    rc = _load().gspn_oracle_prop2d_backward(_ptr(x), _ptr(lam), _ptr(u), _ptr(w4), _ptr(gy),
                                             float(eps), _ptr(gx), _ptr(glam), _ptr(gu), _ptr(gw4),
                                             B, C, H, W)
    if rc != 0:
        raise MemoryError("oracle backward could not allocate scratch")
    return gx, glam, gu, gw4


def prop2d_ex(x, lam, u, w4g, groups: int, k_chunk: int = 1, eps: float = 1e-6) -> np.ndarray:
    """prop2d with taps shared by `groups` contiguous channel groups (w4g:
    [4][B][groups][3][..][..]) and each scan cut into k_chunk segments."""
    x, lam, u, w4g = _f64(x), _f64(lam), _f64(u), _f64(w4g)
    B, C, H, W = x.shape
    assert w4g.size == 12 * B * groups * H * W
    y = np.empty_like(x)
    rc = _load().gspn_oracle_prop2d_ex(_ptr(x), _ptr(lam), _ptr(u), _ptr(w4g), int(groups),
                                       int(k_chunk), float(eps), _ptr(y), B, C, H, W)
    if rc == -2:
        raise ValueError("groups must divide C and k_chunk must be >= 1")
    if rc != 0:
        raise MemoryError("oracle propagation could not allocate scratch")
    return y


def prop2d_ex_backward(x, lam, u, w4g, gy, groups: int, k_chunk: int = 1, eps: float = 1e-6):
    """Gradient of <gy, prop2d_ex(x, lam, u, w4g, groups, k_chunk)> with respect
    to x, lam, u and w4g (the tap gradient has the grouped layout of w4g)."""
    x, lam, u, w4g, gy = _f64(x), _f64(lam), _f64(u), _f64(w4g), _f64(gy)
    B, C, H, W = x.shape
    assert w4g.size == 12 * B * groups * H * W and gy.shape == x.shape
    gx, glam, gu = np.empty_like(x), np.empty_like(x), np.empty_like(x)
    gw4 = np.empty_like(w4g)
    rc = _load().gspn_oracle_prop2d_ex_backward(_ptr(x), _ptr(lam), _ptr(u), _ptr(w4g), _ptr(gy),
                                                int(groups), int(k_chunk), float(eps), _ptr(gx),
                                                _ptr(glam), _ptr(gu), _ptr(gw4), B, C, H, W)
    if rc == -2:
        raise ValueError("groups must divide C and k_chunk must be >= 1")
    if rc != 0:
        raise MemoryError("oracle backward could not allocate scratch")
    return gx, glam, gu, gw4


def _to_storage(a: np.ndarray, storage: str | None) -> np.ndarray:
    """Values of `a` once stored as `storage` (None: kept in fp64).  fp32:
    round to nearest even; bf16: to fp32, then to the nearest even bf16 (the
    upper 16 bits of the fp32 pattern after adding 0x7fff plus the lowest kept
    bit), as a tensor of that type written from an fp32 result holds."""
    if storage is None:
        return a
    f = np.ascontiguousarray(a, dtype=np.float32)
    if storage == "fp32":
        return f.astype(np.float64)
    assert storage == "bf16"
    bits = f.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def latent_sublayer(x_tok, p_down, w_param, p_up, H: int, W: int, groups: int, k_chunk: int = 1,
                    eps: float = 1e-6, storage: str | None = None, with_scale: bool = False):
    """Latent-space propagation sublayer (paper text §5.1; reading notes, key
    design 1): tokens x_tok [B][H*W][C] are projected to Cc latent channels
    by the 1x1 convolution p_down [Cc][C]; per-position propagation
    parameters come from the 1x1 convolution w_param [2 Cc + 12 G][Cc] of
    the latent (rows: lambda for the Cc channels, u for the Cc channels,
    then the raw taps in [direction TD, BU, LR, RL][group][tap] order); the
    latent is propagated in four directions (prop2d_ex, G tap groups,
    k_chunk segments) and projected back by p_up [C][Cc].  Returns
    y_tok [B][H*W][C] in fp64.  Every matrix product is a plain numpy
    matmul in fp64.  With `storage` ("fp32" or "bf16") the latent, the
    parameters and the scan output are rounded to that type where a layer
    storing its activations in it writes them (the inputs are taken as
    given).  with_scale: also return |y_c^T| |p_up^T|, the componentwise
    magnitudes of the output projection's terms."""
    x_tok, p_down, w_param, p_up = _f64(x_tok), _f64(p_down), _f64(w_param), _f64(p_up)
    B, N, C = x_tok.shape
    Cc = p_down.shape[0]
    G = groups
    assert N == H * W and p_down.shape == (Cc, C) and p_up.shape == (C, Cc)
    assert w_param.shape == (2 * Cc + 12 * G, Cc)
    z = _to_storage(np.matmul(p_down, np.transpose(x_tok, (0, 2, 1))), storage)   # [B][Cc][N]
    par = _to_storage(np.matmul(w_param, z), storage)                # [B][2Cc+12G][N]
    lam = par[:, :Cc].reshape(B, Cc, H, W)
    u = par[:, Cc:2 * Cc].reshape(B, Cc, H, W)
    taps = par[:, 2 * Cc:].reshape(B, 4, G, 3, H, W)
    w4 = np.empty((4, B, G, 3, H * W))
    for d in range(4):
        t = taps[:, d]
        if d in (LR, RL):             # column-major lines: [3][W][H]
            t = np.transpose(t, (0, 1, 2, 4, 3))
        w4[d] = t.reshape(B, G, 3, H * W)
    yc = _to_storage(prop2d_ex(z.reshape(B, Cc, H, W), lam, u, w4, G, k_chunk, eps), storage)
    yt = yc.reshape(B, Cc, N).transpose(0, 2, 1)
    y = np.matmul(yt, p_up.T)                                        # [B][N][C]
    if with_scale:
        return y, np.matmul(np.abs(yt), np.abs(p_up.T))
    return y
