"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the propagation operator; it only draws
numbers.  Values are a pure function of (seed, tensor id, element index), so
any slice of any tensor can be regenerated on its own and the result does not
depend on draw order, chunking or platform.

Generator: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014; finaliser constants as
published) used as a counter-based hash, and the Box-Muller transform
(G. Box, M. Muller, 1958) for standard normals:

    key      = mix(mix(seed) ^ (GAMMA * (tensor_id + 1)))
    bits(j)  = mix(key + GAMMA * (j + 1))
    u(j)     = ((bits(j) >> 11) + 1) * 2^-53          in (0, 1]
    z(e)     = sqrt(-2 ln u(2e)) * cos(2 pi u(2e+1))   float64

Storage rounding: fp32 tensors hold float32(z) (round to nearest even);
bf16 tensors hold bf16(float32(z)) (round to nearest even on the fp32 bits).

Tensor ids: x = 0, lambda = 1, u = 2, taps of all four directions = 3,
upstream gradient gy (dL/dy, for the backward) = 4; latent sublayer: tokens
x_tok = 5, p_down = 6, w_param = 7, p_up = 8 (each weight matrix is drawn
N(0, 1), scaled by 1 / sqrt(its fan-in) in float32, then rounded to the
storage type).
"""
from __future__ import annotations

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

TENSOR_IDS = {"x": 0, "lam": 1, "u": 2, "w": 3, "gy": 4, "x_tok": 5, "p_down": 6, "w_param": 7,
              "p_up": 8}
_CHUNK = 1 << 22


def _mix(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _key(seed: int, tensor_id: int) -> np.uint64:
    with np.errstate(over="ignore"):
        s = _mix(np.array([seed & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64))
        t = GAMMA * np.uint64(tensor_id + 1)
        return _mix(s ^ t)[0]


def normal_f64(seed: int, tensor_id: int, start: int, count: int) -> np.ndarray:
    """Standard normals z(start) .. z(start + count - 1) of one tensor stream."""
    key = _key(seed, tensor_id)
    out = np.empty(count, dtype=np.float64)
    with np.errstate(over="ignore"):
        for lo in range(0, count, _CHUNK):
            n = min(_CHUNK, count - lo)
            e = np.arange(start + lo, start + lo + n, dtype=np.uint64)
            j1 = np.uint64(2) * e + np.uint64(1)     # counter of u(2e), offset by one
            b1 = _mix(key + GAMMA * j1)
            b2 = _mix(key + GAMMA * (j1 + np.uint64(1)))
            u1 = ((b1 >> np.uint64(11)) + np.uint64(1)).astype(np.float64) * 2.0 ** -53
            u2 = ((b2 >> np.uint64(11)) + np.uint64(1)).astype(np.float64) * 2.0 ** -53
            out[lo:lo + n] = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)
    return out


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest even); returns uint16 bit patterns."""
    bits = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))
    return ((bits + bias) >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32 values."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def draw(seed: int, name: str, shape, dtype: str, start: int = 0) -> np.ndarray:
    """Values of one tensor (or of the slice starting at element `start`).

    Returns float32 values; for dtype 'bf16' they are already rounded to bf16.
    """
    count = int(np.prod(shape))
    z = normal_f64(seed, TENSOR_IDS[name], start, count).astype(np.float32)
    if dtype == "bf16":
        z = f32_from_bf16_bits(bf16_bits_from_f32(z))
    elif dtype != "fp32":
        raise ValueError("dtype must be 'fp32' or 'bf16'")
    return z.reshape(shape)


def problem(B: int, C: int, H: int, W: int, seed: int, dtype: str) -> dict:
    """All inputs of one propagation problem as float32 numpy arrays.

    x, lam, u: [B][C][H][W]; w: [4][B][C][3][H*W] taps (per direction laid out
    [3][lines][line length] of that direction).
    """
    shp = (B, C, H, W)
    return {
        "x": draw(seed, "x", shp, dtype),
        "lam": draw(seed, "lam", shp, dtype),
        "u": draw(seed, "u", shp, dtype),
        "w": draw(seed, "w", (4, B, C, 3, H * W), dtype),
    }


def plane_slice(B: int, C: int, H: int, W: int, seed: int, dtype: str, b: int, c: int) -> dict:
    """Inputs of the single (b, c) plane of the problem drawn by `problem`.

    Same values as slicing the full tensors, computed without drawing them.
    """
    n = H * W
    pl = b * C + c
    out = {name: draw(seed, name, (1, 1, H, W), dtype, start=pl * n) for name in ("x", "lam", "u")}
    w = np.empty((4, 1, 1, 3, n), dtype=np.float32)
    for d in range(4):
        w[d, 0, 0] = draw(seed, "w", (3, n), dtype, start=((d * B + b) * C + c) * 3 * n)
    out["w"] = w
    return out


# ------------------------------------------------------------------ torch path
#
# The same generator written with torch int64 tensors (two's-complement
# wrap-around equals arithmetic modulo 2^64; logical shifts are masked), so
# large problems can be drawn on the device.  The integer stream is identical
# bit for bit; the float64 log/cos may differ from numpy's in the last bit,
# which changes a rounded fp32 value with probability about 2^-28.

def _signed(v: int) -> int:
    v &= 0xFFFFFFFFFFFFFFFF
    return v - (1 << 64) if v >= (1 << 63) else v


_GAMMA_S = _signed(int(GAMMA))
_M1_S = _signed(int(_M1))
_M2_S = _signed(int(_M2))


def _srl(z, k: int):
    return (z >> k) & ((1 << (64 - k)) - 1)


def _mix_t(z):
    z = (z ^ _srl(z, 30)) * _M1_S
    z = (z ^ _srl(z, 27)) * _M2_S
    return z ^ _srl(z, 31)


def draw_torch(seed: int, name: str, shape, dtype: str, device, start: int = 0):
    """Tensor of the values `draw` returns, generated on `device`.

    dtype 'fp32' gives a float32 tensor, 'bf16' a bfloat16 tensor.
    """
    import torch
    count = int(np.prod(shape))
    key = _signed(int(_key(seed, TENSOR_IDS[name])))
    out = torch.empty(count, dtype=torch.float32, device=device)
    chunk = 1 << 24
    for lo in range(0, count, chunk):
        n = min(chunk, count - lo)
        e = torch.arange(start + lo, start + lo + n, dtype=torch.int64, device=device)
        j1 = e * 2 + 1
        b1 = _mix_t(key + _GAMMA_S * j1)
        b2 = _mix_t(key + _GAMMA_S * (j1 + 1))
        u1 = (_srl(b1, 11) + 1).to(torch.float64) * 2.0 ** -53
        u2 = (_srl(b2, 11) + 1).to(torch.float64) * 2.0 ** -53
        z = torch.sqrt(-2.0 * torch.log(u1)) * torch.cos(2.0 * np.pi * u2)
        out[lo:lo + n] = z.to(torch.float32)
        del e, j1, b1, b2, u1, u2, z
    if dtype == "bf16":
        out = out.to(torch.bfloat16)
    elif dtype != "fp32":
        raise ValueError("dtype must be 'fp32' or 'bf16'")
    return out.reshape(shape)


def problem_torch(B: int, C: int, H: int, W: int, seed: int, dtype: str, device) -> dict:
    """`problem` drawn directly as device tensors."""
    shp = (B, C, H, W)
    return {
        "x": draw_torch(seed, "x", shp, dtype, device),
        "lam": draw_torch(seed, "lam", shp, dtype, device),
        "u": draw_torch(seed, "u", shp, dtype, device),
        "w": draw_torch(seed, "w", (4, B, C, 3, H * W), dtype, device),
    }


def to_torch(a: np.ndarray, dtype: str, device="cpu"):
    """A torch tensor holding exactly the values of `a` in the storage dtype."""
    import torch
    if dtype == "bf16":
        bits = bf16_bits_from_f32(a)
        t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32).copy())
    return t.reshape(a.shape).to(device)


def sublayer_problem_torch(B: int, C: int, Cc: int, G: int, H: int, W: int, seed: int, dtype: str,
                           device) -> dict:
    """Inputs of one latent sublayer call: tokens [B][H*W][C] and the three
    weight matrices, drawn on `device`."""
    import torch
    out = {"x_tok": draw_torch(seed, "x_tok", (B, H * W, C), dtype, device)}
    for name, shape, fan_in in (("p_down", (Cc, C), C), ("w_param", (2 * Cc + 12 * G, Cc), Cc),
                                ("p_up", (C, Cc), Cc)):
        w = draw_torch(seed, name, shape, "fp32", device) * np.float32(1.0 / np.sqrt(fan_in))
        out[name] = w.to(torch.bfloat16) if dtype == "bf16" else w
    return out
