"""ctypes binding of libgspn (include/gspn.h).  Argument marshalling only.

Every function here checks torch-level facts (device, dtype, contiguity,
element counts), allocates the output with torch when none is given, and
calls the C ABI on torch's current HIP stream.  All arithmetic happens in the
library's gfx950 kernels; there is no fallback.  If libgspn.so is missing the
first call raises.

Tensor layouts (see include/gspn.h):
  x, lam, u, y   [B, C, H, W]
  taps of a direction  B*C*3*H*W elements, laid out [B][C][3][lines][length]
      (TD/BU: lines are rows; LR/RL: lines are columns, i.e. transposed)
  w4             4*B*C*3*H*W elements, directions in the order TD, BU, LR, RL
  grouped taps   4*B*G*3*H*W elements ([4][B][G][3][..][..]); channel c reads
                 group c // (C // G)
"""
from __future__ import annotations

import ctypes
import os

import torch

TD, BU, LR, RL, ALL4 = 0, 1, 2, 3, 4
FP32, BF16 = 0, 1

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgspn.so")
_lib = None

_STATUS_EXC = {1: ValueError, 2: ValueError, 3: TypeError, 4: ValueError, 5: ValueError,
               6: ValueError, 7: ValueError, 8: RuntimeError, 9: ValueError}


def library_path() -> str:
    return _LIB_PATH


def lib():
    """The loaded libgspn (ctypes.CDLL).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("libgspn.so is not built (%s); run `python -m "
                               "spatial_line_scan_amd.build` or __graft_entry__.build()" % _LIB_PATH)
        L = ctypes.CDLL(_LIB_PATH)
        vp, i64, ci, cf = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
        L.gspn_abi_version.argtypes = []
        L.gspn_abi_version.restype = ci
        L.gspn_status_str.argtypes = [ci]
        L.gspn_status_str.restype = ctypes.c_char_p
        L.gspn_normalize_weights.argtypes = [vp, vp, ci, i64, i64, i64, i64, ci, cf, vp]
        L.gspn_normalize_weights.restype = ci
        L.gspn_scan_dir.argtypes = [vp, vp, vp, vp, ci, cf, vp, ci, ci, i64, i64, i64, i64, ci, vp]
        L.gspn_scan_dir.restype = ci
        L.gspn_prop2d_4dir.argtypes = [vp, vp, vp, vp, cf, vp, ci, i64, i64, i64, i64, vp]
        L.gspn_prop2d_4dir.restype = ci
        L.gspn_prop2d_4dir_ex.argtypes = [vp, vp, vp, vp, i64, i64, cf, vp, ci, i64, i64, i64,
                                          i64, vp]
        L.gspn_prop2d_4dir_ex.restype = ci
        L.gspn_prop2d_4dir_ex_ws.argtypes = [vp, vp, vp, vp, i64, i64, cf, vp, vp, i64, ci, i64, i64,
                                             i64, i64, vp]
        L.gspn_prop2d_4dir_ex_ws.restype = ci
        L.gspn_prop2d_4dir_ex_workspace.argtypes = [ci, i64, i64, i64, i64, i64]
        L.gspn_prop2d_4dir_ex_workspace.restype = i64
        L.gspn_latent_sublayer.argtypes = [vp, vp, vp, vp, i64, i64, cf, vp, vp, i64, ci, i64,
                                           i64, i64, i64, i64, vp]
        L.gspn_latent_sublayer.restype = ci
        L.gspn_latent_sublayer_workspace.argtypes = [ci, i64, i64, i64, i64, i64, i64]
        L.gspn_latent_sublayer_workspace.restype = i64
        L.gspn_prop2d_4dir_backward.argtypes = [vp, vp, vp, vp, vp, cf, vp, vp, vp, vp, vp, i64,
                                                ci, i64, i64, i64, i64, vp]
        L.gspn_prop2d_4dir_backward.restype = ci
        L.gspn_prop2d_4dir_backward_workspace.argtypes = [i64, i64, i64, i64]
        L.gspn_prop2d_4dir_backward_workspace.restype = i64
        L.gspn_prop2d_4dir_ex_backward.argtypes = [vp, vp, vp, vp, i64, i64, vp, cf, vp, vp, vp, vp,
                                                   vp, i64, ci, i64, i64, i64, i64, vp]
        L.gspn_prop2d_4dir_ex_backward.restype = ci
        L.gspn_prop2d_4dir_ex_backward_workspace.argtypes = [i64, i64, i64, i64, i64]
        L.gspn_prop2d_4dir_ex_backward_workspace.restype = i64
        L.gspn_prop2d_4dir_ex_backward_noalloc.argtypes = [vp, vp, vp, vp, i64, i64, vp, cf, vp,
                                                           vp, vp, vp, ci, i64, i64, i64, i64, vp]
        L.gspn_prop2d_4dir_ex_backward_noalloc.restype = ci
        L.gspn_noalloc_scratch_bytes.argtypes = []
        L.gspn_noalloc_scratch_bytes.restype = i64
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        msg = lib().gspn_status_str(status).decode()
        raise _STATUS_EXC.get(status, RuntimeError)(msg)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return FP32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError("gspn tensors must be float32 or bfloat16, got %s" % t.dtype)


def _same(ref: torch.Tensor, *ts: torch.Tensor):
    for t in ts:
        if t.device != ref.device or t.dtype != ref.dtype:
            raise ValueError("all tensors must share device and dtype")
        if not t.is_contiguous():
            raise ValueError("gspn tensors must be contiguous")
    if ref.device.type != "cuda":
        raise ValueError("gspn tensors must be on a GPU device")


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _p(t: torch.Tensor):
    return ctypes.c_void_p(t.data_ptr())


def normalize_weights(w: torch.Tensor, dir: int, B: int, C: int, H: int, W: int,
                      eps: float = 1e-6, out: torch.Tensor | None = None) -> torch.Tensor:
    """Row-stochastic taps from raw logits (one direction, or ALL4)."""
    _same(w, w)
    n = 3 * B * C * H * W * (4 if dir == ALL4 else 1)
    if w.numel() != n:
        raise ValueError("w has %d elements, expected %d" % (w.numel(), n))
    if out is None:
        out = torch.empty_like(w)
    _same(w, out)
    with torch.cuda.device(w.device):
        _check(lib().gspn_normalize_weights(_p(w), _p(out), _dtype_code(w), B, C, H, W, dir,
                                            float(eps), _stream(w)))
    return out


def scan_dir(x: torch.Tensor, lam: torch.Tensor, u: torch.Tensor, w: torch.Tensor, dir: int,
             w_is_raw: bool = True, out: torch.Tensor | None = None, accumulate: bool = False,
             eps: float = 1e-6) -> torch.Tensor:
    """u * h of one direction (accumulate: out += u * h)."""
    _same(x, lam, u, w)
    if x.dim() != 4 or lam.shape != x.shape or u.shape != x.shape:
        raise ValueError("x, lam, u must share one [B, C, H, W] shape")
    B, C, H, W = x.shape
    if w.numel() != 3 * x.numel():
        raise ValueError("w must hold 3*B*C*H*W elements")
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs an output tensor")
        out = torch.empty_like(x)
    _same(x, out)
    if out.shape != x.shape:
        raise ValueError("out must have x's shape")
    with torch.cuda.device(x.device):
        _check(lib().gspn_scan_dir(_p(x), _p(lam), _p(u), _p(w), int(bool(w_is_raw)), float(eps),
                                   _p(out), int(bool(accumulate)), _dtype_code(x), B, C, H, W,
                                   dir, _stream(x)))
    return out


def prop2d_4dir(x: torch.Tensor, lam: torch.Tensor, u: torch.Tensor, w4: torch.Tensor,
                eps: float = 1e-6, out: torch.Tensor | None = None) -> torch.Tensor:
    """y = u * (h_TD + h_BU + h_LR + h_RL) with fused tap normalisation."""
    _same(x, lam, u, w4)
    if x.dim() != 4 or lam.shape != x.shape or u.shape != x.shape:
        raise ValueError("x, lam, u must share one [B, C, H, W] shape")
    B, C, H, W = x.shape
    if w4.numel() != 12 * x.numel():
        raise ValueError("w4 must hold 4*B*C*3*H*W elements")
    if out is None:
        out = torch.empty_like(x)
    _same(x, out)
    if out.shape != x.shape:
        raise ValueError("out must have x's shape")
    with torch.cuda.device(x.device):
        _check(lib().gspn_prop2d_4dir(_p(x), _p(lam), _p(u), _p(w4), float(eps), _p(out),
                                      _dtype_code(x), B, C, H, W, _stream(x)))
    return out


def prop2d_4dir_ex_workspace_bytes(dtype: torch.dtype, B: int, C: int, groups: int, H: int,
                                   W: int) -> int:
    """Scratch bytes prop2d_4dir_ex uses to normalise each tap group once
    (0: none; every channel then normalises its group's taps)."""
    code = FP32 if dtype == torch.float32 else BF16
    n = lib().gspn_prop2d_4dir_ex_workspace(code, B, C, groups, H, W)
    if n < 0:
        raise ValueError("sizes not accepted by gspn_prop2d_4dir_ex")
    return n


def prop2d_4dir_ex(x: torch.Tensor, lam: torch.Tensor, u: torch.Tensor, w4: torch.Tensor,
                   groups: int, k_chunk: int = 1, eps: float = 1e-6,
                   out: torch.Tensor | None = None, workspace="auto") -> torch.Tensor:
    """prop2d_4dir with taps shared by `groups` contiguous channel groups and
    each scan cut into k_chunk segments (include/gspn.h).

    workspace: "auto" allocates (with torch) the scratch that lets each tap
    group be normalised once when the library would use it
    (gspn_prop2d_4dir_ex_ws); a tensor is used as that scratch; None calls
    gspn_prop2d_4dir_ex, which normalises the taps in every channel."""
    _same(x, lam, u, w4)
    if x.dim() != 4 or lam.shape != x.shape or u.shape != x.shape:
        raise ValueError("x, lam, u must share one [B, C, H, W] shape")
    B, C, H, W = x.shape
    if groups < 1 or C % groups:
        raise ValueError("groups must divide C")
    if w4.numel() != 12 * B * groups * H * W:
        raise ValueError("w4 must hold 4*B*groups*3*H*W elements")
    if out is None:
        out = torch.empty_like(x)
    _same(x, out)
    if out.shape != x.shape:
        raise ValueError("out must have x's shape")
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto', None or a tensor")
        need = prop2d_4dir_ex_workspace_bytes(x.dtype, B, C, groups, H, W)
        workspace = torch.empty(need // 4, dtype=torch.float32, device=x.device) if need else None
        use_ws = True
    else:
        use_ws = workspace is not None
    if workspace is not None and (workspace.device != x.device or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on x's device")
    with torch.cuda.device(x.device):
        if use_ws:
            ws_ptr = ctypes.c_void_p(workspace.data_ptr() if workspace is not None else 0)
            ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
            _check(lib().gspn_prop2d_4dir_ex_ws(_p(x), _p(lam), _p(u), _p(w4), int(groups),
                                                int(k_chunk), float(eps), _p(out), ws_ptr, ws_bytes,
                                                _dtype_code(x), B, C, H, W, _stream(x)))
        else:
            _check(lib().gspn_prop2d_4dir_ex(_p(x), _p(lam), _p(u), _p(w4), int(groups),
                                             int(k_chunk), float(eps), _p(out), _dtype_code(x), B,
                                             C, H, W, _stream(x)))
    return out


def prop2d_4dir_backward_workspace_bytes(B: int, C: int, H: int, W: int) -> int:
    """Scratch bytes prop2d_4dir_backward needs for these sizes (0: none)."""
    n = lib().gspn_prop2d_4dir_backward_workspace(B, C, H, W)
    if n < 0:
        raise ValueError("sizes not accepted by gspn_prop2d_4dir_backward")
    return n


def prop2d_4dir_backward(x: torch.Tensor, lam: torch.Tensor, u: torch.Tensor, w4: torch.Tensor,
                         gy: torch.Tensor, eps: float = 1e-6, workspace: torch.Tensor | None = None):
    """Gradients (gx, glam, gu, gw4) of prop2d_4dir given gy = dL/dy.

    The workspace (fp32 scratch, only needed for planes too large for on-chip
    memory) is allocated here with torch when none is given."""
    _same(x, lam, u, w4, gy)
    if x.dim() != 4 or lam.shape != x.shape or u.shape != x.shape or gy.shape != x.shape:
        raise ValueError("x, lam, u, gy must share one [B, C, H, W] shape")
    B, C, H, W = x.shape
    if w4.numel() != 12 * x.numel():
        raise ValueError("w4 must hold 4*B*C*3*H*W elements")
    need = prop2d_4dir_backward_workspace_bytes(B, C, H, W)
    if workspace is None and need > 0:
        workspace = torch.empty(need // 4, dtype=torch.float32, device=x.device)
    ws_ptr = ctypes.c_void_p(workspace.data_ptr() if workspace is not None else 0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if workspace is not None and (workspace.device != x.device or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on x's device")
    gx, glam, gu = torch.empty_like(x), torch.empty_like(x), torch.empty_like(x)
    gw4 = torch.empty_like(w4)
    with torch.cuda.device(x.device):
        _check(lib().gspn_prop2d_4dir_backward(_p(x), _p(lam), _p(u), _p(w4), _p(gy), float(eps),
                                               _p(gx), _p(glam), _p(gu), _p(gw4), ws_ptr, ws_bytes,
                                               _dtype_code(x), B, C, H, W, _stream(x)))
    return gx, glam, gu, gw4


def prop2d_4dir_ex_backward_workspace_bytes(B: int, C: int, groups: int, H: int, W: int) -> int:
    """Scratch bytes prop2d_4dir_ex_backward needs for these sizes (0: none)."""
    n = lib().gspn_prop2d_4dir_ex_backward_workspace(B, C, groups, H, W)
    if n < 0:
        raise ValueError("sizes not accepted by gspn_prop2d_4dir_ex_backward")
    return n


def prop2d_4dir_ex_backward(x: torch.Tensor, lam: torch.Tensor, u: torch.Tensor, w4: torch.Tensor,
                            gy: torch.Tensor, groups: int, k_chunk: int = 1, eps: float = 1e-6,
                            workspace: torch.Tensor | None = None):
    """Gradients (gx, glam, gu, gw4) of prop2d_4dir_ex given gy = dL/dy; gw4
    has w4's grouped layout.  The workspace is allocated here with torch when
    none is given."""
    _same(x, lam, u, w4, gy)
    if x.dim() != 4 or lam.shape != x.shape or u.shape != x.shape or gy.shape != x.shape:
        raise ValueError("x, lam, u, gy must share one [B, C, H, W] shape")
    B, C, H, W = x.shape
    if groups < 1 or C % groups:
        raise ValueError("groups must divide C")
    if w4.numel() != 12 * B * groups * H * W:
        raise ValueError("w4 must hold 4*B*groups*3*H*W elements")
    need = prop2d_4dir_ex_backward_workspace_bytes(B, C, groups, H, W)
    if workspace is None and need > 0:
        workspace = torch.empty(need // 4, dtype=torch.float32, device=x.device)
    if workspace is not None and (workspace.device != x.device or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on x's device")
    ws_ptr = ctypes.c_void_p(workspace.data_ptr() if workspace is not None else 0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    gx, glam, gu = torch.empty_like(x), torch.empty_like(x), torch.empty_like(x)
    gw4 = torch.empty_like(w4)
    with torch.cuda.device(x.device):
        _check(lib().gspn_prop2d_4dir_ex_backward(_p(x), _p(lam), _p(u), _p(w4), int(groups),
                                                  int(k_chunk), _p(gy), float(eps), _p(gx), _p(glam),
                                                  _p(gu), _p(gw4), ws_ptr, ws_bytes, _dtype_code(x),
                                                  B, C, H, W, _stream(x)))
    return gx, glam, gu, gw4


def prop2d_4dir_ex_backward_noalloc(x: torch.Tensor, lam: torch.Tensor, u: torch.Tensor,
                                    w4: torch.Tensor, gy: torch.Tensor, groups: int,
                                    k_chunk: int = 1, eps: float = 1e-6, out=None):
    """prop2d_4dir_ex_backward through the library's allocation-free entry
    point: its kernels use the library's static device scratch (at most
    noalloc_scratch_bytes() of workspace, else ValueError).  `out` =
    (gx, glam, gu, gw4) preallocated by the caller; allocated here with torch
    when None (the library call itself allocates nothing).  Calls overlapping
    in time on one GPU race on the shared scratch."""
    _same(x, lam, u, w4, gy)
    if x.dim() != 4 or lam.shape != x.shape or u.shape != x.shape or gy.shape != x.shape:
        raise ValueError("x, lam, u, gy must share one [B, C, H, W] shape")
    B, C, H, W = x.shape
    if groups < 1 or C % groups:
        raise ValueError("groups must divide C")
    if w4.numel() != 12 * B * groups * H * W:
        raise ValueError("w4 must hold 4*B*groups*3*H*W elements")
    if out is None:
        out = (torch.empty_like(x), torch.empty_like(x), torch.empty_like(x), torch.empty_like(w4))
    gx, glam, gu, gw4 = out
    _same(x, gx, glam, gu, gw4)
    if gx.shape != x.shape or glam.shape != x.shape or gu.shape != x.shape or \
            gw4.numel() != w4.numel():
        raise ValueError("out tensors must have the shapes of x, x, x, w4")
    with torch.cuda.device(x.device):
        _check(lib().gspn_prop2d_4dir_ex_backward_noalloc(
            _p(x), _p(lam), _p(u), _p(w4), int(groups), int(k_chunk), _p(gy), float(eps), _p(gx),
            _p(glam), _p(gu), _p(gw4), _dtype_code(x), B, C, H, W, _stream(x)))
    return gx, glam, gu, gw4


def noalloc_scratch_bytes() -> int:
    """Bytes of the library's static device scratch (per GPU)."""
    return lib().gspn_noalloc_scratch_bytes()


class Prop2d4Dir(torch.autograd.Function):
    """Autograd wrapper: forward prop2d_4dir, backward prop2d_4dir_backward."""

    @staticmethod
    def forward(ctx, x, lam, u, w4, eps=1e-6):
        ctx.eps = float(eps)
        ctx.save_for_backward(x, lam, u, w4)
        return prop2d_4dir(x, lam, u, w4, eps)

    @staticmethod
    def backward(ctx, gy):
        x, lam, u, w4 = ctx.saved_tensors
        gx, glam, gu, gw4 = prop2d_4dir_backward(x, lam, u, w4, gy.contiguous(), ctx.eps)
        return gx, glam, gu, gw4, None


class Prop2d4DirEx(torch.autograd.Function):
    """Autograd wrapper of the grouped / chunked operator: forward
    prop2d_4dir_ex, backward prop2d_4dir_ex_backward (w4 has the grouped
    layout [4][B][groups][3][H*W])."""

    @staticmethod
    def forward(ctx, x, lam, u, w4, groups, k_chunk=1, eps=1e-6):
        ctx.groups, ctx.k_chunk, ctx.eps = int(groups), int(k_chunk), float(eps)
        ctx.save_for_backward(x, lam, u, w4)
        return prop2d_4dir_ex(x, lam, u, w4, groups, k_chunk, eps)

    @staticmethod
    def backward(ctx, gy):
        x, lam, u, w4 = ctx.saved_tensors
        gx, glam, gu, gw4 = prop2d_4dir_ex_backward(x, lam, u, w4, gy.contiguous(), ctx.groups,
                                                    ctx.k_chunk, ctx.eps)
        return gx, glam, gu, gw4, None, None, None


def latent_sublayer_workspace_bytes(dtype: torch.dtype, B: int, C: int, Cc: int, groups: int,
                                    H: int, W: int) -> int:
    code = FP32 if dtype == torch.float32 else BF16
    n = lib().gspn_latent_sublayer_workspace(code, B, C, Cc, groups, H, W)
    if n < 0:
        raise ValueError("sizes not accepted by gspn_latent_sublayer")
    return n


def latent_sublayer(x_tok: torch.Tensor, p_down: torch.Tensor, w_param: torch.Tensor,
                    p_up: torch.Tensor, H: int, W: int, groups: int, k_chunk: int = 1,
                    eps: float = 1e-6, workspace: torch.Tensor | None = None,
                    out: torch.Tensor | None = None) -> torch.Tensor:
    """Latent propagation sublayer on tokens [B][H*W][C] (include/gspn.h):
    P_down, the 1x1 parameter convolutions, the four-direction scan and P_up.
    The workspace (bytes) is allocated here with torch when none is given."""
    _same(x_tok, p_down, w_param, p_up)
    if x_tok.dim() != 3 or x_tok.shape[1] != H * W:
        raise ValueError("x_tok must be [B, H*W, C]")
    B, _, C = x_tok.shape
    Cc = p_down.shape[0]
    if p_down.shape != (Cc, C) or p_up.shape != (C, Cc) or \
            w_param.shape != (2 * Cc + 12 * groups, Cc):
        raise ValueError("weights must be p_down [Cc, C], w_param [2Cc+12G, Cc], p_up [C, Cc]")
    need = latent_sublayer_workspace_bytes(x_tok.dtype, B, C, Cc, groups, H, W)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x_tok.device)
    if workspace.device != x_tok.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on x_tok's device")
    if out is None:
        out = torch.empty_like(x_tok)
    _same(x_tok, out)
    with torch.cuda.device(x_tok.device):
        _check(lib().gspn_latent_sublayer(
            _p(x_tok), _p(p_down), _p(w_param), _p(p_up), int(groups), int(k_chunk), float(eps),
            _p(out), _p(workspace), workspace.numel() * workspace.element_size(),
            _dtype_code(x_tok), B, C, Cc, H, W, _stream(x_tok)))
    return out
