"""gspn_prop2d_4dir_ex_backward_noalloc (the entry point that uses the
library's static device scratch instead of a caller's workspace) against
gspn_prop2d_4dir_ex_backward on the same inputs, both called through the C
ABI.  The two run the same kernels on the same inputs, so their results agree
bit for bit.  Two calls in a row, the second on a smaller problem, so the
second reads a scratch buffer that still holds the first call's contents."""
import ctypes

import pytest
import torch

from spatial_line_scan_amd import gspn
from spatial_line_scan_amd import inputs

pytestmark = pytest.mark.gpu

# (dtype, B, C, H, W, groups, k_chunk): the first is the larger problem; the
# second is smaller and takes another kernel form (fp32, odd sides, shared
# taps, chunked scans)
CALLS = [("bf16", 2, 8, 74, 74, 8, 1), ("fp32", 1, 4, 21, 26, 2, 3)]


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _run(L, x, lam, u, w4, gy, groups, k, noalloc):
    B, C, H, W = x.shape
    dt = gspn.FP32 if x.dtype == torch.float32 else gspn.BF16
    outs = [torch.full_like(x, float("nan")) for _ in range(3)] + [torch.full_like(w4, float("nan"))]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if noalloc:
        st = L.gspn_prop2d_4dir_ex_backward_noalloc(
            _p(x), _p(lam), _p(u), _p(w4), groups, k, _p(gy), 1e-6, *[_p(o) for o in outs], dt,
            B, C, H, W, stream)
    else:
        need = L.gspn_prop2d_4dir_ex_backward_workspace(B, C, groups, H, W)
        ws = torch.full((max(need, 4) // 4,), float("nan"), device=x.device)
        st = L.gspn_prop2d_4dir_ex_backward(
            _p(x), _p(lam), _p(u), _p(w4), groups, k, _p(gy), 1e-6, *[_p(o) for o in outs],
            _p(ws), need, dt, B, C, H, W, stream)
    assert st == 0, L.gspn_status_str(st).decode()
    torch.cuda.synchronize()
    return outs


def test_noalloc_matches_workspace_entry_point_twice():
    L = gspn.lib()
    for seed, (dtype, B, C, H, W, groups, k) in enumerate(CALLS):
        print("noalloc case", dtype, B, C, H, W, "groups", groups, "k", k, flush=True)
        assert L.gspn_prop2d_4dir_ex_backward_workspace(B, C, groups, H, W) <= \
            L.gspn_noalloc_scratch_bytes()
        shp = (B, C, H, W)
        x, lam, u, gy = (inputs.draw_torch(40 + seed, nm, shp, dtype, "cuda")
                         for nm in ("x", "lam", "u", "gy"))
        w4 = inputs.draw_torch(40 + seed, "w", (4, B, groups, 3, H * W), dtype, "cuda")
        ref = _run(L, x, lam, u, w4, gy, groups, k, noalloc=False)
        got = _run(L, x, lam, u, w4, gy, groups, k, noalloc=True)
        for name, a, b in zip(("gx", "glam", "gu", "gw4"), ref, got):
            assert torch.isfinite(a).all(), name
            assert torch.equal(a, b), (name, (a.float() - b.float()).abs().max().item())


def test_noalloc_rejects_oversized_problem_without_touching_outputs():
    L = gspn.lib()
    B, C, H, W = 32, 64, 74, 74
    assert L.gspn_prop2d_4dir_ex_backward_workspace(B, C, C, H, W) > L.gspn_noalloc_scratch_bytes()
    # sizes are validated before any pointer is used: small real buffers, so
    # nothing could be read or written even if the check were missing
    n = 12 * B * C * H * W
    big = torch.zeros(8, dtype=torch.bfloat16, device="cuda")
    outs = [torch.full((8,), 7.0, dtype=torch.bfloat16, device="cuda") for _ in range(4)]
    ins = [big.clone() for _ in range(5)]
    st = L.gspn_prop2d_4dir_ex_backward_noalloc(
        _p(ins[0]), _p(ins[1]), _p(ins[2]), _p(ins[3]), C, 1, _p(ins[4]), 1e-6,
        *[_p(o) for o in outs], gspn.BF16, B, C, H, W, None)
    assert n > 0 and st == 9, L.gspn_status_str(st).decode()
    with pytest.raises(ValueError, match="scratch"):
        gspn._check(st)
    torch.cuda.synchronize()
    for o in outs:
        assert (o == 7.0).all()
