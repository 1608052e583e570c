"""Throughput of the four-direction GSPN propagation on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload latent1k]

One step = one gspn_prop2d_4dir launch over the whole workload (normalise
the 12 taps of every pixel-channel, scan all four directions, write y), on
inputs already resident in HBM.  Input sets are rotated so that successive
steps do not hit the 256 MB Infinity Cache.  Prints one JSON line.

value     : algorithmic GB/s = 16 values per pixel-channel (read x, lambda, u
            and 4 x 3 taps, write y) x bytes per value / wall time per step
roofline  : the same bytes / average kernel duration (HIP events on the
            launch stream at the two ends of the timed region, the same K
            back-to-back launches the wall clock times, divided by K; the
            minimum and median of 100 single launches from events around
            each), against the
            MI355X HBM peak of 8 TB/s; `traffic`
            is the measured HBM bytes per launch from the committed rocprofv3
            counter summary when it was taken on the current kernel source
cpu_baseline : the fp64 C oracle on the host, single thread, on a bounded
            sample of the same workload (whole planes)
variants  : gspn_prop2d_4dir_ex on the same workload shape, timed the same
            way (not part of `value`): taps shared by all channels of an image
            (groups = 1; algorithmic bytes 4 + 12 G / C values per
            pixel-channel) and a chunked scan (k_chunk = 4, per-channel taps)
sublayer  : gspn_latent_sublayer (P_down, parameter 1x1 convolutions, scan,
            P_up) on the pages' 1K shape: B=32 images of 74 x 74 tokens, C=1152
            compressed to Cc=64, bf16; per-channel taps (G = 64) and shared taps
            (G = 1).  Bytes: tokens in + tokens out (the least any
            implementation moves)
backward  : the gradient entry point (gspn_prop2d_4dir_backward) on the same
            workload and rotated sets, timed the same way (not part of
            `value`); algorithmic bytes = 31 values per pixel-channel (read x,
            lambda, u, gy and 12 taps, write gx, glambda, gu and 12 tap
            gradients)
pixel_ordered_taps : what a caller holding the LR / RL taps in pixel order
            ([3][H][W]) pays: a torch transpose of those 6 tap planes into the
            library's line-major layout, then the call
workloads : the other configurations, each timed the same way with its own
            roofline: latent2k (4 x 64 x 148^2 bf16, forward and backward),
            the same at 147^2 (odd side), base378 (8 x 64 x 27^2 fp32) with one
            input set (warm: it fits the Infinity Cache) and rotated, wide256
            (1 x 1024 x 256^2 fp32, forward and backward)
backward_variants : gspn_prop2d_4dir_ex_backward on the same shape: shared
            taps (groups = 1) and per-channel taps, each with four-segment
            scans (k_chunk = 4); algorithmic bytes 7 + 24 G / C values per
            pixel-channel
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "4-dir GSPN propagation GB/s & ms (B=32,C_c=64,74×74) + % of HBM peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prop2d_latent1k_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "spatial_line_scan_amd", "csrc", f)
                  for f in ("gspn_kernels.hip", "gspn_prop2d_quad.hip", "gspn_internal.h",
                            "gspn_device.h", "gspn_lane.h")]
BWD_VALUES_PER_PIXEL = 31


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed counter summary, if current."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("workload") != workload or t.get("kernel_source_sha") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(wl, budget_s: float, gpu_inputs: dict, gpu_out):
    """Time the fp64 oracle on whole planes of the workload, single-threaded,
    pinned to one host core; the median of three runs of a third of the
    budget each.

    The planes are those of the first rotated input set, in order, until a
    run's time is spent (whole passes again when the workload takes less);
    the next run continues where the last stopped.  The GPU output of the
    first pass's planes from the timed steps is compared with the oracle's
    as a by-product.
    """
    import ctypes

    import numpy as np
    import torch

    import oracle
    from oracle.tolerance import RTOL, compare

    lib = oracle._load()
    dp = ctypes.POINTER(ctypes.c_double)
    n = wl.H * wl.W
    f64 = lambda t: t.to("cpu", torch.float32).numpy().astype(np.float64)
    X, LAM, U, Wt = (f64(gpu_inputs[k]) for k in ("x", "lam", "u", "w"))
    Wt = Wt.reshape(4, wl.B, wl.C, 3 * n)
    Y = f64(gpu_out)
    planes, all_ok, details = 0, True, []
    order = [(b, c) for b in range(wl.B) for c in range(wl.C)]
    per_plane_bytes = 16 * wl.elem_bytes * n
    old_affinity = os.sched_getaffinity(0)
    core = max(old_affinity)
    os.sched_setaffinity(0, {core})
    rates, total_spent = [], 0.0
    try:
        for _ in range(3):
            spent, done = 0.0, 0
            while spent < budget_s / 3:
                b, c = order[planes % len(order)]
                arrs = [np.ascontiguousarray(a[b, c]) for a in (X, LAM, U)]
                arrs.append(np.ascontiguousarray(Wt[:, b, c]))
                y = np.empty_like(arrs[0])
                t0 = time.perf_counter()
                rc = lib.gspn_oracle_prop2d(*(a.ctypes.data_as(dp) for a in arrs), 1e-6,
                                            y.ctypes.data_as(dp), 1, 1, wl.H, wl.W)
                spent += time.perf_counter() - t0
                if rc != 0:
                    raise MemoryError("oracle failed")
                if planes < len(order):
                    ok, msg = compare(Y[b, c], y, RTOL[wl.dtype])
                    all_ok &= ok
                    if len(details) < 2 or not ok:
                        details.append("(%d,%d): %s" % (b, c, msg))
                planes += 1
                done += 1
            rates.append(done * per_plane_bytes / spent / 1e9)
            total_spent += spent
    finally:
        os.sched_setaffinity(0, old_affinity)
    return {
        "value": float(np.median(rates)),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": "%d planes (%.1f passes over the %d planes, %dx%d, %s values, of the timed "
                  "inputs), fp64 C loop on host core %d, three runs of %.1f s, median" % (
                      planes, planes / len(order), len(order), wl.H, wl.W, wl.dtype, core,
                      budget_s / 3),
        "runs_GBps": [round(r, 4) for r in rates],
        "seconds": total_spent,
        "cpu": _cpu_model(),
        "host_cores_visible": os.cpu_count(),
        "gpu_output_matches_oracle_on_sample": bool(all_ok),
        "parity_detail": details[:6],
    }


def _region(fn, steps, stream):
    """One timed region of `steps` back-to-back calls: its wall time, and its
    kernel time per call from a pair of HIP events recorded on the launch
    stream at the region's two ends (inside the wall clock), divided by
    `steps`."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    a.record(stream)
    for i in range(steps):
        fn(i)
    b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, float(a.elapsed_time(b)) / steps


def _single_calls(fn, n, stream):
    """Event pairs around each of n single calls (each pair's own overhead
    included): the fastest and the median call, in ms."""
    import numpy as np
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for i in range(n):
        ev[i][0].record(stream)
        fn(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    t = [x.elapsed_time(y) for x, y in ev]
    return float(np.min(t)), float(np.median(t))


def _single_min(fn, steps, stream):
    """The fastest single call, from event pairs around each of `steps`
    calls (each pair's own overhead included)."""
    return _single_calls(fn, steps, stream)[0]


def _timed(fn, steps, warmup, stream):
    """Wall time of `steps` calls, their kernel time per call from HIP events
    around the same calls, and the fastest single call."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    wall, kavg = _region(fn, steps, stream)
    return wall, kavg, _single_min(fn, steps, stream)


def variant_leg(wl, args, dev, G, k):
    """gspn_prop2d_4dir_ex with `G` tap groups and k-chunk scans on the
    workload's shape, over rotated input sets of at least --rotate-bytes."""
    import numpy as np
    import torch

    from spatial_line_scan_amd import gspn, inputs

    shp = (wl.B, wl.C, wl.H, wl.W)
    base = {n: inputs.draw_torch(0, n, shp, wl.dtype, dev) for n in ("x", "lam", "u")}
    base["w"] = inputs.draw_torch(0, "w", (4, wl.B, G, 3, wl.H * wl.W), wl.dtype, dev)
    nbytes = int(round((4 + 12.0 * G / wl.C) * wl.elem_bytes * wl.pixels))
    nsets = max(1, int(np.ceil(args.rotate_bytes / nbytes)))
    sets = [base] + [{n: t.clone() for n, t in base.items()} for _ in range(nsets - 1)]
    outs = [torch.empty_like(base["x"]) for _ in range(nsets)]
    # the scratch in which shared taps are normalised once per group,
    # allocated before the timed region
    need = gspn.prop2d_4dir_ex_workspace_bytes(base["x"].dtype, wl.B, wl.C, G, wl.H, wl.W)
    ws = torch.empty(max(need, 4) // 4, dtype=torch.float32, device=dev) if need else None
    torch.cuda.synchronize()

    def fn(i):
        s = sets[i % nsets]
        gspn.prop2d_4dir_ex(s["x"], s["lam"], s["u"], s["w"], G, k, out=outs[i % nsets],
                            workspace=ws)

    wall, kavg, kmin = _timed(fn, args.steps, args.warmup, torch.cuda.current_stream(dev))
    achieved = nbytes / (kavg * 1e-3) / 1e9
    del sets, outs
    torch.cuda.empty_cache()
    return {"groups": G, "k_chunk": k, "ms_per_step": round(wall * 1e3 / args.steps, 5),
            "value": round(nbytes / (wall / args.steps) / 1e9, 2), "unit": "GB/s",
            "algorithmic_bytes_per_step": nbytes, "rotated_input_sets": nsets,
            "shared_normalisation_workspace_bytes": need,
            "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                         "kernel_ms_avg": round(kavg, 5), "kernel_ms_min": round(kmin, 5)}}


def ex_backward_leg(wl, args, dev, G, k):
    """gspn_prop2d_4dir_ex_backward (tap groups, chunked scans) on the
    workload's shape over rotated input sets: reads x, lambda, u, gy and the
    grouped taps, writes gx, glambda, gu and the grouped tap gradients."""
    import numpy as np
    import torch

    from spatial_line_scan_amd import gspn, inputs

    shp = (wl.B, wl.C, wl.H, wl.W)
    base = {n: inputs.draw_torch(0, n, shp, wl.dtype, dev) for n in ("x", "lam", "u", "gy")}
    base["w"] = inputs.draw_torch(0, "w", (4, wl.B, G, 3, wl.H * wl.W), wl.dtype, dev)
    nbytes = int(round((7 + 24.0 * G / wl.C) * wl.elem_bytes * wl.pixels))
    nsets = max(1, int(np.ceil(args.rotate_bytes / nbytes)))
    sets = [base] + [{n: t.clone() for n, t in base.items()} for _ in range(nsets - 1)]
    need = gspn.prop2d_4dir_ex_backward_workspace_bytes(wl.B, wl.C, G, wl.H, wl.W)
    ws = torch.empty(max(need, 4) // 4, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def fn(i):
        s = sets[i % nsets]
        gspn.prop2d_4dir_ex_backward(s["x"], s["lam"], s["u"], s["w"], s["gy"], G, k, workspace=ws)

    wall, kavg, kmin = _timed(fn, args.steps, args.warmup, torch.cuda.current_stream(dev))
    achieved = nbytes / (kavg * 1e-3) / 1e9
    del sets, ws
    torch.cuda.empty_cache()
    return {"groups": G, "k_chunk": k, "ms_per_step": round(wall * 1e3 / args.steps, 5),
            "value": round(nbytes / (wall / args.steps) / 1e9, 2), "unit": "GB/s",
            "algorithmic_bytes_per_step": nbytes, "rotated_input_sets": nsets,
            "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                         "kernel_ms_avg": round(kavg, 5), "kernel_ms_min": round(kmin, 5)}}


def sublayer_leg(args, dev, G, B=32, C=1152, Cc=64, H=74, W=74):
    """gspn_latent_sublayer at the pages' 1K shape (bf16), over rotated token sets."""
    import numpy as np
    import torch

    from spatial_line_scan_amd import gspn, inputs

    base = inputs.sublayer_problem_torch(B, C, Cc, G, H, W, 0, "bf16", dev)
    tok_bytes = B * H * W * C * 2
    nbytes = 2 * tok_bytes
    nsets = max(1, int(np.ceil(args.rotate_bytes / nbytes)))
    toks = [base["x_tok"]] + [base["x_tok"].clone() for _ in range(nsets - 1)]
    outs = [torch.empty_like(base["x_tok"]) for _ in range(nsets)]
    need = gspn.latent_sublayer_workspace_bytes(torch.bfloat16, B, C, Cc, G, H, W)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def fn(i):
        gspn.latent_sublayer(toks[i % nsets], base["p_down"], base["w_param"], base["p_up"], H, W,
                             G, 1, workspace=ws, out=outs[i % nsets])

    wall, kavg, kmin = _timed(fn, args.steps, args.warmup, torch.cuda.current_stream(dev))
    del toks, outs, ws
    torch.cuda.empty_cache()
    return {"groups": G, "B": B, "C": C, "Cc": Cc, "H": H, "W": W, "dtype": "bf16",
            "ms_per_step": round(wall * 1e3 / args.steps, 5), "event_ms_avg": round(kavg, 5),
            "event_ms_min": round(kmin, 5), "token_bytes_per_step": nbytes,
            "token_GBps": round(nbytes / (kavg * 1e-3) / 1e9, 2), "rotated_token_sets": nsets,
            "pages_sublayer_ms_A100": 0.18}


def backward_leg(wl, sets, args, dev):
    """Warmup + K backward launches over the rotated sets: wall time and
    HIP-event kernel times on the launch stream (_region, _single_min)."""
    import numpy as np
    import torch

    from spatial_line_scan_amd import gspn

    nsets = len(sets)
    need = gspn.prop2d_4dir_backward_workspace_bytes(wl.B, wl.C, wl.H, wl.W)
    ws = torch.empty(max(1, need // 4), dtype=torch.float32, device=dev) if need else None
    grads = []
    for s in sets:
        grads.append([torch.empty_like(s["x"]) for _ in range(3)] + [torch.empty_like(s["w"])])
    lib = gspn.lib()
    code = gspn.FP32 if wl.dtype == "fp32" else gspn.BF16
    stream = torch.cuda.current_stream(dev)
    sp = gspn.ctypes.c_void_p(stream.cuda_stream)
    wsp = gspn.ctypes.c_void_p(ws.data_ptr() if ws is not None else 0)
    wsb = ws.numel() * 4 if ws is not None else 0

    def bstep(i):
        s, g = sets[i % nsets], grads[i % nsets]
        st = lib.gspn_prop2d_4dir_backward(
            *(gspn.ctypes.c_void_p(t.data_ptr()) for t in (s["x"], s["lam"], s["u"], s["w"], s["gy"])),
            1e-6, *(gspn.ctypes.c_void_p(t.data_ptr()) for t in g), wsp, wsb, code,
            wl.B, wl.C, wl.H, wl.W, sp)
        if st != 0:
            raise RuntimeError(lib.gspn_status_str(st).decode())

    for i in range(args.warmup):
        bstep(i)
    torch.cuda.synchronize()
    wall, kavg = _region(bstep, args.steps, stream)
    kmin = _single_min(bstep, args.steps, stream)
    nbytes = BWD_VALUES_PER_PIXEL * wl.elem_bytes * wl.pixels
    achieved = nbytes / (kavg * 1e-3) / 1e9
    del grads, ws
    return {"ms_per_step": round(wall * 1e3 / args.steps, 5),
            "value": round(nbytes / (wall / args.steps) / 1e9, 2), "unit": "GB/s",
            "algorithmic_bytes_per_step": nbytes,
            "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                         "kernel_ms_avg": round(kavg, 5),
                         "kernel_ms_min": round(kmin, 5)}}


def shape_leg(args, dev, B, C, H, W, dtype, backward=False, rotate=True):
    """gspn_prop2d_4dir (and, with backward, gspn_prop2d_4dir_backward) on a
    B x C x H x W workload of the given storage type: inputs rotated over
    sets of at least --rotate-bytes (rotate) or one set reused (warm, cache
    resident when it fits); HIP-event kernel times and roofline per leg."""
    import numpy as np
    import torch

    from spatial_line_scan_amd import gspn, inputs
    from spatial_line_scan_amd.workloads import Workload

    wl = Workload("shape", B, C, H, W, dtype, (0,))
    base = inputs.problem_torch(B, C, H, W, 0, dtype, dev)
    if backward:
        base["gy"] = inputs.draw_torch(0, "gy", (B, C, H, W), dtype, dev)
    nsets = max(1, int(np.ceil(args.rotate_bytes / wl.algorithmic_bytes))) if rotate else 1
    sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(nsets - 1)]
    outs = [torch.empty_like(base["x"]) for _ in range(nsets)]
    # bf16 planes whose direction sum leaves LDS run only with a workspace
    # (gspn_prop2d_4dir_ex_ws, groups = C), allocated before the timed region
    need = gspn.prop2d_4dir_ex_workspace_bytes(base["x"].dtype, B, C, C, H, W)
    ws = torch.empty(need // 4, dtype=torch.float32, device=dev) if need else None
    torch.cuda.synchronize()

    def fn(i):
        st = sets[i % nsets]
        if ws is None:
            gspn.prop2d_4dir(st["x"], st["lam"], st["u"], st["w"], out=outs[i % nsets])
        else:
            gspn.prop2d_4dir_ex(st["x"], st["lam"], st["u"], st["w"], C, 1, out=outs[i % nsets], workspace=ws)

    wall, kavg, kmin = _timed(fn, args.steps, args.warmup, torch.cuda.current_stream(dev))
    nbytes = wl.algorithmic_bytes
    achieved = nbytes / (kavg * 1e-3) / 1e9
    out = {"B": B, "C": C, "H": H, "W": W, "dtype": dtype,
           "inputs": "rotated over %d sets" % nsets if rotate else "warm (one set)",
           "forward_workspace_bytes": need,
           "forward": {"ms_per_step": round(wall * 1e3 / args.steps, 5),
                       "value": round(nbytes / (wall / args.steps) / 1e9, 2), "unit": "GB/s",
                       "algorithmic_bytes_per_step": nbytes,
                       "roofline": {"bound": "hbm", "achieved": round(achieved, 2),
                                    "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                    "frac": round(achieved / HBM_PEAK_GBPS, 4),
                                    "kernel_ms_avg": round(kavg, 5), "kernel_ms_min": round(kmin, 5)}}}
    del outs, ws
    if backward:
        out["backward"] = backward_leg(wl, sets, args, dev)
    del sets
    torch.cuda.empty_cache()
    return out


def scan_dir_leg(wl, args, dev):
    """gspn_scan_dir on the workload's shape over rotated input sets.  One
    direction alone (y = u h) reads x, lambda, u and that direction's three
    tap planes and writes y: 7 values a pixel.  Timed for each direction with
    raw taps, for top-down with pre-normalised taps, and for the four
    directions as four calls into one output (top-down writes y, the other
    three add to it and so also read it: 31 values a pixel)."""
    import numpy as np
    import torch

    from spatial_line_scan_amd import gspn, inputs

    B, C, H, W = wl.B, wl.C, wl.H, wl.W
    base = inputs.problem_torch(B, C, H, W, 0, wl.dtype, dev)
    base["w"] = base["w"].view(4, B, C, 3, H * W)
    base["wn"] = (0.5 * torch.tanh(base["w"][0].float())).to(base["w"].dtype).contiguous()
    one = 7 * wl.elem_bytes * wl.pixels
    nsets = max(1, int(np.ceil(args.rotate_bytes / one)))
    sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(nsets - 1)]
    outs = [torch.empty_like(base["x"]) for _ in range(nsets)]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)

    def leg(fn, nbytes):
        wall, kavg, kmin = _timed(fn, args.steps, args.warmup, stream)
        achieved = nbytes / (kavg * 1e-3) / 1e9
        return {"ms_per_step": round(wall * 1e3 / args.steps, 5),
                "value": round(nbytes / (wall / args.steps) / 1e9, 2), "unit": "GB/s",
                "algorithmic_bytes_per_step": nbytes,
                "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                             "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                             "kernel_ms_avg": round(kavg, 5), "kernel_ms_min": round(kmin, 5)}}

    def one_dir(d, key="w"):
        def fn(i):
            st = sets[i % nsets]
            w = st[key] if key == "wn" else st["w"][d]
            gspn.scan_dir(st["x"], st["lam"], st["u"], w, d, w_is_raw=key == "w", out=outs[i % nsets])
        return fn

    def four(i):
        st = sets[i % nsets]
        for d in range(4):
            gspn.scan_dir(st["x"], st["lam"], st["u"], st["w"][d], d, out=outs[i % nsets],
                          accumulate=d > 0)

    res = {"B": B, "C": C, "H": H, "W": W, "dtype": wl.dtype, "rotated_input_sets": nsets}
    for d, name in enumerate(("top_down", "bottom_up", "left_right", "right_left")):
        res[name] = leg(one_dir(d), one)
    res["top_down_normalised_taps"] = leg(one_dir(0, "wn"), one)
    res["four_calls_accumulated"] = leg(four, 31 * wl.elem_bytes * wl.pixels)
    del sets, outs
    torch.cuda.empty_cache()
    return res


def pixel_ordered_leg(wl, args, dev):
    """The call a caller holding every direction's taps in pixel order
    ([4][B][C][3][H][W]) makes: transpose the LR and RL tap planes to the
    library's line-major layout (a torch copy into a preallocated tensor),
    then gspn_prop2d_4dir.  Times the transpose, the call and both."""
    import torch

    from spatial_line_scan_amd import gspn, inputs

    base = inputs.problem_torch(wl.B, wl.C, wl.H, wl.W, 0, wl.dtype, dev)
    w_pix = base["w"].reshape(4, wl.B, wl.C, 3, wl.H, wl.W).clone()
    w_lib = torch.empty_like(w_pix)
    w_lib[:2].copy_(w_pix[:2])
    y = torch.empty_like(base["x"])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)

    def transpose(i):
        w_lib[2:].copy_(w_pix[2:].transpose(-1, -2).reshape(2, wl.B, wl.C, 3, wl.H, wl.W))

    def call(i):
        gspn.prop2d_4dir(base["x"], base["lam"], base["u"], w_lib, out=y)

    def both(i):
        transpose(i)
        call(i)

    res = {}
    for name, fn in (("transpose", transpose), ("call", call), ("transpose_and_call", both)):
        wall, kavg, kmin = _timed(fn, args.steps, args.warmup, stream)
        res[name + "_ms"] = round(kavg, 5)
    res["transposed_bytes"] = 2 * 6 * wl.B * wl.C * wl.H * wl.W * wl.elem_bytes
    res["note"] = ("one input set, no rotation; the transpose moves 6 of the 12 tap planes "
                   "(read and write)")
    del w_pix, w_lib, base
    torch.cuda.empty_cache()
    return res


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="latent1k")
    ap.add_argument("--rotate-bytes", type=float, default=1.0e9,
                    help="total bytes of rotated input sets (defeats the 256 MB cache)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward leg")
    ap.add_argument("--no-variants", action="store_true", help="skip the grouped / chunked legs")
    ap.add_argument("--no-sublayer", action="store_true", help="skip the latent sublayer legs")
    ap.add_argument("--no-scan-dir", action="store_true", help="skip the one-direction legs")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the other workloads (latent2k, 147 x 147, base378, wide256) and the "
                         "pixel-ordered tap leg")
    ap.add_argument("--sublayer-only", type=int, default=None, metavar="G",
                    help="run only the latent sublayer leg with G tap groups and print it "
                         "(for profiling its kernels on their own)")
    ap.add_argument("--scan-dir-only", action="store_true",
                    help="run only the one-direction legs and print them")
    ap.add_argument("--shape-only", default=None, metavar="B,C,H,W,DTYPE",
                    help="run only the forward and backward legs on one B x C x H x W grid "
                         "(dtype fp32 or bf16) and print them (for profiling)")
    ap.add_argument("--backward-only", action="store_true",
                    help="run only warmup + K backward launches and print their timing "
                         "(for profiling the backward kernel on its own)")
    ap.add_argument("--copy-only", action="store_true",
                    help="run only the device copy used for calibration (--steps copies of "
                         "256 Mi fp32 = 1 GiB read + 1 GiB written), e.g. under rocprofv3 --pmc "
                         "to scale FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: the propagation shards over independent (b, c) "
              "planes with no exchange, so there is no multi-GPU code path; run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from spatial_line_scan_amd import gspn, inputs
    from spatial_line_scan_amd.workloads import WORKLOADS

    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_only:
        src = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_launches": args.steps, "bytes_read_per_launch": src.numel() * 4,
                          "bytes_written_per_launch": dst.numel() * 4}), flush=True)
        return
    if args.sublayer_only is not None:
        print(json.dumps({"sublayer": sublayer_leg(args, dev, args.sublayer_only)}), flush=True)
        return
    if args.shape_only:
        f = args.shape_only.split(",")
        B, C, H, W = (int(v) for v in f[:4])
        print(json.dumps({"shape": shape_leg(args, dev, B, C, H, W, f[4], backward=True)}), flush=True)
        return
    if args.scan_dir_only:
        print(json.dumps({"scan_dir": scan_dir_leg(wl, args, dev)}), flush=True)
        return
    print("bench: drawing %s inputs" % wl.name, file=sys.stderr, flush=True)
    base = inputs.problem_torch(wl.B, wl.C, wl.H, wl.W, 0, wl.dtype, dev)
    if not args.no_backward:
        base["gy"] = inputs.draw_torch(0, "gy", (wl.B, wl.C, wl.H, wl.W), wl.dtype, dev)
    nsets = max(1, int(np.ceil(args.rotate_bytes / wl.algorithmic_bytes)))
    sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(nsets - 1)]
    if args.backward_only:
        print(json.dumps({"backward": backward_leg(wl, sets, args, dev)}), flush=True)
        return
    outs = [torch.empty_like(base["x"]) for _ in range(nsets)]
    torch.cuda.synchronize()

    def step(i):
        s = sets[i % nsets]
        gspn.prop2d_4dir(s["x"], s["lam"], s["u"], s["w"], out=outs[i % nsets])

    print("bench: warmup %d" % args.warmup, file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # exactly K steps: their wall time, and their kernel time per launch from
    # HIP events on the launch stream at the two ends of the same region (a
    # step is one launch of the four-direction kernel)
    stream = torch.cuda.current_stream(dev)
    wall, kern_avg = _region(step, args.steps, stream)
    # single launches, an event pair around each: the fastest and the median
    # of 100 (or K if more)
    kern_min, kern_median = _single_calls(step, max(100, args.steps), stream)

    # calibration: a plain device copy of ~1 GB through the same HBM
    cal = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    cal2 = torch.empty_like(cal)
    cal2.copy_(cal)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(10):
        cal2.copy_(cal)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * cal.numel() * 4 * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del cal, cal2

    nbytes = wl.algorithmic_bytes
    ms_per_step = wall * 1e3 / args.steps
    value = nbytes / (wall / args.steps) / 1e9
    achieved = nbytes / (kern_avg * 1e-3) / 1e9
    traffic = measured_traffic(wl.name)
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "C": wl.C, "H": wl.H, "W": wl.W,
                   "storage": wl.dtype, "arithmetic": "fp32", "rotated_input_sets": nsets,
                   "algorithmic_bytes_per_step": nbytes},
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "traffic_source": ("profiles/prop2d_latent1k_traffic.json: rocprofv3 FETCH_SIZE and "
                                        "WRITE_SIZE taken on this kernel source (source hash matched), "
                                        "scaled by a 1 GiB copy's reading; not counted in this run"
                                        if traffic is not None else None),
                     "kernel_ms_avg": round(kern_avg, 5),
                     "kernel_ms_min": round(kern_min, 5),
                     "kernel_ms_median_single": round(kern_median, 5)},
        "calibration": {"torch_copy_GBps": round(copy_gbps, 1),
                        "frac_of_copy": round(achieved / copy_gbps, 4)},
    }
    if not args.no_variants:
        print("bench: variants", file=sys.stderr, flush=True)
        out["variants"] = [variant_leg(wl, args, dev, G, k) for G, k in ((1, 1), (wl.C, 4))]
    if not args.no_sublayer and wl.name == "latent1k":
        print("bench: sublayer", file=sys.stderr, flush=True)
        out["sublayer"] = [sublayer_leg(args, dev, G) for G in (64, 1)]
    if not args.no_backward:
        print("bench: backward", file=sys.stderr, flush=True)
        out["backward"] = backward_leg(wl, sets, args, dev)
        if not args.no_variants:
            print("bench: grouped / chunked backward", file=sys.stderr, flush=True)
            out["backward_variants"] = [ex_backward_leg(wl, args, dev, G, k) for G, k in ((1, 4), (wl.C, 4))]
    if not args.no_scan_dir:
        print("bench: one-direction scans", file=sys.stderr, flush=True)
        out["scan_dir"] = scan_dir_leg(wl, args, dev)
    if not args.no_workloads and wl.name == "latent1k":
        print("bench: pixel-ordered taps", file=sys.stderr, flush=True)
        out["pixel_ordered_taps"] = pixel_ordered_leg(wl, args, dev)
        print("bench: other workloads", file=sys.stderr, flush=True)
        l2, b3, wd = WORKLOADS["latent2k"], WORKLOADS["base378"], WORKLOADS["wide256"]
        out["workloads"] = {
            "latent2k": shape_leg(args, dev, l2.B, l2.C, l2.H, l2.W, l2.dtype, backward=True),
            "latent2k_odd_147": shape_leg(args, dev, l2.B, l2.C, 147, 147, l2.dtype, backward=True),
            "base378_warm": shape_leg(args, dev, b3.B, b3.C, b3.H, b3.W, b3.dtype, rotate=False),
            "base378_rotated": shape_leg(args, dev, b3.B, b3.C, b3.H, b3.W, b3.dtype, backward=True),
            "wide256": shape_leg(args, dev, wd.B, wd.C, wd.H, wd.W, wd.dtype, backward=True),
        }
    if not args.no_cpu_baseline:
        print("bench: cpu baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget, sets[0], outs[0])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
