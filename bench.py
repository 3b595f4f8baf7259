#!/usr/bin/env python3
"""Throughput of the MI355X Fourier-slice projector on the D=128 cubic workload.

One step = the whole hot path over one batch: the cubic forward projection of
16384 poses from a 128^3 rfft blob volume (radius cutoff 64, shifts
U(-5,5) px), then the full backward (volume, rotation and shift gradients)
for a random complex upstream gradient.  Inputs are resident in HBM before the
timed region; outputs are preallocated.  W warmup steps, then K timed steps
between device synchronisations (HIP events on the library's stream).

Prints ONE JSON line on stdout.  Per-kernel timings, the roofline terms and
the other workloads go to stderr (and to --details FILE).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "projections/sec fwd+bwd (cubic, D=128) on 1 MI355X; % of HBM/L2 roofline"
UNIT = "projections/s"

# MI355X public figures; the L2 figure is derived from them (8 XCDs x 16
# channels x 128 B/clk x 2.4 GHz), as is the fp32 vector rate.
HBM_PEAK_GBS = 8000.0
L2_PEAK_GBS = 8 * 16 * 128 * 2.4          # = 39321.6 GB/s
FP32_VECTOR_TFLOPS = 157.3


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


def in_mask_pixels(H, r):
    import numpy as np
    kx = np.arange(H // 2 + 1)
    ky = np.fft.fftfreq(H, 1.0 / H)
    m = (r < 0) | (kx[None, :] ** 2 + ky[:, None] ** 2 <= r * r)
    return int(m.sum())


def kernel_model(w, op):
    """Algorithmic bytes of one launch of `op` on workload `w` (per pose x poses).
    tap bytes: in-mask pixels x taps x 8 B (complex tap read or accumulate);
    hbm bytes: compulsory reads/writes of images, volumes and pose params."""
    T = 64 if w.interp == 1 else 8
    npose = w.B * w.P
    n_in = in_mask_pixels(w.H, w.radius)
    img = npose * w.H * (w.H // 2 + 1) * 8
    vol = w.vol.size * 8 if w.vol is not None else w.D * w.D * (w.D // 2 + 1) * 8
    params = npose * (9 + 2) * 4
    tap = npose * n_in * T * 8
    if op == "forward":
        hbm = img + vol + params
    elif op == "backward_vol":
        hbm = img + vol + params
    elif op == "backward_rot":
        hbm = img + vol + params + npose * 11 * 4
    else:
        raise ValueError(op)
    return {"tap_bytes": tap, "hbm_bytes": hbm, "n_in": n_in, "poses": npose, "taps": T}


def time_calls(fn, n, torch):
    """Average ms of fn() over n calls, with HIP events on the current stream."""
    st = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    evs[0].record(st)
    for i in range(n):
        fn()
        evs[i + 1].record(st)
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(n)]
    return sum(per) / n, per


def cpu_baseline(w, sample, eprint):
    """The oracle, untouched, on the first `sample` poses of the workload."""
    import oracle
    P = min(sample, w.P)
    t0 = time.perf_counter()
    oracle.project(w.vol, w.rot[:, :P], w.shifts[:, :P], interp=w.interp, r=w.radius)
    oracle.project_backward(w.grad_out[:, :P], w.vol, w.rot[:, :P], w.shifts[:, :P], interp=w.interp, r=w.radius)
    dt = time.perf_counter() - t0
    res = {"value": round(P * w.B / dt, 2), "unit": UNIT, "cores": oracle.num_threads(), "kind": "oracle",
           "sample": f"first {P} of {w.P} poses of the D=128 cubic workload, forward + full backward, "
                     f"fp64 C oracle with OpenMP ({dt:.1f} s)"}
    eprint(f"[bench] cpu baseline: {res}")
    return res


def run_workload_ops(cfg, steps, warmup, bp, workloads, torch, details):
    """Per-operation timing of one workload (stderr/details only)."""
    w = workloads.make(cfg)
    dev = torch.device("cuda:0")
    res = {"workload": w.name}
    npose = w.B * (w.P if w.rot is not None else 0)
    if cfg == 4:
        ti = torch.from_numpy(w.images).to(dev)
        tw = torch.from_numpy(w.weights).to(dev)
        tr = torch.from_numpy(w.rot).to(dev)
        dv = torch.empty((1, w.D, w.D, w.D // 2 + 1), dtype=torch.complex64, device=dev)
        wv = torch.empty((1, w.D, w.D, w.D // 2 + 1), dtype=torch.float32, device=dev)
        fn = lambda: bp.backproject_2d_to_3d(ti, tr, tw, None, D=w.D, data_vol=dv, weight_vol=wv)  # noqa: E731
        for _ in range(warmup):
            fn()
        ms, _ = time_calls(fn, steps, torch)
        res["backproject_ms"] = ms
        res["backproject_proj_per_s"] = w.P / (ms * 1e-3)
        n_in = in_mask_pixels(w.H, w.radius)
        res["tap_bytes"] = w.P * n_in * 64 * 12
        res["l2_frac"] = res["tap_bytes"] / (ms * 1e-3) / (L2_PEAK_GBS * 1e9)
    else:
        tv = torch.from_numpy(w.vol).to(dev)
        tr = torch.from_numpy(w.rot).to(dev)
        ts = torch.from_numpy(w.shifts).to(dev) if w.shifts is not None else None
        out = torch.empty((w.B, w.P, w.H, w.H // 2 + 1), dtype=torch.complex64, device=dev)
        interp = "cubic" if w.interp == 1 else "linear"
        f = lambda: bp.project_3d_to_2d(tv, tr, ts, out=out, interp=interp, radius_cutoff=w.radius)  # noqa: E731
        for _ in range(warmup):
            f()
        ms, _ = time_calls(f, steps, torch)
        m = kernel_model(w, "forward")
        res["forward_ms"] = ms
        res["forward_proj_per_s"] = npose / (ms * 1e-3)
        res["forward_l2_frac"] = m["tap_bytes"] / (ms * 1e-3) / (L2_PEAK_GBS * 1e9)
        if w.grad_out is not None:
            tg = torch.from_numpy(w.grad_out).to(dev)
            need_s = "backward_shifts" in w.ops
            gv = torch.empty_like(tv)
            gr = torch.empty_like(tr)
            gs = torch.empty_like(ts) if (need_s and ts is not None) else None
            b = lambda: bp.project_3d_to_2d_backward(tg, tv, tr, ts, interp=interp, radius_cutoff=w.radius,  # noqa
                                                     need_shifts=need_s, grad_vol=gv, grad_rot=gr, grad_shifts=gs)
            for _ in range(warmup):
                b()
            ms_b, _ = time_calls(b, steps, torch)
            res["backward_ms"] = ms_b
            res["fwd_bwd_proj_per_s"] = npose / ((ms + ms_b) * 1e-3)
    eprint(f"[bench] workload {cfg}: {json.dumps(res)}")
    details.setdefault("workloads", {})[str(cfg)] = res


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-sample", type=int, default=8192, help="poses of the oracle CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--all-workloads", action="store_true", help="also time the other four workloads (stderr)")
    ap.add_argument("--details", default=None, help="write per-kernel details as JSON to this file")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        eprint("bench.py measures the single-GPU hot path only; this build runs on one GPU "
               f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).  Multi-GPU sharding is "
               "described, not built.")
        sys.exit(2)

    import torch
    import back_projection_amd as bp
    from back_projection_amd import workloads

    if not torch.cuda.is_available():
        eprint("bench.py needs a GPU")
        sys.exit(1)
    bp.lib()   # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    w = workloads.make(3)
    eprint(f"[bench] workload generated in {time.perf_counter() - t0:.1f} s: {w.name}")
    tv = torch.from_numpy(w.vol).to(dev)
    tr = torch.from_numpy(w.rot).to(dev)
    ts = torch.from_numpy(w.shifts).to(dev)
    tg = torch.from_numpy(w.grad_out).to(dev)
    out = torch.empty((w.B, w.P, w.H, w.H // 2 + 1), dtype=torch.complex64, device=dev)
    gv, gr, gs = torch.empty_like(tv), torch.empty_like(tr), torch.empty_like(ts)
    r = w.radius
    npose = w.B * w.P

    def fwd():
        bp.project_3d_to_2d(tv, tr, ts, out=out, interp="cubic", radius_cutoff=r)

    def bwd():
        bp.project_3d_to_2d_backward(tg, tv, tr, ts, interp="cubic", radius_cutoff=r, grad_vol=gv, grad_rot=gr,
                                     grad_shifts=gs)

    def step():
        fwd()
        bwd()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    e0.record(st)
    for _ in range(args.steps):
        step()
    e1.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = e0.elapsed_time(e1)
    ms_per_step = total_ms / args.steps
    value = npose / (ms_per_step * 1e-3)
    eprint(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step (event), wall {wall / args.steps * 1e3:.3f} "
           f"ms/step -> {value:.1f} proj/s")

    # per-kernel breakdown, each call timed live with events on the same stream
    n = max(3, args.steps)
    parts = {
        "forward": fwd,
        "backward_vol": lambda: bp.project_3d_to_2d_backward(tg, tv, tr, ts, interp="cubic", radius_cutoff=r,
                                                             need_rot=False, need_shifts=False, grad_vol=gv),
        "backward_rot": lambda: bp.project_3d_to_2d_backward(tg, tv, tr, ts, interp="cubic", radius_cutoff=r,
                                                             need_vol=False, grad_rot=gr, grad_shifts=gs),
    }
    kernels = {}
    for name, fn in parts.items():
        ms, _ = time_calls(fn, n, torch)
        m = kernel_model(w, name)
        kernels[name] = {
            "ms": round(ms, 4),
            "tap_GBps": round(m["tap_bytes"] / (ms * 1e-3) / 1e9, 1),
            "hbm_GBps": round(m["hbm_bytes"] / (ms * 1e-3) / 1e9, 1),
            "l2_frac": round(m["tap_bytes"] / (ms * 1e-3) / 1e9 / L2_PEAK_GBS, 4),
            "hbm_frac": round(m["hbm_bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            **m,
        }
        eprint(f"[bench] {name}: {kernels[name]}")
    dom = max(kernels, key=lambda k: kernels[k]["ms"])
    kd = kernels[dom]
    achieved = kd["tap_bytes"] / (kd["ms"] * 1e-3) / 1e9
    roofline = {
        "bound": "l2",
        "achieved": round(achieved, 1),
        "peak": round(L2_PEAK_GBS, 1),
        "unit": "GB/s",
        "frac": round(achieved / L2_PEAK_GBS, 4),
        "traffic": None,
        "kernel": dom,
        "hbm": {"achieved": round(kd["hbm_bytes"] / (kd["ms"] * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": kd["hbm_frac"]},
    }

    details = {"kernels": kernels, "ms_per_step": ms_per_step}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_sample, eprint)
    if args.all_workloads:
        del tg, out
        torch.cuda.empty_cache()
        for cfg in (1, 2, 4, 5):
            run_workload_ops(cfg, max(3, args.steps // 2), 1, bp, workloads, torch, details)
    if args.details:
        with open(args.details, "w") as f:
            json.dump(details, f, indent=1)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": UNIT,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "D128 cubic forward + full backward (volume, rotation, shift grads)",
                   "D": w.D, "H": w.H, "poses": npose, "interp": "cubic", "radius_cutoff": r,
                   "shifts": "U(-5,5) px", "volume": "800 Gaussian blobs, rfft complex64 128x128x65"},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
