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
import ctypes
import hashlib
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
LDS_PEAK_GBS = 256 * 128 * 2.4            # 256 CUs x 128 B/clk x 2.4 GHz = 78643.2 GB/s
# fp32 vector: 256 CUs x 4 SIMDs x 32 lanes per clock x 2 flop x 2.4 GHz.  The
# kernels are built without packed FP32 instructions; the FMA probe of
# `--peaks` (non-packed v_fma_f32 only) issues 1.72 wave64 FMAs per CU clock,
# 135.6 TFLOP/s, so the published figure is the ceiling of non-packed FMAs too.
FP32_VECTOR_TFLOPS = 157.3
FP32_FMA_PROBE_TFLOPS = 135.6             # measured, bench.py --peaks

# Algorithmic fp32 flops per in-mask pixel of the separable tricubic
# interpolation each kernel class performs (2 flops per multiply-add; the
# contraction only, not the weights, coordinates or enumeration):
#   forward   value: 64 taps x 2 (complex x weight) + 16 x 2 + 4 x 2 = 168 FMA
#   gradient  value and three derivatives: 64 x 4 + 16 x 6 + 4 x 8 = 384 FMA
#   backward  scatter: 64 taps x 2 (weight x complex, the fixed-point
#             rounding multiply-add) + 16 column weights + 8 row factors = 152
FLOPS_PER_PIXEL_CUBIC = {"forward": 2 * 168, "gradient": 2 * 384, "backward": 2 * 152, "fold": 0}
# the same for the real weight channel (one multiply-add where the complex
# channel has two): forward 64 + 16 + 4, gradient 64 x 2 + 16 x 3 + 4 x 4,
# scatter 64 + 16 + 8
FLOPS_PER_PIXEL_CUBIC_REAL = {"forward": 2 * 84, "gradient": 2 * 192, "backward": 2 * 88}


def op_rates(ms, poses, n_in, tap_bytes_per_pixel, flops_per_pixel):
    """ms, proj/s, tap-delivery rate and fraction of the L2 figure, and (when
    a flop model is given) TFLOP/s and fraction of the fp32 vector peak."""
    sec = ms * 1e-3
    r = {"ms": round(ms, 4), "proj_per_s": round(poses / sec, 1),
         "tap_GBps": round(poses * n_in * tap_bytes_per_pixel / sec / 1e9, 1),
         "l2_frac": round(poses * n_in * tap_bytes_per_pixel / sec / 1e9 / L2_PEAK_GBS, 4)}
    if flops_per_pixel:
        r["tflops"] = round(poses * n_in * flops_per_pixel / sec / 1e12, 2)
        r["alu_frac"] = round(r["tflops"] / FP32_VECTOR_TFLOPS, 4)
    return r


# HBM traffic per launch of a kernel class, from two rocprofv3 PMC runs of this
# script (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by what the
# same counter reads for a plain device copy of known size (--copy-calibration).
# A figure is valid only for the kernel sources it was taken on: it is
# reported when the digest of the 3D kernel sources matches, else null.
TRAFFIC = {
    # profiles/brick_kernels_D128_cubic_step_hbm_traffic.txt
    "forward": {"sources_sha256": "20cee6cd58dcf625671338898f6e16074eacfe26b088f23712dc2566fbc66e4a",
               "fetch_bytes": 313479764, "write_bytes": 1183410253},
    "backward": {"sources_sha256": "20cee6cd58dcf625671338898f6e16074eacfe26b088f23712dc2566fbc66e4a",
                "fetch_bytes": 3003110149, "write_bytes": 301123570},
    "gradient": {"sources_sha256": "20cee6cd58dcf625671338898f6e16074eacfe26b088f23712dc2566fbc66e4a",
                "fetch_bytes": 2783879413, "write_bytes": 120424608},
    "fold": {"sources_sha256": "20cee6cd58dcf625671338898f6e16074eacfe26b088f23712dc2566fbc66e4a",
            "fetch_bytes": 223195580, "write_bytes": 33390592},
}

# VALU issue per kernel class, from the SQ counter pass of the same sessions
# (SQ_INSTS_VALU / SQ_BUSY_CU_CYCLES: wave64 VALU instructions per CU clock),
# valid for the same kernel sources digest as the traffic figures.  A CU
# issues at most 2 per clock (4 SIMDs, a wave64 fp32 instruction every two
# clocks); the FMA probe of --peaks reaches 1.72.
VALU_ISSUE = {
    # profiles/brick_kernels_D128_cubic_counters.txt
    "forward": {"sources_sha256": "20cee6cd58dcf625671338898f6e16074eacfe26b088f23712dc2566fbc66e4a",
                "valu_per_cu_clock": 1.056},
    "backward": {"sources_sha256": "20cee6cd58dcf625671338898f6e16074eacfe26b088f23712dc2566fbc66e4a",
                 "valu_per_cu_clock": 0.799},
    "gradient": {"sources_sha256": "20cee6cd58dcf625671338898f6e16074eacfe26b088f23712dc2566fbc66e4a",
                 "valu_per_cu_clock": 1.339},
}
VALU_ISSUE_PEAK = 2.0
VALU_ISSUE_PROBE = 1.72


def valu_issue(kclass):
    """The kernel class's counter-measured VALU issue rate against the CU's
    issue limit, or None once the kernel sources have changed."""
    t = VALU_ISSUE.get(kclass)
    if not t or t["sources_sha256"] != sources_digest():
        return None
    a = t["valu_per_cu_clock"]
    return {"achieved": a, "peak": VALU_ISSUE_PEAK, "probe": VALU_ISSUE_PROBE,
            "unit": "wave64 VALU instructions per CU clock", "frac": round(a / VALU_ISSUE_PEAK, 4),
            "scope": "kernel alone (the counter passes run one kernel at a time)"}


def sources_digest():
    """Digest of the sources the 3D kernels are built and launched from (the
    2D-only kernel files are left out: the 3D kernels do not include them)."""
    d = hashlib.sha256()
    csrc = os.path.join(ROOT, "back_projection_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h", ".cpp")) and "_2d" not in name:
            d.update(name.encode())
            with open(os.path.join(csrc, name), "rb") as f:
                d.update(f.read())
    return d.hexdigest()


def measured_traffic(kclass):
    t = TRAFFIC.get(kclass)
    if not t or t["sources_sha256"] != sources_digest():
        return None
    return t["fetch_bytes"] + t["write_bytes"]


def copy_calibration(torch, gib=1):
    """A plain device-to-device copy of `gib` GiB, three times (for the PMC scale factor)."""
    n = gib << 28   # float32 elements
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    eprint(f"[bench] copied {gib} GiB three times ({n * 4} bytes read and written per copy)")


def measure_peaks(torch):
    """The bandwidths the rooflines rest on, measured on this GPU with
    libtproj_probes.so (include/tproj_probes.h): HBM stream read, 8-byte
    gathers from a cache-resident buffer, LDS 4x4x4 tap reads / 64-bit
    atomics under four bank-key regimes, the FP32 FMA issue rate, and the
    scatter's tap mix (FMAs forming 64-bit words) with and without its LDS
    atomics.  Printed to stderr as one JSON
    object; nothing here runs in the default benchmark."""
    from back_projection_amd import build_lib
    P = ctypes.CDLL(build_lib.PROBES_LIB)
    vp = ctypes.c_void_p
    P.tpp_stream_read.argtypes = [vp, ctypes.c_size_t, vp, ctypes.c_int, vp]
    P.tpp_l2_gather.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, ctypes.c_int, vp]
    P.tpp_lds_taps.argtypes = [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    blocks = 8192
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def timed(call, reps=5):
        rc = call()
        if rc != 0:
            raise RuntimeError(f"probe launch failed ({rc})")
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            call()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e-3   # seconds per call

    out = {"clock_GHz_assumed": 2.4, "cus": 256}
    big = torch.empty(1 << 32, dtype=torch.uint8, device="cuda:0")     # 4 GiB
    big.fill_(1)
    t = timed(lambda: P.tpp_stream_read(vp(big.data_ptr()), big.numel(), vp(sink.data_ptr()), blocks, st))
    out["hbm_stream_read_GBps"] = round(big.numel() / t / 1e9, 1)
    del big
    for log2, name in ((18, "gather_2MiB_GBps"), (21, "gather_16MiB_GBps"), (24, "gather_128MiB_GBps")):
        buf = torch.zeros(2 << log2, dtype=torch.float32, device="cuda:0")
        iters = 64
        t = timed(lambda: P.tpp_l2_gather(vp(buf.data_ptr()), log2, vp(sink.data_ptr()), iters, blocks, st))
        out[name] = round(blocks * 256 * iters * 128 / t / 1e9, 1)
    clk = 256 * 2.4e9
    for atomic in (0, 1):
        for mode, name in ((0, "random"), (1, "rank_permuted"), (2, "conflict_free"), (3, "bank_split_rotated")):
            iters = 64
            t = timed(lambda: P.tpp_lds_taps(vp(sink.data_ptr()), mode, atomic, iters, blocks, st))
            key = ("lds_atomic_" if atomic else "lds_read_") + name + "_taps_per_clk_cu"
            out[key] = round(blocks * 256 * iters * 64 / t / clk, 2)
    P.tpp_lds_width.argtypes = [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    for width, atomic in ((4, 0), (8, 0), (16, 0), (4, 1), (8, 1)):
        iters = 64
        t = timed(lambda: P.tpp_lds_width(vp(sink.data_ptr()), width, atomic, iters, blocks, st))
        if atomic:
            out[f"lds_atomic_u{8 * width}_lanes_per_clk_cu"] = round(blocks * 256 * iters * 16 / t / clk, 2)
        else:
            out[f"lds_read_b{8 * width}_bytes_per_clk_cu"] = round(blocks * 256 * iters * 16 * width / t / clk, 1)
    P.tpp_valu.argtypes = [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    iters = 256
    t = timed(lambda: P.tpp_valu(vp(sink.data_ptr()), 0, iters, blocks, st))
    out["fp32_fma_TFLOPs"] = round(blocks * 256 * iters * 128 / t / 1e12, 2)
    out["fp32_fma_wave_insts_per_clk_cu"] = round(blocks * 4 * iters * 64 / t / clk, 3)
    # non-FP32 VALU issue: wave64 instructions per CU clock for one kind at a
    # time (the select kinds take two instructions per operation)
    iters = 256
    for mode, name, insts in ((7, "int_add", 1), (8, "bitwise_select", 2), (9, "cmp_cndmask", 2),
                              (10, "add_u64", 1)):
        t = timed(lambda: P.tpp_valu(vp(sink.data_ptr()), mode, iters, blocks, st))
        out[f"{name}_wave_insts_per_clk_cu"] = round(blocks * 4 * iters * 64 * insts / t / clk, 3)
    # the scatter's mix: taps per clock per CU with and without the atomics
    iters = 32
    for mode, extra, atomic in ((1, 0, True), (2, 0, False), (3, 2, True), (4, 2, False), (5, 6, True),
                                (6, 6, False)):
        t = timed(lambda: P.tpp_valu(vp(sink.data_ptr()), mode, iters, blocks, st))
        key = f"tap_mix_fma{2 + extra}_" + ("atomic" if atomic else "no_lds") + "_taps_per_clk_cu"
        out[key] = round(blocks * 256 * iters * 64 / t / clk, 2)
    eprint("[bench] peaks " + json.dumps(out))
    return out


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


def in_mask_pixels(H, r):
    import numpy as np
    kx = np.arange(H // 2 + 1)
    ky = np.fft.fftfreq(H, 1.0 / H)
    m = (r < 0) | (kx[None, :] ** 2 + ky[:, None] ** 2 <= r * r)
    return int(m.sum())


def kernel_model(w, kclass, ws_bytes=0):
    """Algorithmic bytes of one launch of a brick-kernel class on workload `w`.
    tap bytes: in-mask pixels x taps x 8 B per complex tap read (gather) or
    accumulated (scatter: the backward class).  hbm bytes: what the
    launch must read or write in HBM at least (images, volume, pose params;
    for the fold, the partial tiles and the volume)."""
    T = 64 if w.interp == 1 else 8
    npose = w.B * w.P
    n_in = in_mask_pixels(w.H, w.radius)
    img = npose * w.H * (w.H // 2 + 1) * 8
    vol = w.D * w.D * (w.D // 2 + 1) * 8
    params = npose * (9 + 2) * 4
    per_px = {"forward": T * 8, "backward": T * 8, "gradient": T * 8, "fold": 0}[kclass]
    hbm = {"forward": img + vol + params,
           "backward": img + vol + params,
           "gradient": img + vol + params + npose * 11 * 4,
           "fold": ws_bytes + vol}[kclass]
    flops_px = FLOPS_PER_PIXEL_CUBIC[kclass] if w.interp == 1 else 0
    return {"tap_bytes": npose * n_in * per_px, "tap_bytes_per_pixel": per_px, "hbm_bytes": hbm, "n_in": n_in,
            "poses": npose, "taps": T, "flops": npose * n_in * flops_px, "flops_per_pixel": flops_px}


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


def cpu_baseline(w, sample, eprint, sample_1core=512):
    """The oracle, untouched, on the first `sample` poses of the workload with
    all the OpenMP threads it gets, then on the first `sample_1core` poses with
    one thread."""
    import oracle
    P = min(sample, w.P)
    threads = oracle.num_threads()
    t0 = time.perf_counter()
    oracle.project(w.vol, w.rot[:, :P], w.shifts[:, :P], interp=w.interp, r=w.radius)
    oracle.project_backward(w.grad_out[:, :P], w.vol, w.rot[:, :P], w.shifts[:, :P], interp=w.interp, r=w.radius)
    dt = time.perf_counter() - t0
    P1 = min(sample_1core, w.P)
    oracle.set_num_threads(1)
    try:
        t1 = time.perf_counter()
        oracle.project(w.vol, w.rot[:, :P1], w.shifts[:, :P1], interp=w.interp, r=w.radius)
        oracle.project_backward(w.grad_out[:, :P1], w.vol, w.rot[:, :P1], w.shifts[:, :P1], interp=w.interp,
                                r=w.radius)
        dt1 = time.perf_counter() - t1
    finally:
        oracle.set_num_threads(threads)
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = os.cpu_count()
    res = {"value": round(P * w.B / dt, 2), "unit": UNIT, "cores": threads, "kind": "oracle",
           "sample": f"first {P} of {w.P} poses of the D=128 cubic workload, forward + full backward, "
                     f"fp64 C oracle with OpenMP over {threads} threads ({dt:.1f} s)",
           "single_core": {"value": round(P1 * w.B / dt1, 2), "unit": UNIT, "cores": 1,
                           "sample": f"first {P1} poses, one thread ({dt1:.1f} s)"},
           "nproc": affinity, "cpu_count": os.cpu_count(),
           "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}
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
        n_in = in_mask_pixels(w.H, w.radius)
        F, FR = FLOPS_PER_PIXEL_CUBIC, FLOPS_PER_PIXEL_CUBIC_REAL
        # taps: 8 B complex + 4 B real accumulated per tap
        res["backproject"] = op_rates(ms, w.P, n_in, 64 * 12, F["backward"] + FR["backward"])
        # its backward (grad images, grad weights, grad rotations) for random
        # upstream volume gradients
        import numpy as np
        rng = np.random.default_rng(4004)
        gdv = torch.from_numpy(workloads.random_complex(rng, tuple(dv.shape))).to(dev)
        gwv = torch.from_numpy(rng.standard_normal(tuple(wv.shape)).astype(np.float32)).to(dev)
        fb = lambda: bp.backproject_2d_to_3d_backward(gdv, ti, tr, gwv, tw, None)  # noqa: E731
        for _ in range(warmup):
            fb()
        ms_b, _ = time_calls(fb, steps, torch)
        # gathers: grad images (8 B taps) and grad weights (4 B), then the
        # rotation gradient over both channels (12 B)
        res["backproject_backward"] = op_rates(ms_b, w.P, n_in, 64 * 24,
                                               F["forward"] + FR["forward"] + F["gradient"] + FR["gradient"])
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
        n_in = in_mask_pixels(w.H, w.radius)
        T = 64 if w.interp == 1 else 8
        F = FLOPS_PER_PIXEL_CUBIC if w.interp == 1 else {}
        res["forward"] = op_rates(ms, npose, n_in, T * 8, F.get("forward"))
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
            # scatter (taps accumulated) and gradient (taps gathered)
            fb = (F["backward"] + F["gradient"]) if F else None
            res["backward"] = op_rates(ms_b, npose, n_in, 2 * T * 8, fb)
            res["forward_backward"] = op_rates(ms + ms_b, npose, n_in, 3 * T * 8, (F["forward"] + fb) if F else None)
    eprint(f"[bench] workload {cfg}: {json.dumps(res)}")
    details.setdefault("workloads", {})[str(cfg)] = res


def run_2d(steps, warmup, bp, workloads, torch, details):
    """The 2D -> 2D ops on the 2D analogue of the D=128 cubic workload
    (stderr/details only): forward, its full backward (source, rotation and
    shift grads), the accumulation with weights and its backward."""
    w = workloads.make_2d()
    dev = torch.device("cuda:0")
    ts, tr, tsh, tg, tw = (torch.from_numpy(w[k]).to(dev) for k in ("src", "rot", "shifts", "grad_out", "weights"))
    r, D, P = w["radius"], w["D"], w["P"]
    n_in = in_mask_pixels(w["H"], r)
    out = torch.empty((1, P, D, D // 2 + 1), dtype=torch.complex64, device=dev)
    calls = {
        "forward": lambda: bp.project_2d_to_2d(ts, tr, tsh, out=out, radius_cutoff=r),
        "backward": lambda: bp.project_2d_to_2d_backward(tg, ts, tr, tsh, radius_cutoff=r),
        "accumulate_weights": lambda: bp.backproject_2d_to_2d(tg, tr, tw, tsh, D=D, radius_cutoff=r),
    }
    # backward of the accumulation: upstream gradients of the data (the source
    # serves) and of the weight reconstruction (uniform random)
    gw = torch.rand((1, D, D // 2 + 1), dtype=torch.float32, device=dev)
    calls["accumulate_backward"] = lambda: bp.backproject_2d_to_2d_backward(ts, tg, tr, gw, tw, tsh, radius_cutoff=r)
    # tap bytes per in-mask pixel: 16 taps x 8 B (complex), x 12 B with the
    # real weight channel; the gradient passes gather value and derivatives
    # from the same taps
    taps = {"forward": 128, "backward": 256, "accumulate_weights": 192, "accumulate_backward": 2 * 192}
    res = {"workload": w["name"]}
    for name, fn in calls.items():
        for _ in range(warmup):
            fn()
        ms, _ = time_calls(fn, steps, torch)
        tb = P * n_in * taps[name]
        res[name] = {"ms": round(ms, 4), "proj_per_s": round(P / (ms * 1e-3), 1),
                     "tap_GBps": round(tb / (ms * 1e-3) / 1e9, 1),
                     "l2_frac": round(tb / (ms * 1e-3) / 1e9 / L2_PEAK_GBS, 4)}
    res["fwd_bwd_proj_per_s"] = round(P / ((res["forward"]["ms"] + res["backward"]["ms"]) * 1e-3), 1)
    eprint(f"[bench] 2d: {json.dumps(res)}")
    details["2d"] = res


def run_sweep(steps, warmup, bp, workloads, torch, details):
    """The 3D ops on the pages' axes (box size, poses per call, linear vs cubic):
    forward alone and forward + full backward (volume, rotation, shift grads),
    radius D/2, shifts U(-5,5) (stderr/details only)."""
    import numpy as np
    dev = torch.device("cuda:0")
    rows = []
    eprint("[bench] sweep:  D  interp     poses   fwd ms  fwd+bwd ms   fwd proj/s  fwd+bwd proj/s  fwd L2 frac")
    for D in (32, 64, 128, 256):
        rng = np.random.default_rng(3000 + D)
        vol = workloads.rfft_volume(workloads.blob_volume_real(D, *workloads.blob_params(rng, 200, D / 3)))
        tv = torch.from_numpy(vol[None]).to(dev)
        n_in = in_mask_pixels(D, D / 2)
        for P in (1024, 16384):
            tr = torch.from_numpy(workloads.random_rotations(rng, P)[None]).to(dev)
            ts = torch.from_numpy(workloads.random_shifts(rng, P, 5.0)[None]).to(dev)
            gen = torch.Generator(device=dev)
            gen.manual_seed(3100 + D + P)
            tg = torch.randn((1, P, D, D // 2 + 1), dtype=torch.complex64, device=dev, generator=gen)
            out = torch.empty_like(tg)
            for interp in ("linear", "cubic"):
                fw = lambda: bp.project_3d_to_2d(tv, tr, ts, interp=interp, radius_cutoff=D / 2, out=out)
                bw = lambda: bp.project_3d_to_2d_backward(tg, tv, tr, ts, interp=interp, radius_cutoff=D / 2)
                for _ in range(warmup):
                    fw()
                    bw()
                f_ms, _ = time_calls(fw, steps, torch)
                b_ms, _ = time_calls(bw, steps, torch)
                taps = 8 if interp == "linear" else 64
                l2 = P * n_in * taps * 8 / (f_ms * 1e-3) / 1e9 / L2_PEAK_GBS
                r = {"D": D, "interp": interp, "poses": P, "fwd_ms": round(f_ms, 4), "fwd_bwd_ms": round(f_ms + b_ms, 4),
                     "fwd_proj_per_s": round(P / (f_ms * 1e-3), 1),
                     "fwd_bwd_proj_per_s": round(P / ((f_ms + b_ms) * 1e-3), 1), "fwd_l2_frac": round(l2, 4)}
                rows.append(r)
                eprint("[bench] sweep: %4d  %-7s %8d %8.3f %11.3f %12.0f %15.0f %12.3f" % (
                    D, interp, P, f_ms, f_ms + b_ms, r["fwd_proj_per_s"], r["fwd_bwd_proj_per_s"], l2))
            del tg, out
        del tv
        torch.cuda.empty_cache()
    details["sweep"] = rows


def run_oversampling(bp, workloads, torch, details, D=128, P_acc=24, n_blobs=80):
    """Interpolation against oversampling: accuracy (FRC with the analytic
    slices, real-space gain by radius) and time of cubic at 1x against linear
    with a 2x zero-padded volume, padded offline (the projection alone) or on
    the fly (front end + projection), and cubic at 2x (stderr/details only)."""
    import numpy as np
    from back_projection_amd import accuracy as acc
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(4000)
    model = acc.blob_model(rng, D, n_blobs, 0.4 * D)
    vol = acc.real_volume(D, model)
    rot = workloads.random_rotations(rng, P_acc)
    ref = acc.analytic_slices(model, rot, D, D, D / 2)
    tv = torch.from_numpy(vol[None]).to(dev)
    tr = torch.from_numpy(rot[None]).to(dev)
    V1 = bp.volume_rfft(tv, pad=1)
    V2 = bp.volume_rfft(tv, pad=2)
    methods = {"linear 1x": (V1, "linear", 1.0), "cubic 1x": (V1, "cubic", 1.0),
               "linear 2x": (V2, "linear", 2.0), "cubic 2x": (V2, "cubic", 2.0)}
    ref_img = bp.images_irfft(torch.from_numpy(ref.astype(np.complex64)).to(dev)).cpu().numpy()
    ring_fr = (0.25, 0.5, 0.75, 0.9, 1.0)
    edges = (0.0, 0.2, 0.4, 0.6, 0.8)
    res = {"workload": f"D{D} blob volume ({n_blobs} Gaussians, sigma U(1,1.5), centres within 0.4 D), "
                       f"{P_acc} uniform rotations, radius D/2, the samples' exact transform as truth",
           "rings_frac_nyquist": ring_fr, "gain_bands_frac_half_box": edges, "methods": {}}
    eprint("[bench] oversampling: method      FRC at " + " ".join("%5.2f" % f for f in ring_fr) +
           "  | 1-FRC mean  | gain by radius " + " ".join("%.1f-%.1f" % e for e in zip(edges[:-1], edges[1:])))
    for name, (V, interp, o) in methods.items():
        Y = bp.project_3d_to_2d(V, tr, H=D, interp=interp, oversampling=o, radius_cutoff=D / 2)
        img = bp.images_irfft(Y).cpu().numpy()
        Yh = Y.cpu().numpy()[0]
        f = acc.frc(Yh, ref, D)
        at = [float(f[int(round(x * D / 2))]) for x in ring_fr]
        g = acc.radial_gain(img[0], ref_img, edges)
        res["methods"][name] = {"frc": at, "one_minus_frc_mean": float(np.mean(1 - f[1:])), "gain": g.tolist()}
        eprint("[bench] oversampling: %-10s        " % name + " ".join("%.4f" % x for x in at) +
               "  | %.2e    | " % np.mean(1 - f[1:]) + "   ".join("%.3f" % x for x in g))
    # time: 16384 and 1024 poses (rotations repeated from a seeded set)
    for P in (1024, 16384):
        trP = torch.from_numpy(workloads.random_rotations(np.random.default_rng(4100 + P), P)[None]).to(dev)
        out = torch.empty((1, P, D, D // 2 + 1), dtype=torch.complex64, device=dev)
        calls = {
            "cubic 1x": lambda: bp.project_3d_to_2d(V1, trP, H=D, interp="cubic", radius_cutoff=D / 2, out=out),
            "linear 2x offline": lambda: bp.project_3d_to_2d(V2, trP, H=D, interp="linear", oversampling=2.0,
                                                             radius_cutoff=D / 2, out=out),
            "linear 2x on the fly": lambda: bp.project_3d_to_2d(bp.volume_rfft(tv, pad=2), trP, H=D, interp="linear",
                                                                oversampling=2.0, radius_cutoff=D / 2, out=out),
            "cubic 2x offline": lambda: bp.project_3d_to_2d(V2, trP, H=D, interp="cubic", oversampling=2.0,
                                                            radius_cutoff=D / 2, out=out),
            "front end 2x alone": lambda: bp.volume_rfft(tv, pad=2, out=V2),
        }
        tt = {}
        for name, fn in calls.items():
            fn()
            ms, _ = time_calls(fn, 5, torch)
            tt[name] = round(ms, 4)
        res[f"time_ms_{P}_poses"] = tt
        eprint(f"[bench] oversampling: {P} poses, ms per call: " + ", ".join(f"{k} {v:.3f}" for k, v in tt.items()))
        del out
    details["oversampling"] = res


def brick_roofline(kernels, isolated):
    """The JSON line's roofline object for the dominant brick kernel (largest
    live time in the step): the gradient kernel, whose limit is fp32 VALU
    issue (SQ counters: VALU instructions and busy cycles, profiles/); its
    roofline is the fp32 FMA rate.  The tap-bandwidth figure of the L2
    roofline and the LDS and HBM fractions go beside it, and the forward
    kernel's figures with them."""
    dom = max(kernels, key=lambda k: kernels[k]["avg_ms"] * kernels[k]["launches"])
    kd = kernels[dom]
    achieved = kd["flops"] / (kd["avg_ms"] * 1e-3) / 1e12
    tap_gbps = kd["tap_bytes"] / (kd["avg_ms"] * 1e-3) / 1e9
    traffic = measured_traffic(dom)
    roofline = {
        "bound": "alu",
        "achieved": round(achieved, 2),
        "peak": round(FP32_VECTOR_TFLOPS, 2),
        "unit": "TFLOP/s",
        "frac": round(achieved / FP32_VECTOR_TFLOPS, 4),
        "traffic": traffic,
        "kernel": dom,
        "flops_per_launch": kd["flops"],
        "flops_per_pixel": kd["flops_per_pixel"],
        "peak_note": (f"published fp32 vector peak ({FP32_VECTOR_TFLOPS} TFLOP/s: 256 CUs x 4 SIMDs x 32 lanes x "
                      "2 flop x 2.4 GHz); the kernels use non-packed FMAs, which a probe on this GPU issues at "
                      f"{FP32_FMA_PROBE_TFLOPS} TFLOP/s"),
        "l2_tap": {"achieved": round(tap_gbps, 1), "peak": round(L2_PEAK_GBS, 1), "unit": "GB/s",
                   "frac": kd["l2_frac"]},
        "lds": {"achieved": round(tap_gbps, 1), "peak": round(LDS_PEAK_GBS, 1), "unit": "GB/s",
                "frac": kd["lds_frac"]},
        "hbm": {"achieved": round(kd["hbm_GBps"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": kd["hbm_frac"]},
        "valu_issue": valu_issue(dom),
    }
    if dom in isolated:
        iso = isolated[dom]
        roofline["overlap"] = ("runs beside the other backward kernel on a second stream; achieved uses "
                               "its live duration in the step")
        roofline["alone"] = {"avg_ms": round(iso, 4),
                             "achieved": round(kd["flops"] / (iso * 1e-3) / 1e12, 2),
                             "frac": round(kd["flops"] / (iso * 1e-3) / 1e12 / FP32_VECTOR_TFLOPS, 4),
                             "l2_tap_frac": round(kd["tap_bytes"] / (iso * 1e-3) / 1e9 / L2_PEAK_GBS, 4)}
    if "forward" in kernels and dom != "forward":
        kf = kernels["forward"]
        roofline["forward"] = {"avg_ms": kf["avg_ms"], "tflops": kf["tflops"], "alu_frac": kf["alu_frac"],
                               "l2_tap_frac": kf["l2_frac"], "lds_frac": kf["lds_frac"],
                               "traffic": measured_traffic("forward"), "valu_issue": valu_issue("forward")}
    return roofline


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-sample", type=int, default=16384, help="poses of the oracle CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--all-workloads", action="store_true", help="also time every workload per operation (stderr)")
    ap.add_argument("--sweep", action="store_true", help="also time the 3D ops over box size, poses and kernel (stderr)")
    ap.add_argument("--oversampling", action="store_true",
                    help="also run the interpolation vs oversampling accuracy study and timing (stderr)")
    ap.add_argument("--twod", action="store_true", help="also time the 2D -> 2D ops on their D=128 workload (stderr)")
    ap.add_argument("--details", default=None, help="write per-kernel details as JSON to this file")
    ap.add_argument("--peaks", action="store_true", help="measure HBM and L2-resident bandwidths and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (scale factor of the HBM traffic counters)")
    ap.add_argument("--sources-digest", action="store_true", help="print the digest of the kernel sources and exit")
    args = ap.parse_args()
    if args.sources_digest:
        print(sources_digest())
        return

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
    if args.copy_calibration:
        copy_calibration(torch)
        return
    if args.peaks:
        measure_peaks(torch)
        return
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
    # the headline: K steps with no instrumentation inside the timed region
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

    # a second pass of K steps with the library's event pairs around every
    # brick kernel (on the stream each kernel is launched on), for the
    # per-kernel durations in the step
    for k in bp.KERNEL_CLASSES:          # drop anything recorded before
        bp.timing_read(k)
    bp.timing_enable(True)
    ei0, ei1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ei0.record(st)
    for _ in range(args.steps):
        step()
    ei1.record(st)
    torch.cuda.synchronize()
    bp.timing_enable(False)
    instr_ms = ei0.elapsed_time(ei1) / args.steps
    eprint(f"[bench] instrumented pass: {instr_ms:.3f} ms/step (per-kernel events on)")

    # per-kernel averages over the timed region (library event pairs on the launch stream)
    g = bp.Geom(B=1, P=w.P, Bv=1, Br=1, Bs=1, D=w.D, H=w.H, interp=1, oversampling=1.0, radius_cutoff=r)
    ws_bwd = bp.lib().tp_workspace_size(ctypes.byref(g), bp.OP_PROJECT_BACKWARD)
    kernels = {}
    for k in bp.KERNEL_CLASSES:
        tot, n = bp.timing_read(k)
        if n == 0:
            continue
        ms = tot / n
        m = kernel_model(w, k, ws_bwd)
        kernels[k] = {
            "launches": n,
            "avg_ms": round(ms, 4),
            "share_of_step": round(tot / (instr_ms * args.steps), 4),
            "tap_GBps": round(m["tap_bytes"] / (ms * 1e-3) / 1e9, 1),
            "hbm_GBps": round(m["hbm_bytes"] / (ms * 1e-3) / 1e9, 1),
            "tflops": round(m["flops"] / (ms * 1e-3) / 1e12, 2),
            "l2_frac": round(m["tap_bytes"] / (ms * 1e-3) / 1e9 / L2_PEAK_GBS, 4),
            "lds_frac": round(m["tap_bytes"] / (ms * 1e-3) / 1e9 / LDS_PEAK_GBS, 4),
            "hbm_frac": round(m["hbm_bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "alu_frac": round(m["flops"] / (ms * 1e-3) / 1e12 / FP32_VECTOR_TFLOPS, 4),
            **m,
        }
        eprint(f"[bench] kernel {k}: {kernels[k]}")
    # The scatter and the gradient kernel share the GPU during the step (two
    # streams); their live durations above include that sharing.  For
    # reference, each alone (untimed region, same inputs):
    isolated = {}
    for k, call in (("backward", lambda: bp.project_3d_to_2d_backward(
            tg, tv, tr, ts, interp="cubic", radius_cutoff=r, grad_vol=gv, need_rot=False, need_shifts=False)),
                    ("gradient", lambda: bp.project_3d_to_2d_backward(
            tg, tv, tr, ts, interp="cubic", radius_cutoff=r, grad_rot=gr, grad_shifts=gs, need_vol=False))):
        call()
        torch.cuda.synchronize()
        for kk in bp.KERNEL_CLASSES:
            bp.timing_read(kk)
        bp.timing_enable(True)
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        bp.timing_enable(False)
        tot, n = bp.timing_read(k)
        for kk in bp.KERNEL_CLASSES:
            bp.timing_read(kk)
        if n:
            isolated[k] = tot / n
            eprint(f"[bench] kernel {k} alone: {tot / n:.4f} ms")
    roofline = None
    if not kernels:   # only the direct kernels ran (TPROJ_KERNELS=direct): no brick kernel timings
        eprint("[bench] no brick-kernel timings (direct kernels): roofline not reported")
    else:
        roofline = brick_roofline(kernels, isolated)
    details = {"kernels": kernels, "ms_per_step": ms_per_step, "instrumented_ms_per_step": instr_ms}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_sample, eprint)
    if args.all_workloads:
        del tg, out
        torch.cuda.empty_cache()
        for cfg in (1, 2, 3, 4, 5):
            run_workload_ops(cfg, max(3, args.steps // 2), 1, bp, workloads, torch, details)
    if args.sweep:
        torch.cuda.empty_cache()
        run_sweep(5, 1, bp, workloads, torch, details)
    if args.oversampling:
        torch.cuda.empty_cache()
        run_oversampling(bp, workloads, torch, details)
    if args.twod or args.all_workloads:
        torch.cuda.empty_cache()
        run_2d(max(3, args.steps // 2), 1, bp, workloads, torch, details)
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
