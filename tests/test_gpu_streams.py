"""GPU tests of the library's stream handling.

Large calls split their kernels over the caller's stream and a library side
stream (event fork and join): the backward's gradients, and the band-maximum
pass of a back-projection that leaves the side stream free.  These tests
check that results do not depend on that: against the one-stream path inside
a HIP graph capture (which never splits), replayed several times with eager
work in between; and with two host threads calling at once on two streams.
"""
import threading

import numpy as np
import pytest
import torch

import back_projection_amd as bp
from back_projection_amd import workloads
from tests.helpers import dev, log, rel

pytestmark = pytest.mark.gpu

# D = 64, 1024 poses: 2.2 M image pixels, above the size from which the
# backward splits (2^20 pixels)
D, P, R = 64, 1024, 32.0


def _inputs(seed):
    rng = np.random.default_rng(seed)
    vol = workloads.random_complex(rng, (1, D, D, D // 2 + 1))
    rot = workloads.random_rotations(rng, P).reshape(1, P, 3, 3)
    sh = rng.uniform(-3, 3, (1, P, 2)).astype(np.float32)
    g = workloads.random_complex(rng, (1, P, D, D // 2 + 1))
    return dev(vol, rot, sh, g)


def _step(tv, tr, ts, tg):
    out = bp.project_3d_to_2d(tv, tr, ts, radius_cutoff=R)
    gv, gr, gs = bp.project_3d_to_2d_backward(tg, tv, tr, ts, radius_cutoff=R)
    return out, gv, gr, gs


def test_graph_capture_and_replay():
    tv, tr, ts, tg = _inputs(71)
    log("[streams] graph capture, D=64, P=1024")
    _step(tv, tr, ts, tg)                       # warm up outside the capture
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            outs = _step(tv, tr, ts, tg)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for k in range(3):
        # new inputs in place, some eager work, then the replay
        nv, nr, ns, ng = _inputs(100 + k)
        tv.copy_(nv), tr.copy_(nr), ts.copy_(ns), tg.copy_(ng)
        eager = _step(tv, tr, ts, tg)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(outs[0], eager[0]), k                  # forward: bitwise
        assert torch.equal(outs[1], eager[1]), k                  # volume gradient: fixed point, bitwise
        assert rel(outs[2], eager[2]) <= 1e-6, (k, rel(outs[2], eager[2]))
        assert rel(outs[3], eager[3]) <= 1e-6, (k, rel(outs[3], eager[3]))


def test_two_host_threads_two_streams():
    inputs = [_inputs(81), _inputs(82)]
    log("[streams] two host threads, D=64, P=1024")
    ref = []
    for t in inputs:
        ref.append(_step(*t))
    torch.cuda.synchronize()
    results = [None, None]
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(3):
                    r = _step(*inputs[i])
                s.synchronize()
            results[i] = r
        except Exception as e:   # surfaced below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=60)
    assert not errors, errors
    assert all(not th.is_alive() for th in threads)
    for i in range(2):
        assert torch.equal(results[i][0], ref[i][0])
        assert torch.equal(results[i][1], ref[i][1])
        assert rel(results[i][2], ref[i][2]) <= 1e-6
        assert rel(results[i][3], ref[i][3]) <= 1e-6


def _bp_inputs(seed):
    rng = np.random.default_rng(seed)
    rot = workloads.random_rotations(rng, P).reshape(1, P, 3, 3)
    sh = rng.uniform(-3, 3, (1, P, 2)).astype(np.float32)
    img = workloads.random_complex(rng, (1, P, D, D // 2 + 1))
    wts = rng.uniform(0.1, 1.0, (1, P, D, D // 2 + 1)).astype(np.float32)
    return dev(img, rot, sh, wts)


def _bp_step(ti, tr, ts, tw):
    # back-projection with weights, and the volume gradient alone: both leave
    # the side stream to their band-maximum pass when they split
    dv, wv = bp.backproject_2d_to_3d(ti, tr, tw, ts, D=D, radius_cutoff=R)
    gv, _, _ = bp.project_3d_to_2d_backward(ti, dv, tr, ts, radius_cutoff=R, need_rot=False, need_shifts=False)
    return dv, wv, gv


def test_back_projection_side_stream_matches_one_stream():
    """The split calls (band maxima on the side stream) against the same calls
    captured in a graph (one stream), replayed with new inputs: the fixed-point
    volumes are bitwise equal."""
    ti, tr, ts, tw = _bp_inputs(91)
    log("[streams] back-projection split vs captured, D=64, P=1024")
    _bp_step(ti, tr, ts, tw)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            outs = _bp_step(ti, tr, ts, tw)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for k in range(3):
        ni, nr, ns, nw = _bp_inputs(110 + k)
        ti.copy_(ni), tr.copy_(nr), ts.copy_(ns), tw.copy_(nw)
        eager = _bp_step(ti, tr, ts, tw)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, eager):
            assert torch.equal(a, b), k
