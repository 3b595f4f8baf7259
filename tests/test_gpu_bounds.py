"""The fixed-point bounds evaluated by the GPU (tp_bounds_device runs the
device build of back_projection_amd/csrc/fixed_point_bound.h, the code the
back-projection kernels call) against the host build of the same source,
which test_fixed_point_bound.py holds against brute-force weight sums.  The
two builds differ in the reciprocal (the hardware approximation on the GPU)
and in how products are contracted and square roots rounded; the weight-sum
bounds widen every such quantity by 1.0001, far more than that.  The results
agree to about ten ulp (2e-6 relative)."""
import ctypes

import numpy as np
import pytest

import back_projection_amd as bp
from back_projection_amd import workloads

pytestmark = pytest.mark.gpu


def _maps3(rng, n):
    rots = workloads.random_rotations(rng, n).reshape(-1, 3, 3).astype(np.float32)
    gen = (rots * rng.uniform(0.5, 2.0, (n, 1, 1)) + 0.3 * rng.standard_normal((n, 3, 3))).astype(np.float32)
    lattice = np.array([np.eye(3), [[0, 1, 0], [0, 0, 1], [1, 0, 0]], [[0, 0, 1], [1, 0, 0], [0, 1, 0]]],
                       dtype=np.float32)
    degenerate = np.array([[[1, 1, 0], [2, 2, 0], [0, 0, 1]]], dtype=np.float32)
    return np.concatenate([rots, gen, lattice, degenerate])


def _maps2(rng, n):
    th = rng.uniform(0, 2 * np.pi, n)
    R = np.stack([np.cos(th), -np.sin(th), np.sin(th), np.cos(th)], 1).reshape(-1, 2, 2)
    gen = R * rng.uniform(0.5, 2.0, (n, 1, 1)) + 0.3 * rng.standard_normal((n, 2, 2))
    return np.concatenate([R, gen, np.eye(2)[None], [[[1, 2], [0.5, 1]]]]).astype(np.float32)


def _device(L, kind, interp, o, kmax, D, maps):
    maps = np.ascontiguousarray(maps, dtype=np.float32)
    out = np.zeros(len(maps), dtype=np.float32)
    st = L.tp_bounds_device(kind, interp, o, kmax, D, maps.ctypes.data_as(ctypes.c_void_p), len(maps),
                            out.ctypes.data_as(ctypes.c_void_p))
    assert st == 0, L.tp_last_error_detail()
    return out


def _agree(dev, host):
    both_inf = np.isinf(dev) & np.isinf(host)
    assert np.array_equal(np.isinf(dev), np.isinf(host))
    fin = ~both_inf
    np.testing.assert_allclose(dev[fin], host[fin], rtol=2e-6, atol=0)


@pytest.mark.parametrize("interp", [1, 0])
@pytest.mark.parametrize("o", [1.0, 2.0])
def test_device_bounds_3d_match_host(interp, o):
    L = bp.lib()
    maps = _maps3(np.random.default_rng(31 + interp), 2000)
    for kind, fn in ((0, L.tp_weight_sum_bound_3d), (1, L.tp_contrib_bound_3d)):
        dev = _device(L, kind, interp, o, 0.0, 0, maps.reshape(-1, 9))
        host = np.array([fn(interp, o, m.ctypes.data_as(ctypes.c_void_p)) for m in maps], dtype=np.float32)
        _agree(dev, host)


@pytest.mark.parametrize("interp", [1, 0])
def test_device_bounds_2d_match_host(interp):
    L = bp.lib()
    maps = _maps2(np.random.default_rng(57 + interp), 2000)
    for o, kmax, D in ((1.0, 64.0, 128), (2.0, 30.0, 64), (1.0, 12.0, 8)):
        dev = _device(L, 2, interp, o, kmax, D, maps.reshape(-1, 4))
        host = np.array([L.tp_weight_sum_bound_2d(interp, o, kmax, D, m.ctypes.data_as(ctypes.c_void_p))
                         for m in maps], dtype=np.float32)
        _agree(dev, host)
