"""The back-projection's fixed-point window scales rest on bounds that the
kernels compute in device code (back_projection_amd/csrc/fixed_point_bound.h):

  * 3D, B(A): the sum of |interpolation weights| one voxel receives from all
    pixels of one pose (A = o [R_:0 R_:1], p = A k),
  * 3D, C(A): the number of pixels of one pose whose taps reach one voxel,
  * 2D, B2(A): the weight sum for one entry of the periodic D x D source,
    periodic translates included, for in-mask pixels |k| <= kmax.

The library exports host builds of that same source (include/tproj_bounds.h).
Here they are held against brute-force sums over the pixel lattice with the
oracle's 1D kernels, for rotations, oversampled rotations and general maps,
at random and adversarial offsets: if a bound ever fell short, a window's
fixed-point sums could overflow.  (No GPU needed; the GPU evaluation of the
same source is compared with these in test_gpu_bounds.py.)
"""
import ctypes
import os

import numpy as np
import pytest

import back_projection_amd as bp
import oracle
from back_projection_amd import build_lib, workloads


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(bp.LIB_PATH):
        build_lib.build()
    return bp.lib()


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def lib_bound3(L, interp, o, R):
    a, p = _f32(R)
    return float(L.tp_weight_sum_bound_3d(interp, o, p))


def lib_contrib3(L, interp, o, R):
    a, p = _f32(R)
    return float(L.tp_contrib_bound_3d(interp, o, p))


def lib_bound2(L, interp, o, kmax, D, R):
    a, p = _f32(R)
    return float(L.tp_weight_sum_bound_2d(interp, o, kmax, D, p))


def lattice(n):
    k = np.stack(np.meshgrid(np.arange(-n, n + 1), np.arange(-n, n + 1)), -1).reshape(-1, 2)
    return k.astype(np.float64)


def weight_sum3(A, v, interp, n=14):
    """Sum over pixels k in [-n, n]^2 of |w(A k - v)| with the oracle's 1D kernel."""
    sup = 2.0 if interp == 1 else 1.0
    d = lattice(n) @ A.T - v
    near = np.all(np.abs(d) < sup, axis=1)
    total = 0.0
    for row in d[near]:
        total += abs(np.prod([oracle.kernel_weight(interp, float(x)) for x in row]))
    return total


def reaching_pixels3(A, t, interp, n=14):
    """Pixels k whose taps (floor(p) - 1 .. floor(p) + 2 cubic, floor(p) ..
    floor(p) + 1 linear, per axis) include voxel 0, p = A k + t."""
    lo, hi = (-1, 2) if interp == 1 else (0, 1)
    f = np.floor(lattice(n) @ A.T + t)
    return int(np.all((-f >= lo) & (-f <= hi), axis=1).sum())


def maps3(rng):
    """(oversampling, 3x3 matrix) pairs: rotations, oversampled rotations,
    general maps, an axis-aligned and a diagonal slice."""
    rots = workloads.random_rotations(rng, 6).reshape(-1, 3, 3).astype(np.float64)
    out = [(1.0, r) for r in rots]
    out += [(1.7, r) for r in rots[:3]]
    out += [(0.6, r) for r in rots[3:]]
    for r in rots[:4]:
        out.append((1.0, r * rng.uniform(0.6, 1.8) + 0.3 * rng.standard_normal((3, 3))))
    out.append((1.0, np.eye(3)))
    out.append((1.0, np.array([[1.0, 0.0, 0.0], [0.0, 1.0, 0.0], [1.0, 1.0, 0.0]])))
    return out


@pytest.mark.parametrize("interp", [1, 0])
def test_weight_sum_bound_3d_holds(L, interp):
    rng = np.random.default_rng(2025 + interp)
    for o, R in maps3(rng):
        A = o * R[:, :2]
        B = lib_bound3(L, interp, o, R)
        assert np.isfinite(B)
        offsets = list(rng.uniform(0, 1, (40, 3)))
        # voxels right on a sample, and half-way between samples
        offsets += [A @ np.array([0.0, 0.0]), A @ np.array([0.5, 0.0]), A @ np.array([0.5, 0.5]),
                    A @ np.array([0.25, 0.75])]
        worst = max(weight_sum3(A, v, interp) for v in offsets)
        assert worst <= B, (o, R, worst, B)


@pytest.mark.parametrize("interp", [1, 0])
def test_contrib_bound_3d_holds(L, interp):
    rng = np.random.default_rng(77 + interp)
    for o, R in maps3(rng):
        A = o * R[:, :2]
        C = lib_contrib3(L, interp, o, R)
        worst = max(reaching_pixels3(A, t, interp) for t in rng.uniform(0, 1, (60, 3)))
        assert worst <= C, (o, R, worst, C)


def test_bounds_3d_known_values(L):
    """The identity slice: the (x, y) pair gives w = (1, 1), so B = 4 cells
    (2 x 2 lattice points per cell); C = (2 a + 1)^2 with a = NT sqrt(3) / 2."""
    R = np.eye(3)
    assert lib_bound3(L, 1, 1.0, R) == pytest.approx(4.6152 * 4, rel=1e-6)
    assert lib_bound3(L, 0, 1.0, R) == pytest.approx(4.0 * 4, rel=1e-6)
    assert lib_contrib3(L, 1, 1.0, R) == pytest.approx((2 * 2 * np.sqrt(3) + 1) ** 2, rel=1e-5)
    assert lib_contrib3(L, 0, 1.0, R) == pytest.approx((2 * np.sqrt(3) + 1) ** 2, rel=1e-5)


def test_bounds_3d_degenerate_maps_are_infinite(L):
    R = np.array([[1.0, 1.0, 0.0], [2.0, 2.0, 0.0], [0.0, 0.0, 1.0]])   # columns 0 and 1 parallel
    assert np.isinf(lib_bound3(L, 1, 1.0, R))
    assert np.isinf(lib_contrib3(L, 1, 1.0, R))
    assert np.isinf(lib_bound3(L, 0, 1.0, np.zeros((3, 3))))


def test_weight_sum_bound_is_tighter_than_the_pixel_count(L):
    """For rotations the bound is far below the pixel-count bound (63 at
    o = 1, cubic): that is what allows windows of 32 poses."""
    rng = np.random.default_rng(7)
    for R in workloads.random_rotations(rng, 50).reshape(-1, 3, 3).astype(np.float64):
        assert lib_bound3(L, 1, 1.0, R) <= 4.6152 * 6 + 1e-4
        assert lib_contrib3(L, 1, 1.0, R) > 62.8


def weight_sum2(A, t, v, interp, kmax, D):
    """Sum over in-mask pixels |k| <= kmax of |w| for entry v of the D-periodic
    source, p = A k + t; each tap offset is taken to its nearest periodic
    representative (with D > 4 at most one is within the kernel's support)."""
    n = int(np.ceil(kmax))
    k = lattice(n)
    k = k[(k ** 2).sum(1) <= kmax * kmax]
    d = k @ A.T + t - v
    d = d - D * np.round(d / D)
    sup = 2.0 if interp == 1 else 1.0
    near = np.all(np.abs(d) < sup, axis=1)
    return sum(abs(oracle.kernel_weight(interp, float(a)) * oracle.kernel_weight(interp, float(b)))
               for a, b in d[near])


@pytest.mark.parametrize("interp", [1, 0])
def test_weight_sum_bound_2d_holds(L, interp):
    rng = np.random.default_rng(515 + interp)
    cases = []
    for th in rng.uniform(0, 2 * np.pi, 5):
        R = np.array([[np.cos(th), -np.sin(th)], [np.sin(th), np.cos(th)]])
        cases += [(1.0, R, 3.0, 64), (1.0, R, 12.0, 8), (2.0, R, 10.0, 16)]
    cases.append((1.0, np.eye(2), 12.0, 8))
    cases.append((1.0, np.array([[1.3, 0.4], [-0.2, 0.8]]), 9.0, 12))
    for o, R, kmax, D in cases:
        A = o * R
        B = lib_bound2(L, interp, o, kmax, D, R)
        assert np.isfinite(B)
        worst = 0.0
        for t in rng.uniform(0, 1, (6, 2)):
            for v in rng.uniform(0, D, (8, 2)):
                worst = max(worst, weight_sum2(A, t, v, interp, kmax, D))
        assert worst <= B, (o, R, kmax, D, worst, B)


def test_bound_2d_known_value_and_degenerate(L):
    # identity, kmax 3, D 64: one translate, (1 + 1)^2 points per cell
    assert lib_bound2(L, 1, 1.0, 3.0, 64, np.eye(2)) == pytest.approx(4.6152 * 4, rel=1e-6)
    # kmax 12, D 8: n = floor(2 (12 sigma_max + NT) / 8) + 1 = 5 translates per axis (NT = 4 taps)
    assert lib_bound2(L, 1, 1.0, 12.0, 8, np.eye(2)) == pytest.approx(4.6152 * 4 * 25, rel=1e-6)
    # linear (NT = 2): floor(2 (12 + 2) / 8) + 1 = 4
    assert lib_bound2(L, 0, 1.0, 12.0, 8, np.eye(2)) == pytest.approx(4.0 * 4 * 16, rel=1e-6)
    assert np.isinf(lib_bound2(L, 1, 1.0, 3.0, 64, np.array([[1.0, 2.0], [0.5, 1.0]])))


def test_bounds_device_rejects_bad_arguments(L):
    """Checked on the host before any device work."""
    r, p = _f32(np.eye(3))
    o, po = _f32(np.zeros(1))
    assert L.tp_bounds_device(3, 1, 1.0, 0.0, 8, p, 1, po) == 3        # TP_E_VALUE: kind
    assert L.tp_bounds_device(0, 2, 1.0, 0.0, 8, p, 1, po) == 3        # interp
    assert L.tp_bounds_device(0, 1, 1.0, 0.0, 8, p, -1, po) == 3       # n
    assert L.tp_bounds_device(2, 1, 1.0, 0.0, 0, p, 1, po) == 3        # D for the 2D bound
    assert L.tp_bounds_device(0, 1, 1.0, 0.0, 8, None, 1, po) == 1     # TP_E_NULL
    assert L.tp_bounds_device(0, 1, 1.0, 0.0, 8, None, 0, None) == 0   # nothing to do
