"""The back-projection's fixed-point scale rests on a bound B(A) on the sum of
|interpolation weights| that one voxel receives from all pixels of one pose
(A = o [R_:0 R_:1], p = A k).  The brick kernel computes

    B(A) = CELLS * min over axis pairs (i, j) of (floor(w_1) + 1)(floor(w_2) + 1),

w_r = the sum of |row r of M^-1| with M the rows i, j of A, CELLS = (2 + 2 *
0.0742)^2 (cubic) or 4 (linear).  Here that formula, restated, is checked
against brute-force sums of the oracle's kernel weights over the pixel lattice
for rotations, oversampled rotations and general maps, at random and at
adversarial voxel offsets: if it ever fell short, a window's fixed-point sums
could overflow.  (No GPU needed.)
"""
import math

import numpy as np
import pytest

import oracle
from back_projection_amd import workloads


def bound(A, interp):
    cells = 4.6152 if interp == 1 else 4.0
    best = math.inf
    for i, j in ((0, 1), (0, 2), (1, 2)):
        M = A[[i, j], :]
        d = abs(np.linalg.det(M))
        if d <= 1e-6 * np.abs(M[0]).sum() * np.abs(M[1]).sum():
            continue
        Mi = np.linalg.inv(M)
        w = np.abs(Mi).sum(axis=1) * 1.0001 + 1e-4
        best = min(best, float(np.prod(np.floor(w) + 1.0)))
    return cells * best


def weight_sum(A, v, interp, n=14):
    """Sum over pixels k in [-n, n]^2 of |w(A k - v)| with the oracle's 1D kernel."""
    sup = 2.0 if interp == 1 else 1.0
    k = np.stack(np.meshgrid(np.arange(-n, n + 1), np.arange(-n, n + 1)), -1).reshape(-1, 2).astype(np.float64)
    d = k @ A.T - v
    near = np.all(np.abs(d) < sup, axis=1)
    total = 0.0
    for row in d[near]:
        total += abs(np.prod([oracle.kernel_weight(interp, float(x)) for x in row]))
    return total


def maps(rng):
    rots = workloads.random_rotations(rng, 6).reshape(-1, 3, 3).astype(np.float64)
    out = [r[:, :2] for r in rots]
    out += [1.7 * r[:, :2] for r in rots[:3]]
    out += [0.6 * r[:, :2] for r in rots[3:]]
    for r in rots[:4]:
        W = r * rng.uniform(0.6, 1.8) + 0.3 * rng.standard_normal((3, 3))
        out.append(W[:, :2])
    # an axis-aligned slice and a diagonal one
    out.append(np.array([[1.0, 0.0], [0.0, 1.0], [0.0, 0.0]]))
    out.append(np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]]))
    return out


@pytest.mark.parametrize("interp", [1, 0])
def test_weight_sum_bound_holds(interp):
    rng = np.random.default_rng(2025 + interp)
    for A in maps(rng):
        B = bound(A, interp)
        offsets = list(rng.uniform(0, 1, (40, 3)))
        # voxels right on a sample, and half-way between samples
        offsets += [A @ np.array([0.0, 0.0]), A @ np.array([0.5, 0.0]), A @ np.array([0.5, 0.5]),
                    A @ np.array([0.25, 0.75])]
        worst = max(weight_sum(A, v, interp) for v in offsets)
        assert worst <= B, (A, worst, B)


def test_weight_sum_bound_is_tighter_than_the_pixel_count():
    """For rotations the bound is far below the old pixel-count bound (63 at
    o = 1, cubic): that is what allows windows of 32 poses."""
    rng = np.random.default_rng(7)
    for R in workloads.random_rotations(rng, 50).reshape(-1, 3, 3).astype(np.float64):
        assert bound(R[:, :2], 1) <= 4.6152 * 6 + 1e-9
