"""Pins of the oracle's linear-kernel gradients where samples sit on the grid.

Every operation is differentiable with respect to the rotation and the shift
(torch-projectors pages: Spanish "Resumen tecnico" section 2, Dutch
"Technische samenvatting", Methodologie).  The tent kernel has a kink at the
grid nodes, so the derivative there needs a convention; the reading taken is
the right derivative in p, i.e. the derivative of the cell
[floor(p), floor(p)+1).

Along the move of one rotation entry R[i][j] only p_i changes, by t * k_j,
and linear interpolation is exactly linear in p_i inside one cell.  So a
one-sided difference quotient is the one-sided derivative with no truncation
error, as long as no sample leaves its cell.  A sample moves to larger p_i
for t > 0 when k_j > 0 and for t < 0 when k_j < 0; splitting the upstream
gradient by the sign of k_j therefore gives two difference quotients that
together must equal the oracle's right-derivative gradient:

    G+ (k_j > 0):  (L(R + h e_ij) - L(R)) / h
    G- (k_j < 0):  (L(R) - L(R - h e_ij)) / h

Identity maps, the 24 lattice rotations, quarter turns in 2D and rotations
about z all put samples exactly on grid nodes or planes, which is where a
dropped slope at the upper tap (or a left derivative) shows.
"""
import itertools

import numpy as np
import pytest

import oracle

H_STEP = 1e-4     # samples move by at most H_STEP * |k| < 1e-3 of a cell


def lattice_rotations_3d():
    out = []
    for perm in itertools.permutations(range(3)):
        for signs in itertools.product([1, -1], repeat=3):
            M = np.zeros((3, 3))
            for i in range(3):
                M[i, perm[i]] = signs[i]
            if round(np.linalg.det(M)) == 1:
                out.append(M)
    assert len(out) == 24
    return np.array(out)


def signed_permutations_2d():
    out = []
    for perm in itertools.permutations(range(2)):
        for signs in itertools.product([1, -1], repeat=2):
            M = np.zeros((2, 2))
            for i in range(2):
                M[i, perm[i]] = signs[i]
            out.append(M)
    return np.array(out)


def rot_z(a):
    c, s = np.cos(a), np.sin(a)
    return np.array([[c, -s, 0.0], [s, c, 0.0], [0.0, 0.0, 1.0]])


def freq_grids(H):
    kx = np.broadcast_to(np.arange(H // 2 + 1, dtype=float)[None, :], (H, H // 2 + 1))
    ky = np.broadcast_to(np.fft.fftfreq(H, 1.0 / H)[:, None], (H, H // 2 + 1))
    return kx, ky


def split_by_sign(G, k):
    """(G where k > 0, G where k < 0); pixels with k = 0 do not move."""
    return G * (k > 0), G * (k < 0)


def one_sided_rot_grads(L_of, R, G, kcols):
    """Right-derivative gradient of L w.r.t. every R[b, n, i, j] with j < len(kcols),
    from the split one-sided difference quotients described above."""
    out = np.zeros_like(R)
    Bq, P, nrow, ncol = R.shape
    for j, kj in enumerate(kcols):
        Gp, Gm = split_by_sign(G, kj)
        for b, n, i in itertools.product(range(Bq), range(P), range(nrow)):
            e = np.zeros_like(R)
            e[b, n, i, j] = H_STEP
            fwd = (L_of(R + e, Gp) - L_of(R, Gp)) / H_STEP
            bwd = (L_of(R, Gm) - L_of(R - e, Gm)) / H_STEP
            out[b, n, i, j] = fwd + bwd
    return out


def central_shift_grads(L_of, s, G, h=1e-6):
    out = np.zeros_like(s)
    for idx in itertools.product(*map(range, s.shape)):
        e = np.zeros_like(s)
        e[idx] = h
        out[idx] = (L_of(s + e, G) - L_of(s - e, G)) / (2 * h)
    return out


def test_tent_slopes_on_the_closed_cell():
    """Tap floor(p) has slope -1 on d in [0, 1); tap floor(p)+1 has slope +1
    on d in [-1, 0), the lower end included; nothing outside."""
    assert oracle.kernel_dweight(0, 0.0) == -1.0
    assert oracle.kernel_dweight(0, -1.0) == 1.0
    assert oracle.kernel_dweight(0, 0.5) == -1.0 and oracle.kernel_dweight(0, -0.5) == 1.0
    for d in (1.0, 1.5, -1.0000001, -2.0):
        assert oracle.kernel_dweight(0, d) == 0.0
    # the weight itself is the tent: a right-sided difference of W matches
    for d in (0.0, -1.0, 0.25, -0.75):
        h = 1e-9
        num = (oracle.kernel_weight(0, d + h) - oracle.kernel_weight(0, d)) / h
        assert abs(num - oracle.kernel_dweight(0, d)) < 1e-6


def _volume(rng, D, Bv=1):
    return rng.standard_normal((Bv, D, D, D // 2 + 1)) + 1j * rng.standard_normal((Bv, D, D, D // 2 + 1))


def _images(rng, B, P, H):
    return rng.standard_normal((B, P, H, H // 2 + 1)) + 1j * rng.standard_normal((B, P, H, H // 2 + 1))


# ---------------------------------------------------------------------------
# 3D forward: grad_rot / grad_shifts of project_backward
# ---------------------------------------------------------------------------

def _check_project3d(R, D, H, r, seed, with_shifts=True):
    rng = np.random.default_rng(seed)
    V = _volume(rng, D)
    P = R.shape[1]
    s = rng.uniform(-3, 3, (1, P, 2)) if with_shifts else None
    G = _images(rng, 1, P, H)
    kx, ky = freq_grids(H)

    def L_rot(R_, G_):
        out = oracle.project(V, R_, shifts=s, H=H, interp=0, r=r)
        return np.real(np.vdot(G_.ravel(), out.ravel()))

    _, gR, gs = oracle.project_backward(G, V, R, shifts=s, interp=0, r=r, need_vol=False)
    num = one_sided_rot_grads(L_rot, R, G, [kx, ky])
    scale = np.abs(num).max()
    assert scale > 0
    assert np.abs(gR - num).max() < 1e-8 * scale, np.abs(gR - num).max() / scale
    assert np.all(gR[..., 2] == 0)
    if with_shifts:
        def L_s(s_, G_):
            out = oracle.project(V, R, shifts=s_, H=H, interp=0, r=r)
            return np.real(np.vdot(G_.ravel(), out.ravel()))
        ns = central_shift_grads(L_s, s, G)
        assert np.abs(gs - ns).max() < 1e-6 * np.abs(ns).max()


def test_project3d_linear_lattice_rotations():
    """All 24 lattice rotations (identity included): every sample is a node."""
    _check_project3d(lattice_rotations_3d()[None], D=8, H=8, r=-1.0, seed=1)


def test_project3d_linear_rotation_about_z_and_cutoff():
    """Rotations about z keep p_z = 0 exactly (a grid plane) while p_x, p_y
    are generic; with a cutoff and H != D."""
    quarter = np.array([[0.0, -1.0, 0.0], [1.0, 0.0, 0.0], [0.0, 0.0, 1.0]])   # exact, unlike rot_z(pi/2)
    R = np.stack([rot_z(0.0), rot_z(0.3), rot_z(1.1), quarter])[None]
    _check_project3d(R, D=10, H=8, r=3.5, seed=2)


def test_project3d_linear_generic_maps():
    """General position: no sample on a cell boundary, so the one-sided and
    two-sided derivatives agree (also non-orthonormal maps)."""
    rng = np.random.default_rng(3)
    R = rng.standard_normal((1, 3, 3, 3))
    _check_project3d(R, D=10, H=10, r=-1.0, seed=4)


def test_planted_left_derivative_fails():
    """The check is not blind to the convention: the left-sided split
    (G+ backward, G- forward) differs from the oracle at lattice rotations."""
    rng = np.random.default_rng(5)
    D = H = 8
    V = _volume(rng, D)
    R = np.eye(3)[None, None]
    G = _images(rng, 1, 1, H)
    kx, ky = freq_grids(H)

    def L(R_, G_):
        return np.real(np.vdot(G_.ravel(), oracle.project(V, R_, H=H, interp=0).ravel()))

    _, gR, _ = oracle.project_backward(G, V, R, interp=0, need_vol=False, need_shifts=False)
    e = np.zeros_like(R)
    e[0, 0, 0, 0] = H_STEP
    left = (L(R, G) - L(R - e, G)) / H_STEP      # kx >= 0: moves p_x to the left
    right = (L(R + e, G) - L(R, G)) / H_STEP
    assert abs(right - gR[0, 0, 0, 0]) < 1e-8 * abs(right)
    assert abs(left - gR[0, 0, 0, 0]) > 1e-3 * abs(right)


# ---------------------------------------------------------------------------
# 3D back-projection backward: grad_rot / grad_shifts
# ---------------------------------------------------------------------------

def test_backproject3d_backward_linear_lattice_rotations():
    rng = np.random.default_rng(6)
    D = H = 8
    R = lattice_rotations_3d()[None, ::3]          # 8 of the 24
    P = R.shape[1]
    Y = _images(rng, 1, P, H)
    W = rng.random((1, P, H, H // 2 + 1))
    s = rng.uniform(-2, 2, (1, P, 2))
    Gd = _volume(rng, D)
    Gw = rng.standard_normal((1, D, D, D // 2 + 1))
    kx, ky = freq_grids(H)

    def L(R_, mask):
        dv, wv = oracle.backproject(Y * mask, R_, weights=W * mask, shifts=s, D=D, interp=0)
        return np.real(np.vdot(Gd.ravel(), dv.ravel())) + float(np.sum(Gw * wv))

    _, _, gR, _ = oracle.backproject_backward(Gd, Y, R, grad_weight_vol=Gw, weights=W, shifts=s, interp=0,
                                              need_images=False, need_weights=False, need_shifts=False)
    ones = np.ones((1, P, H, H // 2 + 1))
    num = one_sided_rot_grads(L, R, ones, [kx, ky])
    assert np.abs(gR - num).max() < 1e-8 * np.abs(num).max()


# ---------------------------------------------------------------------------
# 2D -> 2D
# ---------------------------------------------------------------------------

def _check_project2d(R, D, H, r, seed):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((1, D, D // 2 + 1)) + 1j * rng.standard_normal((1, D, D // 2 + 1))
    P = R.shape[1]
    s = rng.uniform(-3, 3, (1, P, 2))
    G = _images(rng, 1, P, H)
    kx, ky = freq_grids(H)

    def L(R_, G_):
        return np.real(np.vdot(G_.ravel(), oracle.project2d(X, R_, shifts=s, H=H, interp=0, r=r).ravel()))

    _, gR, gs = oracle.project2d_backward(G, X, R, shifts=s, interp=0, r=r, need_src=False)
    num = one_sided_rot_grads(L, R, G, [kx, ky])
    assert np.abs(gR - num).max() < 1e-8 * np.abs(num).max(), np.abs(gR - num).max()

    def Ls(s_, G_):
        return np.real(np.vdot(G_.ravel(), oracle.project2d(X, R, shifts=s_, H=H, interp=0, r=r).ravel()))

    ns = central_shift_grads(Ls, s, G)
    assert np.abs(gs - ns).max() < 1e-6 * np.abs(ns).max()


def test_project2d_linear_signed_permutations():
    _check_project2d(signed_permutations_2d()[None], D=8, H=8, r=-1.0, seed=7)


def test_project2d_linear_generic_maps():
    rng = np.random.default_rng(8)
    _check_project2d(rng.standard_normal((1, 3, 2, 2)), D=10, H=10, r=4.5, seed=9)


def test_backproject2d_backward_linear_signed_permutations():
    rng = np.random.default_rng(10)
    D = H = 8
    R = signed_permutations_2d()[None]
    P = R.shape[1]
    Y = _images(rng, 1, P, H)
    W = rng.random((1, P, H, H // 2 + 1))
    s = rng.uniform(-2, 2, (1, P, 2))
    Gd = rng.standard_normal((1, D, D // 2 + 1)) + 1j * rng.standard_normal((1, D, D // 2 + 1))
    Gw = rng.standard_normal((1, D, D // 2 + 1))
    kx, ky = freq_grids(H)

    def L(R_, mask):
        dv, wv = oracle.backproject2d(Y * mask, R_, weights=W * mask, shifts=s, D=D, interp=0)
        return np.real(np.vdot(Gd.ravel(), dv.ravel())) + float(np.sum(Gw * wv))

    _, _, gR, _ = oracle.backproject2d_backward(Gd, Y, R, grad_weight=Gw, weights=W, shifts=s, interp=0,
                                                need_images=False, need_weights=False, need_shifts=False)
    num = one_sided_rot_grads(L, R, np.ones((1, P, H, H // 2 + 1)), [kx, ky])
    assert np.abs(gR - num).max() < 1e-8 * np.abs(num).max()
