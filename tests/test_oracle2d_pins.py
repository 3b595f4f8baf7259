"""Pins of the oracle's 2D -> 2D ops (rotation of 2D Fourier data and its
adjoint, the accumulation into a 2D reconstruction; torch-projectors pages:
Dutch Methodologie, operations 1 and 2) against what mathematics fixes: the
rotation of a real image by a signed permutation and integer shifts (numpy's
FFT), interpolation at lattice points, the adjoint identity and finite
differences of every gradient.
"""
import itertools

import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(2024)


def signed_permutations_2d():
    out = []
    for perm in itertools.permutations(range(2)):
        for signs in itertools.product([1, -1], repeat=2):
            M = np.zeros((2, 2))
            for i in range(2):
                M[i, perm[i]] = signs[i]
            out.append(M)
    assert len(out) == 8   # rotations by multiples of 90 degrees and reflections
    return out


def mask2d(H, r):
    kx = np.arange(H // 2 + 1)
    ky = np.fft.fftfreq(H, 1.0 / H)
    return (r < 0) | (kx[None, :] ** 2 + ky[:, None] ** 2 <= r * r)


def inner(a, b):
    return float(np.real(np.vdot(np.ravel(a), np.ravel(b))))


@pytest.mark.parametrize("D", [8, 12])
@pytest.mark.parametrize("interp", [0, 1])
def test_identity_map_returns_the_source(D, interp):
    """At lattice points both kernels interpolate exactly."""
    X = np.fft.rfft2(RNG.standard_normal((2, D, D)))
    out = oracle.project2d(X, np.tile(np.eye(2), (2, 3, 1, 1)), H=D, interp=interp)
    for n in range(3):
        assert np.abs(out[:, n] - X).max() < 1e-12 * np.abs(X).max()


@pytest.mark.parametrize("D,H", [(8, 8), (12, 12), (12, 8)])
@pytest.mark.parametrize("interp", [0, 1])
def test_signed_permutations_match_the_full_fft(D, H, interp):
    """A signed permutation maps the lattice to itself, so output pixel
    (kx, ky) is the full spectrum of the real source at R (kx, ky) mod D --
    which exercises the per-tap Friedel rule for every negative kx."""
    f = RNG.standard_normal((D, D))
    X = np.fft.rfft2(f)[None]
    F = np.fft.fft2(f)                      # F[ky, kx]
    ky = np.round(np.fft.fftfreq(H, 1.0 / H)).astype(int)
    kx = np.arange(H // 2 + 1)
    for R in signed_permutations_2d():
        for r in (-1.0, H / 2 - 1):
            out = oracle.project2d(X, R[None, None], H=H, interp=interp, r=r)[0, 0]
            k2 = np.stack(np.broadcast_arrays(kx[None, :], ky[:, None]))
            p = np.einsum("ij,j...->i...", R.astype(int), k2) % D
            exp = F[p[1], p[0]] * mask2d(H, r)
            assert np.abs(out - exp).max() < 1e-9 * np.abs(exp).max(), (R, r)


def test_rotation_of_real_image_by_quarter_turn():
    """Rotating the real image by a quarter turn about index 0, g[y, x] =
    f[x, -y mod D], is the map (kx, ky) -> (-ky, kx) in Fourier space."""
    D = 10
    f = RNG.standard_normal((D, D))
    y, x = np.meshgrid(np.arange(D), np.arange(D), indexing="ij")
    g = f[x, (-y) % D]
    R = np.array([[0.0, -1.0], [1.0, 0.0]])
    out = oracle.project2d(np.fft.rfft2(f)[None], R[None, None], H=D, interp=1)[0, 0]
    exp = np.fft.rfft2(g)
    assert np.abs(out - exp).max() < 1e-9 * np.abs(exp).max()


@pytest.mark.parametrize("D", [8, 12])
def test_shift_theorem_integer_shifts(D):
    f = RNG.standard_normal((D, D))
    X = np.fft.rfft2(f)[None]
    for sx, sy in itertools.product(range(-3, 4), repeat=2):
        s = np.array([[[sx, sy]]], np.float64)
        out = oracle.project2d(X, np.eye(2)[None, None], shifts=s, H=D, interp=1)[0, 0]
        exp = np.fft.rfft2(np.roll(f, (sy, sx), axis=(0, 1)))
        assert np.abs(out - exp).max() < 1e-9 * np.abs(exp).max(), (sx, sy)


def test_linear_reproduction_of_a_plane_wave_phase():
    """Both kernels reproduce linear functions of the coordinate: a source
    that is linear in (tx, ty) over the taps' reach is interpolated exactly at
    any sample, here checked on a source whose stored half-spectrum is a
    linear ramp away from the wrap and Friedel edges."""
    D = 32
    ty = np.fft.fftfreq(D, 1.0 / D)[:, None]
    tx = np.arange(D // 2 + 1)[None, :]
    X = (0.25 * tx + 0.5 * ty + 1.0 + 0.0j)[None]
    rng = np.random.default_rng(5)
    for interp in (0, 1):
        for _ in range(20):
            p = np.array([rng.uniform(4, 10), rng.uniform(-6, 6)])
            # a diagonal map with H = 1 pixel scaled to land at p: use o and R
            R = np.array([[p[0], 0.0], [0.0, p[1]]])
            out = oracle.project2d(X, R[None, None], H=4, interp=interp)[0, 0]
            # pixel (kx, ky) = (1, 1) samples p
            assert abs(out[1, 1] - (0.25 * p[0] + 0.5 * p[1] + 1.0)) < 1e-12, (interp, p)


CASES = [
    (1, 1, 1, 1, 12, 12, 1, 1.0, -1.0),
    (1, 1, 1, 1, 12, 12, 0, 1.0, 4.0),
    (2, 1, 2, 1, 10, 12, 1, 2.0, 5.0),
    (2, 2, 1, 2, 12, 10, 1, 1.0, -1.0),
    (3, 3, 3, 0, 8, 8, 0, 2.0, -1.0),
]


@pytest.mark.parametrize("B,Bv,Br,Bs,D,H,interp,o,r", CASES)
def test_adjoint_identity(B, Bv, Br, Bs, D, H, interp, o, r):
    rng = np.random.default_rng(B * 100 + D + 7)
    P = 3
    x = rng.standard_normal((Bv, D, D // 2 + 1)) + 1j * rng.standard_normal((Bv, D, D // 2 + 1))
    y = rng.standard_normal((B, P, H, H // 2 + 1)) + 1j * rng.standard_normal((B, P, H, H // 2 + 1))
    R = rng.standard_normal((Br, P, 2, 2))
    s = rng.uniform(-4, 4, (Bs, P, 2)) if Bs else None
    Px = oracle.project2d(x, R, shifts=s, H=H, interp=interp, o=o, r=r, B=B)
    PTy, _ = oracle.backproject2d(y, R, shifts=s, D=D, Bv=Bv, interp=interp, o=o, r=r)
    lhs, rhs = inner(Px, y), inner(x, PTy)
    assert abs(lhs - rhs) < 1e-11 * (abs(lhs) + np.linalg.norm(Px) * np.linalg.norm(y))
    u = rng.standard_normal((Bv, D, D // 2 + 1))
    w = rng.standard_normal((B, P, H, H // 2 + 1))
    _, PTw = oracle.backproject2d(y, R, weights=w, shifts=s, D=D, Bv=Bv, interp=interp, o=o, r=r)
    _, P0u, _, _ = oracle.backproject2d_backward(x, y, R, grad_weight=u, weights=w, shifts=s, interp=interp, o=o,
                                                 r=r, need_images=False, need_rot=False, need_shifts=False)
    lhs, rhs = float(np.sum(P0u * w)), float(np.sum(u * PTw))
    assert abs(lhs - rhs) < 1e-11 * (abs(lhs) + np.linalg.norm(P0u) * np.linalg.norm(w))


def _fd(fun, x, idx, h):
    xp = x.copy(); xp[idx] += h
    xm = x.copy(); xm[idx] -= h
    return (fun(xp) - fun(xm)) / (2 * abs(h))


@pytest.mark.parametrize("B,Bv,Br,Bs,o", [(1, 1, 1, 1, 1.0), (2, 1, 2, 1, 1.5), (2, 2, 1, 2, 1.0)])
def test_project2d_backward_finite_differences(B, Bv, Br, Bs, o):
    rng = np.random.default_rng(55 + B + Br)
    D = H = 12
    P, r = 2, 5.5
    X = np.fft.rfft2(rng.standard_normal((Bv, D, D))) + 0.3 * (rng.standard_normal((Bv, D, D // 2 + 1)) +
                                                                1j * rng.standard_normal((Bv, D, D // 2 + 1)))
    ang = rng.uniform(0, 2 * np.pi, (Br, P))
    R = np.stack([np.stack([np.cos(ang), -np.sin(ang)], -1), np.stack([np.sin(ang), np.cos(ang)], -1)], -2)
    R += 0.05 * rng.standard_normal(R.shape)        # all 4 entries are free
    s = rng.uniform(-3, 3, (Bs, P, 2))
    c = rng.standard_normal((B, P, H, H // 2 + 1)) + 1j * rng.standard_normal((B, P, H, H // 2 + 1))

    def L(X_, R_, s_):
        return inner(c, oracle.project2d(X_, R_, shifts=s_, H=H, interp=1, o=o, r=r, B=B))

    gX, gR, gs = oracle.project2d_backward(c, X, R, shifts=s, interp=1, o=o, r=r)
    h = 1e-6
    for idx in itertools.product(range(Br), range(P), range(2), range(2)):
        num = _fd(lambda x: L(X, x, s), R, idx, h)
        assert abs(num - gR[idx]) < 1e-6 * max(1.0, np.abs(gR).max()), idx
    for idx in itertools.product(range(Bs), range(P), range(2)):
        num = _fd(lambda x: L(X, R, x), s, idx, h)
        assert abs(num - gs[idx]) < 1e-6 * max(1.0, np.abs(gs).max()), idx
    for _ in range(12):
        idx = (rng.integers(Bv), rng.integers(D), rng.integers(D // 2 + 1))
        nre = _fd(lambda x: L(x, R, s), X, idx, 1e-3)
        nim = _fd(lambda x: L(x, R, s), X, idx, 1e-3j)
        assert abs(nre - gX[idx].real) < 1e-8 * max(1.0, np.abs(gX).max())
        assert abs(nim - gX[idx].imag) < 1e-8 * max(1.0, np.abs(gX).max())


def test_backproject2d_backward_finite_differences():
    rng = np.random.default_rng(93)
    D = H = 10
    B, P, r, o = 2, 2, 4.5, 1.0
    Y = rng.standard_normal((B, P, H, H // 2 + 1)) + 1j * rng.standard_normal((B, P, H, H // 2 + 1))
    Wt = rng.random((B, P, H, H // 2 + 1))
    R = rng.standard_normal((B, P, 2, 2))
    s = rng.uniform(-3, 3, (B, P, 2))
    Gd = rng.standard_normal((1, D, D // 2 + 1)) + 1j * rng.standard_normal((1, D, D // 2 + 1))
    Gw = rng.standard_normal((1, D, D // 2 + 1))

    def L(Y_, W_, R_, s_):
        dv, wv = oracle.backproject2d(Y_, R_, weights=W_, shifts=s_, D=D, Bv=1, interp=1, o=o, r=r)
        return inner(Gd, dv) + float(np.sum(Gw * wv))

    gY, gW, gR, gs = oracle.backproject2d_backward(Gd, Y, R, grad_weight=Gw, weights=Wt, shifts=s, interp=1, o=o, r=r)
    h = 1e-6
    for idx in itertools.product(range(B), range(P), range(2), range(2)):
        num = _fd(lambda x: L(Y, Wt, x, s), R, idx, h)
        assert abs(num - gR[idx]) < 1e-6 * max(1.0, np.abs(gR).max()), idx
    for idx in itertools.product(range(B), range(P), range(2)):
        num = _fd(lambda x: L(Y, Wt, R, x), s, idx, h)
        assert abs(num - gs[idx]) < 1e-6 * max(1.0, np.abs(gs).max()), idx
    for _ in range(10):
        idx = (rng.integers(B), rng.integers(P), rng.integers(H), rng.integers(H // 2 + 1))
        nre = _fd(lambda x: L(x, Wt, R, s), Y, idx, 1e-3)
        nim = _fd(lambda x: L(x, Wt, R, s), Y, idx, 1e-3j)
        nw = _fd(lambda x: L(Y, x, R, s), Wt, idx, 1e-3)
        assert abs(nre - gY[idx].real) < 1e-8 * max(1.0, np.abs(gY).max())
        assert abs(nim - gY[idx].imag) < 1e-8 * max(1.0, np.abs(gY).max())
        assert abs(nw - gW[idx]) < 1e-8 * max(1.0, np.abs(gW).max())


def test_oracle2d_rejects_bad_geometry():
    X = np.zeros((1, 8, 5), np.complex128)
    with pytest.raises(ValueError):
        oracle.project2d(X, np.zeros((1, 1, 2, 2)), H=7)
