"""Accuracy study of interpolation against oversampling (measurement only).

The pages compare cubic interpolation at 1x against linear interpolation of
a 2x zero-padded volume, by the Fourier ring correlation of the projections
with the truth and by the attenuation of real-space intensity away from the
centre (torch-projectors pages: Spanish "Resumen tecnico" 4, Dutch
Resultaten, French "Resume technique" 4).  Truth here is analytic: the
volume is a sum of isotropic Gaussians sampled over the whole box (no
window).  What an ideal interpolator (or padding without limit) returns at
a frequency xi (cycles per voxel) is the transform of those samples, which
by Poisson summation is the continuous transform summed over its aliases:

    T(xi) = sum_m sum_b a_b (2 pi s_b^2)^(3/2) exp(-2 pi^2 s_b^2 |xi + m|^2) exp(-2 pi i (xi + m) . c_b),

m over integer vectors, c_b the blob centre relative to the box centre,
xi = R (kx, ky, 0) / D.  The sum factors over the three axes; for widths
s_b >= 1 voxel and |xi| <= 1/2 the terms with |m_i| >= 2 are below 1e-19,
and with the blobs at least five widths inside the box the cut-off mass is
~1e-5 of the DC term, so every deviation measured is the interpolation's.
This module holds no step of the projection itself: the
projections come from the library's entry points.
"""
from __future__ import annotations

import numpy as np


def blob_model(rng, D: int, n_blobs: int, ball: float, smin: float = 1.0, smax: float = 1.5):
    """Centres (x, y, z offsets from the box centre) uniform in a ball of
    radius `ball` voxels, widths ~ U(smin, smax), amplitudes ~ U(0.5, 1)."""
    d = rng.standard_normal((n_blobs, 3))
    d /= np.linalg.norm(d, axis=1, keepdims=True)
    c = d * (ball * rng.random(n_blobs) ** (1.0 / 3.0))[:, None]
    return c, rng.uniform(smin, smax, n_blobs), rng.uniform(0.5, 1.0, n_blobs)


def real_volume(D: int, model) -> np.ndarray:
    """float32 [D, D, D] (z, y, x): the Gaussians evaluated at every voxel
    (separable outer products), centre at index D/2."""
    c, s, a = model
    u = np.arange(D, dtype=np.float64) - D // 2
    f = np.zeros((D, D, D))
    for (cx, cy, cz), sb, ab in zip(c, s, a):
        gx = np.exp(-(u - cx) ** 2 / (2 * sb * sb))
        gy = np.exp(-(u - cy) ** 2 / (2 * sb * sb))
        gz = np.exp(-(u - cz) ** 2 / (2 * sb * sb))
        f += ab * gz[:, None, None] * (gy[:, None] * gx[None, :])[None]
    return f.astype(np.float32)


def pixel_freqs(H: int):
    """(kx, ky) of every rfft2 pixel [H, H//2+1] (fftfreq rows, halved x)."""
    ky = np.fft.fftfreq(H, 1.0 / H)[:, None] * np.ones((1, H // 2 + 1))
    kx = np.arange(H // 2 + 1)[None, :] * np.ones((H, 1))
    return kx, ky


def analytic_slices(model, rot: np.ndarray, D: int, H: int, radius: float) -> np.ndarray:
    """complex128 [P, H, H//2+1]: T at the slice frequencies of the maps rot
    [P, 3, 3] (p = R (kx, ky, 0)), zero outside kx^2 + ky^2 <= radius^2."""
    c, s, a = model
    kx, ky = pixel_freqs(H)
    mask = kx ** 2 + ky ** 2 <= radius * radius
    out = np.zeros((rot.shape[0], H, H // 2 + 1), np.complex128)
    for n, R in enumerate(rot.astype(np.float64)):
        xi = (R[:, 0][:, None, None] * kx + R[:, 1][:, None, None] * ky) / D      # [3, H, W]
        acc = np.zeros((H, H // 2 + 1), np.complex128)
        for cb, sb, ab in zip(c, s, a):
            term = ab * (2 * np.pi * sb * sb) ** 1.5
            for i in range(3):                    # per axis: sum over its aliases m_i = -1, 0, 1
                f = 0
                for m in (-1.0, 0.0, 1.0):
                    x = xi[i] + m
                    f = f + np.exp(-2 * np.pi ** 2 * sb * sb * x * x - 2j * np.pi * x * cb[i])
                term = term * f
            acc += term
        out[n] = np.where(mask, acc, 0)
    return out


def frc(A: np.ndarray, B: np.ndarray, H: int, rings: int | None = None) -> np.ndarray:
    """Fourier ring correlation of the spectra A and B ([..., H, H//2+1],
    summed over the leading axes) per integer ring |k| = 0 .. H/2.  The kx = 0
    and kx = H/2 columns carry no mirrored half, so they count once and the
    others twice (the full spectrum's ring sums)."""
    kx, ky = pixel_freqs(H)
    ring = np.rint(np.sqrt(kx ** 2 + ky ** 2)).astype(int)
    mult = np.where((kx == 0) | (kx == H // 2), 1.0, 2.0)
    A = A.reshape(-1, H, H // 2 + 1).astype(np.complex128)
    B = B.reshape(-1, H, H // 2 + 1).astype(np.complex128)
    n = (rings or H // 2) + 1
    num = np.zeros(n)
    da = np.zeros(n)
    db = np.zeros(n)
    sel = ring < n
    for a, b in zip(A, B):
        np.add.at(num, ring[sel], (mult * (a * np.conj(b)).real)[sel])
        np.add.at(da, ring[sel], (mult * np.abs(a) ** 2)[sel])
        np.add.at(db, ring[sel], (mult * np.abs(b) ** 2)[sel])
    return num / np.sqrt(np.maximum(da * db, 1e-300))


def radial_gain(img: np.ndarray, ref: np.ndarray, edges) -> np.ndarray:
    """Least-squares gain sum(img ref) / sum(ref^2) of real images [..., H, H]
    in bands of real-space radius (fractions of H/2 about the centre H/2):
    1 means no attenuation."""
    H = img.shape[-1]
    u = np.arange(H) - H // 2
    r = np.sqrt(u[:, None] ** 2 + u[None, :] ** 2) / (H / 2)
    img = img.reshape(-1, H, H).astype(np.float64)
    ref = ref.reshape(-1, H, H).astype(np.float64)
    out = []
    for lo, hi in zip(edges[:-1], edges[1:]):
        m = (r >= lo) & (r < hi)
        out.append(float((img[:, m] * ref[:, m]).sum() / max((ref[:, m] ** 2).sum(), 1e-300)))
    return np.array(out)
