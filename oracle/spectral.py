"""Steps either side of the Fourier-slice path, in plain fp64 numpy -- TEST
INFRASTRUCTURE ONLY (the test suite, the smoke check and the benchmark's
CPU-baseline leg may use it; the GPU library never does).

Each function is the definition written out, with numpy's FFT as the one
library step:

* ``volume_rfft``: the real-space front end of a volume.  The pages keep
  every Fourier array in the PyTorch rfft layout (DC at index 0, last axis
  halved: Spanish "Resumen tecnico" 2, French "Resume technique" 2) and
  compare cubic interpolation against oversampling by zero padding in real
  space (Spanish page 4, Dutch Resultaten, French page 4).  The volume is
  placed centred in a box of N = pad * D, its centre N/2 moved to index 0,
  and transformed with rfftn.
* ``images_irfft``: the real-space back end of projections: irfft2 (1/H^2
  normalised) and the centre back at H/2.
* ``weight_images``: the per-image weight (CTF) multiply of the weight
  channel's use for CTF correction (French page 2).
* ``finish_reconstruction``: an accumulated data volume divided by its
  accumulated weights plus a constant regulariser, zero where that sum is
  not positive (the reading taken for the finishing step, which the pages
  name only through CTF correction).
"""
from __future__ import annotations

import numpy as np


def volume_rfft(vol, pad: int = 1) -> np.ndarray:
    """vol [Bv, D, D, D] (z, y, x) real, centre at index D/2 ->
    complex128 [Bv, N, N, N//2+1], N = pad * D."""
    v = np.asarray(vol, dtype=np.float64)
    if v.ndim == 3:
        v = v[None]
    D = v.shape[-1]
    N = pad * D
    off = (N - D) // 2
    g = np.zeros((v.shape[0], N, N, N))
    g[:, off:off + D, off:off + D, off:off + D] = v
    h = np.fft.ifftshift(g, axes=(1, 2, 3))
    return np.fft.rfftn(h, axes=(1, 2, 3))


def images_irfft(images) -> np.ndarray:
    """spectra [..., H, H//2+1] -> real [..., H, H], index 0 at the centre."""
    x = np.asarray(images, dtype=np.complex128)
    H = x.shape[-2]
    r = np.fft.irfft2(x, s=(H, H), axes=(-2, -1))
    return np.fft.fftshift(r, axes=(-2, -1))


def weight_images(images, weights) -> np.ndarray:
    """images * weights, weights matching the trailing dims of images."""
    return np.asarray(images, dtype=np.complex128) * np.asarray(weights, dtype=np.float64)


def finish_reconstruction(data, weights, lam: float = 0.0) -> np.ndarray:
    """data / (weights + lam) where weights + lam > 0, else 0."""
    d = np.asarray(data, dtype=np.complex128)
    w = np.asarray(weights, dtype=np.float64) + float(lam)
    out = np.zeros_like(d)
    pos = w > 0
    out[pos] = d[pos] / w[pos]
    return out
