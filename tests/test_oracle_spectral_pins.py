"""Pins of the spectral steps of the oracle (oracle/spectral.py) to facts that
do not come from the oracle itself: exact transforms of deltas, the
continuous Fourier transform of a Gaussian (for sigma = 2.5 voxels the
aliasing of the sampled Gaussian is ~1e-13 and the part cut off by the box
~1e-8 of the DC term), the
exact subsampling relation of zero padding, a brute-force DFT round trip,
the shift convention of the projection ops, and exact recovery of a source
from noise-free, lattice-aligned, CTF-weighted projections."""
import itertools

import numpy as np
import pytest

import oracle as O
from oracle import spectral as S


def centred_delta(D, dz=0, dy=0, dx=0):
    v = np.zeros((D, D, D))
    v[D // 2 + dz, D // 2 + dy, D // 2 + dx] = 1.0
    return v


@pytest.mark.parametrize("pad", [1, 2, 3])
def test_delta_at_the_centre_has_a_flat_spectrum(pad):
    X = S.volume_rfft(centred_delta(8), pad)
    assert X.shape == (1, 8 * pad, 8 * pad, 4 * pad + 1)
    np.testing.assert_allclose(X, 1.0, atol=1e-14)


@pytest.mark.parametrize("pad", [1, 2])
@pytest.mark.parametrize("axis", [0, 1, 2])
def test_delta_off_centre_is_a_plane_wave_along_its_own_axis(pad, axis):
    """A delta one voxel past the centre along z, y or x gives exp(-2 pi i f / N)
    in that axis' frequency f (fftfreq order, x halved): the axis order
    (z, y, x) and the sign of the forward transform."""
    D = 8
    N = pad * D
    off = [0, 0, 0]
    off[axis] = 1
    X = S.volume_rfft(centred_delta(D, *off), pad)[0]
    fz = np.fft.fftfreq(N, 1.0 / N)[:, None, None]
    fy = np.fft.fftfreq(N, 1.0 / N)[None, :, None]
    fx = np.arange(N // 2 + 1)[None, None, :]
    f = (fz, fy, fx)[axis]
    np.testing.assert_allclose(X, np.broadcast_to(np.exp(-2j * np.pi * f / N), X.shape), atol=1e-13)


def test_gaussian_blob_matches_its_continuous_fourier_transform():
    """Off-centre Gaussian: a (2 pi s^2)^(3/2) exp(-2 pi^2 s^2 |k/N|^2) exp(-2 pi i k.c / N)."""
    D, pad, s, a = 32, 2, 2.5, 0.8
    c = np.array([1.5, -2.25, 0.75])                       # (x, y, z) offsets from the centre
    z, y, x = np.meshgrid(*(np.arange(D) - D // 2,) * 3, indexing="ij")
    v = a * np.exp(-((x - c[0]) ** 2 + (y - c[1]) ** 2 + (z - c[2]) ** 2) / (2 * s * s))
    X = S.volume_rfft(v, pad)[0]
    N = pad * D
    kz = np.fft.fftfreq(N, 1.0 / N)[:, None, None]
    ky = np.fft.fftfreq(N, 1.0 / N)[None, :, None]
    kx = np.arange(N // 2 + 1)[None, None, :]
    ref = a * (2 * np.pi * s * s) ** 1.5 * np.exp(-2 * np.pi ** 2 * s * s * (kx ** 2 + ky ** 2 + kz ** 2) / N ** 2) \
        * np.exp(-2j * np.pi * (kx * c[0] + ky * c[1] + kz * c[2]) / N)
    assert np.abs(X - ref).max() < 1e-7 * abs(ref[0, 0, 0])


def test_padding_samples_the_same_spectrum_twice_as_finely():
    """With the support inside the original box, the pad-2 spectrum at even
    indices is the pad-1 spectrum."""
    rng = np.random.default_rng(5)
    v = rng.standard_normal((2, 8, 8, 8))
    X1 = S.volume_rfft(v, 1)
    X2 = S.volume_rfft(v, 2)
    np.testing.assert_allclose(X2[:, ::2, ::2, ::2], X1, atol=1e-12)
    assert not np.allclose(X2[:, 1::2, ::2, ::2], 0)


def brute_rfft2(img):
    """rfft2 of a real H x H image by direct summation (no FFT library)."""
    H = img.shape[0]
    n = np.arange(H)
    out = np.zeros((H, H // 2 + 1), complex)
    for ky in range(H):
        for kx in range(H // 2 + 1):
            out[ky, kx] = np.sum(img * np.exp(-2j * np.pi * (ky * n[:, None] + kx * n[None, :]) / H))
    return out


def test_images_irfft_inverts_a_brute_force_transform_of_a_centred_image():
    rng = np.random.default_rng(6)
    H = 6
    img = rng.standard_normal((H, H))
    spec = brute_rfft2(np.fft.ifftshift(img))              # centre H/2 moved to index 0
    np.testing.assert_allclose(S.images_irfft(spec), img, atol=1e-12)


@pytest.mark.parametrize("sx,sy", [(0, 0), (1, 0), (0, 1), (2, -3)])
def test_shift_phase_of_the_projection_moves_a_centred_delta_by_the_shift(sx, sy):
    """The projection ops' shift phase exp(-2 pi i (kx sx + ky sy) / H),
    applied to a flat spectrum, comes back as a delta at (H/2 + sy, H/2 + sx):
    a positive shift moves content to larger indices."""
    H = 8
    src = np.ones((1, H, H // 2 + 1), complex)                # flat source: delta at the centre
    rot = np.eye(2)[None, None]
    Y = O.project2d(src, rot, shifts=np.array([[[sx, sy]]], float), interp=0)
    img = S.images_irfft(Y[0, 0])
    ref = np.zeros((H, H))
    ref[H // 2 + sy, H // 2 + sx] = 1.0
    np.testing.assert_allclose(img, ref, atol=1e-12)


def test_weight_images_and_finishing_by_hand():
    img = np.array([[1 + 2j, -3j], [0.5, 4 - 1j]])
    w = np.array([2.0, -0.5])
    np.testing.assert_array_equal(S.weight_images(img, w), [[2 + 4j, 1.5j], [1.0, -2 + 0.5j]])
    d = np.array([2 + 2j, 1j, 3.0, -1.0])
    ws = np.array([1.0, 0.0, -0.5, 3.0])
    np.testing.assert_array_equal(S.finish_reconstruction(d, ws), [2 + 2j, 0, 0, -1 / 3])
    np.testing.assert_array_equal(S.finish_reconstruction(d, ws, 1.0), [1 + 1j, 1j, 6.0, -0.25])


def signed_permutations_2d():
    out = []
    for perm in itertools.permutations(range(2)):
        for sg in itertools.product((1, -1), repeat=2):
            R = np.zeros((2, 2))
            for i in range(2):
                R[i, perm[i]] = sg[i]
            out.append(R)
    return np.array(out)


@pytest.mark.parametrize("interp", [0, 1])
def test_finishing_recovers_the_source_from_ctf_weighted_lattice_projections(interp):
    """Observations w * P_n(S) for the eight lattice rotations; accumulating
    w * observation with weights w^2 and dividing gives S back exactly (every
    stored entry is hit; at lattice points both kernels take the entry itself)."""
    rng = np.random.default_rng(7)
    D = 12
    src = (rng.standard_normal((1, D, D // 2 + 1)) + 1j * rng.standard_normal((1, D, D // 2 + 1)))
    rot = signed_permutations_2d()[None]
    w = rng.uniform(0.2, 1.0, (1, 8, D, D // 2 + 1))
    obs = S.weight_images(O.project2d(src, rot, interp=interp), w)
    data, wsum = O.backproject2d(S.weight_images(obs, w), rot, weights=w * w, D=D, interp=interp)
    assert wsum.min() > 0
    np.testing.assert_allclose(S.finish_reconstruction(data, wsum), src, atol=1e-12)
    # a plain division without the CTF weights would not recover the source
    data0, cnt = O.backproject2d(obs, rot, weights=np.ones_like(w), D=D, interp=interp)
    assert np.abs(S.finish_reconstruction(data0, cnt) - src).max() > 1e-3
