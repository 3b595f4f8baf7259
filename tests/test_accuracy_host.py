"""Host checks of the accuracy-study helpers (back_projection_amd.accuracy):
the analytic slice agrees with the DFT of the sampled model (oracle front
end, identity map, lattice frequencies), the FRC of a spectrum with itself
is 1 and with its negative -1, and the radial gain of a scaled image is the
scale."""
import numpy as np

from back_projection_amd import accuracy as acc
from oracle import spectral as S


def test_analytic_slice_matches_the_dft_of_the_sampled_model():
    D = 48
    rng = np.random.default_rng(11)
    model = acc.blob_model(rng, D, 12, 14.0)         # >= 6.6 widths inside the box
    vol = acc.real_volume(D, model).astype(np.float64)
    X = S.volume_rfft(vol, 1)[0]                      # [z, y, x]
    ref = acc.analytic_slices(model, np.eye(3)[None], D, D, D / 2)[0]
    kx, ky = acc.pixel_freqs(D)
    mask = kx ** 2 + ky ** 2 <= (D / 2) ** 2
    got = np.where(mask, X[0], 0)                     # kz = 0 plane
    assert np.abs(got - ref).max() < 1e-6 * abs(ref[0, 0])


def test_frc_and_gain_basics():
    rng = np.random.default_rng(12)
    H = 16
    A = rng.standard_normal((3, H, H // 2 + 1)) + 1j * rng.standard_normal((3, H, H // 2 + 1))
    np.testing.assert_allclose(acc.frc(A, A, H), 1.0, atol=1e-12)
    np.testing.assert_allclose(acc.frc(A, -A, H), -1.0, atol=1e-12)
    img = rng.standard_normal((2, H, H))
    np.testing.assert_allclose(acc.radial_gain(0.5 * img, img, (0.0, 0.5, 1.0)), 0.5, atol=1e-12)
