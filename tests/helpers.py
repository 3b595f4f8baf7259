"""Shared helpers for the parity tests (no method arithmetic here)."""
import numpy as np
import torch


def rel(a, b):
    a = a.detach().cpu().numpy() if isinstance(a, torch.Tensor) else np.asarray(a)
    b = b.detach().cpu().numpy() if isinstance(b, torch.Tensor) else np.asarray(b)
    den = np.linalg.norm(b.ravel().astype(np.complex128))
    num = np.linalg.norm((a.astype(np.complex128) - b.astype(np.complex128)).ravel())
    return float(num / den) if den > 0 else float(num)


def dev(*arrays, device="cuda:0"):
    return [None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(device) for a in arrays]


def host(t):
    return None if t is None else t.detach().cpu().numpy()


def log(msg):
    print(msg, flush=True)


def volume_kmag(D):
    """|k| of every stored entry of an rfft volume [D, D, D//2+1] (x halved,
    z and y in fftfreq order)."""
    f = np.fft.fftfreq(D, 1.0 / D)
    kz, ky, kx = np.meshgrid(f, f, np.arange(D // 2 + 1), indexing="ij")
    return np.sqrt(kx * kx + ky * ky + kz * kz)


def image_kmag(H):
    """|k| of every pixel of an rfft image [H, H//2+1]."""
    ky, kx = np.meshgrid(np.fft.fftfreq(H, 1.0 / H), np.arange(H // 2 + 1), indexing="ij")
    return np.sqrt(kx * kx + ky * ky)


def shell_rels(a, b, kmag, nshells=8):
    """Relative L2 error of a against b in each of `nshells` equal-width
    radial shells of |k| (the trailing dims of a and b are those of kmag),
    over the range where b is nonzero.  Returns [(k_lo, k_hi, rel)], shells
    with no nonzero reference skipped.  A global relative L2 is dominated by
    the large low-frequency entries; this checks the small outer ones too."""
    a = a.detach().cpu().numpy() if isinstance(a, torch.Tensor) else np.asarray(a)
    b = np.asarray(b)
    a = a.reshape((-1,) + kmag.shape)
    b = b.reshape((-1,) + kmag.shape)
    nz = np.any(b != 0, axis=0)
    kmax = float(kmag[nz].max()) if nz.any() else 0.0
    edges = np.linspace(0.0, kmax, nshells + 1)
    edges[-1] = np.nextafter(kmax, np.inf)
    out = []
    for lo, hi in zip(edges[:-1], edges[1:]):
        m = (kmag >= lo) & (kmag < hi)
        bs = b[:, m].astype(np.complex128)
        den = np.linalg.norm(bs.ravel())
        if den == 0:
            continue
        num = np.linalg.norm((a[:, m].astype(np.complex128) - bs).ravel())
        out.append((float(lo), float(hi), float(num / den)))
    return out
