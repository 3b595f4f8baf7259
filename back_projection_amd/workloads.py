"""Seeded synthetic inputs for the Fourier-slice projection workloads.

This module only makes inputs: Gaussian-blob volumes and their rfft, uniform
random rotations from normalised Gaussian quaternions, uniform shifts,
Gaussian upstream gradients, noisy analytic blob projections and CTF^2-like
weight images.  It holds none of the projector's own arithmetic (no slicing,
interpolation, phase or accumulation), so both the GPU path and the CPU
oracle can be fed from it.

The five workloads follow the cryo-EM setting of the torch-projectors pages
(rfft volumes and images in PyTorch/FFTW layout, DC at index 0; Spanish page,
"Resumen tecnico" section 2).  Everything is float32 / complex64, generated on
the CPU from ``numpy.random.default_rng(seed)``.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

# ---------------------------------------------------------------------------
# primitives
# ---------------------------------------------------------------------------


def blob_params(rng, n_blobs: int, ball_radius: float):
    """Centres uniform in a ball (offsets from the box centre), sigma ~ U(1,3)
    voxels, peak amplitude ~ U(0.5, 1)."""
    d = rng.standard_normal((n_blobs, 3))
    d /= np.linalg.norm(d, axis=1, keepdims=True)
    rad = ball_radius * rng.random(n_blobs) ** (1.0 / 3.0)
    centres = d * rad[:, None]                     # (x, y, z) offsets
    sigma = rng.uniform(1.0, 3.0, n_blobs)
    amp = rng.uniform(0.5, 1.0, n_blobs)
    return centres, sigma, amp


def blob_volume_real(D: int, centres, sigma, amp) -> np.ndarray:
    """Real float32 [D, D, D] (z, y, x) sum of isotropic Gaussians about the box
    centre D/2, each evaluated in a 4-sigma window (separable product)."""
    f = np.zeros((D, D, D), np.float32)
    c0 = D // 2
    for (cx, cy, cz), s, a in zip(centres, sigma, amp):
        h = int(np.ceil(4 * s))
        px, py, pz = c0 + cx, c0 + cy, c0 + cz
        xs = np.arange(int(np.floor(px)) - h, int(np.floor(px)) + h + 2)
        ys = np.arange(int(np.floor(py)) - h, int(np.floor(py)) + h + 2)
        zs = np.arange(int(np.floor(pz)) - h, int(np.floor(pz)) + h + 2)
        gx = np.exp(-(xs - px) ** 2 / (2 * s * s))
        gy = np.exp(-(ys - py) ** 2 / (2 * s * s))
        gz = np.exp(-(zs - pz) ** 2 / (2 * s * s))
        blk = (a * gz[:, None, None] * gy[None, :, None] * gx[None, None, :]).astype(np.float32)
        f[np.ix_(zs % D, ys % D, xs % D)] += blk
    return f


def rfft_volume(f: np.ndarray) -> np.ndarray:
    """ifftshift (box centre -> index 0) then rfftn over (z, y, x); complex64
    [D, D, D//2+1] with DC at index 0."""
    t = torch.from_numpy(np.fft.ifftshift(f).copy())
    return torch.fft.rfftn(t).numpy().astype(np.complex64)


def random_rotations(rng, n: int) -> np.ndarray:
    """Uniform rotations on SO(3): normalised Gaussian quaternions -> matrices,
    float32 [n, 3, 3]."""
    q = rng.standard_normal((n, 4))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    w, x, y, z = q.T
    R = np.empty((n, 3, 3))
    R[:, 0, 0] = 1 - 2 * (y * y + z * z)
    R[:, 0, 1] = 2 * (x * y - z * w)
    R[:, 0, 2] = 2 * (x * z + y * w)
    R[:, 1, 0] = 2 * (x * y + z * w)
    R[:, 1, 1] = 1 - 2 * (x * x + z * z)
    R[:, 1, 2] = 2 * (y * z - x * w)
    R[:, 2, 0] = 2 * (x * z - y * w)
    R[:, 2, 1] = 2 * (y * z + x * w)
    R[:, 2, 2] = 1 - 2 * (x * x + y * y)
    return R.astype(np.float32)


def random_shifts(rng, n: int, amax: float) -> np.ndarray:
    return rng.uniform(-amax, amax, (n, 2)).astype(np.float32)


def random_complex(rng, shape) -> np.ndarray:
    """Complex64 with Re and Im iid N(0, 1)."""
    re = rng.standard_normal(shape, dtype=np.float32)
    im = rng.standard_normal(shape, dtype=np.float32)
    return (re + 1j * im).astype(np.complex64)


def noisy_blob_projections(rng, H: int, centres, sigma, amp, rots: np.ndarray, snr: float = 0.1,
                           batch: int = 64, device=None) -> np.ndarray:
    """rfft2 of noisy analytic projections of a blob volume: each rotation maps
    the blob centre c to (R^T c)_xy on the image, the z-integral of a Gaussian
    of width sigma and peak a is a 2D Gaussian of peak a*sqrt(2 pi)*sigma.
    Gaussian noise (numpy-seeded) with variance var(clean)/snr per image.
    The dense Gaussian sums run with torch on ``device`` (a GPU when present:
    they are input preparation only).  complex64 [n, H, H//2+1]."""
    if device is None:
        device = "cuda" if torch.cuda.is_available() else "cpu"
    n = rots.shape[0]
    out = np.empty((n, H, H // 2 + 1), np.complex64)
    c = torch.from_numpy(centres.astype(np.float32)).to(device)
    s = torch.from_numpy(sigma.astype(np.float32)).to(device)
    a2 = torch.from_numpy((amp * np.sqrt(2 * np.pi) * sigma).astype(np.float32)).to(device)
    grid = torch.arange(H, dtype=torch.float32, device=device) - H // 2
    inv2s2 = 1.0 / (2 * s * s)
    for i0 in range(0, n, batch):
        R = torch.from_numpy(rots[i0:i0 + batch]).to(device)   # [b, 3, 3]
        cp = torch.einsum("bji,nj->bni", R, c)                  # R^T c  -> [b, nb, 3]
        gx = torch.exp(-torch.square(grid[None, :, None] - cp[:, None, :, 0]) * inv2s2)   # [b, H, nb]
        gy = torch.exp(-torch.square(grid[None, :, None] - cp[:, None, :, 1]) * inv2s2)
        img = torch.bmm((gy * a2).contiguous(), gx.transpose(1, 2).contiguous())       # [b, H(y), H(x)]
        var = img.var(dim=(1, 2), keepdim=True)
        noise = torch.from_numpy(rng.standard_normal(tuple(img.shape), dtype=np.float32)).to(device)
        img = img + noise * torch.sqrt(var / snr)
        img = torch.fft.ifftshift(img, dim=(1, 2))
        out[i0:i0 + batch] = torch.fft.rfft2(img).cpu().numpy()
    return out


def ctf2_like_weights(rng, n: int, H: int, n_keep: int | None = None) -> np.ndarray:
    """Real weights in [0, 1]: sin^2(pi c rho^2 + 0.07) exp(-b rho^2) with
    rho = |k| / (H/2), c ~ U(5, 20), b ~ U(0, 2) per image; float32
    [n_keep, H, H//2+1] (the first n_keep of n images)."""
    kx = np.arange(H // 2 + 1, dtype=np.float32)
    ky = np.fft.fftfreq(H, 1.0 / H).astype(np.float32)
    rho2 = (kx[None, :] ** 2 + ky[:, None] ** 2) / (H / 2) ** 2
    n_keep = n if n_keep is None else n_keep
    c = rng.uniform(5, 20, n).astype(np.float32)[:n_keep]
    b = rng.uniform(0, 2, n).astype(np.float32)[:n_keep]
    return (np.sin(np.pi * c[:, None, None] * rho2[None] + 0.07) ** 2 * np.exp(-b[:, None, None] * rho2[None])).astype(
        np.float32)


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------


@dataclass
class Workload:
    """One synthetic workload.  Array shapes follow the library's layout:
    vol [Bv, D, D, D//2+1] c64, rot [Br, P, 3, 3] f32, shifts [Bs, P, 2] f32 or
    None, grad_out [B, P, H, H//2+1] c64 or None, images/weights for the
    back-projection workload."""
    name: str
    D: int
    H: int
    B: int
    P: int
    interp: int
    radius: float
    ops: tuple
    vol: np.ndarray | None = None
    rot: np.ndarray | None = None
    shifts: np.ndarray | None = None
    grad_out: np.ndarray | None = None
    images: np.ndarray | None = None
    weights: np.ndarray | None = None
    oversampling: float = 1.0
    notes: dict = field(default_factory=dict)


NAMES = {
    1: "D32 linear forward, 64 poses, r=16",
    2: "D64 cubic forward+backward (volume, rotation grads), 1024 poses, shifts U(-3,3)",
    3: "D128 cubic forward+backward (volume, rotation, shift grads), 16384 poses, shifts U(-5,5), r=64",
    4: "D256 cubic back-projection with weights, 4096 images",
    5: "4 x D192 cubic forward+backward (volume, rotation, shift grads), 8192 poses each, shifts U(-8,8), r=96",
}


def make(cfg: int, P: int | None = None, with_grad: bool = True) -> Workload:
    """Build workload ``cfg`` (1..5).  ``P`` truncates the pose count (the same
    seed gives the same leading poses)."""
    seed = 1000 + cfg
    rng = np.random.default_rng(seed)
    if cfg == 1:
        D, nb, ball, Pf, interp, r, amax = 32, 50, 10.0, 64, 0, 16.0, None
        ops = ("forward",)
    elif cfg == 2:
        D, nb, ball, Pf, interp, r, amax = 64, 200, 64 / 3, 1024, 1, -1.0, 3.0
        ops = ("forward", "backward_vol", "backward_rot")
    elif cfg == 3:
        D, nb, ball, Pf, interp, r, amax = 128, 800, 128 / 3, 16384, 1, 64.0, 5.0
        ops = ("forward", "backward_vol", "backward_rot", "backward_shifts")
    elif cfg == 4:
        D, nb, ball, Pf, interp, r, amax = 256, 3200, 256 / 3, 4096, 1, -1.0, None
        ops = ("backproject",)
    elif cfg == 5:
        D, nb, ball, Pf, interp, r, amax = 192, 1800, 192 / 3, 8192, 1, 96.0, 8.0
        ops = ("forward", "backward_vol", "backward_rot", "backward_shifts")
    else:
        raise ValueError(cfg)
    P = Pf if P is None else P
    B = 4 if cfg == 5 else 1
    w = Workload(NAMES[cfg], D, D, B, P, interp, r, ops)
    if cfg == 4:
        centres, sigma, amp = blob_params(rng, nb, ball)
        rot = random_rotations(rng, Pf)[:P]
        w.rot = rot[None]
        w.images = noisy_blob_projections(np.random.default_rng(seed + 7), D, centres, sigma, amp, rot)[None]
        w.weights = ctf2_like_weights(np.random.default_rng(seed + 11), Pf, D, P)[None]
        return w
    vols, rots, shifts = [], [], []
    for b in range(B):
        sub = rng if B == 1 else np.random.default_rng(seed * 10 + b)
        centres, sigma, amp = blob_params(sub, nb, ball)
        vols.append(rfft_volume(blob_volume_real(D, centres, sigma, amp)))
        rots.append(random_rotations(sub, Pf)[:P])
        if amax is not None:
            shifts.append(random_shifts(sub, Pf, amax)[:P])
    w.vol = np.stack(vols)
    w.rot = np.stack(rots)
    w.shifts = np.stack(shifts) if shifts else None
    if with_grad and any(op.startswith("backward") for op in ops):
        w.grad_out = upstream_grads(seed + 99, B, P, D)
    return w


def upstream_grads(seed: int, B: int, P: int, H: int, block: int = 256) -> np.ndarray:
    """Complex64 [B, P, H, H//2+1], Re and Im iid N(0,1), drawn in blocks of
    poses with their own seeds so that a truncated P gives the leading rows of
    the full array."""
    out = np.empty((B, P, H, H // 2 + 1), np.complex64)
    for b in range(B):
        for j0 in range(0, P, block):
            g = np.random.default_rng([seed, b, j0 // block])
            blk = random_complex(g, (block, H, H // 2 + 1))
            out[b, j0:j0 + block] = blk[:min(block, P - j0)]
    return out


# ---------------------------------------------------------------------------
# 2D -> 2D workload (the 2D analogue of workload 3)
# ---------------------------------------------------------------------------
NAME_2D = ("2D D128 cubic forward+backward (source, rotation, shift grads) and accumulation with weights, "
           "16384 poses, shifts U(-5,5), r=64")


def random_rotations_2d(rng, n: int) -> np.ndarray:
    """float32 [n, 2, 2] rotations by angles uniform in [0, 2 pi)."""
    a = rng.uniform(0.0, 2.0 * np.pi, n)
    c, s = np.cos(a), np.sin(a)
    return np.stack([np.stack([c, -s], -1), np.stack([s, c], -1)], -2).astype(np.float32)


def blob_image_rfft(rng, D: int, n_blobs: int, radius: float) -> np.ndarray:
    """rfft2 (after ifftshift) of a real D x D image of isotropic 2D Gaussians,
    centres uniform in a disc about the box centre, sigma ~ U(1,3), amplitude
    ~ U(0.5,1); complex64 [D, D//2+1], DC at index 0."""
    f = np.zeros((D, D), np.float32)
    ang = rng.uniform(0, 2 * np.pi, n_blobs)
    rad = radius * np.sqrt(rng.random(n_blobs))
    sig = rng.uniform(1.0, 3.0, n_blobs)
    amp = rng.uniform(0.5, 1.0, n_blobs)
    y, x = np.meshgrid(np.arange(D), np.arange(D), indexing="ij")
    for a, r, s_, m in zip(ang, rad, sig, amp):
        cx, cy = D // 2 + r * np.cos(a), D // 2 + r * np.sin(a)
        f += (m * np.exp(-((x - cx) ** 2 + (y - cy) ** 2) / (2 * s_ * s_))).astype(np.float32)
    return np.fft.rfft2(np.fft.ifftshift(f)).astype(np.complex64)


def make_2d(P: int = 16384, D: int = 128) -> dict:
    """Seeded 2D workload: source, rotations, shifts, upstream gradients,
    images and CTF^2-like weights for the accumulation."""
    rng = np.random.default_rng(2002)
    src = blob_image_rfft(rng, D, 200, D / 3)[None]
    rot = random_rotations_2d(rng, P)[None]
    shifts = random_shifts(rng, P, 5.0)[None]
    grad_out = upstream_grads(2101, 1, P, D)
    weights = ctf2_like_weights(np.random.default_rng(2111), P, D, P)[None]
    return dict(name=NAME_2D, D=D, H=D, P=P, radius=64.0, src=src, rot=rot, shifts=shifts, grad_out=grad_out,
                weights=weights)
