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
