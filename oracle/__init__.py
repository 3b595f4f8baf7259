"""Fourier-slice projection oracle -- TEST INFRASTRUCTURE ONLY.

Python binding (ctypes + numpy) of the plain fp64 C oracle in ``oracle.c``.
Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package; the GPU library never does, and the two share no code.

Array conventions (all numpy, C-contiguous; inputs are cast to fp64 exactly):
  vol     complex [Bv, D, D, D//2+1]   rfft volume, x (last axis) halved
  rot     real    [Br, P, 3, 3]        rows/cols ordered (x, y, z)
  shifts  real    [Bs, P, 2]           (sx, sy) in pixels, or None
  images  complex [B, P, H, H//2+1]    rfft images
  weights real    [B, P, H, H//2+1]    or None
The 2D -> 2D ops (``project2d`` ...) take a 2D rfft source [Bv, D, D//2+1]
(complex; real for the weight channel) and 2x2 maps rot [Br, P, 2, 2].
Each of Bv, Br, Bs is 1 or B.  ``interp`` is 0 (linear) or 1 (cubic),
``o`` the oversampling factor and ``r`` the radius cutoff (< 0: none).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_D = ctypes.c_double
_I = ctypes.c_int
_P = ctypes.c_void_p


def build(verbose: bool = False) -> str:
    """Compile oracle.c into liboracle.so (gcc, OpenMP)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", _LIB_PATH,
           os.path.join(_HERE, "oracle.c"), "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        geom = [_I] * 8 + [_D, _D]
        lib.oracle_project.argtypes = geom + [_P] * 4
        lib.oracle_backproject.argtypes = geom + [_P] * 6
        lib.oracle_project_backward.argtypes = geom + [_P] * 7
        lib.oracle_backproject_backward.argtypes = geom + [_P] * 10
        lib.oracle_project2d.argtypes = geom + [_P] * 4
        lib.oracle_backproject2d.argtypes = geom + [_P] * 6
        lib.oracle_project2d_backward.argtypes = geom + [_P] * 7
        lib.oracle_backproject2d_backward.argtypes = geom + [_P] * 10
        for f in ("oracle_project", "oracle_backproject", "oracle_project_backward",
                  "oracle_backproject_backward", "oracle_project2d", "oracle_backproject2d",
                  "oracle_project2d_backward", "oracle_backproject2d_backward"):
            getattr(lib, f).restype = _I
        lib.oracle_kernel_weight.argtypes = [_I, _D]
        lib.oracle_kernel_weight.restype = _D
        lib.oracle_kernel_dweight.argtypes = [_I, _D]
        lib.oracle_kernel_dweight.restype = _D
        lib.oracle_num_threads.restype = _I
        lib.oracle_set_num_threads.argtypes = [_I]
        lib.oracle_set_num_threads.restype = _I
        _lib = lib
    return _lib


def _c(a, dtype):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a), dtype=dtype)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_P)


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"oracle {name} rejected its arguments (code {rc})")


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> int:
    """OpenMP threads of later calls (returns the count now in effect)."""
    return int(_load().oracle_set_num_threads(int(n)))


def kernel_weight(interp: int, d: float) -> float:
    return float(_load().oracle_kernel_weight(int(interp), float(d)))


def kernel_dweight(interp: int, d: float) -> float:
    return float(_load().oracle_kernel_dweight(int(interp), float(d)))


def _batch(*bs):
    bs = [b for b in bs if b is not None]
    B = max(bs)
    for b in bs:
        if b not in (1, B):
            raise ValueError(f"batch sizes {bs} are not 1 or a common B")
    return B


def project(vol, rot, shifts=None, H=None, interp=1, o=1.0, r=-1.0, B=None):
    """3D -> 2D forward: out[b, n] = M * phi * I(vol[bv], o R (kx, ky, 0))."""
    vol = _c(vol, np.complex128)
    rot = _c(rot, np.float64)
    shifts = _c(shifts, np.float64)
    Bv, D = vol.shape[0], vol.shape[1]
    Br, P = rot.shape[0], rot.shape[1]
    Bs = shifts.shape[0] if shifts is not None else 0
    B = B or _batch(Bv, Br, Bs if shifts is not None else None)
    H = H or D
    out = np.empty((B, P, H, H // 2 + 1), np.complex128)
    rc = _load().oracle_project(B, P, Bv, Br, Bs, D, H, interp, o, r, _ptr(vol), _ptr(rot), _ptr(shifts), _ptr(out))
    _check(rc, "project")
    return out


def backproject(images, rot, weights=None, shifts=None, D=None, Bv=1, interp=1, o=1.0, r=-1.0):
    """2D -> 3D back-projection (adjoint of project); returns (data_vol, weight_vol or None)."""
    images = _c(images, np.complex128)
    rot = _c(rot, np.float64)
    weights = _c(weights, np.float64)
    shifts = _c(shifts, np.float64)
    B, P, H = images.shape[0], images.shape[1], images.shape[2]
    Br = rot.shape[0]
    Bs = shifts.shape[0] if shifts is not None else 0
    D = D or H
    data = np.empty((Bv, D, D, D // 2 + 1), np.complex128)
    wvol = np.empty((Bv, D, D, D // 2 + 1), np.float64) if weights is not None else None
    rc = _load().oracle_backproject(B, P, Bv, Br, Bs, D, H, interp, o, r, _ptr(images), _ptr(weights), _ptr(rot),
                                    _ptr(shifts), _ptr(data), _ptr(wvol))
    _check(rc, "backproject")
    return data, wvol


def project_backward(grad_out, vol, rot, shifts=None, interp=1, o=1.0, r=-1.0,
                     need_vol=True, need_rot=True, need_shifts=True):
    """Backward of project; returns (grad_vol, grad_rot, grad_shifts) (None where not requested)."""
    grad_out = _c(grad_out, np.complex128)
    vol = _c(vol, np.complex128)
    rot = _c(rot, np.float64)
    shifts = _c(shifts, np.float64)
    B, P, H = grad_out.shape[0], grad_out.shape[1], grad_out.shape[2]
    Bv, D = vol.shape[0], vol.shape[1]
    Br = rot.shape[0]
    Bs = shifts.shape[0] if shifts is not None else 0
    gv = np.empty((Bv, D, D, D // 2 + 1), np.complex128) if need_vol else None
    gr = np.empty((Br, P, 3, 3), np.float64) if need_rot else None
    gs = np.empty((Bs, P, 2), np.float64) if (need_shifts and shifts is not None) else None
    rc = _load().oracle_project_backward(B, P, Bv, Br, Bs, D, H, interp, o, r, _ptr(grad_out), _ptr(vol), _ptr(rot),
                                         _ptr(shifts), _ptr(gv), _ptr(gr), _ptr(gs))
    _check(rc, "project_backward")
    return gv, gr, gs


def backproject_backward(grad_data_vol, images, rot, grad_weight_vol=None, weights=None, shifts=None,
                         interp=1, o=1.0, r=-1.0, need_images=True, need_weights=True, need_rot=True,
                         need_shifts=True):
    """Backward of backproject; returns (grad_images, grad_weights, grad_rot, grad_shifts)."""
    gdv = _c(grad_data_vol, np.complex128)
    gwv = _c(grad_weight_vol, np.float64)
    images = _c(images, np.complex128)
    weights = _c(weights, np.float64)
    rot = _c(rot, np.float64)
    shifts = _c(shifts, np.float64)
    B, P, H = images.shape[0], images.shape[1], images.shape[2]
    Bv, D = gdv.shape[0], gdv.shape[1]
    Br = rot.shape[0]
    Bs = shifts.shape[0] if shifts is not None else 0
    gi = np.empty((B, P, H, H // 2 + 1), np.complex128) if need_images else None
    gw = np.empty((B, P, H, H // 2 + 1), np.float64) if (need_weights and gwv is not None) else None
    gr = np.empty((Br, P, 3, 3), np.float64) if need_rot else None
    gs = np.empty((Bs, P, 2), np.float64) if (need_shifts and shifts is not None) else None
    rc = _load().oracle_backproject_backward(B, P, Bv, Br, Bs, D, H, interp, o, r, _ptr(gdv), _ptr(gwv), _ptr(images),
                                             _ptr(weights), _ptr(rot), _ptr(shifts), _ptr(gi), _ptr(gw), _ptr(gr),
                                             _ptr(gs))
    _check(rc, "backproject_backward")
    return gi, gw, gr, gs


# ---------------------------------------------------------------------------
# 2D -> 2D
# ---------------------------------------------------------------------------
def project2d(src, rot, shifts=None, H=None, interp=1, o=1.0, r=-1.0, B=None):
    """2D -> 2D forward: out[b, n] = M * phi * I(src[bv], o R (kx, ky))."""
    src = _c(src, np.complex128)
    rot = _c(rot, np.float64)
    shifts = _c(shifts, np.float64)
    Bv, D = src.shape[0], src.shape[1]
    Br, P = rot.shape[0], rot.shape[1]
    Bs = shifts.shape[0] if shifts is not None else 0
    B = B or _batch(Bv, Br, Bs if shifts is not None else None)
    H = H or D
    out = np.empty((B, P, H, H // 2 + 1), np.complex128)
    rc = _load().oracle_project2d(B, P, Bv, Br, Bs, D, H, interp, o, r, _ptr(src), _ptr(rot), _ptr(shifts), _ptr(out))
    _check(rc, "project2d")
    return out


def backproject2d(images, rot, weights=None, shifts=None, D=None, Bv=1, interp=1, o=1.0, r=-1.0):
    """2D -> 2D accumulation (adjoint of project2d); returns (data, weight or None)."""
    images = _c(images, np.complex128)
    rot = _c(rot, np.float64)
    weights = _c(weights, np.float64)
    shifts = _c(shifts, np.float64)
    B, P, H = images.shape[0], images.shape[1], images.shape[2]
    Br = rot.shape[0]
    Bs = shifts.shape[0] if shifts is not None else 0
    D = D or H
    data = np.empty((Bv, D, D // 2 + 1), np.complex128)
    wimg = np.empty((Bv, D, D // 2 + 1), np.float64) if weights is not None else None
    rc = _load().oracle_backproject2d(B, P, Bv, Br, Bs, D, H, interp, o, r, _ptr(images), _ptr(weights), _ptr(rot),
                                      _ptr(shifts), _ptr(data), _ptr(wimg))
    _check(rc, "backproject2d")
    return data, wimg


def project2d_backward(grad_out, src, rot, shifts=None, interp=1, o=1.0, r=-1.0,
                       need_src=True, need_rot=True, need_shifts=True):
    """Backward of project2d; returns (grad_src, grad_rot, grad_shifts)."""
    grad_out = _c(grad_out, np.complex128)
    src = _c(src, np.complex128)
    rot = _c(rot, np.float64)
    shifts = _c(shifts, np.float64)
    B, P, H = grad_out.shape[0], grad_out.shape[1], grad_out.shape[2]
    Bv, D = src.shape[0], src.shape[1]
    Br = rot.shape[0]
    Bs = shifts.shape[0] if shifts is not None else 0
    gx = np.empty((Bv, D, D // 2 + 1), np.complex128) if need_src else None
    gr = np.empty((Br, P, 2, 2), np.float64) if need_rot else None
    gs = np.empty((Bs, P, 2), np.float64) if (need_shifts and shifts is not None) else None
    rc = _load().oracle_project2d_backward(B, P, Bv, Br, Bs, D, H, interp, o, r, _ptr(grad_out), _ptr(src), _ptr(rot),
                                           _ptr(shifts), _ptr(gx), _ptr(gr), _ptr(gs))
    _check(rc, "project2d_backward")
    return gx, gr, gs


def backproject2d_backward(grad_data, images, rot, grad_weight=None, weights=None, shifts=None,
                           interp=1, o=1.0, r=-1.0, need_images=True, need_weights=True, need_rot=True,
                           need_shifts=True):
    """Backward of backproject2d; returns (grad_images, grad_weights, grad_rot, grad_shifts)."""
    gd = _c(grad_data, np.complex128)
    gw = _c(grad_weight, np.float64)
    images = _c(images, np.complex128)
    weights = _c(weights, np.float64)
    rot = _c(rot, np.float64)
    shifts = _c(shifts, np.float64)
    B, P, H = images.shape[0], images.shape[1], images.shape[2]
    Bv, D = gd.shape[0], gd.shape[1]
    Br = rot.shape[0]
    Bs = shifts.shape[0] if shifts is not None else 0
    gi = np.empty((B, P, H, H // 2 + 1), np.complex128) if need_images else None
    gwo = np.empty((B, P, H, H // 2 + 1), np.float64) if (need_weights and gw is not None) else None
    gr = np.empty((Br, P, 2, 2), np.float64) if need_rot else None
    gs = np.empty((Bs, P, 2), np.float64) if (need_shifts and shifts is not None) else None
    rc = _load().oracle_backproject2d_backward(B, P, Bv, Br, Bs, D, H, interp, o, r, _ptr(gd), _ptr(gw), _ptr(images),
                                               _ptr(weights), _ptr(rot), _ptr(shifts), _ptr(gi), _ptr(gwo), _ptr(gr),
                                               _ptr(gs))
    _check(rc, "backproject2d_backward")
    return gi, gwo, gr, gs
