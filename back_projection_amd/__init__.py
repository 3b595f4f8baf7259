"""MI355X (gfx950) differentiable Fourier-slice projection.

Thin ctypes binding of ``libtproj.so`` (C ABI in ``include/tproj.h``): the
functions below only check and marshal arguments -- every step of the
computation runs in the library's HIP kernels.  PyTorch supplies device
memory (tensors) and the current HIP stream.  If the library is missing the
calls raise; there is no fallback.

Operations (torch-projectors pages: Spanish "Resumen tecnico" 2, Dutch
Methodologie, French "Resume technique" 2):
  project_3d_to_2d               rotated central slices of an rfft volume
  project_3d_to_2d_backward      volume, rotation and shift gradients
  backproject_2d_to_3d           accumulate rfft images (+ real weights)
  backproject_2d_to_3d_backward  image, weight, rotation and shift gradients
  project_2d_to_2d               rotation of a 2D rfft source (Dutch page, op. 1)
  project_2d_to_2d_backward      source, rotation and shift gradients
  backproject_2d_to_2d           accumulation into 2D reconstructions (op. 2)
  backproject_2d_to_2d_backward  image, weight, rotation and shift gradients

Tensor layout (CUDA/HIP tensors, contiguous):
  vol      complex64 [Bv, D, D, D//2+1]      weight vol float32 [Bv, D, D, D//2+1]
  images   complex64 [B, P, H, H//2+1]       weights    float32 [B, P, H, H//2+1]
  rot      float32   [Br, P, 3, 3]           shifts     float32 [Bs, P, 2]
with each of Bv, Br, Bs equal to 1 or B.  The 2D -> 2D calls take a source
complex64 [Bv, D, D//2+1] (weight source float32 [Bv, D, D//2+1]) and
rot float32 [Br, P, 2, 2].
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "project_3d_to_2d", "project_3d_to_2d_backward", "backproject_2d_to_3d", "backproject_2d_to_3d_backward",
    "project_2d_to_2d", "project_2d_to_2d_backward", "backproject_2d_to_2d", "backproject_2d_to_2d_backward",
    "project_3d_to_2d_noalloc", "NOALLOC_SCRATCH_BYTES", "volume_rfft", "images_irfft", "weight_images", "finish_reconstruction",
    "TprojError", "lib", "Geom", "LIB_PATH", "HEADER_SYMBOLS", "SPECTRAL_SYMBOLS", "BOUNDS_SYMBOLS", "timing_enable",
    "timing_read", "KERNEL_CLASSES",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtproj.so")

# Every symbol that include/tproj.h declares.
HEADER_SYMBOLS = (
    "project_3d_to_2d", "project_3d_to_2d_backward", "backproject_2d_to_3d", "backproject_2d_to_3d_backward",
    "project_2d_to_2d", "project_2d_to_2d_backward", "backproject_2d_to_2d", "backproject_2d_to_2d_backward",
    "tp_workspace_size", "tp_validate", "tp_status_string", "tp_last_error_detail", "tp_abi_version",
    "tp_timing_enable", "tp_timing_read", "project_3d_to_2d_noalloc",
)

# TP_NOALLOC_SCRATCH_BYTES of include/tproj.h: the static work area of
# project_3d_to_2d_noalloc (per GPU).
NOALLOC_SCRATCH_BYTES = 32 << 20

# Every symbol that include/tproj_bounds.h declares.
BOUNDS_SYMBOLS = ("tp_weight_sum_bound_3d", "tp_contrib_bound_3d", "tp_weight_sum_bound_2d", "tp_bounds_device")

# Every symbol that include/tproj_spectral.h declares.
SPECTRAL_SYMBOLS = (
    "tp_volume_rfft_workspace", "tp_volume_rfft", "tp_images_irfft_workspace", "tp_images_irfft",
    "tp_weight_images", "tp_finish_reconstruction",
)

OP_PROJECT, OP_PROJECT_BACKWARD, OP_BACKPROJECT, OP_BACKPROJECT_BACKWARD = 0, 1, 2, 3
OP_PROJECT_2D, OP_PROJECT_2D_BACKWARD, OP_BACKPROJECT_2D, OP_BACKPROJECT_2D_BACKWARD = 4, 5, 6, 7


class TprojError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"tproj status {status}: {detail}")
        self.status = status
        self.detail = detail


class Geom(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("P", ctypes.c_int32), ("Bv", ctypes.c_int32), ("Br", ctypes.c_int32),
                ("Bs", ctypes.c_int32), ("D", ctypes.c_int32), ("H", ctypes.c_int32), ("interp", ctypes.c_int32),
                ("oversampling", ctypes.c_float), ("radius_cutoff", ctypes.c_float)]


_lib = None
_vp = ctypes.c_void_p


def lib():
    """Load libtproj.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with back_projection_amd.build_lib.build() "
                              "(or __graft_entry__.build()); there is no non-HIP fallback")
        L = ctypes.CDLL(LIB_PATH)
        G = ctypes.POINTER(Geom)
        L.project_3d_to_2d.argtypes = [G, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.project_3d_to_2d_backward.argtypes = [G, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.backproject_2d_to_3d.argtypes = [G, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.backproject_2d_to_3d_backward.argtypes = [G] + [_vp] * 11 + [ctypes.c_size_t, _vp]
        L.project_3d_to_2d_noalloc.argtypes = [G, _vp, _vp, _vp, _vp, _vp]
        L.project_3d_to_2d_noalloc.restype = ctypes.c_int
        L.project_2d_to_2d.argtypes = L.project_3d_to_2d.argtypes
        L.project_2d_to_2d_backward.argtypes = L.project_3d_to_2d_backward.argtypes
        L.backproject_2d_to_2d.argtypes = L.backproject_2d_to_3d.argtypes
        L.backproject_2d_to_2d_backward.argtypes = L.backproject_2d_to_3d_backward.argtypes
        for f in ("project_3d_to_2d", "project_3d_to_2d_backward", "backproject_2d_to_3d",
                  "backproject_2d_to_3d_backward", "project_2d_to_2d", "project_2d_to_2d_backward",
                  "backproject_2d_to_2d", "backproject_2d_to_2d_backward", "tp_validate"):
            getattr(L, f).restype = ctypes.c_int
        L.tp_validate.argtypes = [G]
        L.tp_workspace_size.argtypes = [G, ctypes.c_int]
        L.tp_workspace_size.restype = ctypes.c_size_t
        L.tp_status_string.argtypes = [ctypes.c_int]
        L.tp_status_string.restype = ctypes.c_char_p
        L.tp_last_error_detail.restype = ctypes.c_char_p
        L.tp_abi_version.restype = ctypes.c_int
        L.tp_timing_enable.argtypes = [ctypes.c_int]
        L.tp_timing_enable.restype = ctypes.c_int
        L.tp_timing_read.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
        L.tp_timing_read.restype = ctypes.c_int
        L.tp_volume_rfft_workspace.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
        L.tp_volume_rfft_workspace.restype = ctypes.c_size_t
        L.tp_volume_rfft.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.tp_images_irfft_workspace.argtypes = [ctypes.c_int, ctypes.c_int64]
        L.tp_images_irfft_workspace.restype = ctypes.c_size_t
        L.tp_images_irfft.argtypes = [ctypes.c_int, ctypes.c_int64, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.tp_weight_images.argtypes = [ctypes.c_int64, ctypes.c_int64, _vp, _vp, _vp, _vp]
        L.tp_finish_reconstruction.argtypes = [ctypes.c_int64, _vp, _vp, ctypes.c_float, _vp, _vp]
        for f in ("tp_volume_rfft", "tp_images_irfft", "tp_weight_images", "tp_finish_reconstruction"):
            getattr(L, f).restype = ctypes.c_int
        for f in ("tp_weight_sum_bound_3d", "tp_contrib_bound_3d"):
            getattr(L, f).argtypes = [ctypes.c_int, ctypes.c_float, _vp]
            getattr(L, f).restype = ctypes.c_float
        L.tp_weight_sum_bound_2d.argtypes = [ctypes.c_int, ctypes.c_float, ctypes.c_float, ctypes.c_int, _vp]
        L.tp_weight_sum_bound_2d.restype = ctypes.c_float
        L.tp_bounds_device.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_float, ctypes.c_int, _vp,
                                       ctypes.c_int64, _vp]
        L.tp_bounds_device.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise TprojError(status, lib().tp_last_error_detail().decode())


# kernel classes of tp_timing_read (include/tproj.h)
KERNEL_CLASSES = {"forward": 0, "backward": 1, "gradient": 2, "fold": 3}


def timing_enable(on: bool = True):
    """Start (or stop) event timing of the brick kernels (tp_timing_enable)."""
    _check(lib().tp_timing_enable(1 if on else 0))


def timing_read(kernel_class: str):
    """(summed milliseconds, launches) of one kernel class since the last read (tp_timing_read)."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    _check(lib().tp_timing_read(KERNEL_CLASSES[kernel_class], ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def _interp(x) -> int:
    if isinstance(x, str):
        return {"linear": 0, "cubic": 1}[x]
    return int(x)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _typ(t, name, dtype, ndim):
    """Type and rank of one argument (no device access)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    return t


def _shape(t, name, shape):
    """Full shape of one argument against what the geometry implies: the C ABI
    receives only pointers and the geometry, so a mis-shaped tensor would be
    read or written out of bounds on the device."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _bcast(B, **sizes):
    """Each broadcast batch size (Bv, Br, Bs; 0 = absent) is 1 or B."""
    for name, n in sizes.items():
        if n and n not in (1, B):
            raise ValueError(f"{name} = {n} must be 1 or the batch size {B}")


def _placed(device, **tensors):
    """Every given tensor on `device` and contiguous (after the shape checks)."""
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be on a GPU device")
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def _req(t, name, dtype, ndim, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _batch(*bs):
    bs = [b for b in bs if b]
    B = max(bs)
    if any(b not in (1, B) for b in bs):
        raise ValueError(f"batch sizes {bs} must each be 1 or a common B")
    return B


def _workspace(g: Geom, op: int, device):
    n = lib().tp_workspace_size(ctypes.byref(g), op)
    if n == ctypes.c_size_t(-1).value:
        _check(lib().tp_validate(ctypes.byref(g)))
    if n == 0:
        return None, 0
    return torch.empty(n, dtype=torch.uint8, device=device), n


def project_3d_to_2d(vol, rot, shifts=None, *, H=None, interp="cubic", oversampling=1.0, radius_cutoff=-1.0,
                     B=None, out=None):
    """Forward: out[b, n] = M * phi * I(vol[bv], o R (kx, ky, 0)).  Returns out
    (complex64 [B, P, H, H//2+1])."""
    _typ(vol, "vol", torch.complex64, 4)
    _typ(rot, "rot", torch.float32, 4)
    if shifts is not None:
        _typ(shifts, "shifts", torch.float32, 3)
    Bv, D = vol.shape[0], vol.shape[1]
    Br, P = rot.shape[0], rot.shape[1]
    Bs = shifts.shape[0] if shifts is not None else 0
    B = B or _batch(Bv, Br, Bs)
    H = H or D
    _shape(vol, "vol", (Bv, D, D, D // 2 + 1))
    _shape(rot, "rot", (Br, P, 3, 3))
    _shape(shifts, "shifts", (Bs, P, 2))
    _bcast(B, Bv=Bv, Br=Br, Bs=Bs)
    if out is not None:
        _typ(out, "out", torch.complex64, 4)
        _shape(out, "out", (B, P, H, H // 2 + 1))
    dev = vol.device
    _placed(dev, vol=vol, rot=rot, shifts=shifts, out=out)
    if out is None:
        out = torch.empty((B, P, H, H // 2 + 1), dtype=torch.complex64, device=dev)
    g = Geom(B, P, Bv, Br, Bs, D, H, _interp(interp), float(oversampling), float(radius_cutoff))
    ws, nws = _workspace(g, OP_PROJECT, dev)
    _check(lib().project_3d_to_2d(ctypes.byref(g), _ptr(vol), _ptr(rot), _ptr(shifts), _ptr(out), _ptr(ws), nws,
                                  _stream(dev)))
    return out


def project_3d_to_2d_noalloc(vol, rot, shifts, out, *, interp="cubic", oversampling=1.0, radius_cutoff=-1.0):
    """project_3d_to_2d for callers that cannot allocate: no workspace, no
    output allocation (out, complex64 [B, P, H, H//2+1], is required and gives
    B and H).  The library's static per-GPU work area holds the scratch;
    geometries that need more than NOALLOC_SCRATCH_BYTES are rejected.
    Calls that overlap on one GPU race (they share that area)."""
    _typ(vol, "vol", torch.complex64, 4)
    _typ(rot, "rot", torch.float32, 4)
    _typ(out, "out", torch.complex64, 4)
    if shifts is not None:
        _typ(shifts, "shifts", torch.float32, 3)
    Bv, D = vol.shape[0], vol.shape[1]
    Br, P = rot.shape[0], rot.shape[1]
    Bs = shifts.shape[0] if shifts is not None else 0
    B, H = out.shape[0], out.shape[2]
    _shape(vol, "vol", (Bv, D, D, D // 2 + 1))
    _shape(rot, "rot", (Br, P, 3, 3))
    _shape(shifts, "shifts", (Bs, P, 2))
    _shape(out, "out", (B, P, H, H // 2 + 1))
    _bcast(B, Bv=Bv, Br=Br, Bs=Bs)
    dev = vol.device
    _placed(dev, vol=vol, rot=rot, shifts=shifts, out=out)
    g = Geom(B, P, Bv, Br, Bs, D, H, _interp(interp), float(oversampling), float(radius_cutoff))
    _check(lib().project_3d_to_2d_noalloc(ctypes.byref(g), _ptr(vol), _ptr(rot), _ptr(shifts), _ptr(out),
                                          _stream(dev)))
    return out


def project_3d_to_2d_backward(grad_out, vol, rot, shifts=None, *, interp="cubic", oversampling=1.0,
                              radius_cutoff=-1.0, need_vol=True, need_rot=True, need_shifts=True,
                              grad_vol=None, grad_rot=None, grad_shifts=None):
    """Backward of project_3d_to_2d; returns (grad_vol, grad_rot, grad_shifts),
    None where not requested.  Preallocated outputs may be passed in."""
    _typ(grad_out, "grad_out", torch.complex64, 4)
    _typ(vol, "vol", torch.complex64, 4)
    _typ(rot, "rot", torch.float32, 4)
    if shifts is not None:
        _typ(shifts, "shifts", torch.float32, 3)
    B, P, H = grad_out.shape[0], grad_out.shape[1], grad_out.shape[2]
    Bv, D = vol.shape[0], vol.shape[1]
    Br = rot.shape[0]
    Bs = shifts.shape[0] if shifts is not None else 0
    _shape(grad_out, "grad_out", (B, P, H, H // 2 + 1))
    _shape(vol, "vol", (Bv, D, D, D // 2 + 1))
    _shape(rot, "rot", (Br, P, 3, 3))
    _shape(shifts, "shifts", (Bs, P, 2))
    _bcast(B, Bv=Bv, Br=Br, Bs=Bs)
    outs = {}
    for t, ref, name, need in ((grad_vol, vol, "grad_vol", need_vol), (grad_rot, rot, "grad_rot", need_rot),
                               (grad_shifts, shifts, "grad_shifts", need_shifts and shifts is not None)):
        if need and t is not None:
            _typ(t, name, ref.dtype, ref.dim())
            _shape(t, name, ref.shape)
            outs[name] = t
    dev = grad_out.device
    _placed(dev, grad_out=grad_out, vol=vol, rot=rot, shifts=shifts, **outs)
    gv = (grad_vol if grad_vol is not None else torch.empty_like(vol)) if need_vol else None
    gr = (grad_rot if grad_rot is not None else torch.empty_like(rot)) if need_rot else None
    gs = (grad_shifts if grad_shifts is not None else torch.empty_like(shifts)) if (
        need_shifts and shifts is not None) else None
    g = Geom(B, P, Bv, Br, Bs, D, H, _interp(interp), float(oversampling), float(radius_cutoff))
    ws, nws = _workspace(g, OP_PROJECT_BACKWARD, dev)
    _check(lib().project_3d_to_2d_backward(ctypes.byref(g), _ptr(grad_out), _ptr(vol), _ptr(rot), _ptr(shifts),
                                           _ptr(gv), _ptr(gr), _ptr(gs), _ptr(ws), nws, _stream(dev)))
    return gv, gr, gs


def backproject_2d_to_3d(images, rot, weights=None, shifts=None, *, D=None, Bv=1, interp="cubic", oversampling=1.0,
                         radius_cutoff=-1.0, data_vol=None, weight_vol=None):
    """Back-projection (adjoint): returns (data_vol, weight_vol or None).
    Preallocated outputs may be passed in."""
    _typ(images, "images", torch.complex64, 4)
    _typ(rot, "rot", torch.float32, 4)
    if weights is not None:
        _typ(weights, "weights", torch.float32, 4)
    if shifts is not None:
        _typ(shifts, "shifts", torch.float32, 3)
    B, P, H = images.shape[0], images.shape[1], images.shape[2]
    Br = rot.shape[0]
    Bs = shifts.shape[0] if shifts is not None else 0
    D = D or H
    _shape(images, "images", (B, P, H, H // 2 + 1))
    _shape(weights, "weights", (B, P, H, H // 2 + 1))
    _shape(rot, "rot", (Br, P, 3, 3))
    _shape(shifts, "shifts", (Bs, P, 2))
    _bcast(B, Bv=Bv, Br=Br, Bs=Bs)
    if data_vol is not None:
        _typ(data_vol, "data_vol", torch.complex64, 4)
        _shape(data_vol, "data_vol", (Bv, D, D, D // 2 + 1))
    if weights is not None and weight_vol is not None:
        _typ(weight_vol, "weight_vol", torch.float32, 4)
        _shape(weight_vol, "weight_vol", (Bv, D, D, D // 2 + 1))
    dev = images.device
    _placed(dev, images=images, rot=rot, weights=weights, shifts=shifts, data_vol=data_vol,
            weight_vol=weight_vol if weights is not None else None)
    data = data_vol if data_vol is not None else torch.empty((Bv, D, D, D // 2 + 1), dtype=torch.complex64,
                                                             device=dev)
    wvol = None
    if weights is not None:
        wvol = weight_vol if weight_vol is not None else torch.empty((Bv, D, D, D // 2 + 1), dtype=torch.float32,
                                                                     device=dev)
    g = Geom(B, P, Bv, Br, Bs, D, H, _interp(interp), float(oversampling), float(radius_cutoff))
    ws, nws = _workspace(g, OP_BACKPROJECT, dev)
    _check(lib().backproject_2d_to_3d(ctypes.byref(g), _ptr(images), _ptr(weights), _ptr(rot), _ptr(shifts),
                                      _ptr(data), _ptr(wvol), _ptr(ws), nws, _stream(dev)))
    return data, wvol


def backproject_2d_to_3d_backward(grad_data_vol, images, rot, grad_weight_vol=None, weights=None, shifts=None, *,
                                  interp="cubic", oversampling=1.0, radius_cutoff=-1.0, need_images=True,
                                  need_weights=True, need_rot=True, need_shifts=True):
    """Backward of backproject_2d_to_3d; returns (grad_images, grad_weights,
    grad_rot, grad_shifts), None where not requested."""
    _typ(grad_data_vol, "grad_data_vol", torch.complex64, 4)
    _typ(images, "images", torch.complex64, 4)
    _typ(rot, "rot", torch.float32, 4)
    if grad_weight_vol is not None:
        _typ(grad_weight_vol, "grad_weight_vol", torch.float32, 4)
    if weights is not None:
        _typ(weights, "weights", torch.float32, 4)
    if shifts is not None:
        _typ(shifts, "shifts", torch.float32, 3)
    B, P, H = images.shape[0], images.shape[1], images.shape[2]
    Bv, D = grad_data_vol.shape[0], grad_data_vol.shape[1]
    Br = rot.shape[0]
    Bs = shifts.shape[0] if shifts is not None else 0
    _shape(grad_data_vol, "grad_data_vol", (Bv, D, D, D // 2 + 1))
    _shape(grad_weight_vol, "grad_weight_vol", (Bv, D, D, D // 2 + 1))
    _shape(images, "images", (B, P, H, H // 2 + 1))
    _shape(weights, "weights", (B, P, H, H // 2 + 1))
    _shape(rot, "rot", (Br, P, 3, 3))
    _shape(shifts, "shifts", (Bs, P, 2))
    _bcast(B, Bv=Bv, Br=Br, Bs=Bs)
    dev = grad_data_vol.device
    _placed(dev, grad_data_vol=grad_data_vol, images=images, rot=rot, grad_weight_vol=grad_weight_vol,
            weights=weights, shifts=shifts)
    gi = torch.empty_like(images) if need_images else None
    gw = torch.empty((B, P, H, H // 2 + 1), dtype=torch.float32, device=dev) if (
        need_weights and weights is not None) else None
    gr = torch.empty_like(rot) if need_rot else None
    gs = torch.empty_like(shifts) if (need_shifts and shifts is not None) else None
    g = Geom(B, P, Bv, Br, Bs, D, H, _interp(interp), float(oversampling), float(radius_cutoff))
    ws, nws = _workspace(g, OP_BACKPROJECT_BACKWARD, dev)
    _check(lib().backproject_2d_to_3d_backward(ctypes.byref(g), _ptr(grad_data_vol), _ptr(grad_weight_vol),
                                               _ptr(images), _ptr(weights), _ptr(rot), _ptr(shifts), _ptr(gi),
                                               _ptr(gw), _ptr(gr), _ptr(gs), _ptr(ws), nws, _stream(dev)))
    return gi, gw, gr, gs


# ---------------------------------------------------------------------------
# 2D -> 2D
# ---------------------------------------------------------------------------
def project_2d_to_2d(src, rot, shifts=None, *, H=None, interp="cubic", oversampling=1.0, radius_cutoff=-1.0,
                     B=None, out=None):
    """Forward: out[b, n] = M * phi * I(src[bv], o R (kx, ky)).  Returns out
    (complex64 [B, P, H, H//2+1])."""
    _typ(src, "src", torch.complex64, 3)
    _typ(rot, "rot", torch.float32, 4)
    if shifts is not None:
        _typ(shifts, "shifts", torch.float32, 3)
    Bv, D = src.shape[0], src.shape[1]
    Br, P = rot.shape[0], rot.shape[1]
    Bs = shifts.shape[0] if shifts is not None else 0
    B = B or _batch(Bv, Br, Bs)
    H = H or D
    _shape(src, "src", (Bv, D, D // 2 + 1))
    _shape(rot, "rot", (Br, P, 2, 2))
    _shape(shifts, "shifts", (Bs, P, 2))
    _bcast(B, Bv=Bv, Br=Br, Bs=Bs)
    if out is not None:
        _typ(out, "out", torch.complex64, 4)
        _shape(out, "out", (B, P, H, H // 2 + 1))
    dev = src.device
    _placed(dev, src=src, rot=rot, shifts=shifts, out=out)
    if out is None:
        out = torch.empty((B, P, H, H // 2 + 1), dtype=torch.complex64, device=dev)
    g = Geom(B, P, Bv, Br, Bs, D, H, _interp(interp), float(oversampling), float(radius_cutoff))
    ws, nws = _workspace(g, OP_PROJECT_2D, dev)
    _check(lib().project_2d_to_2d(ctypes.byref(g), _ptr(src), _ptr(rot), _ptr(shifts), _ptr(out), _ptr(ws), nws,
                                  _stream(dev)))
    return out


def project_2d_to_2d_backward(grad_out, src, rot, shifts=None, *, interp="cubic", oversampling=1.0,
                              radius_cutoff=-1.0, need_src=True, need_rot=True, need_shifts=True):
    """Backward of project_2d_to_2d; returns (grad_src, grad_rot, grad_shifts),
    None where not requested."""
    _typ(grad_out, "grad_out", torch.complex64, 4)
    _typ(src, "src", torch.complex64, 3)
    _typ(rot, "rot", torch.float32, 4)
    if shifts is not None:
        _typ(shifts, "shifts", torch.float32, 3)
    B, P, H = grad_out.shape[0], grad_out.shape[1], grad_out.shape[2]
    Bv, D = src.shape[0], src.shape[1]
    Br = rot.shape[0]
    Bs = shifts.shape[0] if shifts is not None else 0
    _shape(grad_out, "grad_out", (B, P, H, H // 2 + 1))
    _shape(src, "src", (Bv, D, D // 2 + 1))
    _shape(rot, "rot", (Br, P, 2, 2))
    _shape(shifts, "shifts", (Bs, P, 2))
    _bcast(B, Bv=Bv, Br=Br, Bs=Bs)
    dev = grad_out.device
    _placed(dev, grad_out=grad_out, src=src, rot=rot, shifts=shifts)
    gx = torch.empty_like(src) if need_src else None
    gr = torch.empty_like(rot) if need_rot else None
    gs = torch.empty_like(shifts) if (need_shifts and shifts is not None) else None
    g = Geom(B, P, Bv, Br, Bs, D, H, _interp(interp), float(oversampling), float(radius_cutoff))
    ws, nws = _workspace(g, OP_PROJECT_2D_BACKWARD, dev)
    _check(lib().project_2d_to_2d_backward(ctypes.byref(g), _ptr(grad_out), _ptr(src), _ptr(rot), _ptr(shifts),
                                           _ptr(gx), _ptr(gr), _ptr(gs), _ptr(ws), nws, _stream(dev)))
    return gx, gr, gs


def backproject_2d_to_2d(images, rot, weights=None, shifts=None, *, D=None, Bv=1, interp="cubic",
                         oversampling=1.0, radius_cutoff=-1.0):
    """Accumulation into 2D reconstructions (adjoint of project_2d_to_2d):
    returns (data, weight or None), complex64 / float32 [Bv, D, D//2+1]."""
    _typ(images, "images", torch.complex64, 4)
    _typ(rot, "rot", torch.float32, 4)
    if weights is not None:
        _typ(weights, "weights", torch.float32, 4)
    if shifts is not None:
        _typ(shifts, "shifts", torch.float32, 3)
    B, P, H = images.shape[0], images.shape[1], images.shape[2]
    Br = rot.shape[0]
    Bs = shifts.shape[0] if shifts is not None else 0
    D = D or H
    _shape(images, "images", (B, P, H, H // 2 + 1))
    _shape(weights, "weights", (B, P, H, H // 2 + 1))
    _shape(rot, "rot", (Br, P, 2, 2))
    _shape(shifts, "shifts", (Bs, P, 2))
    _bcast(B, Bv=Bv, Br=Br, Bs=Bs)
    dev = images.device
    _placed(dev, images=images, rot=rot, weights=weights, shifts=shifts)
    data = torch.empty((Bv, D, D // 2 + 1), dtype=torch.complex64, device=dev)
    wimg = torch.empty((Bv, D, D // 2 + 1), dtype=torch.float32, device=dev) if weights is not None else None
    g = Geom(B, P, Bv, Br, Bs, D, H, _interp(interp), float(oversampling), float(radius_cutoff))
    ws, nws = _workspace(g, OP_BACKPROJECT_2D, dev)
    _check(lib().backproject_2d_to_2d(ctypes.byref(g), _ptr(images), _ptr(weights), _ptr(rot), _ptr(shifts),
                                      _ptr(data), _ptr(wimg), _ptr(ws), nws, _stream(dev)))
    return data, wimg


def backproject_2d_to_2d_backward(grad_data, images, rot, grad_weight=None, weights=None, shifts=None, *,
                                  interp="cubic", oversampling=1.0, radius_cutoff=-1.0, need_images=True,
                                  need_weights=True, need_rot=True, need_shifts=True):
    """Backward of backproject_2d_to_2d; returns (grad_images, grad_weights,
    grad_rot, grad_shifts), None where not requested."""
    _typ(grad_data, "grad_data", torch.complex64, 3)
    _typ(images, "images", torch.complex64, 4)
    _typ(rot, "rot", torch.float32, 4)
    if grad_weight is not None:
        _typ(grad_weight, "grad_weight", torch.float32, 3)
    if weights is not None:
        _typ(weights, "weights", torch.float32, 4)
    if shifts is not None:
        _typ(shifts, "shifts", torch.float32, 3)
    B, P, H = images.shape[0], images.shape[1], images.shape[2]
    Bv, D = grad_data.shape[0], grad_data.shape[1]
    Br = rot.shape[0]
    Bs = shifts.shape[0] if shifts is not None else 0
    _shape(grad_data, "grad_data", (Bv, D, D // 2 + 1))
    _shape(grad_weight, "grad_weight", (Bv, D, D // 2 + 1))
    _shape(images, "images", (B, P, H, H // 2 + 1))
    _shape(weights, "weights", (B, P, H, H // 2 + 1))
    _shape(rot, "rot", (Br, P, 2, 2))
    _shape(shifts, "shifts", (Bs, P, 2))
    _bcast(B, Bv=Bv, Br=Br, Bs=Bs)
    dev = grad_data.device
    _placed(dev, grad_data=grad_data, images=images, rot=rot, grad_weight=grad_weight, weights=weights,
            shifts=shifts)
    gi = torch.empty_like(images) if need_images else None
    gw = torch.empty((B, P, H, H // 2 + 1), dtype=torch.float32, device=dev) if (
        need_weights and weights is not None) else None
    gr = torch.empty_like(rot) if need_rot else None
    gs = torch.empty_like(shifts) if (need_shifts and shifts is not None) else None
    g = Geom(B, P, Bv, Br, Bs, D, H, _interp(interp), float(oversampling), float(radius_cutoff))
    ws, nws = _workspace(g, OP_BACKPROJECT_2D_BACKWARD, dev)
    _check(lib().backproject_2d_to_2d_backward(ctypes.byref(g), _ptr(grad_data), _ptr(grad_weight), _ptr(images),
                                               _ptr(weights), _ptr(rot), _ptr(shifts), _ptr(gi), _ptr(gw), _ptr(gr),
                                               _ptr(gs), _ptr(ws), nws, _stream(dev)))
    return gi, gw, gr, gs


# ---------------------------------------------------------------------------
# Steps either side of the path (include/tproj_spectral.h)
# ---------------------------------------------------------------------------
def _spectral_ws(n, device):
    if n == ctypes.c_size_t(-1).value:
        raise TprojError(4, lib().tp_last_error_detail().decode())
    return (torch.empty(n, dtype=torch.uint8, device=device), n) if n else (None, 0)


def volume_rfft(vol, pad=1, out=None):
    """Real volume(s) [Bv, D, D, D] (or [D, D, D]) float32, centre at D/2 ->
    zero-padded to N = pad * D, centre moved to index 0, rfftn: complex64
    [Bv, N, N, N//2+1] (tp_volume_rfft)."""
    if vol.dim() == 3:
        vol = vol.unsqueeze(0)
    _req(vol, "vol", torch.float32, 4)
    Bv, D = vol.shape[0], vol.shape[-1]
    if tuple(vol.shape[1:]) != (D, D, D):
        raise ValueError(f"vol must be [Bv, D, D, D], got {tuple(vol.shape)}")
    N = int(pad) * D
    dev = vol.device
    if out is None:
        out = torch.empty((Bv, N, N, N // 2 + 1), dtype=torch.complex64, device=dev)
    _req(out, "out", torch.complex64, 4, dev)
    if tuple(out.shape) != (Bv, N, N, N // 2 + 1):
        raise ValueError(f"out must be {(Bv, N, N, N // 2 + 1)}, got {tuple(out.shape)}")
    with torch.cuda.device(dev):
        ws, nws = _spectral_ws(lib().tp_volume_rfft_workspace(D, int(pad), Bv), dev)
        _check(lib().tp_volume_rfft(D, int(pad), Bv, _ptr(vol), _ptr(out), _ptr(ws), nws, _stream(dev)))
    return out


def images_irfft(images, out=None):
    """Spectra [..., H, H//2+1] complex64 -> real images [..., H, H] float32:
    normalised inverse DFT, index 0 moved to the centre (tp_images_irfft)."""
    if not isinstance(images, torch.Tensor) or images.dim() < 2:
        raise ValueError("images must be a tensor [..., H, H//2+1]")
    _req(images, "images", torch.complex64, images.dim())
    H = images.shape[-2]
    if images.shape[-1] != H // 2 + 1:
        raise ValueError(f"images must be [..., H, H//2+1], got {tuple(images.shape)}")
    n = images.numel() // (H * (H // 2 + 1))
    dev = images.device
    shape = tuple(images.shape[:-2]) + (H, H)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=dev)
    _req(out, "out", torch.float32, len(shape), dev)
    if tuple(out.shape) != shape:
        raise ValueError(f"out must be {shape}, got {tuple(out.shape)}")
    with torch.cuda.device(dev):
        ws, nws = _spectral_ws(lib().tp_images_irfft_workspace(H, n), dev)
        _check(lib().tp_images_irfft(H, n, _ptr(images), _ptr(out), _ptr(ws), nws, _stream(dev)))
    return out


def weight_images(images, weights, out=None):
    """images * weights (per-image CTF multiply): weights' shape must match
    the trailing dims of images (e.g. [P, H, H//2+1] for [B, P, H, H//2+1])
    (tp_weight_images).  out may be images (in place)."""
    _req(images, "images", torch.complex64, images.dim())
    _req(weights, "weights", torch.float32, weights.dim(), images.device)
    if weights.dim() > images.dim() or tuple(images.shape[images.dim() - weights.dim():]) != tuple(weights.shape):
        raise ValueError(f"weights {tuple(weights.shape)} must match the trailing dims of images {tuple(images.shape)}")
    if out is None:
        out = torch.empty_like(images)
    _req(out, "out", torch.complex64, images.dim(), images.device)
    if out.shape != images.shape:
        raise ValueError("out must have the shape of images")
    dev = images.device
    with torch.cuda.device(dev):
        _check(lib().tp_weight_images(images.numel(), weights.numel(), _ptr(images), _ptr(weights), _ptr(out),
                                      _stream(dev)))
    return out


def finish_reconstruction(data, weights, lam=0.0, out=None):
    """data / (weights + lam) where that is > 0, else 0 (tp_finish_reconstruction);
    data complex64 and weights float32 of one shape."""
    _req(data, "data", torch.complex64, data.dim())
    _req(weights, "weights", torch.float32, data.dim(), data.device)
    if weights.shape != data.shape:
        raise ValueError(f"weights {tuple(weights.shape)} must have the shape of data {tuple(data.shape)}")
    if out is None:
        out = torch.empty_like(data)
    _req(out, "out", torch.complex64, data.dim(), data.device)
    dev = data.device
    with torch.cuda.device(dev):
        _check(lib().tp_finish_reconstruction(data.numel(), _ptr(data), _ptr(weights), float(lam), _ptr(out),
                                              _stream(dev)))
    return out
