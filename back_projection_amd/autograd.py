"""torch.autograd wrappers of the four operations: every input of the pages'
operations is differentiable (volume or source, images, weights, rotations,
shifts; torch-projectors pages: Dutch Methodologie, Spanish "Resumen
tecnico" 2), with the forward and backward passes both served by the
library's entry points, and nothing kept between them but the inputs.

Complex gradients follow torch's convention for real losses (dL/dRe +
i dL/dIm, so that |z|^2 has gradient 2z), which is the convention of the
library's backward entry points.  Inputs that do not require grad are not
computed in the backward call.
"""
from __future__ import annotations

import torch

from . import (backproject_2d_to_2d, backproject_2d_to_2d_backward, backproject_2d_to_3d,
               backproject_2d_to_3d_backward, project_2d_to_2d, project_2d_to_2d_backward, project_3d_to_2d,
               project_3d_to_2d_backward)

__all__ = ["project_3d_to_2d_ag", "backproject_2d_to_3d_ag", "project_2d_to_2d_ag", "backproject_2d_to_2d_ag"]


def _c(t):
    return None if t is None else t.contiguous()


class _Project(torch.autograd.Function):
    @staticmethod
    def forward(ctx, vol, rot, shifts, twod, H, interp, oversampling, radius_cutoff):
        fwd = project_2d_to_2d if twod else project_3d_to_2d
        out = fwd(vol, rot, shifts, H=H, interp=interp, oversampling=oversampling, radius_cutoff=radius_cutoff)
        ctx.save_for_backward(vol, rot, shifts)
        ctx.cfg = (twod, interp, oversampling, radius_cutoff)
        return out

    @staticmethod
    def backward(ctx, gout):
        vol, rot, shifts = ctx.saved_tensors
        twod, interp, o, r = ctx.cfg
        nv, nr, ns = ctx.needs_input_grad[:3]
        ns = ns and shifts is not None
        if not (nv or nr or ns):
            return (None,) * 8
        if twod:
            gv, gr, gs = project_2d_to_2d_backward(_c(gout), vol, rot, shifts, interp=interp, oversampling=o,
                                                   radius_cutoff=r, need_src=nv, need_rot=nr, need_shifts=ns)
        else:
            gv, gr, gs = project_3d_to_2d_backward(_c(gout), vol, rot, shifts, interp=interp, oversampling=o,
                                                   radius_cutoff=r, need_vol=nv, need_rot=nr, need_shifts=ns)
        return gv, gr, gs, None, None, None, None, None


class _Backproject(torch.autograd.Function):
    @staticmethod
    def forward(ctx, images, rot, weights, shifts, twod, D, Bv, interp, oversampling, radius_cutoff):
        bwd = backproject_2d_to_2d if twod else backproject_2d_to_3d
        data, wvol = bwd(images, rot, weights, shifts, D=D, Bv=Bv, interp=interp, oversampling=oversampling,
                         radius_cutoff=radius_cutoff)
        ctx.save_for_backward(images, rot, weights, shifts)
        ctx.cfg = (twod, interp, oversampling, radius_cutoff)
        # unused outputs get zero upstream gradients (torch materialises them)
        if wvol is None:
            return data
        return data, wvol

    @staticmethod
    def backward(ctx, gdata, gweight=None):
        images, rot, weights, shifts = ctx.saved_tensors
        twod, interp, o, r = ctx.cfg
        ni, nr, nw, ns = ctx.needs_input_grad[:4]
        nw = nw and weights is not None
        ns = ns and shifts is not None
        if not (ni or nr or nw or ns):
            return (None,) * 10
        fn = backproject_2d_to_2d_backward if twod else backproject_2d_to_3d_backward
        gi, gw, gr, gs = fn(_c(gdata), images, rot, _c(gweight) if weights is not None else None, weights, shifts,
                            interp=interp, oversampling=o, radius_cutoff=r, need_images=ni, need_weights=nw,
                            need_rot=nr, need_shifts=ns)
        return gi, gr, gw, gs, None, None, None, None, None, None


def project_3d_to_2d_ag(vol, rot, shifts=None, *, H=None, interp="cubic", oversampling=1.0, radius_cutoff=-1.0):
    """Differentiable project_3d_to_2d (gradients for vol, rot, shifts)."""
    return _Project.apply(vol, rot, shifts, False, H, interp, oversampling, radius_cutoff)


def project_2d_to_2d_ag(src, rot, shifts=None, *, H=None, interp="cubic", oversampling=1.0, radius_cutoff=-1.0):
    """Differentiable project_2d_to_2d (gradients for src, rot, shifts)."""
    return _Project.apply(src, rot, shifts, True, H, interp, oversampling, radius_cutoff)


def backproject_2d_to_3d_ag(images, rot, weights=None, shifts=None, *, D=None, Bv=1, interp="cubic",
                            oversampling=1.0, radius_cutoff=-1.0):
    """Differentiable backproject_2d_to_3d: data volume, or (data, weight volume)
    with weights (gradients for images, rot, weights, shifts)."""
    return _Backproject.apply(images, rot, weights, shifts, False, D, Bv, interp, oversampling, radius_cutoff)


def backproject_2d_to_2d_ag(images, rot, weights=None, shifts=None, *, D=None, Bv=1, interp="cubic",
                            oversampling=1.0, radius_cutoff=-1.0):
    """Differentiable backproject_2d_to_2d (as backproject_2d_to_3d_ag, in 2D)."""
    return _Backproject.apply(images, rot, weights, shifts, True, D, Bv, interp, oversampling, radius_cutoff)
