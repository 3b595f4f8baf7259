"""Host-side argument checks of the Python binding (no GPU, no launch).

The C ABI receives plain pointers and the geometry (B, P, D, H, Bv, Br, Bs),
so the binding must reject any tensor whose full shape disagrees with the
geometry the other arguments imply: such a tensor would be read or written
out of bounds on the device.  Shapes are checked before device placement, so
CPU tensors exercise every check here: a consistent set gets as far as the
"must be on a GPU device" check, and every single mismatch stops earlier with
a shape error.
"""
import pytest
import torch

import back_projection_amd as bp

C64, F32 = torch.complex64, torch.float32


def z(shape, dtype):
    return torch.zeros(shape, dtype=dtype)


B, P, D, H = 2, 3, 8, 10
W2 = H // 2 + 1


def args_3d():
    """name -> (function, positional args builder, keyword args) with a
    consistent set of 3D tensors; each entry of `tensors` may be replaced."""
    vol = z((1, D, D, D // 2 + 1), C64)
    rot = z((B, P, 3, 3), F32)
    sh = z((B, P, 2), F32)
    img = z((B, P, H, W2), C64)
    wts = z((B, P, H, W2), F32)
    wvol = z((1, D, D, D // 2 + 1), F32)
    return {
        "project_3d_to_2d": (bp.project_3d_to_2d, dict(vol=vol, rot=rot, shifts=sh), dict(H=H)),
        "project_3d_to_2d_backward": (bp.project_3d_to_2d_backward,
                                      dict(grad_out=img, vol=vol, rot=rot, shifts=sh), {}),
        "backproject_2d_to_3d": (bp.backproject_2d_to_3d, dict(images=img, rot=rot, weights=wts, shifts=sh),
                                 dict(D=D)),
        "backproject_2d_to_3d_backward": (bp.backproject_2d_to_3d_backward,
                                          dict(grad_data_vol=vol, images=img, rot=rot, grad_weight_vol=wvol,
                                               weights=wts, shifts=sh), {}),
    }


def args_2d():
    src = z((1, D, D // 2 + 1), C64)
    rot = z((B, P, 2, 2), F32)
    sh = z((B, P, 2), F32)
    img = z((B, P, H, W2), C64)
    wts = z((B, P, H, W2), F32)
    wsrc = z((1, D, D // 2 + 1), F32)
    return {
        "project_2d_to_2d": (bp.project_2d_to_2d, dict(src=src, rot=rot, shifts=sh), dict(H=H)),
        "project_2d_to_2d_backward": (bp.project_2d_to_2d_backward,
                                      dict(grad_out=img, src=src, rot=rot, shifts=sh), {}),
        "backproject_2d_to_2d": (bp.backproject_2d_to_2d, dict(images=img, rot=rot, weights=wts, shifts=sh),
                                 dict(D=D)),
        "backproject_2d_to_2d_backward": (bp.backproject_2d_to_2d_backward,
                                          dict(grad_data=src, images=img, rot=rot, grad_weight=wsrc, weights=wts,
                                               shifts=sh), {}),
    }


ALL = {**args_3d(), **args_2d()}


def bad_variants(t):
    """Same rank, one dimension two larger (each dimension in turn; by two so
    that a box edge stays even and the half axis D//2+1 still moves)."""
    for d in range(t.dim()):
        shape = list(t.shape)
        shape[d] += 2
        yield d, z(tuple(shape), t.dtype)


@pytest.mark.parametrize("name", sorted(ALL))
def test_consistent_shapes_pass_the_shape_checks(name):
    fn, tensors, kw = ALL[name]
    with pytest.raises(ValueError, match="must be on a GPU device"):
        fn(**tensors, **kw)


@pytest.mark.parametrize("name", sorted(ALL))
def test_every_mismatched_dimension_is_rejected(name):
    fn, tensors, kw = ALL[name]
    checked = 0
    for arg in tensors:
        for d, bad in bad_variants(tensors[arg]):
            args = dict(tensors)
            args[arg] = bad
            with pytest.raises(ValueError) as ei:
                fn(**args, **kw)
            msg = str(ei.value)
            assert "must be on a GPU device" not in msg, (name, arg, d, msg)
            checked += 1
    assert checked >= 10


def test_broadcast_sources_may_hold_one_or_B_entries():
    """A lone source with B entries instead of 1 is consistent; 3 is not."""
    for name, arg in (("project_3d_to_2d", "vol"), ("project_2d_to_2d", "src")):
        fn, tensors, kw = ALL[name]
        t = tensors[arg]
        ok = z((B,) + tuple(t.shape[1:]), t.dtype)
        with pytest.raises(ValueError, match="must be on a GPU device"):
            fn(**{**tensors, arg: ok}, **kw)
        bad = z((B + 1,) + tuple(t.shape[1:]), t.dtype)
        with pytest.raises(ValueError, match="batch"):
            fn(**{**tensors, arg: bad}, **kw)


def test_wrong_rank_and_dtype():
    fn, tensors, kw = ALL["project_3d_to_2d"]
    with pytest.raises(ValueError, match="dims"):
        fn(**{**tensors, "rot": z((B, P, 9), F32)}, **kw)
    with pytest.raises(TypeError):
        fn(**{**tensors, "rot": z((B, P, 3, 3), torch.float64)}, **kw)
    fn, tensors, kw = ALL["project_2d_to_2d"]
    with pytest.raises(ValueError, match="shape"):
        fn(**{**tensors, "rot": z((B, P, 3, 3), F32)}, **kw)


def test_preallocated_outputs_are_checked():
    fn, tensors, kw = ALL["project_3d_to_2d"]
    with pytest.raises(ValueError, match="out must have shape"):
        fn(**tensors, **kw, out=z((B, P, H, W2 + 1), C64))
    fn, tensors, kw = ALL["project_3d_to_2d_backward"]
    with pytest.raises(ValueError, match="grad_rot must have shape"):
        fn(**tensors, **kw, grad_rot=z((B, P, 3, 2), F32))
    fn, tensors, kw = ALL["backproject_2d_to_3d"]
    with pytest.raises(ValueError, match="data_vol must have shape"):
        fn(**tensors, **kw, data_vol=z((1, D, D, D // 2), C64))
