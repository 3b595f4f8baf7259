"""The autograd wrappers (back_projection_amd.autograd) on the GPU: their
gradients equal the backward entry points' for the same upstream gradient,
inputs without requires_grad are skipped, the complex convention matches
torch's (a loss sum |out|^2 gives upstream 2 out), and a directional finite
difference of a real loss agrees with the autograd gradient to the
precision fp32 allows."""
import numpy as np
import pytest
import torch

import back_projection_amd as bp
from back_projection_amd import autograd as ag
from back_projection_amd import workloads
from tests.helpers import log, rel

pytestmark = pytest.mark.gpu


def setup3d(seed=900, D=24, P=6):
    rng = np.random.default_rng(seed)
    vol = workloads.rfft_volume(workloads.blob_volume_real(D, *workloads.blob_params(rng, 30, D / 3)))[None]
    rot = workloads.random_rotations(rng, P)[None]
    sh = workloads.random_shifts(rng, P, 3.0)[None]
    return [torch.from_numpy(a).cuda() for a in (vol, rot, sh)]


def test_project_autograd_matches_the_backward_entry_point():
    log("[autograd] project 3D")
    tv, tr, ts = setup3d()
    v, r, s = (t.clone().requires_grad_(True) for t in (tv, tr, ts))
    out = ag.project_3d_to_2d_ag(v, r, s, radius_cutoff=12.0)
    # sum |out|^2 alone does not depend on the shifts; a fixed complex weight
    # makes every gradient nonzero: upstream = w + 2 out
    w = torch.from_numpy(workloads.random_complex(np.random.default_rng(905), tuple(out.shape))).cuda()
    loss = (out * w.conj()).real.sum() + (out.abs() ** 2).sum()
    loss.backward()
    gv, gr, gs = bp.project_3d_to_2d_backward((w + 2 * out).detach().contiguous(), tv, tr, ts, radius_cutoff=12.0)
    torch.cuda.synchronize()
    # float atomics in the rotation/shift sums: agreement to rounding, not bitwise
    assert rel(v.grad, gv) <= 1e-6 and rel(r.grad, gr) <= 1e-5 and rel(s.grad, gs) <= 1e-5


def test_project_autograd_directional_derivative():
    """d/dt L(R + t dR, s + t ds) by central differences against <grad, d>."""
    log("[autograd] directional derivative")
    tv, tr, ts = setup3d(901)
    rng = np.random.default_rng(902)
    dR = torch.from_numpy(rng.standard_normal(tr.shape).astype(np.float32)).cuda() * 1e-2
    dS = torch.from_numpy(rng.standard_normal(ts.shape).astype(np.float32)).cuda() * 1e-1
    w = torch.from_numpy(workloads.random_complex(rng, (1, 6, 24, 13))).cuda()

    def L(r, s):
        out = ag.project_3d_to_2d_ag(tv, r, s, radius_cutoff=12.0)
        return (out * w.conj()).real.sum()

    r = tr.clone().requires_grad_(True)
    s = ts.clone().requires_grad_(True)
    L(r, s).backward()
    pred = float((r.grad * dR).sum() + (s.grad * dS).sum())
    h = 0.5
    with torch.no_grad():
        fd = (float(L(tr + h * dR, ts + h * dS)) - float(L(tr - h * dR, ts - h * dS))) / (2 * h)
    log(f"  predicted {pred:.6e}, central difference {fd:.6e}")
    assert abs(fd - pred) <= 2e-2 * abs(pred)


def test_backproject_autograd_with_weights_and_partial_requires_grad():
    log("[autograd] backproject 3D with weights")
    rng = np.random.default_rng(903)
    D, P = 20, 5
    img = torch.from_numpy(workloads.random_complex(rng, (1, P, D, D // 2 + 1))).cuda()
    wts = torch.from_numpy(workloads.ctf2_like_weights(rng, P, D, P)[None].astype(np.float32)).cuda()
    rot = torch.from_numpy(workloads.random_rotations(rng, P)[None]).cuda()
    sh = torch.from_numpy(workloads.random_shifts(rng, P, 2.0)[None]).cuda()
    gd = torch.from_numpy(workloads.random_complex(rng, (1, D, D, D // 2 + 1))).cuda()
    gw = torch.from_numpy(rng.standard_normal((1, D, D, D // 2 + 1)).astype(np.float32)).cuda()
    i, r = img.clone().requires_grad_(True), rot.clone().requires_grad_(True)
    data, wvol = ag.backproject_2d_to_3d_ag(i, r, wts, sh, D=D)
    ((data * gd.conj()).real.sum() + (wvol * gw).sum()).backward()
    gi, gwt, gr, gs = bp.backproject_2d_to_3d_backward(gd, img, rot, gw, wts, sh)
    torch.cuda.synchronize()
    assert rel(i.grad, gi) <= 1e-6 and rel(r.grad, gr) <= 1e-5


def test_2d_autograd_round_trip():
    log("[autograd] 2D project + accumulate")
    rng = np.random.default_rng(904)
    D, P = 16, 4
    src = torch.from_numpy(workloads.blob_image_rfft(rng, D, 10, D / 3)[None]).cuda()
    ang = rng.uniform(0, 2 * np.pi, P)
    rot = torch.from_numpy(np.stack([np.stack([np.cos(ang), -np.sin(ang)], -1),
                                     np.stack([np.sin(ang), np.cos(ang)], -1)], -2)[None].astype(np.float32)).cuda()
    s = src.clone().requires_grad_(True)
    r = rot.clone().requires_grad_(True)
    out = ag.project_2d_to_2d_ag(s, r, radius_cutoff=8.0)
    rec = ag.backproject_2d_to_2d_ag(out, r, D=D, radius_cutoff=8.0)
    (rec.abs() ** 2).sum().backward()
    assert s.grad is not None and r.grad is not None
    assert torch.isfinite(s.grad).all() and torch.isfinite(r.grad).all()
    # the same chain through the entry points by hand
    g_rec = 2 * rec.detach()
    gi, _, gr2, _ = bp.backproject_2d_to_2d_backward(g_rec.contiguous(), out.detach().contiguous(), rot,
                                                     radius_cutoff=8.0, need_weights=False, need_shifts=False)
    gs, gr1, _ = bp.project_2d_to_2d_backward(gi, src, rot, need_shifts=False, radius_cutoff=8.0)
    torch.cuda.synchronize()
    assert rel(s.grad, gs) <= 1e-5
    assert rel(r.grad, gr1 + gr2) <= 1e-5
