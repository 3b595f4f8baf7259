"""Dense full-size parity: every pose of the benchmarked workloads against the
fp64 oracle, in the launch configuration the benchmark times.

* D = 128 cubic, 16384 poses, shifts, cutoff 64: the forward and the full
  backward with the benchmark's dense N(0, 1) upstream gradient.
* D = 256 cubic back-projection of all 4096 noisy blob images with their
  CTF^2-like weights.
* 4 x D = 192 cubic, 8192 poses each: forward and full backward, one GPU call
  for all four volumes, checked volume by volume.

Besides the global relative L2 (1e-5 forward, 1e-4 back-projection and
gradients), every output is checked per radial shell of |k| (8 equal-width
shells) against the same bar: the global figure is dominated by the large
low-frequency entries, while the fixed-point accumulation's quantum is set per
radial band, so the small outer-shell values need a check of their own.
"""
import numpy as np
import pytest
import torch

import back_projection_amd as bp
import oracle
from back_projection_amd import workloads
from tests.helpers import dev, host, image_kmag, log, rel, shell_rels, volume_kmag

pytestmark = pytest.mark.gpu

FWD_TOL = 1e-5
BWD_TOL = 1e-4


def check(name, got, ref, tol, kmag):
    g = rel(got, ref)
    shells = shell_rels(got, ref, kmag)
    worst = max(s[2] for s in shells)
    log(f"[dense] {name}: global {g:.2e}, per shell " + " ".join(f"{s[2]:.1e}" for s in shells))
    assert g <= tol, (name, g)
    assert worst <= tol, (name, shells)
    return g, worst


def per_pose_rel(got, ref):
    """Largest per-pose relative L2 error of a [.., P, k] gradient."""
    got = np.asarray(got, np.float64).reshape(-1, int(np.prod(ref.shape[-2:])) if ref.ndim == 4 else ref.shape[-1])
    ref = np.asarray(ref, np.float64).reshape(got.shape)
    num = np.linalg.norm(got - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    return float(np.max(num / np.maximum(den, 1e-30)))


def test_workload3_dense():
    w = workloads.make(3)
    log(f"[dense] workload 3: D={w.D} P={w.P}, all poses, dense upstream")
    tv, tr, ts, tg = dev(w.vol, w.rot, w.shifts, w.grad_out)
    kw = dict(interp="cubic", radius_cutoff=w.radius)
    out = host(bp.project_3d_to_2d(tv, tr, ts, **kw))
    gv, gr, gs = bp.project_3d_to_2d_backward(tg, tv, tr, ts, **kw)
    gv, gr, gs = host(gv), host(gr), host(gs)
    del tg
    torch.cuda.empty_cache()
    ref = oracle.project(w.vol, w.rot, w.shifts, interp=1, r=w.radius)
    check("forward", out, ref, FWD_TOL, image_kmag(w.H))
    del ref, out
    rgv, rgr, rgs = oracle.project_backward(w.grad_out, w.vol, w.rot, w.shifts, interp=1, r=w.radius)
    check("grad_vol", gv, rgv, BWD_TOL, volume_kmag(w.D))
    for name, a, b in (("grad_rot", gr, rgr), ("grad_shifts", gs, rgs)):
        e = rel(a, b)
        log(f"[dense] {name}: global {e:.2e}, worst pose {per_pose_rel(a, b):.2e}")
        assert e <= BWD_TOL, (name, e)
    assert np.all(gr[..., 2] == 0)


def test_workload4_dense():
    w = workloads.make(4)
    log(f"[dense] workload 4: D={w.D} P={w.P}, all images and weights")
    ti, tw, tr = dev(w.images, w.weights, w.rot)
    dvol, wvol = bp.backproject_2d_to_3d(ti, tr, tw, None, D=w.D, interp="cubic")
    dvol, wvol = host(dvol), host(wvol)
    del ti, tw
    torch.cuda.empty_cache()
    rdv, rwv = oracle.backproject(w.images, w.rot, w.weights, None, D=w.D, interp=1)
    k = volume_kmag(w.D)
    check("data volume", dvol, rdv, BWD_TOL, k)
    check("weight volume", wvol, rwv, BWD_TOL, k)


@pytest.fixture(scope="module")
def workload5_gpu():
    """One GPU call per op over all four volumes (the benchmarked launch);
    results on the host."""
    w = workloads.make(5)
    log(f"[dense] workload 5: B={w.B} D={w.D} P={w.P}, one launch for all volumes")
    tv, tr, ts, tg = dev(w.vol, w.rot, w.shifts, w.grad_out)
    kw = dict(interp="cubic", radius_cutoff=w.radius)
    out = host(bp.project_3d_to_2d(tv, tr, ts, **kw))
    gv, gr, gs = bp.project_3d_to_2d_backward(tg, tv, tr, ts, **kw)
    res = dict(w=w, out=out, gv=host(gv), gr=host(gr), gs=host(gs))
    del tv, tr, ts, tg, gv, gr, gs
    torch.cuda.empty_cache()
    return res


@pytest.mark.slow
@pytest.mark.parametrize("b", range(4))
def test_workload5_dense(workload5_gpu, b):
    r = workload5_gpu
    w = r["w"]
    sl = slice(b, b + 1)
    log(f"[dense] workload 5, volume {b}: oracle over its {w.P} poses")
    ref = oracle.project(w.vol[sl], w.rot[sl], w.shifts[sl], interp=1, r=w.radius)
    check(f"forward[{b}]", r["out"][sl], ref, FWD_TOL, image_kmag(w.H))
    del ref
    rgv, rgr, rgs = oracle.project_backward(w.grad_out[sl], w.vol[sl], w.rot[sl], w.shifts[sl], interp=1,
                                            r=w.radius)
    check(f"grad_vol[{b}]", r["gv"][sl], rgv, BWD_TOL, volume_kmag(w.D))
    for name, a, ref_ in (("grad_rot", r["gr"][sl], rgr), ("grad_shifts", r["gs"][sl], rgs)):
        e = rel(a, ref_)
        log(f"[dense] {name}[{b}]: global {e:.2e}, worst pose {per_pose_rel(a, ref_):.2e}")
        assert e <= BWD_TOL, (name, b, e)
