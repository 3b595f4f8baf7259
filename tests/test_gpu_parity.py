"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Tolerances (relative L2 over the whole output): 1e-5 for the fp32 forward
gathers, 1e-4 for the accumulated back-projection and every gradient.
Small cases span several workgroup tiles, ragged image rows (H/2+1 pixels),
odd-sized boxes, oversampling, cutoffs, batch broadcasting, non-Hermitian
volumes and non-orthonormal maps (the general wrap path).
"""
import zlib

import numpy as np
import pytest
import torch

import back_projection_amd as bp
import oracle
from back_projection_amd import workloads
from tests.helpers import dev, host, log, rel

pytestmark = pytest.mark.gpu

FWD_TOL = 1e-5
BWD_TOL = 1e-4

# name, D, H, P, B, Bv, Br, Bs, interp, o, r, hermitian, rot_kind
SMALL = [
    ("cubic-basic", 16, 16, 5, 1, 1, 1, 1, 1, 1.0, -1.0, True, "rot"),
    ("linear-ragged-cut", 24, 20, 7, 1, 1, 1, 0, 0, 1.0, 9.5, True, "rot"),
    ("cubic-bcast-vol", 20, 24, 4, 2, 1, 2, 1, 1, 1.5, 10.0, False, "rot"),
    ("cubic-bcast-rot", 16, 16, 3, 3, 3, 1, 3, 1, 1.0, -1.0, False, "rot"),
    ("linear-oversampled", 12, 12, 3, 2, 2, 2, 0, 0, 2.5, -1.0, True, "rot"),
    ("cubic-general-map", 32, 32, 6, 1, 1, 1, 1, 1, 1.0, 16.0, False, "wild"),
    ("cubic-H-neq-D", 18, 30, 9, 1, 1, 1, 1, 1, 1.0, 14.0, True, "rot"),
    ("cubic-oversampled-cut", 14, 16, 4, 1, 1, 1, 1, 1, 2.0, 7.0, True, "rot"),
    ("linear-bcast-shifts", 16, 18, 5, 2, 2, 2, 1, 0, 1.0, -1.0, False, "rot"),
    ("cubic-tiny-D", 8, 8, 6, 1, 1, 1, 1, 1, 1.0, -1.0, False, "rot"),
    # images much larger than the box: every voxel has a dozen periodic
    # preimages per axis, more than the fold's per-axis table holds, so the
    # back-projection takes the untabled fold
    ("cubic-many-aliases", 8, 48, 3, 1, 1, 1, 1, 1, 1.0, -1.0, False, "rot"),
    # hundreds of poses per brick and two volumes: several chunks per brick,
    # so the back-projection sums each brick's chunk tiles before the fold
    ("cubic-multivolume-chunks", 24, 24, 512, 2, 2, 2, 2, 1, 1.0, -1.0, True, "rot"),
    ("linear-multivolume-chunks", 32, 32, 1024, 2, 2, 1, 1, 0, 1.0, 15.0, False, "rot"),
]


def make_small(D, H, P, B, Bv, Br, Bs, interp, o, r, herm, rot_kind, seed):
    rng = np.random.default_rng(seed)
    if herm:
        f = rng.standard_normal((Bv, D, D, D)).astype(np.float32)
        vol = np.fft.rfftn(f, axes=(1, 2, 3)).astype(np.complex64)
    else:
        vol = workloads.random_complex(rng, (Bv, D, D, D // 2 + 1))
    rot = workloads.random_rotations(rng, Br * P).reshape(Br, P, 3, 3)
    if rot_kind == "wild":
        rot = (rot * rng.uniform(0.5, 2.5, (Br, P, 1, 1)) + 0.3 * rng.standard_normal((Br, P, 3, 3))).astype(np.float32)
    sh = rng.uniform(-4, 4, (Bs, P, 2)).astype(np.float32) if Bs else None
    imgs = workloads.random_complex(rng, (B, P, H, H // 2 + 1))
    wts = rng.random((B, P, H, H // 2 + 1)).astype(np.float32)
    gwv = rng.standard_normal((Bv, D, D, D // 2 + 1)).astype(np.float32)
    gdv = workloads.random_complex(rng, (Bv, D, D, D // 2 + 1))
    return vol, rot, sh, imgs, wts, gdv, gwv


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_all_ops(case):
    name, D, H, P, B, Bv, Br, Bs, interp, o, r, herm, rot_kind = case
    log(f"[parity] small case {name}")
    vol, rot, sh, imgs, wts, gdv, gwv = make_small(D, H, P, B, Bv, Br, Bs, interp, o, r, herm, rot_kind,
                                                   seed=zlib.crc32(name.encode()))
    tv, tr, ts, ti, tw, tgd, tgw = dev(vol, rot, sh, imgs, wts, gdv, gwv)
    kw = dict(interp=interp, oversampling=o, radius_cutoff=r)
    okw = dict(interp=interp, o=o, r=r)

    out = bp.project_3d_to_2d(tv, tr, ts, H=H, B=B, **kw)
    ref = oracle.project(vol, rot, sh, H=H, B=B, **okw)
    assert rel(out, ref) <= FWD_TOL, ("forward", rel(out, ref))

    gv, gr, gs = bp.project_3d_to_2d_backward(ti, tv, tr, ts, **kw)
    rgv, rgr, rgs = oracle.project_backward(imgs, vol, rot, sh, **okw)
    assert rel(gv, rgv) <= BWD_TOL, ("grad_vol", rel(gv, rgv))
    assert rel(gr, rgr) <= BWD_TOL, ("grad_rot", rel(gr, rgr))
    assert np.all(host(gr)[..., 2] == 0)
    if sh is not None:
        assert rel(gs, rgs) <= BWD_TOL, ("grad_shifts", rel(gs, rgs))

    dvol, wvol = bp.backproject_2d_to_3d(ti, tr, tw, ts, D=D, Bv=Bv, **kw)
    rdv, rwv = oracle.backproject(imgs, rot, wts, sh, D=D, Bv=Bv, **okw)
    assert rel(dvol, rdv) <= BWD_TOL, ("bp data", rel(dvol, rdv))
    assert rel(wvol, rwv) <= BWD_TOL, ("bp weights", rel(wvol, rwv))
    dvol2, none = bp.backproject_2d_to_3d(ti, tr, None, ts, D=D, Bv=Bv, **kw)
    assert none is None and rel(dvol2, rdv) <= BWD_TOL

    gi, gw, gr2, gs2 = bp.backproject_2d_to_3d_backward(tgd, ti, tr, tgw, tw, ts, **kw)
    rgi, rgw, rgr2, rgs2 = oracle.backproject_backward(gdv, imgs, rot, gwv, wts, sh, **okw)
    assert rel(gi, rgi) <= FWD_TOL, ("grad_images", rel(gi, rgi))
    assert rel(gw, rgw) <= FWD_TOL, ("grad_weights", rel(gw, rgw))
    assert rel(gr2, rgr2) <= BWD_TOL, ("bp grad_rot", rel(gr2, rgr2))
    if sh is not None:
        assert rel(gs2, rgs2) <= BWD_TOL, ("bp grad_shifts", rel(gs2, rgs2))


def test_more_poses_than_a_chunk_holds():
    """70000 poses against one volume: the pose list is longer than the 65535
    poses a work item's hit list can address, so every brick is split."""
    log("[parity] 70000 poses, D=8")
    vol, rot, sh, imgs, wts, gdv, gwv = make_small(8, 8, 70000, 1, 1, 1, 1, 1, 1.0, -1.0, True, "rot", 11)
    tv, tr, ts, ti, tw = dev(vol, rot, sh, imgs, wts)
    out = bp.project_3d_to_2d(tv, tr, ts, H=8)
    assert rel(out, oracle.project(vol, rot, sh, H=8, interp=1)) <= FWD_TOL
    gv, gr, gs = bp.project_3d_to_2d_backward(ti, tv, tr, ts)
    rgv, rgr, rgs = oracle.project_backward(imgs, vol, rot, sh, interp=1)
    assert rel(gv, rgv) <= BWD_TOL and rel(gr, rgr) <= BWD_TOL and rel(gs, rgs) <= BWD_TOL
    dvol, wvol = bp.backproject_2d_to_3d(ti, tr, tw, ts, D=8)
    rdv, rwv = oracle.backproject(imgs, rot, wts, sh, D=8, interp=1)
    assert rel(dvol, rdv) <= BWD_TOL and rel(wvol, rwv) <= BWD_TOL


def test_requested_outputs_only():
    """NULL outputs are skipped; a missing weight upstream gives zero grad_weights."""
    vol, rot, sh, imgs, wts, gdv, gwv = make_small(16, 16, 3, 1, 1, 1, 1, 1, 1.0, -1.0, True, "rot", 5)
    tv, tr, ts, ti, tw, tgd = dev(vol, rot, sh, imgs, wts, gdv)
    gv, gr, gs = bp.project_3d_to_2d_backward(ti, tv, tr, ts, need_vol=False, need_shifts=False)
    assert gv is None and gs is None
    rgv, rgr, _ = oracle.project_backward(imgs, vol, rot, sh, interp=1)
    assert rel(gr, rgr) <= BWD_TOL
    gi, gw, gr2, gs2 = bp.backproject_2d_to_3d_backward(tgd, ti, tr, None, tw, ts, need_images=False)
    assert gi is None
    assert float(gw.abs().max()) == 0.0
    _, _, rgr2, rgs2 = oracle.backproject_backward(gdv, imgs, rot, None, wts, sh, interp=1)
    assert rel(gr2, rgr2) <= BWD_TOL and rel(gs2, rgs2) <= BWD_TOL


def test_empty_and_degenerate():
    """A zero volume projects to exact zeros; r = 0 keeps only DC; P = 1."""
    D = 16
    rng = np.random.default_rng(9)
    vol = workloads.random_complex(rng, (1, D, D, D // 2 + 1))
    rot = workloads.random_rotations(rng, 1)[None]
    tv, tr = dev(vol, rot)
    z = bp.project_3d_to_2d(torch.zeros_like(tv), tr)
    assert float(z.abs().max()) == 0.0
    out = bp.project_3d_to_2d(tv, tr, radius_cutoff=0.0)
    h = host(out)[0, 0]
    assert np.count_nonzero(h) <= 1 and abs(h[0, 0] - vol[0, 0, 0, 0]) < 1e-6 * abs(vol[0, 0, 0, 0])
    gz, _ = bp.backproject_2d_to_3d(torch.zeros((1, 1, D, D // 2 + 1), dtype=torch.complex64, device="cuda:0"), tr)
    assert float(gz.abs().max()) == 0.0


def test_repeatable_forward_and_grads():
    """The forward and the (fixed-point) volume gradient are bitwise repeatable;
    the rotation/shift gradients add per-brick partial sums with float atomics
    and repeat up to rounding."""
    vol, rot, sh, imgs, *_ = make_small(32, 32, 16, 1, 1, 1, 1, 1, 1.0, 16.0, True, "rot", 11)
    tv, tr, ts, ti = dev(vol, rot, sh, imgs)
    a = bp.project_3d_to_2d(tv, tr, ts, radius_cutoff=16.0)
    b = bp.project_3d_to_2d(tv, tr, ts, radius_cutoff=16.0)
    assert torch.equal(a, b)
    v1, r1, s1 = bp.project_3d_to_2d_backward(ti, tv, tr, ts, radius_cutoff=16.0)
    v2, r2, s2 = bp.project_3d_to_2d_backward(ti, tv, tr, ts, radius_cutoff=16.0)
    assert torch.equal(v1, v2)
    assert rel(r1, r2) <= 1e-6 and rel(s1, s2) <= 1e-6
    d1, w1 = bp.backproject_2d_to_3d(ti, tr, ti.real.abs().contiguous(), ts, radius_cutoff=16.0)
    d2, w2 = bp.backproject_2d_to_3d(ti, tr, ti.real.abs().contiguous(), ts, radius_cutoff=16.0)
    assert torch.equal(d1, d2) and torch.equal(w1, w2)


def test_adjoint_identity_fp32():
    """<P x, y> = <x, P^T y> with both sides from the GPU."""
    D, H, P = 32, 32, 40
    rng = np.random.default_rng(13)
    x = workloads.random_complex(rng, (1, D, D, D // 2 + 1))
    y = workloads.random_complex(rng, (1, P, H, H // 2 + 1))
    rot = workloads.random_rotations(rng, P)[None]
    sh = workloads.random_shifts(rng, P, 4.0)[None]
    tx, ty, tr, ts = dev(x, y, rot, sh)
    Px = host(bp.project_3d_to_2d(tx, tr, ts, radius_cutoff=15.0)).astype(np.complex128)
    PTy = host(bp.backproject_2d_to_3d(ty, tr, None, ts, radius_cutoff=15.0)[0]).astype(np.complex128)
    lhs = np.real(np.vdot(Px.ravel(), y.ravel().astype(np.complex128)))
    rhs = np.real(np.vdot(x.ravel().astype(np.complex128), PTy.ravel()))
    scale = np.linalg.norm(Px) * np.linalg.norm(y)
    assert abs(lhs - rhs) <= 1e-5 * scale


# ---------------------------------------------------------------------------
# the five workloads, at full size, in the launch configuration the bench uses
# ---------------------------------------------------------------------------

def _sample(rng, P, k):
    return np.sort(rng.choice(P, size=min(k, P), replace=False))


def test_workload1_full():
    w = workloads.make(1)
    log("[parity] workload 1 full")
    tv, tr = dev(w.vol, w.rot)
    out = bp.project_3d_to_2d(tv, tr, None, interp="linear", radius_cutoff=w.radius)
    ref = oracle.project(w.vol, w.rot, None, interp=0, r=w.radius)
    assert rel(out, ref) <= FWD_TOL


def test_workload2_full():
    w = workloads.make(2)
    log("[parity] workload 2 full")
    tv, tr, ts, tg = dev(w.vol, w.rot, w.shifts, w.grad_out)
    out = bp.project_3d_to_2d(tv, tr, ts, interp="cubic", radius_cutoff=w.radius)
    ref = oracle.project(w.vol, w.rot, w.shifts, interp=1, r=w.radius)
    assert rel(out, ref) <= FWD_TOL, rel(out, ref)
    gv, gr, _ = bp.project_3d_to_2d_backward(tg, tv, tr, ts, interp="cubic", radius_cutoff=w.radius,
                                             need_shifts=False)
    rgv, rgr, _ = oracle.project_backward(w.grad_out, w.vol, w.rot, w.shifts, interp=1, r=w.radius, need_shifts=False)
    assert rel(gv, rgv) <= BWD_TOL, rel(gv, rgv)
    assert rel(gr, rgr) <= BWD_TOL, rel(gr, rgr)


def _fwd_bwd_full(cfg, nsample):
    w = workloads.make(cfg, with_grad=False)
    B, P, H = w.B, w.P, w.H
    rng = np.random.default_rng(cfg)
    idx = _sample(rng, P, nsample)
    log(f"[parity] workload {cfg} full: B={B} P={P} D={w.D}, {len(idx)} sampled poses")
    tv, tr, ts = dev(w.vol, w.rot, w.shifts)
    out = bp.project_3d_to_2d(tv, tr, ts, interp="cubic", radius_cutoff=w.radius)
    ref = oracle.project(w.vol, w.rot[:, idx], w.shifts[:, idx], interp=1, r=w.radius)
    assert rel(out[:, idx], ref) <= FWD_TOL, rel(out[:, idx], ref)
    # upstream gradient that is nonzero only on the sampled poses: the full
    # launch then has to reproduce the oracle on those poses and give exact
    # zeros for the rotation/shift grads of the others
    gsub = np.stack([workloads.random_complex(np.random.default_rng([cfg, b]), (len(idx), H, H // 2 + 1))
                     for b in range(B)])
    tg = torch.zeros((B, P, H, H // 2 + 1), dtype=torch.complex64, device="cuda:0")
    tg[:, torch.from_numpy(idx).cuda()] = torch.from_numpy(gsub).cuda()
    gv, gr, gs = bp.project_3d_to_2d_backward(tg, tv, tr, ts, interp="cubic", radius_cutoff=w.radius)
    rgv, rgr, rgs = oracle.project_backward(gsub, w.vol, w.rot[:, idx], w.shifts[:, idx], interp=1, r=w.radius)
    assert rel(gv, rgv) <= BWD_TOL, rel(gv, rgv)
    assert rel(gr[:, idx], rgr) <= BWD_TOL, rel(gr[:, idx], rgr)
    assert rel(gs[:, idx], rgs) <= BWD_TOL, rel(gs[:, idx], rgs)
    rest = np.setdiff1d(np.arange(P), idx)
    assert float(gr[:, rest].abs().max()) == 0.0 and float(gs[:, rest].abs().max()) == 0.0
    # adjoint identity over the full launch: <P V, G> = <V, P^T G>
    lhs = np.real(np.vdot(host(out[:, idx]).astype(np.complex128).ravel(), gsub.astype(np.complex128).ravel()))
    rhs = np.real(np.vdot(w.vol.astype(np.complex128).ravel(), host(gv).astype(np.complex128).ravel()))
    assert abs(lhs - rhs) <= 1e-5 * np.linalg.norm(host(out[:, idx])) * np.linalg.norm(gsub)


def test_workload3_full_sampled():
    _fwd_bwd_full(3, 96)


def test_workload5_full_sampled():
    _fwd_bwd_full(5, 24)


def test_workload4_full_sampled():
    w = workloads.make(4)
    P, H, D = w.P, w.H, w.D
    idx = _sample(np.random.default_rng(4), P, 48)
    log(f"[parity] workload 4 full: P={P} D={D}, {len(idx)} sampled images")
    imgs = np.zeros_like(w.images)
    wts = np.zeros_like(w.weights)
    imgs[:, idx] = w.images[:, idx]
    wts[:, idx] = w.weights[:, idx]
    ti, tw, tr = dev(imgs, wts, w.rot)
    dvol, wvol = bp.backproject_2d_to_3d(ti, tr, tw, None, D=D, interp="cubic")
    rdv, rwv = oracle.backproject(w.images[:, idx], w.rot[:, idx], w.weights[:, idx], None, D=D, interp=1)
    assert rel(dvol, rdv) <= BWD_TOL, rel(dvol, rdv)
    assert rel(wvol, rwv) <= BWD_TOL, rel(wvol, rwv)
    # linearity over the full launch: BP(all) = BP(sampled) + BP(rest)
    ti_all, tw_all = dev(w.images, w.weights)
    dall, wall = bp.backproject_2d_to_3d(ti_all, tr, tw_all, None, D=D, interp="cubic")
    drest, wrest = bp.backproject_2d_to_3d(ti_all - ti, tr, tw_all - tw, None, D=D, interp="cubic")
    assert rel(dvol + drest, dall) <= BWD_TOL
    assert rel(wvol + wrest, wall) <= BWD_TOL


def test_direct_path_large_image():
    """H = 4096 is past the brick enumeration's limits: the direct kernels run.
    (o = 1/4 keeps |p| <= 50 inside a few periods of the D = 64 box, where fp32
    sample coordinates hold the forward tolerance.)"""
    D, H, r, o = 64, 4096, 200.0, 0.25
    rng = np.random.default_rng(41)
    vol = workloads.random_complex(rng, (1, D, D, D // 2 + 1))
    rot = workloads.random_rotations(rng, 2).reshape(1, 2, 3, 3)
    sh = rng.uniform(-3, 3, (1, 2, 2)).astype(np.float32)
    g = workloads.random_complex(rng, (1, 2, H, H // 2 + 1))
    tv, tr, ts, tg = dev(vol, rot, sh, g)
    log("[parity] direct path, H=4096")
    out = bp.project_3d_to_2d(tv, tr, ts, H=H, radius_cutoff=r, oversampling=o)
    assert rel(out, oracle.project(vol, rot, sh, H=H, interp=1, r=r, o=o)) <= FWD_TOL
    gv, gr, gs = bp.project_3d_to_2d_backward(tg, tv, tr, ts, radius_cutoff=r, oversampling=o)
    rgv, rgr, rgs = oracle.project_backward(g, vol, rot, sh, interp=1, r=r, o=o)
    assert rel(gv, rgv) <= BWD_TOL and rel(gr, rgr) <= BWD_TOL and rel(gs, rgs) <= BWD_TOL


def test_large_volume_sampled():
    """D = 384 (cubic, cutoff D/2, shifts): sampled poses against the oracle and
    the adjoint identity for the volume gradient over the whole launch."""
    D, H, P, r = 384, 384, 40, 192.0
    rng = np.random.default_rng(43)
    vol = workloads.random_complex(rng, (1, D, D, D // 2 + 1))
    rot = workloads.random_rotations(rng, P).reshape(1, P, 3, 3)
    sh = rng.uniform(-6, 6, (1, P, 2)).astype(np.float32)
    idx = np.sort(rng.choice(P, 3, replace=False))
    log(f"[parity] large volume D={D}, P={P}, sampled poses {idx.tolist()}")
    tv, tr, ts = dev(vol, rot, sh)
    out = bp.project_3d_to_2d(tv, tr, ts, radius_cutoff=r)
    ref = oracle.project(vol, rot[:, idx], sh[:, idx], interp=1, r=r)
    assert rel(out[:, idx], ref) <= FWD_TOL, rel(out[:, idx], ref)
    g = workloads.random_complex(rng, (1, P, H, H // 2 + 1))
    tg, = dev(g)
    gv, gr, gs = bp.project_3d_to_2d_backward(tg, tv, tr, ts, radius_cutoff=r)
    _, rgr, rgs = oracle.project_backward(g[:, idx], vol, rot[:, idx], sh[:, idx], interp=1, r=r,
                                          need_vol=False)
    assert rel(gr[:, idx], rgr) <= BWD_TOL, rel(gr[:, idx], rgr)
    assert rel(gs[:, idx], rgs) <= BWD_TOL, rel(gs[:, idx], rgs)
    lhs = np.real(np.vdot(host(out).astype(np.complex128).ravel(), g.astype(np.complex128).ravel()))
    rhs = np.real(np.vdot(vol.astype(np.complex128).ravel(), host(gv).astype(np.complex128).ravel()))
    assert abs(lhs - rhs) <= 1e-5 * np.linalg.norm(host(out)) * np.linalg.norm(g), (lhs, rhs)


def test_lattice_rotations_are_exact():
    """The 24 signed permutations map every pixel to a lattice point, where
    both kernels take the stored entry itself (weights exactly 1 and 0): the
    GPU forward must equal the oracle bit for bit, Friedel conjugation
    included.  The backward there meets the linear kernel's kink: the volume,
    rotation and shift gradients (linear and cubic) must match the oracle's
    derivative of the cell [floor(p), floor(p)+1)."""
    import itertools
    D = 16
    rng = np.random.default_rng(29)
    vol = workloads.random_complex(rng, (1, D, D, D // 2 + 1))
    mats = []
    for perm in itertools.permutations(range(3)):
        for sg in itertools.product((1, -1), repeat=3):
            R = np.zeros((3, 3), np.float32)
            for i in range(3):
                R[i, perm[i]] = sg[i]
            if np.linalg.det(R) > 0:
                mats.append(R)
    rot = np.array(mats)[None]
    P = rot.shape[1]
    sh = rng.uniform(-3, 3, (1, P, 2)).astype(np.float32)
    g = workloads.random_complex(rng, (1, P, D, D // 2 + 1))
    wts = rng.random((1, P, D, D // 2 + 1)).astype(np.float32)
    gwv = rng.standard_normal((1, D, D, D // 2 + 1)).astype(np.float32)
    log(f"[parity] {P} lattice rotations, D={D}")
    tv, tr, ts, tg, tw, tgw = dev(vol, rot, sh, g, wts, gwv)
    for interp, code in (("linear", 0), ("cubic", 1)):
        out = host(bp.project_3d_to_2d(tv, tr, interp=interp))
        ref = oracle.project(vol, rot, interp=code).astype(np.complex64)
        assert np.array_equal(out, ref), (interp, float(np.abs(out - ref).max()))
        gv, gr, gs = bp.project_3d_to_2d_backward(tg, tv, tr, ts, interp=interp)
        rgv, rgr, rgs = oracle.project_backward(g, vol, rot, sh, interp=code)
        errs = (rel(gv, rgv), rel(gr, rgr), rel(gs, rgs))
        log(f"[parity] lattice {interp}: grad_vol {errs[0]:.2e} grad_rot {errs[1]:.2e} grad_shifts {errs[2]:.2e}")
        assert max(errs) <= BWD_TOL, (interp, errs)
        assert np.all(host(gr)[..., 2] == 0)
        # back-projection backward: images g, weights, grad volumes (vol, gwv)
        gi, gw, gr2, gs2 = bp.backproject_2d_to_3d_backward(tv, tg, tr, tgw, tw, ts, interp=interp)
        rgi, rgw, rgr2, rgs2 = oracle.backproject_backward(vol, g, rot, gwv, wts, sh, interp=code)
        errs = (rel(gi, rgi), rel(gw, rgw), rel(gr2, rgr2), rel(gs2, rgs2))
        assert max(errs) <= BWD_TOL, (interp, errs)
