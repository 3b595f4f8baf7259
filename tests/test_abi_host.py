"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/tproj.h declares, and rejects bad arguments with the
documented status codes before it enqueues anything."""
import ctypes
import os
import re
import subprocess

import pytest

import back_projection_amd as bp
from back_projection_amd import build_lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tproj.h")

TP_OK, TP_E_NULL, TP_E_SHAPE, TP_E_VALUE, TP_E_DEVICE, TP_E_LAUNCH, TP_E_WORKSPACE = range(7)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(bp.LIB_PATH):
        build_lib.build()
    return bp.lib()


def header_functions(path=HEADER):
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


def test_header_declares_the_binding_symbols():
    assert header_functions() == sorted(bp.HEADER_SYMBOLS)


def test_library_exports_every_header_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", bp.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    missing = [f for f in header_functions() if f not in exported]
    assert not missing, missing
    for f in header_functions():
        assert hasattr(L, f)


SPECTRAL_HEADER = os.path.join(ROOT, "include", "tproj_spectral.h")


def test_spectral_header_declares_the_binding_symbols(L):
    assert header_functions(SPECTRAL_HEADER) == sorted(bp.SPECTRAL_SYMBOLS)
    out = subprocess.run(["nm", "-D", "--defined-only", bp.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    assert set(bp.SPECTRAL_SYMBOLS) <= exported
    for f in bp.SPECTRAL_SYMBOLS:
        assert hasattr(L, f)


BOUNDS_HEADER = os.path.join(ROOT, "include", "tproj_bounds.h")


def test_bounds_header_declares_the_binding_symbols(L):
    assert header_functions(BOUNDS_HEADER) == sorted(bp.BOUNDS_SYMBOLS)
    out = subprocess.run(["nm", "-D", "--defined-only", bp.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    assert set(bp.BOUNDS_SYMBOLS) <= exported
    for f in bp.BOUNDS_SYMBOLS:
        assert hasattr(L, f)


def test_spectral_entry_points_reject_bad_arguments(L):
    """Checked before anything is enqueued (no device needed)."""
    assert L.tp_volume_rfft(7, 1, 1, None, None, None, 0, None) == TP_E_SHAPE        # odd D
    assert L.tp_volume_rfft(64, 0, 1, None, None, None, 0, None) == TP_E_SHAPE       # pad 0
    assert L.tp_volume_rfft(512, 4, 1, None, None, None, 0, None) == TP_E_SHAPE      # N > 1024
    assert L.tp_volume_rfft(64, 2, 1, None, None, None, 0, None) == TP_E_NULL
    assert L.tp_volume_rfft_workspace(63, 1, 1) == ctypes.c_size_t(-1).value
    assert L.tp_images_irfft(9, 1, None, None, None, 0, None) == TP_E_SHAPE
    assert L.tp_images_irfft(64, 0, None, None, None, 0, None) == TP_OK               # nothing to do
    assert L.tp_images_irfft(64, 3, None, None, None, 0, None) == TP_E_NULL
    assert L.tp_images_irfft_workspace(64, 0) == 0
    assert L.tp_weight_images(10, 3, None, None, None, None) == TP_E_SHAPE            # 3 does not divide 10
    assert L.tp_weight_images(0, 1, None, None, None, None) == TP_OK
    assert L.tp_weight_images(12, 3, None, None, None, None) == TP_E_NULL
    assert L.tp_finish_reconstruction(4, None, None, ctypes.c_float(-1.0), None, None) == TP_E_VALUE
    assert L.tp_finish_reconstruction(4, None, None, ctypes.c_float(float("nan")), None, None) == TP_E_VALUE
    assert L.tp_finish_reconstruction(4, None, None, ctypes.c_float(0.5), None, None) == TP_E_NULL
    assert b"lambda" in L.tp_last_error_detail() or b"required" in L.tp_last_error_detail()


def test_probe_library_exports_its_header():
    """libtproj_probes.so (bench.py --peaks) exports what include/tproj_probes.h declares."""
    if not os.path.exists(build_lib.PROBES_LIB):
        build_lib.build()
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "tproj_probes.h")).read(), flags=re.S)
    declared = sorted(set(re.findall(r"^int\s+([A-Za-z_][A-Za-z0-9_]*)\s*\(", text, flags=re.M)))
    assert declared == ["tpp_l2_gather", "tpp_lds_taps", "tpp_lds_width", "tpp_stream_read", "tpp_valu"]
    out = subprocess.run(["nm", "-D", "--defined-only", build_lib.PROBES_LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    assert set(declared) <= exported
    P = ctypes.CDLL(build_lib.PROBES_LIB)
    P.tpp_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    assert P.tpp_stream_read(None, 16, None, 1, None) == -1        # rejected on the host, nothing launched
    assert P.tpp_stream_read(ctypes.c_void_p(0x10000), 24, ctypes.c_void_p(0x10000), 1, None) == -1
    P.tpp_valu.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    assert P.tpp_valu(None, 0, 1, 1, None) == -1                        # no sink
    assert P.tpp_valu(ctypes.c_void_p(0x10000), 11, 1, 1, None) == -1  # no such mode
    assert P.tpp_valu(ctypes.c_void_p(0x10000), -1, 1, 1, None) == -1  # no such mode
    assert P.tpp_valu(ctypes.c_void_p(0x10000), 0, 0, 1, None) == -1   # iters


def test_abi_version_and_strings(L):
    assert L.tp_abi_version() == 1
    for s in range(7):
        assert L.tp_status_string(s)
    assert L.tp_status_string(99) == b"unknown status"


def geom(**kw):
    d = dict(B=1, P=4, Bv=1, Br=1, Bs=0, D=16, H=16, interp=1, oversampling=1.0, radius_cutoff=-1.0)
    d.update(kw)
    return bp.Geom(**d)


@pytest.mark.parametrize("kw,status", [
    (dict(), TP_OK),
    (dict(D=15), TP_E_SHAPE),
    (dict(H=7), TP_E_SHAPE),
    (dict(D=0), TP_E_SHAPE),
    (dict(D=2048), TP_E_SHAPE),
    (dict(P=0), TP_E_SHAPE),
    (dict(B=2, Bv=3), TP_E_SHAPE),
    (dict(B=2, Br=2, Bv=2, Bs=3), TP_E_SHAPE),
    (dict(interp=2), TP_E_VALUE),
    (dict(oversampling=0.0), TP_E_VALUE),
    (dict(oversampling=float("inf")), TP_E_VALUE),
    (dict(radius_cutoff=float("nan")), TP_E_VALUE),
    (dict(B=3, Bv=1, Br=3, Bs=1), TP_OK),
])
def test_validate(L, kw, status):
    g = geom(**kw)
    assert L.tp_validate(ctypes.byref(g)) == status
    if status != TP_OK:
        assert L.tp_last_error_detail()


def test_null_geometry(L):
    assert L.tp_validate(None) == TP_E_NULL


def test_workspace_size(L):
    g = geom()
    sizes = [L.tp_workspace_size(ctypes.byref(g), op) for op in range(8)]
    assert all(0 <= s < (1 << 32) for s in sizes)
    assert sizes[0] > 0 and sizes[0] % 256 == 0     # brick work list of the forward gather
    # 2D ops: the source extension [Bv][D+4][D+5] complex64 at least
    assert all(s >= g.Bv * (g.D + 4) * (g.D + 5) * 8 for s in (sizes[4], sizes[5], sizes[7]))
    assert sizes[6] > 0 and all(s % 256 == 0 for s in sizes[4:])
    assert L.tp_workspace_size(ctypes.byref(g), 8) == ctypes.c_size_t(-1).value
    bad = geom(D=3)
    assert L.tp_workspace_size(ctypes.byref(bad), 0) == ctypes.c_size_t(-1).value


FAKE = ctypes.c_void_p(0x10000)      # an aligned, never-dereferenced address
ODD = ctypes.c_void_p(0x10004)       # 4- but not 8-byte aligned


def test_entry_points_reject_before_launch(L):
    g = geom()
    gp = ctypes.byref(g)
    # forward
    assert L.project_3d_to_2d(gp, None, FAKE, None, FAKE, None, 0, None) == TP_E_NULL
    assert L.project_3d_to_2d(gp, FAKE, None, None, FAKE, None, 0, None) == TP_E_NULL
    assert L.project_3d_to_2d(gp, FAKE, FAKE, None, None, None, 0, None) == TP_E_NULL
    assert L.project_3d_to_2d(gp, ODD, FAKE, None, FAKE, None, 0, None) == TP_E_VALUE
    assert L.project_3d_to_2d(gp, FAKE, FAKE, FAKE, FAKE, None, 0, None) == TP_E_VALUE   # shifts but Bs = 0
    gs = geom(Bs=1)
    assert L.project_3d_to_2d(ctypes.byref(gs), FAKE, FAKE, None, FAKE, None, 0, None) == TP_E_VALUE
    bad = geom(D=9)
    assert L.project_3d_to_2d(ctypes.byref(bad), FAKE, FAKE, None, FAKE, None, 0, None) == TP_E_SHAPE
    # forward backward: rotation grads need the volume, shift grads need shifts
    assert L.project_3d_to_2d_backward(gp, FAKE, None, FAKE, None, None, FAKE, None, None, 0, None) == TP_E_NULL
    assert L.project_3d_to_2d_backward(gp, FAKE, FAKE, FAKE, None, None, None, FAKE, None, 0, None) == TP_E_NULL
    assert L.project_3d_to_2d_backward(gp, None, FAKE, FAKE, None, FAKE, None, None, None, 0, None) == TP_E_NULL
    # back-projection: weights and weight volume come together
    assert L.backproject_2d_to_3d(gp, FAKE, FAKE, FAKE, None, FAKE, None, None, 0, None) == TP_E_NULL
    assert L.backproject_2d_to_3d(gp, FAKE, None, FAKE, None, FAKE, FAKE, None, 0, None) == TP_E_NULL
    assert L.backproject_2d_to_3d(gp, FAKE, None, FAKE, None, None, None, None, 0, None) == TP_E_NULL
    # back-projection backward
    assert L.backproject_2d_to_3d_backward(gp, None, None, FAKE, None, FAKE, None, FAKE, None, None, None, None, 0,
                                           None) == TP_E_NULL
    assert L.backproject_2d_to_3d_backward(gp, FAKE, None, None, None, FAKE, None, None, None, FAKE, None, None, 0,
                                           None) == TP_E_NULL
    assert L.backproject_2d_to_3d_backward(gp, FAKE, FAKE, FAKE, None, FAKE, None, None, None, FAKE, None, None, 0,
                                           None) == TP_E_NULL


def test_python_binding_requires_gpu_tensors():
    import torch
    v = torch.zeros((1, 8, 8, 5), dtype=torch.complex64)
    r = torch.zeros((1, 2, 3, 3), dtype=torch.float32)
    with pytest.raises(ValueError):
        bp.project_3d_to_2d(v, r)
    with pytest.raises(TypeError):
        bp.project_3d_to_2d(v.to(torch.complex128), r)


def test_timing_api_host_side(L):
    """Event timing: state switches and reads need no GPU when nothing was recorded."""
    ms, n = ctypes.c_double(-1.0), ctypes.c_int64(-1)
    assert L.tp_timing_read(0, ctypes.byref(ms), ctypes.byref(n)) == TP_OK
    assert (ms.value, n.value) == (0.0, 0)
    assert L.tp_timing_enable(1) == TP_OK
    assert L.tp_timing_enable(0) == TP_OK
    assert L.tp_timing_read(4, ctypes.byref(ms), ctypes.byref(n)) == TP_E_VALUE
    assert L.tp_timing_read(-1, ctypes.byref(ms), ctypes.byref(n)) == TP_E_VALUE
    assert L.tp_timing_read(1, None, ctypes.byref(n)) == TP_E_NULL
    assert bp.timing_read("fold") == (0.0, 0)


def test_noalloc_forward_rejects_before_launch(L):
    """The allocation-free forward checks its arguments and the size of its
    static work area on the host; on a machine without a GPU a valid call
    stops at the device check (TP_E_DEVICE), never at a launch."""
    g = geom()
    gp = ctypes.byref(g)
    assert L.project_3d_to_2d_noalloc(gp, None, FAKE, None, FAKE, None) == TP_E_NULL
    assert L.project_3d_to_2d_noalloc(gp, FAKE, FAKE, None, None, None) == TP_E_NULL
    assert L.project_3d_to_2d_noalloc(gp, ODD, FAKE, None, FAKE, None) == TP_E_VALUE
    assert L.project_3d_to_2d_noalloc(gp, FAKE, FAKE, FAKE, FAKE, None) == TP_E_VALUE    # shifts but Bs = 0
    big = geom(P=65536, D=128, H=128, radius_cutoff=64.0)
    need = L.tp_workspace_size(ctypes.byref(big), 0)
    assert need > bp.NOALLOC_SCRATCH_BYTES
    assert L.project_3d_to_2d_noalloc(ctypes.byref(big), FAKE, FAKE, None, FAKE, None) == TP_E_WORKSPACE
    assert b"static" in L.tp_last_error_detail()
    # the D = 128 workload with 16384 poses fits
    cfg = geom(P=16384, D=128, H=128, Bs=1, radius_cutoff=64.0)
    assert L.tp_workspace_size(ctypes.byref(cfg), 0) <= bp.NOALLOC_SCRATCH_BYTES
    import torch
    if not torch.cuda.is_available():
        assert L.project_3d_to_2d_noalloc(gp, FAKE, FAKE, None, FAKE, None) == TP_E_DEVICE
        assert L.project_3d_to_2d(gp, FAKE, FAKE, None, FAKE, FAKE, 1 << 20, None) == TP_E_DEVICE
