"""Host-side logic of bench.py (no GPU): the one-GPU contract, the roofline
object of the JSON line, the digest rule for counter-measured traffic, and
the operation-rate helper."""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("argv, env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_exits_with_a_message(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                       env=dict(os.environ, **env), timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_sources_digest_is_stable_and_hex(bench):
    a, b = bench.sources_digest(), bench.sources_digest()
    assert a == b and len(a) == 64
    int(a, 16)


def test_traffic_is_null_when_the_sources_changed(bench, monkeypatch):
    real = bench.sources_digest()
    monkeypatch.setattr(bench, "TRAFFIC", {"gradient": {"sources_sha256": "0" * 64, "fetch_bytes": 10,
                                                         "write_bytes": 5}})
    assert bench.measured_traffic("gradient") is None
    monkeypatch.setattr(bench, "TRAFFIC", {"gradient": {"sources_sha256": real, "fetch_bytes": 10,
                                                         "write_bytes": 5}})
    assert bench.measured_traffic("gradient") == 15
    assert bench.measured_traffic("no-such-kernel") is None


def test_valu_issue_follows_the_digest(bench, monkeypatch):
    real = bench.sources_digest()
    monkeypatch.setattr(bench, "VALU_ISSUE", {"gradient": {"sources_sha256": real, "valu_per_cu_clock": 1.5}})
    v = bench.valu_issue("gradient")
    assert v["achieved"] == 1.5 and v["peak"] == 2.0 and v["frac"] == pytest.approx(0.75)
    monkeypatch.setattr(bench, "VALU_ISSUE", {"gradient": {"sources_sha256": "0" * 64, "valu_per_cu_clock": 1.5}})
    assert bench.valu_issue("gradient") is None


def _kernel(avg_ms, flops, tap_bytes, launches=20):
    return {"avg_ms": avg_ms, "launches": launches, "flops": flops, "flops_per_pixel": 768, "tap_bytes": tap_bytes,
            "l2_frac": 0.5, "lds_frac": 0.25, "hbm_GBps": 100.0, "hbm_frac": 0.0125, "tflops": 1.0,
            "alu_frac": 0.01}


def test_roofline_object(bench):
    kernels = {"forward": _kernel(1.0, 3.0e10, 5.0e10), "gradient": _kernel(4.0, 8.0e10, 5.0e10)}
    r = bench.brick_roofline(kernels, {"gradient": 2.0})
    # the dominant kernel is the one with the largest total time
    assert r["kernel"] == "gradient"
    assert r["bound"] == "alu" and r["unit"] == "TFLOP/s"
    assert r["peak"] == pytest.approx(bench.FP32_VECTOR_TFLOPS)
    assert r["achieved"] == pytest.approx(8.0e10 / 4.0e-3 / 1e12, rel=1e-3)
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], rel=1e-3)
    assert r["alone"]["avg_ms"] == 2.0
    assert r["alone"]["frac"] == pytest.approx(8.0e10 / 2.0e-3 / 1e12 / bench.FP32_VECTOR_TFLOPS, rel=1e-3)
    assert r["l2_tap"]["achieved"] == pytest.approx(5.0e10 / 4.0e-3 / 1e9, rel=1e-3)
    assert r["forward"]["avg_ms"] == 1.0
    for key in ("achieved", "peak", "frac", "traffic", "valu_issue"):
        assert key in r


def test_op_rates(bench):
    # the D = 128 forward's shape: 16384 poses, 6490 in-mask pixels, 64 taps of 8 B, 336 flops
    r = bench.op_rates(1.29, 16384, 6490, 512, 336)
    assert r["ms"] == 1.29
    assert r["proj_per_s"] == pytest.approx(16384 / 1.29e-3, rel=1e-6)
    assert r["tap_GBps"] == pytest.approx(16384 * 6490 * 512 / 1.29e-3 / 1e9, rel=1e-4)
    assert r["l2_frac"] == pytest.approx(r["tap_GBps"] / bench.L2_PEAK_GBS, rel=1e-3)
    assert r["tflops"] == pytest.approx(16384 * 6490 * 336 / 1.29e-3 / 1e12, rel=1e-3)
    assert r["alu_frac"] == pytest.approx(r["tflops"] / bench.FP32_VECTOR_TFLOPS, rel=1e-3)
    assert "tflops" not in bench.op_rates(1.0, 64, 414, 64, None)   # linear: tap rate only
