"""Host-side checks of bench.py: the one-GPU refusal and the rule that the
roofline's traffic figure is reported only for the GEMM source it was measured on."""
import hashlib
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr
    assert not r.stdout.strip().startswith("{")  # no result line


def test_traffic_is_reported_only_for_the_measured_source(tmp_path, monkeypatch):
    bench = _bench_module()
    src = tmp_path / "gemm.hip"
    src.write_bytes(b"// kernel source as measured\n")
    (tmp_path / "profiles").mkdir()
    prof = tmp_path / "profiles" / "gemm1_wl_traffic.txt"
    sha = hashlib.sha256(src.read_bytes()).hexdigest()
    prof.write_text("# header: not a field\nhbm_bytes_per_launch: 12345\n" f"gemm_source_sha256: {sha}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "GEMM_SOURCE", str(src))
    assert bench.traffic_from_profile("gemm1", "wl") == 12345.0
    assert bench.traffic_from_profile("gemm1", "other") is None  # no summary for that workload
    src.write_bytes(b"// kernel source changed since the counters were taken\n")
    assert bench.traffic_from_profile("gemm1", "wl") is None
