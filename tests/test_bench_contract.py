"""bench.py's host-side contract, checked without a GPU: it measures one GPU
only, so asking for more exits with a message (status 2) before touching a
device; and its roofline traffic is read only from a profile summary made
from the current kernel sources."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_profiled_traffic_follows_the_sources(tmp_path, monkeypatch):
    import hashlib
    import importlib.util
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    # a tree whose summary was made from its current kernel sources reports the traffic
    fake = tmp_path / "repo"
    csrc = fake / "rejection_sampling_verify_rs_amd" / "csrc"
    csrc.mkdir(parents=True)
    (fake / "profiles").mkdir()
    (csrc / "a.hip").write_text("// kernel\n")
    (csrc / "b.hpp").write_text("// header\n")
    sha = hashlib.sha256(b"// kernel\n" + b"// header\n").hexdigest()
    (fake / "profiles" / "rs_verify_B256_K8_V151936_hbm_bytes.md").write_text(
        'traffic_bytes_per_dispatch: {"stream": 123}\n' f"kernel_source_sha256: {sha}\n")
    monkeypatch.setattr(bench, "ROOT", str(fake))
    assert bench.profiled_traffic("stream") == 123
    # once a kernel source changes, the counters no longer describe it
    (csrc / "b.hpp").write_text("// header, edited\n")
    assert bench.profiled_traffic("stream") is None
