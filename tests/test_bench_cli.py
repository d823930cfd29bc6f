"""bench.py's command line and its counter-traffic lookup, on the CPU (no
GPU is touched: every case exits before the first device call)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_exits_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode != 0
    assert "one GPU only" in r.stderr


@pytest.mark.parametrize("args", [["--warmup", "0"], ["--warmup", "-1"]])
def test_inconsistent_options_are_refused(args):
    r = _run(*args)
    assert r.returncode == 2 and "error" in r.stderr


def test_counter_traffic_needs_matching_sources(tmp_path, monkeypatch):
    """Traffic is the committed ratio times the bytes while the kernel
    sources hash as profiled, and None once any of them differs."""
    sys.path.insert(0, ROOT)
    import bench

    sha = bench.kernel_sources_sha()
    prof = tmp_path / "profiles"
    prof.mkdir()
    line = ("machine-readable: traffic_ratio_attend=1.5000 traffic_ratio_select=1.0000 "
            f"traffic_ratio_retrieve=2.0000 sha_kernels={sha}")
    (prof / "cx_hbm_counters.md").write_text(line + "\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "sparse_attention_tiered_amd").symlink_to(os.path.join(ROOT, "sparse_attention_tiered_amd"))
    assert bench.counter_traffic("cx", "attend", 1000.0) == pytest.approx(1500.0)
    stale = line.replace(f"sha_kernels={sha}", "sha_kernels=000000000000")
    (prof / "cx_hbm_counters.md").write_text(stale + "\n")
    assert bench.counter_traffic("cx", "attend", 1000.0) is None
    assert bench.counter_traffic("nope", "attend", 1000.0) is None
