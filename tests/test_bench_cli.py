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


def test_timed_window():
    """The default window is every configured step after min(8, steps / 4)
    warm-up steps; an explicit K times the last K configured steps, not
    before the warm-up; past the configured steps the queries continue."""
    sys.path.insert(0, ROOT)
    import bench
    assert bench.timed_window(128) == (8, 128, 128)         # the 128K workloads: steps 8-127
    assert bench.timed_window(64) == (8, 64, 64)
    assert bench.timed_window(16) == (4, 16, 16)            # min(8, 16 / 4)
    assert bench.timed_window(128, 5, 20) == (108, 128, 128)
    assert bench.timed_window(128, 8, 120) == (8, 128, 128)
    assert bench.timed_window(64, 8, 120) == (8, 128, 128)  # runs past the configured 64


def test_cpu_baseline_runs_the_oracle_on_the_window():
    """The CPU baseline (the oracle, one thread) on the tiny workload: state
    brought to the window's first step untimed, then timed whole steps from
    there, never past the window."""
    sys.path.insert(0, ROOT)
    import numpy as np

    import bench
    from sparse_attention_tiered_amd import workload as W
    w = W.get("c1")
    geo = W.geometry(w)
    draws = W.draw_queries(w, geo)
    host = [np.zeros(w.Hkv * geo.pages[b] * W.PAGE_ELEMS, np.uint16) for b in range(w.B)]
    W.fill_all(w, geo, draws, host)
    r = bench.cpu_baseline(w, geo, draws, host, 4, 7, budget_s=30.0)
    assert r["cores"] == 1 and r["blas_threads_used"] == 1 and r["kind"] == "oracle"
    assert r["steps_timed"] == [4, 6] and r["value"] > 0
