"""bench.py on the host: more than one GPU is refused with a message, before any
GPU work; the clock summary flags readings that move."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "single GPU" in r.stderr
    assert r.stdout == ""


def test_clock_summary_marks_moving_readings():
    """The clock-scaled peak is reported only for readings that stay within 20%:
    the telemetry has been seen swinging between 1.2 and 2.3 GHz in one run."""
    sys.path.insert(0, ROOT)
    import bench
    c = bench.ClockSampler.__new__(bench.ClockSampler)
    c.samples = [2400.0] * 10 + [2300.0, 2250.0, 2300.0, 2280.0]
    s = c.summary()
    assert s["steady"] and s["min_mhz"] == 2250.0 and s["samples"] == 7
    c.samples = [2339.0] * 10 + [1241.0, 2339.0, 1241.0, 1241.0]
    s = c.summary()  # the second half: 2339 x 3, then 1241, 2339, 1241, 1241
    assert not s["steady"] and (s["min_mhz"], s["max_mhz"], s["median_mhz"]) == (1241.0, 2339.0, 2339.0)
    c.samples = [2341.0] * 10 + [2068.0, 2341.0, 2341.0, 2200.0]
    assert c.summary()["steady"]  # ordinary clock steps, 12% apart
    c.samples = []
    assert c.summary() is None


def test_kernel_digest_ignores_comments(tmp_path, monkeypatch):
    """The digest that ties committed counters to the kernels they were taken on
    changes with the code, not with a comment."""
    import shutil
    sys.path.insert(0, ROOT)
    import bench
    src = os.path.join(ROOT, "reproducible_causal_attention_amd", "csrc")
    dst = tmp_path / "reproducible_causal_attention_amd" / "csrc"
    shutil.copytree(src, dst)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    d0 = bench.kernel_sources_digest()
    f = dst / "cdna4.hpp"
    f.write_text(f.read_text() + "\n// a remark\n/* and a block\n   remark */\n")
    assert bench.kernel_sources_digest() == d0
    f.write_text(f.read_text() + "\nconstexpr int kUnused = 1;\n")
    assert bench.kernel_sources_digest() != d0
