"""bench.py's command line, on the CPU: more than one GPU is refused with a
message (the layer runs on one MI355X) before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1", "--warmup", "0"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""                  # no result line


def test_bench_lists_its_workloads():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 0
    for wl in ("decode80b", "decode35b", "refill80b", "batch80b", "prefill80b", "prefill80b_zipf", "chain80b", "ceiling"):
        assert wl in r.stdout
