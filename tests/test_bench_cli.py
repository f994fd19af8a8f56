"""bench.py's command line on the host (no GPU): more than one GPU is refused
with a message and exit status 2, before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stdout and "--gpus 1" in res.stdout


def test_workloads_listed():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True, text=True,
                         timeout=120)
    assert res.returncode == 0
    for w in ("layer4", "layer2", "batch32", "tier4"):
        assert w in res.stdout
