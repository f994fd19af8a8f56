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
    for w in ("layer4", "layer2", "batch32", "tier4", "stack60", "tiny", "gdn", "stream", "gap", "exchange"):
        assert w in res.stdout


def _bench():
    import importlib.util
    spec = importlib.util.spec_from_file_location("_bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_single_token_bytes_count_five_experts():
    """The roofline's bytes for the headline layer: the 4 selected experts and
    the shared one, 2,359,296 bytes per matrix (codes + scale/bias), so
    23,592,960 bytes for gate/up and 11,796,480 for down."""
    import numpy as np
    import synthetic as syn
    b = _bench()
    dims = syn.WORKLOADS["layer4"].dims
    assert b.matrix_bytes(dims) == 2_359_296
    n = b.distinct_experts(np.array([[7, 300, 2, 511]]))
    assert n == 5
    sb = b.stage_bytes(dims, ["k_router", "k_gateup", "k_down"], n, 1)
    assert sb[1] == 23_592_960 and sb[2] == 11_796_480
    assert sb[0] == 513 * 4096 * 2 + 4096 * 2 + 4096 * 4
    # the 2-bit layer: 1,048,576 + 262,144 bytes per matrix
    d2 = syn.WORKLOADS["layer2"].dims
    assert b.stage_bytes(d2, ["k_router", "k_gateup", "k_down"], 5, 1)[1] == 5 * 2 * 1_310_720


def test_unrouted_rows_are_refused():
    """A route row that no forward call has written (still -1) cannot enter the
    byte count (it once counted as ~2 experts instead of 5)."""
    import numpy as np
    import pytest
    b = _bench()
    with pytest.raises(ValueError):
        b.distinct_experts(np.full((1, 4), -1))
    # a batch: shared experts among tokens count once
    assert b.distinct_experts(np.array([[1, 2], [2, 3]])) == 4


def test_default_steps_per_workload():
    b = _bench()
    assert b.parse_args([]).steps == 2048 and b.parse_args([]).workload == "layer4"
    assert b.parse_args(["--workload", "stack60"]).steps == 64
    assert b.parse_args(["--workload", "stack60", "--steps", "5"]).steps == 5


def test_gdn_bytes():
    """One token through 64 heads of 128 x 128 fp32 state: 4 MiB read and
    4 MiB written, plus q, k, v and the output (4 x 32 KiB) and the gates."""
    b = _bench()
    assert b.gdn_step_bytes(64, 128) == 2 * 4 * 1024 * 1024 + 4 * 32 * 1024 + 64 * 8
