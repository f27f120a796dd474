"""Host checks of bench.py's contract that need no GPU: more than one GPU is
refused with a message before anything touches a device, and the JSON helpers
that need no device behave."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused_with_a_message(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and f"--gpus {n}" in r.stderr
    assert r.stdout == ""


def test_traffic_record_is_tied_to_the_kernel_sources():
    sys.path.insert(0, ROOT)
    import bench
    import synthgen

    h = bench.kernel_source_hash()
    assert len(h) == 16
    t = bench.load_traffic()
    # either the committed counters match the current kernel sources, or no traffic is claimed
    assert t is None or t > synthgen.WORKLOADS[bench.WORKLOAD].algorithmic_bytes * 0.9


def test_host_cpu_description():
    import bench

    h = bench.host_cpu()
    assert set(h) == {"cpu_model", "cpu_family_model_stepping", "affinity", "online"}
    assert 1 <= h["affinity"] <= h["online"]
    assert isinstance(h["cpu_model"], str) and h["cpu_model"]


def test_cpu_baseline_on_a_tiny_workload():
    """The CPU baseline's threaded oracle split reproduces the oracle and reports
    one-thread and all-core rates with the host description."""
    import bench
    import synthgen

    wl = synthgen.small_workload(4, 64, 2, 64, "bf16", seed=1, tile=(16, 1, 64))
    rec = bench.cpu_baseline(wl, synthgen.make_inputs(wl), run_s=0.05)
    assert rec["parity_with_oracle"] is True
    assert rec["kind"] == "oracle" and rec["value"] > 0 and rec["one_thread"]["value"] > 0
    assert rec["cores"] == rec["host"]["affinity"] and rec["gemm_fp64"]["value"] > 0
