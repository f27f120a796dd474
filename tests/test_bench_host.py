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
    assert set(h) == {"cpu_model", "affinity", "online"}
    assert 1 <= h["affinity"] <= h["online"]
    assert isinstance(h["cpu_model"], str) and h["cpu_model"]
