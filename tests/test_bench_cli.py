"""bench.py's host-side contract, on the CPU: more than one GPU is refused before anything touches
a GPU, and the HBM traffic figures it reports are those measured on the current kernel sources
(each is stored with a hash of the sources it was taken on; a stale figure is reported as null).
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n, "--steps", "1"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_figures_match_the_current_sources():
    for key, m in bench.MEASURED_TRAFFIC.items():
        assert m["sources_sha256_16"] == bench.sources_digest(key), (
            f"{key}: the kernel sources changed since its HBM traffic was measured")
        assert bench.traffic(key) == m["bytes_per_launch"] > 0


def test_unknown_traffic_key_is_null():
    assert bench.traffic("no such kernel") is None
