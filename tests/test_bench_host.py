"""CPU checks of bench.py's host logic: the one-GPU guard, the algorithmic
byte counts, and the rule that measured HBM traffic is reported only for the
kernel sources it was measured on."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_bytes_per_element():
    # read bf16 (2 B) + codes (0.5 B FP4, 0.75 B E2M3) + one scale byte per 32
    assert bench.quant_bytes_per_elem(0) == 2.53125
    assert bench.quant_bytes_per_elem(1) == 2.78125


def test_traffic_only_for_the_measured_sources(monkeypatch):
    for variant, kernels in bench.MEASURED_TRAFFIC.items():
        for name, m in kernels.items():
            assert name in bench.KERNEL_SOURCES
            got = bench.measured_traffic(variant, name)
            if m["sha"] == bench.source_sha(name):
                assert got == m["read"] + m["write"]
            else:
                assert got is None
            stale = dict(kernels)
            stale[name] = dict(m, sha="0" * 16)
            monkeypatch.setitem(bench.MEASURED_TRAFFIC, variant, stale)
            assert bench.measured_traffic(variant, name) is None
            monkeypatch.setitem(bench.MEASURED_TRAFFIC, variant, kernels)
    assert bench.measured_traffic("e1m2", "no_such_kernel") is None
