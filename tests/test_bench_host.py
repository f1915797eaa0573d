"""CPU checks of bench.py's host logic: the one-GPU guard, the algorithmic
byte counts, the per-launch percentiles, and the rule that measured HBM traffic
is reported only for the kernel sources it was measured on."""
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


def test_launch_percentiles():
    import numpy as np
    xs = [float(v) for v in np.random.default_rng(5).permutation(101)]   # 0 .. 100
    d = bench.launch_percentiles(xs)
    assert (d["median_us"], d["p10_us"], d["p90_us"], d["launches"]) == (50.0, 10.0, 90.0, 101)
    # interpolation agrees with numpy's default (linear) percentile
    ys = list(np.random.default_rng(6).exponential(40.0, 37))
    d = bench.launch_percentiles(ys)
    for key, p in (("median_us", 50), ("p10_us", 10), ("p90_us", 90)):
        assert abs(d[key] - round(float(np.percentile(ys, p)), 3)) < 1e-9
    assert bench.launch_percentiles([7.0])["median_us"] == 7.0


def test_split_range_covers_in_order():
    for n, parts in ((4096, 16), (10, 3), (5, 8), (1, 1), (7, 1)):
        r = bench.split_range(n, parts)
        assert r[0][0] == 0 and r[-1][1] == n
        assert all(a < b for a, b in r)
        assert all(r[i][1] == r[i + 1][0] for i in range(len(r) - 1))
        sizes = [b - a for a, b in r]
        assert max(sizes) - min(sizes) <= 1
    assert 1 <= bench.oracle_threads() <= 16


def test_threaded_oracle_matches_one_call():
    # the all-core baseline concatenates per-thread column ranges: same codes as one call
    import numpy as np
    from oracle import oracle as orc
    from fp4_microscaling_quantization_amd import synth
    x = synth.normal(64, 96, seed=11)
    p = orc.qparams(grid=1, round=1, hadamard_n=16, sign_mask=0x5A5A, sr_seed=9)
    whole = orc.quantize_lines(x, orc.AXIS_COL, p, 0, 96, 1)
    parts = [orc.quantize_lines(x, orc.AXIS_COL, p, a, b - a, 1) for a, b in bench.split_range(96, 5)]
    assert np.array_equal(np.concatenate([c for c, _ in parts]), whole[0])
    assert np.array_equal(np.concatenate([s for _, s in parts]), whole[1])


def test_rotating_sets_span_the_last_level_cache():
    # every timed loop rotates at least 4 sets, together above 512 MB (the
    # MI355X last-level cache is 256 MB)
    for set_bytes in (2_654_208, 84_934_656, 179_830_784, 169_869_312, 700 << 20):
        n = bench.n_sets(set_bytes)
        assert n >= 4 and n * set_bytes > 512 << 20, (set_bytes, n)
