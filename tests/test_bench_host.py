"""Host-side checks of bench.py (no GPU): the multi-GPU refusal, the profile
records' source-hash gate and the timing statistics."""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_profile_records_only_used_for_matching_sources():
    sys.path.insert(0, ROOT)
    import bench
    h = bench.kernel_source_hash()
    assert len(h) == 16 and h == bench.kernel_source_hash()
    for key in bench.WORKLOAD_KEY.values():
        for kind, getter, field in (("traffic", bench.load_traffic, "bytes_per_launch"),):
            path = os.path.join(ROOT, "profiles", f"{key}_{kind}.json")
            got = getter(key, h)
            if os.path.exists(path):
                rec = json.load(open(path))
                assert got == (rec[field] if rec["kernel_source_hash"] == h else None)
            else:
                assert got is None
            assert getter(key, "0" * 16) is None
        assert bench.load_counter_clock(key, "0" * 16) is None


def test_stats_median_and_percentiles():
    sys.path.insert(0, ROOT)
    import bench
    s = bench.stats(np.array([1.0, 2.0, 3.0, 4.0, 100.0]))
    assert s["median"] == 3.0 and s["mean"] == 22.0
    assert s["p10"] <= s["median"] <= s["p90"]
