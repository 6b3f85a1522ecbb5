"""Host-side checks of bench.py (no GPU): the multi-GPU refusal and the
traffic record's source-hash gate."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_record_only_used_for_matching_sources(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    h = bench.kernel_source_hash()
    assert len(h) == 16 and h == bench.kernel_source_hash()
    rec_path = os.path.join(ROOT, "profiles", "fused_llama7b_gate_up_traffic.json")
    if os.path.exists(rec_path):
        rec = json.load(open(rec_path))
        got = bench.load_traffic(h)
        assert got is None or got == rec["hbm_bytes_per_launch"]
        assert got == (rec["hbm_bytes_per_launch"] if rec["kernel_source_hash"] == h else None)
    assert bench.load_traffic("0" * 16) is None
