"""bench.py's command-line contract (CPU only)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_traffic_is_reported_only_for_matching_sources():
    sys.path.insert(0, ROOT)
    import json

    import bench
    p = os.path.join(ROOT, "profiles", "traffic.json")
    d = json.load(open(p))
    v = bench.load_traffic("qdq_mxfp4_rot0")
    if d["source_hash"] == bench.source_hash():
        assert isinstance(v, int) and v > 0
    else:
        assert v is None
