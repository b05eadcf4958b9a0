"""bench.py pieces that need no GPU: the one-GPU refusal and the record of
profiled HBM traffic that the roofline entry reads."""
import json
import os
import re
import subprocess
import sys

from conftest import ROOT

BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2, (r.returncode, r.stdout, r.stderr)
    assert "one GPU" in r.stdout + r.stderr
    assert not r.stdout.strip().startswith("{")   # no result line


def test_traffic_record_is_well_formed():
    import bench
    tr = json.load(open(bench.TRAFFIC_FILE))
    for key in ("kernel", "read_bytes_per_launch", "write_bytes_per_launch", "bytes_per_launch", "read_factor",
                "write_factor", "kernel_source_hash"):
        assert key in tr, key
    assert abs(tr["read_bytes_per_launch"] + tr["write_bytes_per_launch"] - tr["bytes_per_launch"]) < 1.0
    # counters against the 269.2 MB the compress launch must move at least
    assert tr["bytes_per_launch"] >= 269_221_888
    assert re.fullmatch(r"[0-9a-f]{16}", tr["kernel_source_hash"])


def test_source_hash_is_stable_and_hex():
    import bench
    h = bench.source_hash()
    assert re.fullmatch(r"[0-9a-f]{16}", h) and h == bench.source_hash()
