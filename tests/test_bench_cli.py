"""Host-side checks of the benchmark script's contract (no GPU): it refuses more than one
GPU with a message and a nonzero status before touching a device, and the HBM traffic
records it reads for its ``roofline.traffic`` field are well formed."""
from __future__ import annotations

import glob
import json
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    for n in (2, 8):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)], cwd=ROOT,
                           capture_output=True, text=True, timeout=120)
        assert r.returncode == 2
        assert "one GPU" in r.stderr and f"--gpus {n}" in r.stderr
        assert r.stdout.strip() == ""   # no JSON line


def test_traffic_records_are_well_formed():
    import bench
    h = bench.source_hash()
    assert re.fullmatch(r"[0-9a-f]{16}", h)
    files = sorted(glob.glob(os.path.join(ROOT, "profiles", "decode_split_*_traffic.json")))
    assert files, "no traffic record under profiles/"
    for f in files:
        rec = json.load(open(f))
        for k in ("kernel", "workload", "source_hash", "dispatches", "fetch_bytes_per_launch",
                  "write_bytes_per_launch", "bytes_per_launch", "copy_fetch_scale", "copy_write_scale", "commands"):
            assert k in rec, (f, k)
        assert re.fullmatch(r"[0-9a-f]{16}", rec["source_hash"])
        assert rec["bytes_per_launch"] == rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
        assert rec["copy_fetch_scale"] > 0 and rec["copy_write_scale"] > 0
        assert rec["dispatches"]["fetch"] > 0 and rec["dispatches"]["write"] > 0
        assert "rocprofv3 --pmc FETCH_SIZE" in rec["commands"] and "rocprofv3 --pmc WRITE_SIZE" in rec["commands"]
        # each record sits beside its summary
        assert os.path.exists(f[: -len(".json")] + ".md")
