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


def test_timed_schedule_routes_and_samples():
    """The timed step / route schedule for the driver's and other (steps, warmup) pairs: a
    routing event follows exactly the decode steps j with (j + 1) % omega == 0, each timed
    step appears once in order, and one step in eight carries the kernel events."""
    import bench
    for steps, warmup in [(20, 5), (128, 16), (7, 3), (1, 0), (0, 4), (64, 0)]:
        for omega in (1, 8, 3):
            sched = bench.timed_schedule(steps, warmup, omega)
            assert [i for i, _, _, _ in sched] == list(range(steps))
            assert [j for _, j, _, _ in sched] == list(range(warmup, warmup + steps))
            routes = [j for _, j, r, _ in sched if r]
            assert routes == [j for j in range(warmup, warmup + steps) if (j + 1) % omega == 0]
            sampled = [i for i, _, _, s in sched if s]
            assert steps // 8 <= len(sampled) <= -(-steps // 8) and (steps == 0 or sampled[0] == 0)
            # the sampled step moves through the 8 positions of successive blocks
            assert all(i % 8 == (i // 8) % 8 for i in sampled)
    # the driver's command: 20 timed steps after 5 warmup steps, routes after steps 7, 15, 23
    sched = bench.timed_schedule(20, 5, 8)
    assert [j for _, j, r, _ in sched if r] == [7, 15, 23]
    # over 64 timed steps every phase of the routing interval is sampled once
    assert sorted(j % 8 for _, j, _, s in bench.timed_schedule(64, 0, 8) if s) == list(range(8))


def test_prompt_sequence_subset_matches_the_batch_draw():
    """``seqs`` draws only some sequences with the rows (and ragged lengths) of the whole batch."""
    import torch
    from recoverable_kv_cache_amd import workload as WL
    wl = WL.Workload("ragged_small", 1, 4, 4, 2, 32, 96, 8, 16, 4, 16, 8, 0.5, 0.7, prompt_len_min=40,
                     n_outlier=2, n_topics=2)
    full = WL.prompt(wl, 0)
    part = WL.prompt(wl, 0, seqs=[2, 0])
    for a, b in zip(part, full):
        assert torch.equal(a[0], b[2]) and torch.equal(a[1], b[0])
    _, k, v = WL.prompt(wl, 0, with_q=False, seqs=[3])
    assert torch.equal(k[0], full[1][3]) and torch.equal(v[0], full[2][3])


def test_decode_inputs_of_one_sequence_match_the_batch_draw():
    """Sequence b's decode inputs do not depend on the batch size (per-sequence streams), so a
    one-sequence oracle sample sees the bytes the batched GPU run sees."""
    import torch
    from recoverable_kv_cache_amd import workload as WL
    wl = WL.CHURN_4K.with_(batch=3)
    for j in (0, 255, 256):
        full = WL.decode_step(wl, 1, j)
        one = WL.decode_step(wl.with_(batch=1), 1, j)
        assert all(torch.equal(a[0], b[0]) for a, b in zip(one, full))
