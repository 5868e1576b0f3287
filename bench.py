"""Decode-attention throughput of the QEvict hot path on one MI355X.

A timed "step" is one generated token of the whole path for every layer:
qevict_decode_attn (append + split-K attention over sinks / recent / Full bf16 /
Quantized INT2 windows + combine + window-mass score update) for each of the L
layers, plus one routing event over all layers (TopK + pack / promote +
compaction) after every Omega-th step.  Inputs are resident in HBM before the
timed region starts.  The prompt-attention column sums that initialise the
scores run once per layer before timing (reported as prefill_s).

Workload: Llama-3-8B-shaped stack, 32 layers, 32 query / 8 KV heads of 128,
batch 1, 32K-token prompt, windows of 32, 4 sinks, 256 recent, budget 20% of
the full bf16 cache, quantized share 0.70, INT2.

    python bench.py [--gpus 1] [--steps 128] [--warmup 16]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E peak, GB/s
TIME_EVERY = 8           # per-kernel timing on every 8th timed step
METRIC = "decode-attn tokens/s + achieved HBM GB/s (% peak) at 32K ctx; route µs/event"


# --ranker choices -> the library flag that selects them (None: the cumulative score)
RANKERS = {"cum": None, "decay": "QEVICT_F_RANK_DECAY", "pnorm": "QEVICT_F_RANK_PNORM",
           "keynorm": "QEVICT_F_RANK_KEYNORM"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash() -> str:
    h = hashlib.sha256()
    for f in ("qevict_decode.hip", "qevict_common.h", "qevict_internal.h", "qevict_mass.h"):
        h.update(open(os.path.join(ROOT, "recoverable_kv_cache_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def timed_schedule(steps: int, warmup: int, omega: int, every: int = TIME_EVERY) -> list[tuple[int, int, bool, bool]]:
    """The timed steps as (i, j, routes, sampled): i counts timed steps from 0, j = warmup + i is
    the decode step index, ``routes`` is true when a routing event follows step j
    ((j + 1) % omega == 0, after the decode of every layer), and ``sampled`` marks the steps
    whose split-K launches carry dispatch-stamped events (one in ``every``, rotating through
    the positions of the block so that every phase of the routing interval is sampled)."""
    if steps < 0 or warmup < 0 or omega < 1 or every < 1:
        raise ValueError("steps, warmup >= 0 and omega, every >= 1")
    return [(i, warmup + i, (warmup + i + 1) % omega == 0, i % every == (i // every) % every)
            for i in range(steps)]


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    import platform
    return platform.processor() or "unknown"


def host_workers() -> int:
    """Threads for drawing inputs on the host: the cores this process may use, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def prompts_in_order(wl, layers, workers: int):
    """Yield (layer, (q, k, v)) for each layer, drawn on the host (the oracle's streams),
    with at most ``workers`` layers drawn ahead at a time."""
    from concurrent.futures import ThreadPoolExecutor
    from recoverable_kv_cache_amd import workload as WL
    layers = list(layers)
    with ThreadPoolExecutor(workers) as ex:
        futs = {}
        nxt = 0
        for l in layers:
            while nxt < len(layers) and len(futs) < workers:
                futs[layers[nxt]] = ex.submit(WL.prompt, wl, layers[nxt])
                nxt += 1
            yield l, futs.pop(l).result()


def cpu_baseline(wl, budget_s: float = 20.0, ranker: str = "cum", quant_bits: int = 2, rope_cs=None) -> dict:
    """Time the fp64 oracle's decode step on the host (layer 0, sequence 0), with a
    synthetic initial score instead of the prompt column sums (those alone are
    ~9 TFLOP of fp64 per layer on a 32K prompt)."""
    import numpy as np
    import torch
    from oracle import qevict_oracle as O
    from recoverable_kv_cache_amd import workload as WL
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    ocfg = O.OracleConfig(wl.h_q, wl.h_kv, wl.d_head, wl.window, wl.n_sink, wl.n_local, wl.omega,
                          wl.quant_frac, wl.budget_frac, wl.n_decode, ranker=ranker, quant_bits=quant_bits,
                          rope=rope_cs is not None)
    S = wl.prompt_lens()[0]
    qp, kp, vp = WL.prompt(wl, 0, with_q=False, seqs=[0])
    f = lambda t: t.to(torch.float64).numpy()
    unit = O.UnitOracle(ocfg, S, rope_cs=None if rope_cs is None else rope_cs.numpy())
    n_win = (wl.prompt_len - wl.n_sink + wl.window - 1) // wl.window
    t0 = time.perf_counter()
    unit.prefill(None, f(kp[0, :, :S]), f(vp[0, :, :S]), score_init=WL.init_scores(wl, 0, n_win)[0].numpy())
    setup_s = time.perf_counter() - t0
    del kp, vp
    times = []
    j = 0
    t_start = time.perf_counter()
    while j < wl.n_decode and (time.perf_counter() - t_start < budget_s or j < 2):
        q, k, v = WL.decode_step(wl.with_(batch=1), 0, j)   # sequence 0's streams
        t1 = time.perf_counter()
        unit.decode(f(q[0]), f(k[0]), f(v[0]))
        times.append(time.perf_counter() - t1)
        j += 1
    per_layer_step = statistics.mean(times)
    return {"value": round(wl.batch / (per_layer_step * wl.n_layers), 4), "unit": "tokens/s", "cores": cores,
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"fp64 NumPy oracle, layer 0 / sequence 0 of the same workload, {len(times)} decode steps "
                      f"({per_layer_step * 1e3:.0f} ms per layer-step, setup {setup_s:.1f} s), "
                      f"extrapolated x{wl.n_layers} layers x batch {wl.batch}"}


def stream_reference(nbytes: int, dev, n_buf: int = 32, passes: int = 4) -> dict:
    """A plain streaming read of the same number of bytes per launch (the library's
    qevict_stream_read), for context beside the HBM peak: launched back to back over n_buf
    distinct buffers (one per layer; together beyond the last-level cache), timed like the
    split kernel (events stamped by each launch's own dispatch, every launch of one pass)
    and as the wall time of back-to-back passes."""
    import torch
    from recoverable_kv_cache_amd import binding as B
    nb = max(1024, nbytes // 1024 * 1024)
    bufs = [torch.ones(nb // 4, dtype=torch.int32, device=dev) for _ in range(n_buf)]
    sink = torch.zeros(B.STREAM_READ_WGS, dtype=torch.int32, device=dev)
    for b in bufs:
        B.stream_read(b, sink)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in bufs]
    for e0, e1 in evs:
        e0.record()
        e1.record()
    torch.cuda.synchronize()
    for b, (e0, e1) in zip(bufs, evs):
        B.stream_read(b, sink, e0, e1)
    torch.cuda.synchronize()
    stamped_us = statistics.mean(e0.elapsed_time(e1) for e0, e1 in evs) * 1e3
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0.record()
    for _ in range(passes):
        for b in bufs:
            B.stream_read(b, sink)
    w1.record()
    torch.cuda.synchronize()
    b2b_us = w0.elapsed_time(w1) * 1e3 / (passes * n_buf)
    del bufs
    torch.cuda.empty_cache()
    return {"what": f"qevict_stream_read of the same bytes, {n_buf} distinct buffers", "bytes": nb,
            "us_per_launch": round(stamped_us, 3), "gbps": round(nb / (stamped_us * 1e-6) / 1e9, 1),
            "us_back_to_back": round(b2b_us, 3)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="llama8b_32k")
    ap.add_argument("--n-splits", type=int, default=0)
    ap.add_argument("--ranker", choices=sorted(RANKERS), default="cum",
                    help="window rank key: cumulative mass (Eq. 1) or an Appendix J alternative")
    ap.add_argument("--quant-bits", type=int, choices=(2, 4), default=2,
                    help="bits per Quantized-tier code: INT2 (default) or INT4")
    ap.add_argument("--rope", action="store_true",
                    help="inputs before RoPE, Quantized tier in the pre-RoPE domain (rotary base 500000)")
    ap.add_argument("--combine", choices=("auto", "launch"), default="auto",
                    help="auto: a decode step is one launch when each (sequence, KV head) has one split; "
                         "launch: always the separate finish launch (QEVICT_F_SEPARATE_FINISH)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=20.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB device copy (for scaling rocprofv3 byte counters) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the decode path here runs on a single GPU.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from recoverable_kv_cache_amd import binding as B
    from recoverable_kv_cache_amd import workload as WL

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": a.numel()}))
        return

    wl = {w.name: w for w in WL.ALL_WORKLOADS}[args.workload]
    if args.steps + args.warmup > wl.n_decode:
        sys.exit(f"--steps + --warmup must be <= {wl.n_decode}")
    flags = (getattr(B, RANKERS[args.ranker]) if RANKERS[args.ranker] else 0) | \
        (B.QEVICT_F_INT4 if args.quant_bits == 4 else 0) | (B.QEVICT_F_ROPE if args.rope else 0) | \
        (B.QEVICT_F_SEPARATE_FINISH if args.combine == "launch" else 0)
    cfg = B.make_config(wl, n_splits=args.n_splits, flags=flags)
    lens = wl.prompt_lens()
    st = B.QEvictState(cfg, lens, device=dev)
    rope_cs = None
    if args.rope:
        rope_cs = WL.rope_table(wl.d_head, max(32, wl.prompt_len + wl.n_decode))
        st.set_rope(rope_cs.to(dev))
    log(f"[bench] {wl.name}: arena {st.info.arena_bytes / 2**30:.2f} GiB, splits {st.info.n_splits}, "
        f"K_f {st.info.max_K_f}, K_q {st.info.max_K_q}")

    # ---- prefill every layer (column sums on MFMA); the prompts are drawn on the host from
    # the same streams the oracle reads and copied to the device
    workers = host_workers()
    torch.cuda.synchronize()
    t_pf = 0.0
    t_gen = time.perf_counter()
    for l, (qp, kp, vp) in prompts_in_order(wl, range(wl.n_layers), workers):
        qp, kp, vp = qp.to(dev), kp.to(dev), vp.to(dev)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        st.prefill_init(l, qp, kp, vp)
        torch.cuda.synchronize()
        t_pf += time.perf_counter() - t0
        del qp, kp, vp
        if l % 8 == 0:
            log(f"[bench] prefill layer {l} done ({t_pf:.1f} s of prefill, {time.perf_counter() - t_gen:.1f} s so far)")
    assert st.poll_status() == 0, "device status after prefill"

    # ---- decode inputs for every (step, layer), drawn on the host and resident in HBM
    from concurrent.futures import ThreadPoolExecutor
    n_total = args.warmup + args.steps
    with ThreadPoolExecutor(workers) as ex:
        host_in = list(ex.map(lambda j: [WL.decode_step(wl, l, j) for l in range(wl.n_layers)], range(n_total)))
    inputs = [[tuple(t.to(dev) for t in qkv) for qkv in row] for row in host_in]
    del host_in
    out = torch.empty((wl.batch, wl.h_q, wl.d_head), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] inputs ready ({time.perf_counter() - t_gen:.1f} s)")

    def new_event():
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def run_step(j, timing=None, route_ev=None, route_k=None):
        for l in range(wl.n_layers):
            if timing is not None:
                st.time_next_decode(timing[l][0], timing[l][1])
            q, k, v = inputs[j][l]
            st.decode_attn(l, q, k, v, out)
        if (j + 1) % wl.omega == 0:
            if route_k is not None:
                st.time_next_route(route_k[0], route_k[1])
            if route_ev is not None:
                route_ev[0].record()
            st.route(-1)
            if route_ev is not None:
                route_ev[1].record()

    for j in range(args.warmup):
        run_step(j)
    torch.cuda.synchronize()
    kv0 = [st.step_bytes(l) for l in range(wl.n_layers)]

    # ---- timed region: wall-clock events around all steps; the split-K kernels of the
    # sampled steps carry events stamped by their own dispatch (start / end), and every
    # routing event is bracketed by events, and also timed by events its kernels' dispatches
    # stamp (the routing kernel's start, the migration kernel's end)
    sched = timed_schedule(args.steps, args.warmup, wl.omega)
    kev = {i: [(new_event(), new_event()) for _ in range(wl.n_layers)] for i, _, _, s_ in sched if s_}
    rev = {i: (new_event(), new_event()) for i, _, r, _ in sched if r}
    rkev = {i: (new_event(), new_event()) for i, _, r, _ in sched if r}
    start, stop = new_event(), new_event()
    torch.cuda.synchronize()
    start.record()
    for i, j, _, _ in sched:
        run_step(j, timing=kev.get(i), route_ev=rev.get(i), route_k=rkev.get(i))
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    route_ms = [e0.elapsed_time(e1) for e0, e1 in rev.values()]   # between stream events
    route_k_ms = [e0.elapsed_time(e1) for e0, e1 in rkev.values()]   # kernels' own dispatch stamps
    n_route = len(route_ms)
    kern_ms = [e0.elapsed_time(e1) for evs in kev.values() for e0, e1 in evs]
    kv1 = [st.step_bytes(l) for l in range(wl.n_layers)]
    status = st.poll_status()
    assert status == 0, f"device status {status}"

    avg_kernel_s = statistics.mean(kern_ms) * 1e-3 if kern_ms else float("nan")
    kv_per_launch = statistics.mean([(a[0] + b[0]) / 2 for a, b in zip(kv0, kv1)])
    io_per_launch = kv0[0][1]
    alg_bytes = kv_per_launch + io_per_launch
    achieved_gbps = alg_bytes / avg_kernel_s / 1e9
    tokens_per_s = wl.batch * args.steps / (total_ms * 1e-3)
    decode_ms = total_ms - sum(route_ms)
    decode_tokens_per_s = wl.batch * args.steps / (decode_ms * 1e-3)

    traffic = None
    tag = "" if (args.quant_bits == 2 and args.ranker == "cum" and not args.rope) else \
        f"_int{args.quant_bits}_{args.ranker}{'_rope' if args.rope else ''}"
    tf = os.path.join(ROOT, "profiles", f"decode_split_{wl.name}{tag}_traffic.json")
    if os.path.exists(tf):
        rec = json.load(open(tf))
        if rec.get("source_hash") == source_hash():
            traffic = rec.get("bytes_per_launch")

    sref = stream_reference(int(alg_bytes), dev)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) ...")
        cpu = cpu_baseline(wl, args.cpu_budget_s, args.ranker, args.quant_bits, rope_cs)

    def stats_us(ms):
        s_ = sorted(ms)
        return {"mean": round(statistics.mean(s_) * 1e3, 2) if s_ else None,
                "p50": round(s_[len(s_) // 2] * 1e3, 2) if s_ else None,
                "p99": round(s_[min(len(s_) - 1, math.ceil(0.99 * len(s_)) - 1)] * 1e3, 2) if s_ else None}
    line = {
        "metric": METRIC,
        "value": round(tokens_per_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"bf16 + int{args.quant_bits} operands, fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": wl.n_layers, "batch": wl.batch, "h_q": wl.h_q, "h_kv": wl.h_kv,
                   "d_head": wl.d_head, "prompt_len": wl.prompt_len, "window": wl.window, "n_sink": wl.n_sink,
                   "n_local": wl.n_local, "omega": wl.omega, "budget_frac": wl.budget_frac,
                   "quant_frac": wl.quant_frac, "storage": f"bf16 + int{args.quant_bits}", "n_splits": st.info.n_splits,
                   "K_f": st.info.max_K_f, "K_q": st.info.max_K_q, "ranker": args.ranker,
                   "rope": "inputs before RoPE, base 500000" if args.rope else None,
                   "finish": "in the split kernel" if st.info.combine_in_kernel else "second launch"},
        "decode_attn_tokens_per_s": round(decode_tokens_per_s, 2),
        "route_us_per_event": {**stats_us(route_k_ms), "events": n_route,
                               "scope": f"all {wl.n_layers} layers x batch {wl.batch}",
                               "timing": "routing kernel's dispatch start to migration kernel's dispatch end"},
        "route_us_per_event_stream_events": {**stats_us(route_ms),
                                             "timing": "hipEventRecord before and after the routing call"},
        "hbm_gbps_split_kernel": round(achieved_gbps, 1),
        "hbm_frac_of_peak": round(achieved_gbps / HBM_PEAK_GBPS, 4),
        "prefill_s": round(t_pf, 3),
        "roofline": {"bound": "hbm", "kernel": B.load_library().qevict_decode_kernel_name().decode(),
                     "achieved": round(achieved_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": int(alg_bytes),
                     "avg_launch_us": round(avg_kernel_s * 1e6, 3), "launches": len(kern_ms),
                     "stream_ref": sref, "frac_of_stream_ref": round(achieved_gbps / sref["gbps"], 4)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
