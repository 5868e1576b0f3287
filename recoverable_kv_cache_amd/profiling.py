"""Summaries of rocprofv3 runs of ``bench.py`` (CSV output) for the ``profiles/`` folder.

    python -m recoverable_kv_cache_amd.profiling trace  <run_kernel_stats.csv> <out.md> "<command>"
    python -m recoverable_kv_cache_amd.profiling traffic <fetch_dir> <write_dir> <copy_fetch_dir> <copy_write_dir> \
        <kernel substring> <workload> <out.json> <out.md> "<commands>"
    python -m recoverable_kv_cache_amd.profiling sq <out.md> <kernel substring> <workload> "<commands>" <dir> [<dir> ...]

``trace`` tabulates per-kernel calls and durations.  ``traffic`` turns the
``FETCH_SIZE`` / ``WRITE_SIZE`` counters (KiB per dispatch) of the decode split
kernel into HBM bytes per launch, each scaled by what the same counter reads for
a plain 1 GiB device copy (read 1 GiB, write 1 GiB), and records the hash of the
kernel sources so that ``bench.py`` only reports it while the kernel is unchanged.
``sq`` tabulates shader-sequencer counters of that kernel (one pass per directory, at most
8 SQ counters each), per dispatch, with the ratios read from them.
"""
from __future__ import annotations

import csv
import glob
import json
import os
import statistics
import sys

COPY_BYTES = 1 << 30


def _rows(path_or_dir: str, suffix: str):
    paths = [path_or_dir] if os.path.isfile(path_or_dir) else glob.glob(os.path.join(path_or_dir, "**", "*" + suffix),
                                                                       recursive=True)
    if not paths:
        raise FileNotFoundError(f"no {suffix} under {path_or_dir}")
    rows = []
    for p in paths:
        with open(p, newline="") as f:
            rows += list(csv.DictReader(f))
    return rows


def trace_summary(stats_csv: str, out_md: str, command: str) -> None:
    rows = _rows(stats_csv, "kernel_stats.csv")
    lines = [f"# Kernel trace: `{command}`", "",
             "rocprofv3 `--kernel-trace --stats` (durations in µs, GPU time per dispatch).", "",
             "| kernel | calls | avg µs | min µs | max µs | total ms |", "|---|---:|---:|---:|---:|---:|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"]
        if len(name) > 70:
            name = name[:67] + "..."
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['TotalDurationNs']) / 1e6:.3f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def _counter_per_dispatch(d: str, counter: str, kernel_sub: str) -> list[float]:
    vals: dict[str, float] = {}
    for r in _rows(d, "counter_collection.csv"):
        name = r.get("Kernel_Name") or r.get("Kernel-Name") or ""
        if kernel_sub not in name or r.get("Counter_Name") != counter:
            continue
        key = r.get("Dispatch_Id") or r.get("Correlation_Id") or str(len(vals))
        vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    return list(vals.values())


def traffic_summary(fetch_dir, write_dir, cfetch_dir, cwrite_dir, kernel_sub, workload, out_json, out_md, commands):
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench
    f = _counter_per_dispatch(fetch_dir, "FETCH_SIZE", kernel_sub)
    w = _counter_per_dispatch(write_dir, "WRITE_SIZE", kernel_sub)
    cf = _counter_per_dispatch(cfetch_dir, "FETCH_SIZE", "copy")
    cw = _counter_per_dispatch(cwrite_dir, "WRITE_SIZE", "copy")
    if not (f and w and cf and cw):
        raise SystemExit(f"missing counters: fetch {len(f)} write {len(w)} copy {len(cf)}/{len(cw)}")
    fetch_scale = statistics.mean(cf) * 1024 / COPY_BYTES     # counted bytes per real byte read
    write_scale = statistics.mean(cw) * 1024 / COPY_BYTES
    fetch_b = statistics.mean(f) * 1024 / fetch_scale
    write_b = statistics.mean(w) * 1024 / write_scale
    rec = {"kernel": kernel_sub, "workload": workload, "source_hash": bench.source_hash(),
           "dispatches": {"fetch": len(f), "write": len(w)},
           "fetch_kib_per_dispatch": statistics.mean(f), "write_kib_per_dispatch": statistics.mean(w),
           "copy_fetch_scale": fetch_scale, "copy_write_scale": write_scale,
           "fetch_bytes_per_launch": fetch_b, "write_bytes_per_launch": write_b,
           "bytes_per_launch": fetch_b + write_b, "commands": commands}
    with open(out_json, "w") as fo:
        json.dump(rec, fo, indent=1)
    with open(out_md, "w") as fo:
        fo.write(f"# HBM traffic of `{kernel_sub}` ({workload})\n\n")
        fo.write("rocprofv3 `--pmc FETCH_SIZE` and `--pmc WRITE_SIZE` in separate runs, KiB per dispatch, each scaled by "
                 "what the same counter reads for a plain 1 GiB device copy (`bench.py --copy-calibration`).\n\n")
        fo.write("| quantity | value |\n|---|---:|\n")
        fo.write(f"| FETCH_SIZE per dispatch (KiB, mean of {len(f)}) | {statistics.mean(f):.1f} |\n")
        fo.write(f"| WRITE_SIZE per dispatch (KiB, mean of {len(w)}) | {statistics.mean(w):.1f} |\n")
        fo.write(f"| copy calibration: FETCH_SIZE bytes per byte read | {fetch_scale:.4f} |\n")
        fo.write(f"| copy calibration: WRITE_SIZE bytes per byte written | {write_scale:.4f} |\n")
        fo.write(f"| HBM bytes read per launch | {fetch_b:,.0f} |\n| HBM bytes written per launch | {write_b:,.0f} |\n")
        fo.write(f"| total per launch | {fetch_b + write_b:,.0f} |\n\n")
        fo.write("Commands:\n\n" + "\n".join(f"    {c}" for c in commands.split(" ;; ")) + "\n")


def _counters(d: str, kernel_sub: str) -> dict[str, list[float]]:
    per: dict[str, dict[str, float]] = {}
    for r in _rows(d, "counter_collection.csv"):
        name = r.get("Kernel_Name") or r.get("Kernel-Name") or ""
        if kernel_sub not in name:
            continue
        key = r.get("Dispatch_Id") or r.get("Correlation_Id") or "0"
        c = r.get("Counter_Name")
        per.setdefault(c, {})
        per[c][key] = per[c].get(key, 0.0) + float(r["Counter_Value"])
    return {c: list(v.values()) for c, v in per.items()}


def _gpu_units(d: str) -> tuple[int, int]:
    """(SIMDs, shader engines) of the GPU agent, from the run's agent_info.csv (0, 0 if absent)."""
    try:
        for r in _rows(d, "agent_info.csv"):
            if int(r.get("Simd_Count") or 0) > 0:
                return int(r["Simd_Count"]), int(r.get("Num_Shader_Banks") or 0)
    except FileNotFoundError:
        pass
    return 0, 0


def sq_summary(out_md: str, kernel_sub: str, workload: str, commands: str, *dirs: str) -> None:
    vals: dict[str, float] = {}
    n_disp: dict[str, int] = {}
    for d in dirs:
        for c, v in _counters(d, kernel_sub).items():
            vals[c] = statistics.mean(v)
            n_disp[c] = len(v)
    if not vals:
        raise SystemExit("no counters of " + kernel_sub)
    lines = [f"# Shader-sequencer counters of `{kernel_sub}` ({workload})", "",
             "rocprofv3 `--pmc`, one pass per group of counters; means per dispatch (sums over the chip). "
             "SQ_WAVE_CYCLES, SQ_WAIT_* and SQ_ACTIVE_INST_* count quad-cycles (4 cycles).", "",
             "| counter | per dispatch | dispatches |", "|---|---:|---:|"]
    for c in sorted(vals):
        lines.append(f"| {c} | {vals[c]:,.0f} | {n_disp[c]} |")
    g = vals.get
    n_simd, n_se = _gpu_units(dirs[0])
    ratios = []
    # SQ_WAVE_CYCLES, SQ_WAIT_ANY, SQ_ACTIVE_INST_* count quad-cycles; SQ_BUSY_CYCLES counts cycles per
    # shader engine; SQ_VALU_MFMA_BUSY_CYCLES cycles per SIMD (all summed over the chip)
    if g("SQ_WAVES"):
        for c in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VMEM_RD", "SQ_INSTS_SMEM"):
            if g(c) is not None:
                ratios.append((f"{c} per wave", g(c) / g("SQ_WAVES")))
        if g("SQ_WAVE_CYCLES"):
            ratios.append(("wave lifetime, cycles (4 SQ_WAVE_CYCLES / SQ_WAVES)", 4 * g("SQ_WAVE_CYCLES") / g("SQ_WAVES")))
    if g("SQ_WAVE_CYCLES"):
        for c in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY"):
            if g(c) is not None:
                ratios.append((f"{c} / SQ_WAVE_CYCLES (share of wave time)", g(c) / g("SQ_WAVE_CYCLES")))
    if g("SQ_BUSY_CYCLES") and n_simd and n_se:
        simd_cycles = g("SQ_BUSY_CYCLES") / n_se * n_simd
        ratios.append(("kernel cycles per shader engine (SQ_BUSY_CYCLES / engines)", g("SQ_BUSY_CYCLES") / n_se))
        for c, name in (("SQ_ACTIVE_INST_VALU", "VALU"), ("SQ_ACTIVE_INST_LDS", "LDS"), ("SQ_ACTIVE_INST_VMEM", "VMEM")):
            if g(c) is not None:
                ratios.append((f"{name} issue share of SIMD cycles (4 {c} / SIMD cycles)", 4 * g(c) / simd_cycles))
        if g("SQ_VALU_MFMA_BUSY_CYCLES") is not None:
            ratios.append(("MFMA busy share of SIMD cycles", g("SQ_VALU_MFMA_BUSY_CYCLES") / simd_cycles))
    if g("SQ_INSTS_LDS") and g("SQ_LDS_BANK_CONFLICT") is not None:
        ratios.append(("SQ_LDS_BANK_CONFLICT cycles per LDS instruction", g("SQ_LDS_BANK_CONFLICT") / g("SQ_INSTS_LDS")))
    if ratios:
        lines += ["", "| ratio | value |", "|---|---:|"] + [f"| {k} | {v:.3f} |" for k, v in ratios]
    lines += ["", "Commands:", ""] + [f"    {c}" for c in commands.split(" ;; ")]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    if sys.argv[1] == "trace":
        trace_summary(sys.argv[2], sys.argv[3], sys.argv[4])
    elif sys.argv[1] == "traffic":
        traffic_summary(*sys.argv[2:11])
    elif sys.argv[1] == "sq":
        sq_summary(*sys.argv[2:])
    else:
        raise SystemExit(__doc__)
