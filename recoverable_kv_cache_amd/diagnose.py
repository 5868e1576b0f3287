"""Appendix I / K routing diagnostics of QEvict on one layer of a synthetic drift workload,
on the GPU:  python -m recoverable_kv_cache_amd.diagnose [--workload NAME] [--steps N]

For each policy (three tiers with and without Q -> F promotion, and the two-tier split
of the same budget) a policy state and an uncompressed reference state decode the same
tokens; the metrics of recoverable_kv_cache_amd/diagnostics.py are printed as one JSON
line per policy, with the time of the per-step mass export.
"""
from __future__ import annotations

import argparse
import json
import sys
import time

import torch

from recoverable_kv_cache_amd import binding as B
from recoverable_kv_cache_amd import diagnostics as D
from recoverable_kv_cache_amd import workload as WL

POLICIES = {
    "three-tier": dict(flags=0),
    "three-tier one-way": dict(flags=B.QEVICT_F_NO_PROMOTE),
    "two-tier": dict(flags=0, quant_frac=0.0),
}


def run(wl: WL.Workload, steps: int, name: str, over: dict, dev) -> dict:
    wl1 = wl.with_(n_layers=1, batch=1)
    over = dict(over)
    flags = over.pop("flags")
    sp = B.QEvictState(B.make_config(wl1, flags=flags, **over), wl1.prompt_lens()[:1], device=dev)
    # the reference: a Full tier that holds every window (a budget just above the whole cache)
    sr = B.QEvictState(B.make_config(wl1, budget_frac=1.1, quant_frac=0.0), wl1.prompt_lens()[:1], device=dev)
    need = -(-(wl1.prompt_len + steps - wl1.n_sink) // wl1.window)
    assert sr.info.max_K_f >= need, "the reference must keep every window"
    qp, kp, vp = WL.prompt(wl1, 0, device=dev)
    for st in (sp, sr):      # scores initialised from the prompt-attention column sums
        st.prefill_init(0, qp, kp, vp)
    del qp, kp, vp
    out = torch.empty((1, wl1.h_q, wl1.d_head), dtype=torch.float32, device=dev)
    inputs = [WL.decode_step(wl1, 0, j, device=dev) for j in range(steps)]
    mass_ms = []

    def run_step(j):
        q, k, v = inputs[j]
        sp.decode_attn(0, q, k, v, out)
        sr.decode_attn(0, q, k, v, out)

    class Timed:                      # times the reference's step-mass export
        def __init__(self, st):
            self.st, self.cfg = st, st.cfg

        def step_mass(self, layer, b):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            m = self.st.step_mass(layer, b)
            e1.record()
            torch.cuda.synchronize()
            mass_ms.append(e0.elapsed_time(e1))
            return m

        def __getattr__(self, k):
            return getattr(self.st, k)

    t0 = time.perf_counter()
    tr = D.record(sp, Timed(sr), 0, 0, run_step, steps, wl1.omega)
    s = D.summarize(tr, horizon=32, m=3, deltas=(1, 8))
    s.update(policy=name, workload=wl.name, steps=steps, K_f=tr.K_f, K_q=sp.info.max_K_q,
             step_mass_us=round(1e3 * sorted(mass_ms)[len(mass_ms) // 2], 2), wall_s=round(time.perf_counter() - t0, 1))
    return s


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="llama8b_32k")
    ap.add_argument("--steps", type=int, default=256)
    args = ap.parse_args()
    wl = {w.name: w for w in WL.ALL_WORKLOADS}[args.workload]
    if args.steps > wl.n_decode:
        sys.exit(f"--steps must be <= {wl.n_decode}")
    dev = torch.device("cuda:0")
    for name, over in POLICIES.items():
        print(json.dumps(run(wl, args.steps, name, over, dev)), flush=True)


if __name__ == "__main__":
    main()
