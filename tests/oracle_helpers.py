"""Shared helpers for the oracle tests: build oracle configs and feed seeded inputs."""
import numpy as np
import torch

from oracle import qevict_oracle as O
from recoverable_kv_cache_amd import workload as WL


def cfg_from(wl: WL.Workload, **kw) -> O.OracleConfig:
    base = dict(h_q=wl.h_q, h_kv=wl.h_kv, d=wl.d_head, window=wl.window, n_sink=wl.n_sink,
                n_local=wl.n_local, omega=wl.omega, quant_frac=wl.quant_frac,
                budget_frac=wl.budget_frac, n_decode=wl.n_decode)
    base.update(kw)
    return O.OracleConfig(**base)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.float64).numpy()


def run_unit(wl: WL.Workload, cfg: O.OracleConfig, b: int = 0, layer: int = 0, steps=None,
             score_init=None, collect=True):
    """Prefill + decode with due routing for one unit; returns (unit, per-step outputs)."""
    qp, kp, vp = WL.prompt(wl, layer)
    S = wl.prompt_lens()[b]
    unit = O.UnitOracle(cfg, S)
    unit.prefill(f64(qp[b, :, :S]), f64(kp[b, :, :S]), f64(vp[b, :, :S]), score_init=score_init)
    outs = []
    for j in range(wl.n_decode if steps is None else steps):
        q, k, v = WL.decode_step(wl, layer, j)
        out = unit.step_and_route(f64(q[b]), f64(k[b]), f64(v[b]))
        if collect:
            outs.append(out)
    return unit, outs
