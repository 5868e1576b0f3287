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


def window_masses(out: dict, h_q: int, n_windows: int) -> np.ndarray:
    """Per-head mass of one oracle decode step on the sinks (column 0) and on each window
    (column 1 + w), from its probabilities and token owners."""
    A, owner = out["probs"], out["owner"]
    m = np.zeros((h_q, n_windows + 1))
    m[:, 0] = A[:, owner < 0].sum(axis=1)
    for w in np.unique(owner[owner >= 0]):
        m[:, 1 + int(w)] = A[:, owner == w].sum(axis=1)
    return m


def oracle_trace(wl: WL.Workload, cfg: O.OracleConfig, steps: int, score_init=None, n_windows: int = 0,
                 ref_kw=None):
    """A policy unit and an uncompressed reference unit (budget over the whole cache, no
    Quantized tier) decode the same tokens; returns (events, masses, s_full, policy unit)
    in the form of oracle/qevict_diagnostics.py: events[r] = dict(t, n, state, s_q)."""
    ref_cfg = O.OracleConfig(**{**cfg.__dict__, "budget_frac": 4.0, "quant_frac": 0.0, **(ref_kw or {})})
    qp, kp, vp = WL.prompt(wl, 0)
    S = wl.prompt_len
    pol, ref = O.UnitOracle(cfg, S), O.UnitOracle(ref_cfg, S)
    for u in (pol, ref):
        u.prefill(f64(qp[0]), f64(kp[0]), f64(vp[0]), score_init=score_init)
    nw = n_windows or (S + wl.n_decode + wl.omega - wl.n_sink + wl.window - 1) // wl.window + 1
    events, masses = [], []
    for j in range(steps):
        q, k, v = WL.decode_step(wl, 0, j)
        pol.decode(f64(q[0]), f64(k[0]), f64(v[0]))
        out = ref.decode(f64(q[0]), f64(k[0]), f64(v[0]))
        masses.append(window_masses(out, cfg.h_q, nw))
        if (j + 1) % wl.omega == 0:
            ev = pol.route()
            ref.route()
            events.append(dict(t=j + 1, n=pol.n, state={w: W.state for w, W in pol.win.items()},
                               s_q=dict(pol.score), s_full=dict(ref.score), promoted=ev["promoted"]))
    return events, masses, pol
