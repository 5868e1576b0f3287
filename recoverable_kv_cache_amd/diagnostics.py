"""Routing diagnostics of QEvict on the GPU state ("QEvict: Recoverable Quantized KV
Eviction for Attention-Drift-Robust Long-Context Decoding", Appendix I, Eqs. 12-19, and
Appendix K).

A policy state and an uncompressed reference state (budget covering the whole cache,
no Quantized tier: every step attends over every token, the FullKV reference of
Appendix I.1) decode the same tokens.  Per decode step the reference's per-head window
masses come from ``qevict_step_mass``; at each routing event the policy's tiers and
scores and the reference's cumulative scores come from ``qevict_export_unit``.  The
metrics are reductions over those arrays, computed here with NumPy:

* Future Missed Mass (Eq. 13) over a horizon H, per head, averaged over heads;
* Selection Churn (Eq. 14) between consecutive events (Full ∪ Quantized windows);
* tier-mass shares of the reference's cumulative mass (Eq. 15);
* Quantized-Score Agreement and the mass ratio R_Q over the Quantized windows (Eqs. 16-17);
* Global LIR (Eq. 18) and lagged transitions (Eq. 19) of the policy's Full tier and of
  the reference's top-K_f selection;
* Q -> F promotions per event (Appendix K).

Conventions (where the pages leave them open): routing is per (sequence, layer), so the
tier sets are shared by all heads; positions existing at an event are counted by window
(the sinks and every window that has started); an inactive episode starts when a window
leaves the selected set, is eligible after m events and rescued if the window is
selected again before the run ends; transitions are counted over windows that have
aged out of the recent region.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# window states as exported
S_NONE, S_LOCAL, S_FULL, S_QUANT, S_EVICTED = 0, 1, 2, 3, 4


@dataclass
class Trace:
    """What one (sequence, layer) unit produced: per event r the policy tiers and scores,
    the reference scores, the step count and token count; per step the reference's
    per-head masses [h][1 + n_windows] (column 0 the sinks)."""
    n_sink: int
    window: int
    K_f: int
    t: list = field(default_factory=list)          # decode steps done at event r
    n: list = field(default_factory=list)          # tokens at event r
    state: list = field(default_factory=list)      # [n_created] int per event
    s_q: list = field(default_factory=list)        # policy scores per event
    s_full: list = field(default_factory=list)     # reference scores per event
    promoted: list = field(default_factory=list)
    masses: list = field(default_factory=list)     # per step: [h][1 + n_windows]


def _pad(x, n, fill=0):
    out = np.full(n, fill, dtype=np.asarray(x).dtype)
    out[: len(x)] = x
    return out


def future_missed_mass(tr: Trace, horizon: int = 32) -> np.ndarray:
    T = len(tr.masses)
    M = np.stack(tr.masses) if T else np.zeros((0, 1, 1))     # [T][h][1 + n_windows]
    nw = M.shape[2] - 1
    out = []
    for t_r, n_r, st in zip(tr.t, tr.n, tr.state):
        if t_r >= T:
            continue
        st = _pad(st, nw)
        starts = tr.n_sink + tr.window * np.arange(nw)
        created = np.arange(nw) < len(st)
        ev = (st == S_EVICTED)
        exist = np.concatenate([[True], (starts < n_r) & created])
        block = M[t_r: min(t_r + horizon, T)]                  # steps t_r + 1 .. (0-based rows)
        num = block[:, :, 1:][:, :, ev].sum(axis=(0, 2))
        den = block[:, :, exist].sum(axis=(0, 2))
        out.append(float(np.mean(np.where(den > 0, num / np.where(den > 0, den, 1.0), 0.0))))
    return np.array(out)


def selection_churn(tr: Trace) -> np.ndarray:
    out = []
    for a, b in zip(tr.state, tr.state[1:]):
        n = max(len(a), len(b))
        ra = np.isin(_pad(a, n), (S_FULL, S_QUANT))
        rb = np.isin(_pad(b, n), (S_FULL, S_QUANT))
        union = np.count_nonzero(ra | rb)
        out.append(0.0 if union == 0 else 1.0 - np.count_nonzero(ra & rb) / union)
    return np.array(out)


def tier_mass_share(tr: Trace, r: int) -> dict:
    st, sf = np.asarray(tr.state[r]), np.asarray(tr.s_full[r])[: len(tr.state[r])]
    tot = sf.sum()
    return {z: float(sf[st == z].sum() / tot) if tot > 0 else 0.0 for z in (S_FULL, S_QUANT, S_EVICTED, S_LOCAL)}


def quantized_score_agreement(tr: Trace, r: int):
    st = np.asarray(tr.state[r])
    q = st == S_QUANT
    if not q.any():
        return None
    a = np.asarray(tr.s_q[r])[: len(st)][q]
    f = np.asarray(tr.s_full[r])[: len(st)][q]
    na, nf = np.linalg.norm(a), np.linalg.norm(f)
    cos = float(a @ f / (na * nf)) if na > 0 and nf > 0 else 0.0
    ratio = float(a.sum() / f.sum()) if f.sum() > 0 else 0.0
    return cos, ratio


def selections(tr: Trace, which: str) -> tuple[np.ndarray, np.ndarray]:
    """X [R][n_windows] (0/1) and the aged mask for the policy's Full tier ("policy") or
    the reference top-K_f of the aged windows ("oracle")."""
    R = len(tr.state)
    nw = max(len(s) for s in tr.state) if R else 0
    X = np.zeros((R, nw), dtype=np.int8)
    aged = np.zeros((R, nw), dtype=bool)
    for r, st in enumerate(tr.state):
        st = _pad(st, nw)
        aged[r] = np.isin(st, (S_FULL, S_QUANT, S_EVICTED))
        if which == "policy":
            X[r] = st == S_FULL
        else:
            sf = _pad(np.asarray(tr.s_full[r])[: len(tr.state[r])], nw, 0.0)
            cand = np.flatnonzero(aged[r])
            order = cand[np.lexsort((cand, -sf[cand]))]        # score descending, index ascending
            X[r, order[: tr.K_f]] = 1
    return X, aged


def global_lir(X: np.ndarray, m: int = 3) -> tuple[int, int, list]:
    R, nw = X.shape
    rescued = eligible = 0
    lengths = []
    for w in range(nw):
        x = X[:, w]
        dep = np.flatnonzero((x[:-1] == 1) & (x[1:] == 0)) + 1     # first inactive event of each episode
        for s in dep:
            back = np.flatnonzero(x[s:] == 1)
            end = s + back[0] if back.size else R
            length = end - s
            if length >= m:
                eligible += 1
                if back.size:
                    rescued += 1
                    lengths.append(int(length))
    return rescued, eligible, lengths


def lagged_transitions(X: np.ndarray, aged: np.ndarray, delta: int) -> dict:
    R = X.shape[0]
    if R <= delta:
        return {(a, b): 0.0 for a in (0, 1) for b in (0, 1)}
    a_now, b_later, mask = X[: R - delta], X[delta:], aged[: R - delta]
    out = {}
    for a in (0, 1):
        sel = mask & (a_now == a)
        n = np.count_nonzero(sel)
        for b in (0, 1):
            out[(a, b)] = float(np.count_nonzero(sel & (b_later == b)) / n) if n else 0.0
    return out


def summarize(tr: Trace, horizon: int = 32, m: int = 3, deltas=(1, 8)) -> dict:
    """All metrics of one trace, averaged over events where the pages average them."""
    fmm = future_missed_mass(tr, horizon)
    churn = selection_churn(tr)
    shares = [tier_mass_share(tr, r) for r in range(len(tr.state))]
    qsa = [x for x in (quantized_score_agreement(tr, r) for r in range(len(tr.state))) if x is not None]
    out = {
        "events": len(tr.state),
        "fmm": float(fmm.mean()) if fmm.size else None,
        "churn": float(churn.mean()) if churn.size else None,
        "mass_share_last": {name: shares[-1][z] for name, z in
                            (("full", S_FULL), ("quantized", S_QUANT), ("evicted", S_EVICTED), ("local", S_LOCAL))}
        if shares else None,
        "qsa": float(np.mean([c for c, _ in qsa])) if qsa else None,
        "r_q": float(np.mean([q for _, q in qsa])) if qsa else None,
        "promotions": int(sum(tr.promoted)),
    }
    for which in ("policy", "oracle"):
        X, aged = selections(tr, which)
        res, eli, lens = global_lir(X, m)
        out[f"lir_{which}"] = {"rescued": res, "eligible": eli, "rate": res / eli if eli else None,
                               "median_return": float(np.median(lens)) if lens else None}
        out[f"transitions_{which}"] = {f"P{a}{b}({d})": v for d in deltas
                                       for (a, b), v in lagged_transitions(X, aged, d).items()}
    return out


def record(policy, reference, layer: int, b: int, run_step, steps: int, omega: int) -> Trace:
    """Drive both states for ``steps`` decode steps of (layer, sequence b) through
    ``run_step(j)`` (which calls decode_attn on both states and nothing else) and route
    both every ``omega`` steps, recording what the metrics need."""
    ex = policy.export_unit(layer, b, tables_only=True)
    tr = Trace(n_sink=policy.cfg.n_sink, window=policy.cfg.window, K_f=ex.K_f)
    for j in range(steps):
        run_step(j)
        tr.masses.append(reference.step_mass(layer, b).cpu().numpy())
        if (j + 1) % omega == 0:
            policy.route(layer)
            reference.route(layer)
            ep = policy.export_unit(layer, b, tables_only=True)
            er = reference.export_unit(layer, b, tables_only=True)
            tr.t.append(j + 1)
            tr.n.append(ep.n)
            tr.state.append(ep.state.copy())
            tr.s_q.append(ep.score[: ep.n_windows].copy())
            tr.s_full.append(er.score[: er.n_windows].copy())
            tr.promoted.append(int(ep.counters["promoted"]))
    return tr
