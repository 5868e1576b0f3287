"""Plain reference implementation of the routing diagnostics of QEvict.

TEST INFRASTRUCTURE.  Only ``tests/`` (and ``bench.py``'s cpu_baseline leg) may import
this module; the library's own diagnostics (``recoverable_kv_cache_amd/diagnostics.py``)
share no code with it.  Plain Python loops over windows and events, float64.

Source: "QEvict: Recoverable Quantized KV Eviction for Attention-Drift-Robust
Long-Context Decoding", Appendix I: Eq. 12 (FullKV reference score), Eq. 13 (Future
Missed Mass), Eq. 14 (Selection Churn), Eq. 15 (tier-mass share), Eq. 16 (Quantized-Score
Agreement), Eq. 17 (mass ratio R_Q), Eq. 18 (Global LIR), Eq. 19 (lagged transition
probabilities); Appendix K (Q -> F promotions, one-way variant).

Readings (the pages leave these open):

* routing is per (sequence, layer), so the evicted / retained sets are the same for
  every head; FMM is computed per head and averaged over heads, then over events;
* a decode-time routing event r follows decode step t_r; its horizon is the steps
  t_r + 1 .. min(t_r + H, T);
* "positions that existed at r" are counted at window granularity: the sinks and every
  window whose first position is below n_r (a partly filled recent window counts whole;
  the recent region is never evicted, so only FMM's denominator sees this);
* the evicted set E_r is every window in the Evicted tier after event r; the retained
  set R_r of Eq. 14 is Full ∪ Quantized (historical windows only, the recent region and
  the sinks excluded); all windows have W tokens, so the Jaccard distance over token
  positions equals the one over windows;
* S^Full (Eqs. 15-17) is the head-averaged cumulative score of the FullKV reference run
  (prefill initialisation included), S^Q the policy's own score;
* an inactive episode (Eq. 18) starts when a window leaves the selected set and lasts
  while it stays out; it is eligible once it has lasted m events and rescued if the
  window is selected again at a later event; episodes running to the end count as not
  rescued; the lagged transitions (Eq. 19) run over windows that are aged (candidates)
  at event r;
* the oracle selection of Appendix I.4 is the top-K_f of the aged windows by S^Full.
"""
from __future__ import annotations

import math
from typing import Optional

from oracle.qevict_oracle import EVICTED, FULL, LOCAL, NONE, QUANT


def future_missed_mass(events: list, masses: list, n_sink: int, window: int, horizon: int = 32) -> list:
    """Eq. 13 per event.  events[r] = dict(t=steps done, n=tokens, state={w: tier});
    masses[tau - 1] = per-head rows [h][1 + n_windows] (column 0 the sinks) of the
    FullKV reference at decode step tau.  Returns FMM per eligible event."""
    T = len(masses)
    out = []
    for ev in events:
        t_r, n_r = ev["t"], ev["n"]
        if t_r >= T:
            continue
        evicted = [w for w, z in ev["state"].items() if z == EVICTED]
        existing = [w for w in ev["state"] if n_sink + w * window < n_r]
        H_q = len(masses[0])
        per_head = []
        for h in range(H_q):
            num = 0.0
            den = 0.0
            for tau in range(t_r + 1, min(t_r + horizon, T) + 1):
                row = masses[tau - 1][h]
                for w in evicted:
                    num += row[1 + w]
                den += row[0]
                for w in existing:
                    den += row[1 + w]
            per_head.append(num / den if den > 0 else 0.0)
        out.append(sum(per_head) / H_q)
    return out


def retained(state: dict) -> set:
    return {w for w, z in state.items() if z in (FULL, QUANT)}


def selection_churn(events: list) -> list:
    """Eq. 14 between consecutive events."""
    out = []
    for a, b in zip(events, events[1:]):
        ra, rb = retained(a["state"]), retained(b["state"])
        union = ra | rb
        out.append(0.0 if not union else 1.0 - len(ra & rb) / len(union))
    return out


def tier_mass_share(state: dict, s_full: dict) -> dict:
    """Eq. 15: share of the FullKV cumulative mass held by each tier."""
    total = sum(s_full[w] for w in state)
    out = {}
    for z in (FULL, QUANT, EVICTED, LOCAL):
        part = sum(s_full[w] for w, zz in state.items() if zz == z)
        out[z] = part / total if total > 0 else 0.0
    return out


def quantized_score_agreement(state: dict, s_q: dict, s_full: dict) -> Optional[tuple]:
    """Eqs. 16-17 over the Quantized windows: (cosine, mass ratio), None without any."""
    Q = [w for w, z in state.items() if z == QUANT]
    if not Q:
        return None
    dot = sum(s_q[w] * s_full[w] for w in Q)
    nq = math.sqrt(sum(s_q[w] ** 2 for w in Q))
    nf = math.sqrt(sum(s_full[w] ** 2 for w in Q))
    cos = dot / (nq * nf) if nq > 0 and nf > 0 else 0.0
    ratio = sum(s_q[w] for w in Q) / sum(s_full[w] for w in Q) if sum(s_full[w] for w in Q) > 0 else 0.0
    return cos, ratio


def oracle_selection(state: dict, s_full: dict, k_f: int) -> set:
    """Appendix I.4: the top-K_f aged windows by the FullKV score (ties: lower index)."""
    aged = [w for w, z in state.items() if z not in (LOCAL, NONE)]
    aged.sort(key=lambda w: (-s_full[w], w))
    return set(aged[:k_f])


def global_lir(selected: list, aged: list, m: int = 3) -> tuple:
    """Eq. 18.  selected[r] / aged[r]: sets of windows at event r.  Returns
    (rescued, eligible, lengths of the rescued episodes)."""
    R = len(selected)
    windows = set().union(*aged) if aged else set()
    rescued = eligible = 0
    lengths = []
    for w in sorted(windows):
        r = 0
        while r < R:
            if w in selected[r] and r + 1 < R and w not in selected[r + 1]:
                start = r + 1          # the window has just left the selected set
                end = start
                while end < R and w not in selected[end]:
                    end += 1
                length = end - start
                if length >= m:
                    eligible += 1
                    if end < R:
                        rescued += 1
                        lengths.append(length)
                r = end
            else:
                r += 1
    return rescued, eligible, lengths


def lagged_transitions(selected: list, aged: list, delta: int) -> dict:
    """Eq. 19: P[X_{r+delta} = b | X_r = a] over windows aged at event r."""
    counts = {(a, b): 0 for a in (0, 1) for b in (0, 1)}
    for r in range(len(selected) - delta):
        for w in aged[r]:
            a = 1 if w in selected[r] else 0
            b = 1 if w in selected[r + delta] else 0
            counts[(a, b)] += 1
    out = {}
    for a in (0, 1):
        n = counts[(a, 0)] + counts[(a, 1)]
        for b in (0, 1):
            out[(a, b)] = counts[(a, b)] / n if n else 0.0
    return out
