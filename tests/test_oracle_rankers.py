"""Pins of the oracle's alternative rankers ([QEvict] Appendix J, Eqs. 20-24).

Decay (Eq. 22) and p-norm (Eq. 23) are checked against closed forms on inputs where
attention is known without the oracle's softmax: with all keys zero every accessible
token gets the same weight, so a window's prefill score is a harmonic sum and its
mass at a decode step is (its tokens present) / (tokens present).  Key-norm (Eq. 24)
is checked on keys whose norm sits in one channel of one head.
"""
from fractions import Fraction

import numpy as np

from oracle import qevict_oracle as O


def _cfg(**kw):
    base = dict(h_q=2, h_kv=1, d=8, window=4, n_sink=2, n_local=8, omega=3, quant_frac=0.0,
                budget_frac=2.0, n_decode=12)   # room for every window in the Full tier
    base.update(kw)
    return O.OracleConfig(**base)


def _uniform_run(cfg, S, steps):
    """Zero keys, random queries and values: prefill + `steps` decode steps with routing
    (nothing is evicted, which the closed forms assume)."""
    rng = np.random.default_rng(3)
    unit = O.UnitOracle(cfg, S)
    qp = O.to_bf16(rng.standard_normal((cfg.h_q, S, cfg.d)))
    kp = np.zeros((cfg.h_kv, S, cfg.d))
    vp = O.to_bf16(rng.standard_normal((cfg.h_kv, S, cfg.d)))
    unit.prefill(qp, kp, vp)
    for _ in range(steps):
        unit.step_and_route(O.to_bf16(rng.standard_normal((cfg.h_q, cfg.d))), np.zeros((cfg.h_kv, cfg.d)),
                            O.to_bf16(rng.standard_normal((cfg.h_kv, cfg.d))))
    assert not unit.ever_evicted
    return unit


def _expected(cfg, S, steps, w):
    """Closed forms for window w: prefill score S_0 = sum over prompt rows u of the
    window's tokens <= u, each weighted 1/(u+1); interval masses u_r = sum over the
    decode steps of the interval of (window tokens < n) / n with n the length after
    the step's append (the budget keeps every token accessible)."""
    a, b = cfg.n_sink + w * cfg.window, cfg.n_sink + (w + 1) * cfg.window
    s0 = sum(Fraction(max(0, min(b, u + 1) - a), u + 1) for u in range(S))
    us, cur = [], Fraction(0)
    for j in range(steps):
        n = S + j + 1
        cur += Fraction(max(0, min(b, n) - a), n)
        if (j + 1) % cfg.omega == 0:
            us.append(cur)
            cur = Fraction(0)
    return s0, us, cur


def test_decay_matches_geometric_closed_form():
    cfg = _cfg(ranker="decay")
    S, steps = 18, 12
    unit = _uniform_run(cfg, S, steps)
    lam = Fraction(cfg.decay_lambda)
    for w in range(3):
        s0, us, rest = _expected(cfg, S, steps, w)
        want = s0
        for u in us:
            want = lam * want + u
        assert abs(unit.score[w] - float(want)) < 1e-12, (w, unit.score[w], float(want))
        assert abs(unit.uacc[w] - float(rest)) < 1e-12


def test_decay_is_applied_per_routing_event_not_per_step():
    cfg = _cfg(ranker="decay")
    S, steps = 18, 6
    unit = _uniform_run(cfg, S, steps)
    s0, us, _ = _expected(cfg, S, steps, 0)
    per_step = s0
    for j in range(steps):   # a per-step decay (the wrong reading) differs from the per-event one
        per_step = Fraction(cfg.decay_lambda) * per_step
    assert abs(unit.score[0] - float(per_step)) > 1e-3


def test_pnorm_matches_sum_of_cubes():
    cfg = _cfg(ranker="pnorm")
    S, steps = 18, 12
    unit = _uniform_run(cfg, S, steps)
    for w in range(3):
        s0, us, _ = _expected(cfg, S, steps, w)
        want = s0 ** 3 + sum(u ** 3 for u in us)
        assert abs(unit.score[w] - float(want)) <= 1e-12 * float(want), (w, unit.score[w], float(want))


def test_pnorm_rank_key_orders_like_its_root():
    rng = np.random.default_rng(5)
    P = {w: float(x) for w, x in enumerate(rng.random(200) ** 3 * 50)}
    root = {w: x ** (1 / 3) for w, x in P.items()}
    assert O.route_order(list(P), P) == O.route_order(list(P), root)


def test_cumulative_default_unchanged_by_the_accumulator():
    cfg = _cfg()
    S, steps = 18, 12
    unit = _uniform_run(cfg, S, steps)
    s0, us, rest = _expected(cfg, S, steps, 1)
    assert abs(unit.score[1] - float(s0 + sum(us) + rest)) < 1e-12
    assert all(v == 0.0 for v in unit.uacc.values())


def test_keynorm_scores_from_known_norms_and_prefers_small_keys():
    """Each prompt token's key carries its whole norm in channel 0 of head 0; windows
    that age get minus their mean norm; with room for half of them in the Full tier,
    the smaller-norm windows are kept there."""
    cfg = _cfg(ranker="keynorm", h_kv=2, h_q=4, budget_frac=0.45, quant_frac=0.0, n_local=4, n_decode=0)
    S = 2 + 4 * 6 + 3
    rng = np.random.default_rng(9)
    norms = O.to_bf16(rng.uniform(0.5, 8.0, S))
    kp = np.zeros((cfg.h_kv, S, cfg.d))
    kp[0, :, 0] = norms
    qp = O.to_bf16(rng.standard_normal((cfg.h_q, S, cfg.d)))
    vp = O.to_bf16(rng.standard_normal((cfg.h_kv, S, cfg.d)))
    unit = O.UnitOracle(cfg, S)
    ev = unit.prefill(qp, kp, vp)["route"]
    aged = [w for w in range(6) if cfg.n_sink + (w + 1) * cfg.window <= S - cfg.n_local]
    assert aged
    for w in aged:
        a = cfg.n_sink + w * cfg.window
        assert unit.score[w] == -float(np.mean(norms[a:a + cfg.window]))
    kept = ev["F"]
    dropped = ev["E"] + ev["Q"]
    assert kept and dropped
    assert max(-unit.score[w] for w in kept) <= min(-unit.score[w] for w in dropped)
