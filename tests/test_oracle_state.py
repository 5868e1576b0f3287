"""Pins of the oracle's accounting, decode attention, scores, prefill and router.

Pins used: the capacities the QEvict paper prints for its diagnostic settings
(Appendix I.1), dense attention from torch's scaled_dot_product_attention when
the budget covers the whole cache with q = 0 (a textbook special case), torch
softmax column sums for the prefill, torch.logsumexp, heapq / brute force for
TopK, and invariants stated in the pages (mass sums to one, the §4.1 budget,
Eq. 6 irreversibility, the write-once ledger of §4.3).
"""
import heapq
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import qevict_oracle as O
from recoverable_kv_cache_amd import workload as WL
from tests.oracle_helpers import cfg_from, f64, run_unit

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------------- accounting
def test_printed_diagnostic_capacities():
    g = json.load(open(os.path.join(GOLDEN, "diagnostic_capacities.json")))
    for case in g["cases"]:
        cfg = O.OracleConfig(h_q=g["h_q"], h_kv=g["h_kv"], d=g["d"], window=case["window"],
                             n_sink=g["n_sink"], n_local=g["n_local"], omega=case["window"],
                             quant_frac=g["quant_frac"], budget_frac=g["budget_frac"],
                             n_decode=g["n_decode"])
        caps = O.capacities(cfg, g["prompt_len"])
        assert (caps["K_f"], caps["K_q"]) == (case["K_f"], case["K_q"]), case["name"]


@pytest.mark.parametrize("bits", [2, 4])
def test_capacities_are_maximal_within_budget(bits):
    for wl in WL.ALL_WORKLOADS:
        cfg = cfg_from(wl, quant_bits=bits)
        caps = O.capacities(cfg, wl.prompt_len)
        assert caps["K_f"] * caps["M_f"] <= (1 - cfg.quant_frac) * caps["B_hist"] < (caps["K_f"] + 1) * caps["M_f"]
        assert caps["K_q"] * caps["M_q"] <= cfg.quant_frac * caps["B_hist"] < (caps["K_q"] + 1) * caps["M_q"]
        used = (cfg.n_sink + cfg.n_local) * caps["b_tok"] + caps["K_f"] * caps["M_f"] + caps["K_q"] * caps["M_q"]
        assert used <= caps["B_total"]


@pytest.mark.parametrize("bits", [2, 4])
def test_quantized_window_bytes_equal_the_stored_record(bits):
    """M_q is what a Quantized window actually stores: its canonical record (codes of
    both tensors + fp16 parameters of every head) + a 4-byte position + the 16-byte
    ledger entry."""
    wl = WL.TINY
    cfg = cfg_from(wl, quant_bits=bits)
    rng = np.random.default_rng(4)
    k = O.to_bf16(rng.standard_normal((cfg.h_kv, cfg.window, cfg.d)))
    v = O.to_bf16(rng.standard_normal((cfg.h_kv, cfg.window, cfg.d)))
    led = O.quantize_window(k, v, 0, bits=bits)
    assert O.quant_window_bytes(cfg) == len(O.canonical_ledger_bytes(led)) + 4 + 16


def test_int2_retains_more_windows_than_int4():
    """[QEvict] Appendix G.3: under one byte budget INT2 keeps more historical windows
    than INT4; the Full tier's share is the same."""
    for wl in WL.ALL_WORKLOADS:
        c2 = O.capacities(cfg_from(wl), wl.prompt_len)
        c4 = O.capacities(cfg_from(wl, quant_bits=4), wl.prompt_len)
        assert c4["K_f"] == c2["K_f"] and c4["M_q"] > c2["M_q"]
        assert c4["K_q"] < c2["K_q"] or c2["K_q"] == 0


def test_quant_share_goes_to_quantized_tier():
    """App. B.5: a fraction q of the historical budget goes to the quantized tier,
    1 - q to the full-precision tier."""
    for q in (0.1, 0.3, 0.7, 0.9):
        cfg = cfg_from(WL.LLAMA8B_32K, quant_frac=q)
        caps = O.capacities(cfg, 32768)
        fq, ff = caps["K_q"] * caps["M_q"], caps["K_f"] * caps["M_f"]
        assert abs(fq / (fq + ff) - q) < 0.01


def test_budget_error_and_zero_full_tier():
    with pytest.raises(O.BudgetError):
        O.capacities(cfg_from(WL.TINY, budget_frac=0.10), 512)
    caps = O.capacities(cfg_from(WL.TINY, budget_frac=0.15), 512)
    assert caps["K_f"] == 0 and caps["K_q"] > 0


def test_eq7_full_cache_bytes():
    # Eq. 7 with L = 1: M_FullKV = 2 H_kv d_h S c_f, c_f = 2 bytes for bf16
    cfg = cfg_from(WL.LLAMA8B_32K)
    assert O.token_bytes(cfg) * 1000 == 2 * 8 * 128 * 1000 * 2


# ---------------------------------------------------------------------------------- decode
def _dense_reference(q, K, V):
    """torch SDPA over the whole cache in float64 (q [H_q][d], K/V [H_kv][n][d])."""
    G = q.shape[0] // K.shape[0]
    qt = torch.from_numpy(q)[:, None, :]
    Kt = torch.from_numpy(K).repeat_interleave(G, 0)
    Vt = torch.from_numpy(V).repeat_interleave(G, 0)
    return torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt)[:, 0, :].numpy()


def test_dense_equivalence_when_budget_covers_cache():
    wl = WL.TINY.with_(n_decode=24)
    cfg = cfg_from(wl, budget_frac=1.0, quant_frac=0.0)
    caps = O.capacities(cfg, wl.prompt_len)
    n_can_age = (wl.prompt_len + wl.n_decode - wl.n_local - wl.n_sink) // wl.window
    assert caps["K_q"] == 0 and caps["K_f"] >= n_can_age
    qp, kp, vp = WL.prompt(wl, 0)
    unit = O.UnitOracle(cfg, wl.prompt_len)
    unit.prefill(f64(qp[0]), f64(kp[0]), f64(vp[0]))
    K_all, V_all = f64(kp[0]), f64(vp[0])
    for j in range(wl.n_decode):
        q, k, v = WL.decode_step(wl, 0, j)
        out = unit.step_and_route(f64(q[0]), f64(k[0]), f64(v[0]))
        K_all = np.concatenate([K_all, f64(k[0])[:, None]], axis=1)
        V_all = np.concatenate([V_all, f64(v[0])[:, None]], axis=1)
        np.testing.assert_allclose(out["o"], _dense_reference(f64(q[0]), K_all, V_all), rtol=0, atol=1e-12)
    assert all(e["evicted"] == 0 and e["n_quant"] == 0 for e in unit.events)


def test_mass_sums_to_one_and_matches_torch_softmax():
    wl = WL.TINY.with_(n_decode=17)
    cfg = cfg_from(wl, budget_frac=0.25)               # forces eviction (K_f=1, K_q=15)
    unit, outs = run_unit(wl, cfg)
    for out in outs:
        tm = out["tier_mass"]
        total = tm["sink"] + tm[O.LOCAL] + tm[O.FULL] + tm[O.QUANT]
        np.testing.assert_allclose(total, 1.0, rtol=0, atol=1e-12)
        A = torch.from_numpy(out["probs"])
        assert torch.allclose(A.sum(1), torch.ones(A.shape[0], dtype=torch.float64), atol=1e-12)


def test_window_mass_against_independent_softmax():
    wl = WL.TINY.with_(n_decode=9)
    cfg = cfg_from(wl, budget_frac=0.25)
    unit, _ = run_unit(wl, cfg, steps=8)
    before = dict(unit.score)
    q, k, v = WL.decode_step(wl, 0, 8)
    out = unit.decode(f64(q[0]), f64(k[0]), f64(v[0]))
    owner, K, V = unit.accessible()
    G = cfg.group
    logits = torch.stack([torch.from_numpy(K[h // G] @ f64(q[0])[h]) for h in range(cfg.h_q)]) / math.sqrt(cfg.d)
    P = torch.softmax(logits, dim=1).numpy()
    for w, u in out["mass"].items():
        assert abs(u - P[:, owner == w].sum() / cfg.h_q) < 1e-13
        assert abs(unit.score[w] - before[w] - u) < 1e-12


def test_score_only_on_routing_steps_flag():
    wl = WL.TINY.with_(n_decode=16)
    cfg = cfg_from(wl, budget_frac=0.25, score_every_step=False)
    unit, outs = run_unit(wl, cfg, steps=7)
    s7 = dict(unit.score)
    q, k, v = WL.decode_step(wl, 0, 7)
    unit.step_and_route(f64(q[0]), f64(k[0]), f64(v[0]))
    # steps 0..6 are not routing steps: the score equals the prefill score
    unit0, _ = run_unit(wl, cfg, steps=0)
    for w in unit0.score:
        assert s7[w] == unit0.score[w]


# ---------------------------------------------------------------------------------- prefill
def test_prefill_scores_against_torch_column_sums():
    wl = WL.TINY.with_(prompt_len=200, n_local=32)
    cfg = cfg_from(wl, budget_frac=0.5)
    qp, kp, vp = WL.prompt(wl, 0)
    unit = O.UnitOracle(cfg, 200)
    info = unit.prefill(f64(qp[0]), f64(kp[0]), f64(vp[0]))
    S, G = 200, cfg.group
    Q, K = torch.from_numpy(f64(qp[0])), torch.from_numpy(f64(kp[0]))
    mask = torch.ones(S, S, dtype=torch.bool).triu(1)
    col = torch.zeros(cfg.h_q, S, dtype=torch.float64)
    for h in range(cfg.h_q):
        lg = (Q[h] @ K[h // G].T) / math.sqrt(cfg.d)
        col[h] = torch.softmax(lg.masked_fill(mask, float("-inf")), dim=1).sum(0)
    np.testing.assert_allclose(info["col"], col.numpy(), rtol=1e-12, atol=1e-12)
    # invariant: every causal row sums to one, so window scores + sink mass = prompt length
    total = sum(unit.score.values()) + info["sink_mass"]
    assert abs(total - S) < 1e-9
    # row LSE against torch.logsumexp
    for u in (0, 7, 150, 199):
        lse = O.row_lse(f64(qp[0])[1][u], f64(kp[0])[0][: u + 1])
        ref = torch.logsumexp(K[0][: u + 1] @ Q[1][u] / math.sqrt(cfg.d), 0).item()
        assert abs(lse - ref) < 1e-12


def test_prefill_routes_only_aged_windows():
    wl = WL.TINY
    cfg = cfg_from(wl, budget_frac=0.25)
    unit, _ = run_unit(wl, cfg, steps=0)
    ev = unit.events[0]
    n_aged = sum(1 for w in range(64) if cfg.n_sink + (w + 1) * cfg.window <= 512 - cfg.n_local)
    assert ev["aged"] == n_aged == len(ev["order"])
    for w, (st, *_rest) in unit.window_table().items():
        if w >= n_aged:
            assert st == O.LOCAL


# ---------------------------------------------------------------------------------- router
def test_route_order_equals_full_sort_and_heap_selection():
    rng = np.random.default_rng(0)
    for trial in range(200):
        n = int(rng.integers(1, 40))
        vals = rng.integers(0, 6, n).astype(float) / 4.0       # many ties
        ids = rng.permutation(1000)[:n].tolist()
        scores = dict(zip(ids, vals))
        order = O.route_order(ids, scores)
        for K in range(0, n + 1):
            top = heapq.nsmallest(K, ids, key=lambda w: (-scores[w], w))
            assert order[:K] == top
    # exhaustive on a tiny pool: the order is the unique permutation that is
    # non-increasing in score and increasing in index within equal scores
    ids = [3, 1, 4, 0, 2]
    scores = {3: 0.5, 1: 0.5, 4: 1.0, 0: 0.25, 2: 0.5}
    ok = [p for p in itertools.permutations(ids)
          if all((scores[a] > scores[b]) or (scores[a] == scores[b] and a < b) for a, b in zip(p, p[1:]))]
    assert ok == [tuple(O.route_order(ids, scores))]


@pytest.mark.parametrize("rho,q", [(0.25, 0.70), (0.15, 0.70), (0.40, 0.0), (0.25, 1.0)])
def test_router_invariants_over_a_run(rho, q):
    wl = WL.TINY
    cfg = cfg_from(wl, budget_frac=rho, quant_frac=q)
    caps = O.capacities(cfg, wl.prompt_len)
    unit, _ = run_unit(wl, cfg, collect=False)
    seen_evicted = set()
    for ev in unit.events:
        assert len(ev["F"]) <= caps["K_f"] and len(ev["Q"]) <= caps["K_q"]
        assert not (set(ev["order"]) & seen_evicted)        # Eq. 6: evicted windows never return
        seen_evicted |= set(ev["E"])
        if caps["K_q"] == 0:
            assert ev["n_quant"] == 0
        if caps["K_f"] == 0:
            assert ev["n_full"] == 0
    assert seen_evicted, "these budgets force eviction"


@pytest.mark.parametrize("bits", [2, 4])
def test_write_once_ledger_and_promoted_values(bits):
    """A window taken F -> Q -> F -> Q keeps the codes of its first demotion, and a
    promoted window holds bf16(x_hat), not its original values."""
    wl = WL.TINY.with_(n_decode=0)
    cfg = cfg_from(wl, budget_frac=0.25, quant_bits=bits)          # K_f = 1
    qp, kp, vp = WL.prompt(wl, 0)
    unit = O.UnitOracle(cfg, 512)
    n_win = 32
    unit.prefill(f64(qp[0]), f64(kp[0]), f64(vp[0]), score_init=np.zeros(n_win))
    w = 5
    s0 = cfg.n_sink + w * cfg.window
    orig_k = f64(kp[0])[:, s0:s0 + cfg.window]
    # zero scores: ties go to the lowest indices, so window 0 is Full and w is Quantized
    assert unit.win[0].state == O.FULL and unit.win[w].state == O.QUANT
    unit.score[w] = 1e6
    unit.route()
    assert unit.win[w].state == O.FULL
    # push it to Q (first demotion creates the ledger)
    unit.score[w] = 0.5
    unit.score[0] = 1e7
    unit.route()
    assert unit.win[w].state == O.QUANT
    first = O.canonical_ledger_bytes(unit.win[w].ledger)
    assert unit.win[w].ledger.bits == bits and unit.win[w].ledger.k_codes.max() <= 2 ** bits - 1
    # promote: bf16 of the dequantized values, ledger dormant
    unit.score[w] = 1e8
    unit.route()
    W = unit.win[w]
    assert W.state == O.FULL and W.ledger.dormant
    np.testing.assert_array_equal(W.k, O.to_bf16(W.ledger.k_hat()))
    assert not np.array_equal(W.k, orig_k)
    # demote again: reactivated, bit-identical record
    unit.score[w] = 0.5
    unit.score[0] = 1e9
    ev = unit.route()
    assert unit.win[w].state == O.QUANT and not unit.win[w].ledger.dormant
    assert ev["reactivated"] >= 1
    assert O.canonical_ledger_bytes(unit.win[w].ledger) == first


def test_drift_workload_exercises_promotion():
    """With a drifting query the tiers churn: windows are demoted and promoted."""
    wl = WL.TINY.with_(n_topics=4, topic_period=16, n_decode=64, n_outlier=2)
    cfg = cfg_from(wl, budget_frac=0.25)
    # flat initial scores so that decode-time mass decides the tiers
    unit, _ = run_unit(wl, cfg, collect=False, score_init=np.zeros(32))
    assert sum(e["promoted"] for e in unit.events) > 0
    assert sum(e["packed"] for e in unit.events) > 0


def _hand_pool(promote: bool):
    """A unit with seven windows of four tokens after two sinks (30 positions, four recent):
    window 0 Quantized (score 10), 1 Full (5), 2 aged recent (8), 3 aged recent (1),
    4 Quantized (0.5), 5 Full (3), 6 still recent (100, not a candidate); K_f = K_q = 2."""
    cfg = O.OracleConfig(h_q=2, h_kv=1, d=16, window=4, n_sink=2, n_local=4, omega=1, quant_frac=0.5,
                         budget_frac=1.0, n_decode=0, promote=promote)
    rng = np.random.default_rng(7)
    unit = O.UnitOracle(cfg, 30)
    for p in range(30):
        unit._store(p, O.to_bf16(rng.standard_normal((1, 16))), O.to_bf16(rng.standard_normal((1, 16))))
    unit.n = 30
    unit.caps = dict(unit.caps, K_f=2, K_q=2)
    for w in (0, 4):
        W = unit.win[w]
        W.ledger = O.quantize_window(W.k, W.v, unit.win_start(w))
        W.state, W.k, W.v = O.QUANT, None, None
    for w in (1, 5):
        unit.win[w].state = O.FULL
    unit.score.update({0: 10.0, 1: 5.0, 2: 8.0, 3: 1.0, 4: 0.5, 5: 3.0, 6: 100.0})
    return unit


def test_route_sets_hand_case_bidirectional():
    """Eqs. 4-5 worked by hand: rank order 0 (10), 2 (8), 1 (5), 5 (3), 3 (1), 4 (0.5); window 6
    has not aged (its end 30 > n - n_local = 26) and is no candidate."""
    unit = _hand_pool(promote=True)
    ev = unit.route()
    assert (ev["F"], ev["Q"], ev["E"]) == ([0, 2], [1, 5], [3, 4])
    assert (ev["promoted"], ev["packed"], ev["demoted"], ev["evicted"]) == (1, 2, 2, 2)
    states = {w: unit.win[w].state for w in range(7)}
    assert states == {0: O.FULL, 1: O.QUANT, 2: O.FULL, 3: O.EVICTED, 4: O.EVICTED, 5: O.QUANT, 6: O.LOCAL}
    assert unit.win[0].ledger.dormant


def test_route_sets_hand_case_one_way():
    """The one-way policy of [QEvict] Appendix K on the same pool: same capacities and rank
    order, but Quantized windows 0 and 4 may not enter Full.  Full = the top two of the eligible
    windows {2 (8), 1 (5), 5 (3), 3 (1)}; Quantized = the next two of everything left in rank
    order {0 (10), 5 (3), 3 (1), 4 (0.5)}: window 0 outranks all and stays Quantized."""
    unit = _hand_pool(promote=False)
    ev = unit.route()
    assert (ev["F"], ev["Q"], ev["E"]) == ([2, 1], [0, 5], [3, 4])
    assert (ev["promoted"], ev["packed"], ev["demoted"], ev["evicted"]) == (0, 1, 1, 2)
    assert len(ev["F"]) == unit.caps["K_f"]               # the Full tier is filled, not left short
    states = {w: unit.win[w].state for w in range(7)}
    assert states == {0: O.QUANT, 1: O.FULL, 2: O.FULL, 3: O.EVICTED, 4: O.EVICTED, 5: O.QUANT, 6: O.LOCAL}
    assert not unit.win[0].ledger.dormant


def _values_from_record(rec: bytes, h_kv: int, W: int, d: int):
    """Dequantized K, V [h_kv][W][d] read straight from a canonical INT2 record (codes four to
    a byte, low bits first; fp16 offsets and scales): x = off + code * scl in float64."""
    cb = W * d // 4
    per = 2 * cb + 4 * d + 4 * W
    ks, vs = [], []
    for h in range(h_kv):
        b = np.frombuffer(rec, np.uint8, count=per, offset=h * per)
        codes = lambda x: np.stack([(x >> (2 * j)) & 3 for j in range(4)], -1).reshape(W, d).astype(np.float64)
        p = np.frombuffer(rec, "<f2", count=2 * d + 2 * W, offset=h * per + 2 * cb).astype(np.float64)
        koff, kscl, voff, vscl = p[:d], p[d:2 * d], p[2 * d:2 * d + W], p[2 * d + W:]
        ks.append(koff[None, :] + codes(b[:cb]) * kscl[None, :])
        vs.append(voff[:, None] + codes(b[cb:2 * cb]) * vscl[:, None])
    return np.stack(ks), np.stack(vs)


@pytest.mark.parametrize("bf16_values", [False, True])
def test_quantized_execution_readings_against_sdpa(bf16_values):
    """Reading R2: inside attention a Quantized window holds its exact dequantized values
    x = off + code * scl, or, in the model's execution dtype, their bf16 rounding.  The oracle's
    attention over sinks, recent / Full pages and Quantized windows equals torch SDPA over a cache
    rebuilt from the stored records (values decoded from the record bytes, rounded by torch's
    bf16 cast for the second reading)."""
    wl = WL.TINY.with_(n_decode=9)
    cfg = cfg_from(wl, budget_frac=0.3)
    qp, kp, vp = WL.prompt(wl, 0)
    unit = O.UnitOracle(cfg, wl.prompt_len)
    unit.prefill(f64(qp[0]), f64(kp[0]), f64(vp[0]), score_init=np.arange(64, dtype=np.float64))
    for j in range(8):
        q, k, v = WL.decode_step(wl, 0, j)
        unit.decode(f64(q[0]), f64(k[0]), f64(v[0]))
    unit.route()
    q, k, v = WL.decode_step(wl, 0, 8)
    out = unit.decode(f64(q[0]), f64(k[0]), f64(v[0]))
    Ks, Vs, n_quant = [torch.from_numpy(unit.sink_k)], [torch.from_numpy(unit.sink_v)], 0
    for w in sorted(unit.win):
        W = unit.win[w]
        if W.state == O.QUANT:
            kx, vx = (torch.from_numpy(x) for x in _values_from_record(O.canonical_ledger_bytes(W.ledger),
                                                                       wl.h_kv, wl.window, wl.d_head))
            if bf16_values:
                kx, vx = kx.to(torch.bfloat16).to(torch.float64), vx.to(torch.bfloat16).to(torch.float64)
            Ks.append(kx)
            Vs.append(vx)
            n_quant += 1
        elif W.state in (O.LOCAL, O.FULL):
            nt = min(wl.window, unit.n - unit.win_start(w))
            Ks.append(torch.from_numpy(W.k[:, :nt]))
            Vs.append(torch.from_numpy(W.v[:, :nt]))
    assert n_quant > 10
    K, V = torch.cat(Ks, dim=1), torch.cat(Vs, dim=1)
    G = wl.h_q // wl.h_kv
    qd = q[0].to(torch.float64)[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(qd, K.repeat_interleave(G, 0), V.repeat_interleave(G, 0))
    o = unit.attend(out["q_rot"], qexec_bf16=bf16_values)[0]
    np.testing.assert_allclose(o, ref[:, 0].numpy(), rtol=0, atol=1e-12)
    if not bf16_values:
        np.testing.assert_array_equal(o, out["o"])       # the step's own output is the exact reading
    else:
        assert np.abs(o - out["o"]).max() > 0            # the two readings differ here
