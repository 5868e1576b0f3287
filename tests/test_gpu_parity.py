"""GPU parity: the HIP path, called through the C ABI, against the fp64 oracle.

Every case runs prefill + decode steps + routing events in lockstep and checks
routing sets, ledger and pages bit-exactly, decode outputs within 2e-3 of
||o||_2 and window scores within 1e-4 (see tests/gpu_harness.py).
"""
import math

import numpy as np
import pytest
import torch

from oracle import qevict_oracle as O
from recoverable_kv_cache_amd import binding as B
from recoverable_kv_cache_amd import workload as WL
from tests.gpu_harness import Lockstep, bf16_bits, rel_err
from tests.oracle_helpers import f64

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


def test_tiny_config_full_lockstep():
    """The tiny single-layer workload: 512-token prompt + 64 decode steps, 8 events."""
    _print("case: tiny full lockstep")
    ls = Lockstep(WL.TINY).run(64)
    _print(f"tiny: max o err {ls.max_o_err:.2e} (bf16 reading {ls.max_o_err_bf16:.2e}, gap {ls.max_reading_gap:.2e}), max score err {ls.max_s_err:.2e}, events {ls.events}")


@pytest.mark.parametrize("rho,q", [(0.25, 0.70), (0.15, 0.70), (1.0, 0.0)], ids=["evict", "no-full-tier", "dense"])
def test_tiny_budget_variants(rho, q):
    _print(f"case: tiny rho={rho} q={q}")
    wl = WL.TINY.with_(budget_frac=rho, quant_frac=q)
    ls = Lockstep(wl).run(40)
    _print(f"rho={rho}: max o err {ls.max_o_err:.2e} (bf16 reading {ls.max_o_err_bf16:.2e}, gap {ls.max_reading_gap:.2e}), max score err {ls.max_s_err:.2e}")


def test_drift_with_promotions_and_splits():
    """Flat initial scores + drifting topic queries: windows are demoted, promoted
    (Q -> F dequantize into a page) and re-demoted (reactivation)."""
    _print("case: drift promotions")
    wl = WL.TINY.with_(n_topics=4, topic_period=16, n_decode=64, n_outlier=2, budget_frac=0.25)
    si = torch.zeros((1, 64), dtype=torch.float64)
    ls = Lockstep(wl, score_init=si, n_splits=5).run(64)
    unit = ls.units[0]
    assert sum(e["promoted"] for e in unit.events) > 0
    ex = ls.st.export_unit(0, 0)
    assert ex.counters["n_full"] == unit.events[-1]["n_full"]
    _print(f"drift: promotions {sum(e['promoted'] for e in unit.events)}, fills after a pack of their page {ex.counters['paired_fills']}")
    assert ex.counters["paired_fills"] > 0


def test_batched_ragged_prompts_gqa8_d128():
    """Ragged prompt lengths, 8 query heads per KV head, d=128, W=32 (reduced sizes)."""
    _print("case: ragged batch")
    wl = WL.Workload("ragged", 1, 3, 16, 2, 128, 640, 24, 32, 4, 64, 8, 0.30, 0.70, prompt_len_min=300,
                     n_outlier=2, n_topics=2, topic_period=8)
    ls = Lockstep(wl).run(24)
    _print(f"ragged: max o err {ls.max_o_err:.2e} (bf16 reading {ls.max_o_err_bf16:.2e}, gap {ls.max_reading_gap:.2e}), max score err {ls.max_s_err:.2e}")


@pytest.mark.parametrize("n_splits", [1, 3], ids=["one-split", "three-splits"])
def test_single_launch_step_and_finish_launch(n_splits):
    """With one split per (sequence, KV head) a decode step is one launch: the split kernel
    writes the output, the log-sum-exps and the token, and the last of a sequence's KV heads
    advances its count; QEVICT_F_SEPARATE_FINISH keeps the finish launch.  Both follow the
    oracle through drift, promotions and routing events (two sequences, 4 KV heads)."""
    wl = WL.Workload("one_launch_b2", 1, 2, 16, 4, 64, 768, 40, 16, 4, 64, 8, 0.30, 0.70, prompt_len_min=600,
                     n_outlier=2, n_topics=3, topic_period=12)
    si = torch.zeros((2, 64), dtype=torch.float64)
    for flags in (0, B.QEVICT_F_SEPARATE_FINISH):
        _print(f"case: n_splits={n_splits} flags={flags}")
        ls = Lockstep(wl, score_init=si, flags=flags, n_splits=n_splits)
        assert ls.st.info.n_splits == n_splits
        assert ls.st.info.combine_in_kernel == int(n_splits == 1 and not flags)
        ls.run(40)
        _print(f"n_splits={n_splits} flags={flags}: max o err {ls.max_o_err:.2e}, max score err {ls.max_s_err:.2e}")
        assert ls.st.poll_status() == 0
        assert sum(e["promoted"] for e in ls.units[0].events) + sum(e["promoted"] for e in ls.units[1].events) > 0
        paired = [ls.st.export_unit(0, b).counters["paired_fills"] for b in range(2)]
        _print("fills after a pack of their page:", paired)
        assert sum(paired) > 0   # (a promotion took a page a pack of the same event read: that path ran)


def test_window64_gqa8_multichunk():
    """70B-shaped heads at reduced size: W = 64 (an INT2 window spans two 32-token
    chunks of pair jobs, a bf16 window four tiles), 8 query heads per KV head, d = 128,
    ragged prompts, drifting queries."""
    _print("case: window 64, GQA 8")
    wl = WL.Workload("w64", 1, 2, 16, 2, 128, 1200, 24, 64, 4, 128, 8, 0.30, 0.70, prompt_len_min=700,
                     n_outlier=2, n_topics=2, topic_period=8)
    ls = Lockstep(wl).run(24)
    _print(f"w64: max o err {ls.max_o_err:.2e} (bf16 reading {ls.max_o_err_bf16:.2e}, gap {ls.max_reading_gap:.2e}), max score err {ls.max_s_err:.2e}, events {ls.events}")


def test_window16_d128_promotions():
    """Churn-shaped heads at reduced size: W = 16 (one 16-token tile per INT2 chunk),
    d = 128, GQA 4, flat initial scores and topic drift, so windows are promoted back to
    bf16 and demoted again."""
    _print("case: window 16, d 128")
    wl = WL.Workload("w16", 1, 2, 8, 2, 128, 700, 48, 16, 4, 64, 8, 0.20, 0.70, prompt_len_min=500,
                     n_outlier=2, n_topics=4, topic_period=16)
    n_win = math.ceil((wl.prompt_len + wl.n_decode - wl.n_sink) / wl.window)
    si = torch.zeros((wl.batch, n_win), dtype=torch.float64)
    ls = Lockstep(wl, score_init=si).run(48)
    assert sum(e["promoted"] for u in ls.units for e in u.events) > 0
    _print(f"w16: max o err {ls.max_o_err:.2e} (bf16 reading {ls.max_o_err_bf16:.2e}, gap {ls.max_reading_gap:.2e}), max score err {ls.max_s_err:.2e}, events {ls.events}")


def test_one_way_and_route_step_scoring_flags():
    _print("case: flags")
    wl = WL.TINY.with_(n_topics=4, topic_period=16, n_decode=32, budget_frac=0.25)
    si = torch.zeros((1, 64), dtype=torch.float64)
    ls = Lockstep(wl, score_init=si, flags=B.QEVICT_F_NO_PROMOTE | B.QEVICT_F_SCORE_ROUTE_ONLY).run(32)
    assert sum(e["promoted"] for e in ls.units[0].events) == 0


def test_mha_one_query_head_per_kv_head():
    """Plain multi-head attention (G = 1: the decode kernel's one-head column layout and the
    prefill passes' one-head workgroups), d = 128, W = 32, ragged batch, topic drift."""
    _print("case: mha")
    wl = WL.Workload("mha", 1, 2, 4, 4, 128, 600, 32, 32, 4, 64, 8, 0.30, 0.70, prompt_len_min=350,
                     n_outlier=2, n_topics=2, topic_period=8)
    ls = Lockstep(wl).run(32)
    assert any(u.win[w].ledger is not None for u in ls.units for w in u.win)
    _print(f"mha: max o err {ls.max_o_err:.2e} (bf16 reading {ls.max_o_err_bf16:.2e}, gap {ls.max_reading_gap:.2e}), max score err {ls.max_s_err:.2e}, events {ls.events}")


def test_short_prompt_edge_cases():
    """Prompts shorter than the sinks, empty prompts and a prompt that ends on a window edge."""
    for S in (0, 3, 4, 20):
        _print(f"case: prompt_len={S}")
        wl = WL.TINY.with_(prompt_len=S, n_decode=40, n_local=16, budget_frac=2.0)
        Lockstep(wl).run(40)


def test_forced_pack_and_promote_entry_points():
    """qevict_pack_int2 / qevict_promote against the oracle's codec and Algorithm 1."""
    _print("case: forced pack/promote")
    wl = WL.TINY.with_(n_decode=8)
    ls = Lockstep(wl)
    ls.prefill()
    unit = ls.units[0]
    full = [w for w, W in unit.win.items() if W.state == O.FULL]
    quant = [w for w, W in unit.win.items() if W.state == O.QUANT]
    assert full and quant
    # demote the Full windows, then promote two Quantized ones
    ids = torch.tensor([full], dtype=torch.int32, device="cuda")
    ls.st.pack_int2(0, ids)
    for w in full:
        W = unit.win[w]
        W.ledger = O.quantize_window(W.k, W.v, unit.win_start(w)) if W.ledger is None else W.ledger
        W.ledger.dormant = False
        W.k = W.v = None
        W.state = O.QUANT
    ls.check("after pack")
    prom = quant[:2]
    ls.st.promote(0, torch.tensor([prom], dtype=torch.int32, device="cuda"))
    for w in prom:
        W = unit.win[w]
        W.k, W.v = O.to_bf16(W.ledger.k_hat()), O.to_bf16(W.ledger.v_hat())
        W.ledger.dormant = True
        W.state = O.FULL
    ls.check("after promote")
    for j in range(8):
        ls.step(j)


def test_prefill_column_sums_mid_size():
    """MFMA column sums vs the oracle's dense causal softmax at S=1536, d=128, G=4."""
    _print("case: prefill column sums S=1536")
    wl = WL.Workload("mid", 1, 1, 8, 2, 128, 1536, 8, 32, 4, 256, 8, 0.2, 0.7, n_outlier=4, n_topics=4)
    cfg = B.make_config(wl)
    st = B.QEvictState(cfg, [1536])
    qp, kp, vp = WL.prompt(wl, 0)
    st.prefill_init(0, qp.cuda(), kp.cuda(), vp.cuda())
    torch.cuda.synchronize()
    lse_gpu, col_gpu = (t.cpu().numpy() for t in st.workspace_views())
    col_ref = O.prefill_column_sums(f64(qp[0]), f64(kp[0]))
    err = np.abs(col_gpu[0] - col_ref).max()
    _print(f"column-sum max abs err {err:.2e}")
    assert err < 2e-5
    for h, u in [(0, 0), (3, 777), (7, 1535)]:
        ref = O.row_lse(f64(qp[0])[h][u], f64(kp[0])[h // 4][: u + 1]) / math.log(2)
        assert abs(lse_gpu[0, h, u] - ref) < 1e-4
    ex = st.export_unit(0, 0)
    unit = O.UnitOracle(O.OracleConfig(8, 2, 128, 32, 4, 256, 8, 0.7, 0.2, 8), 1536)
    unit.prefill(f64(qp[0]), f64(kp[0]), f64(vp[0]))
    ref = np.array([unit.score[w] for w in range(ex.n_windows)])
    assert np.abs(ex.score[: ex.n_windows] - ref).max() < 1e-4
    assert abs(ex.score[: ex.n_windows].sum() + ex.sink_mass - 1536) < 1e-3


SINGLE_LAUNCH_CASES = {
    # name: (workload, flags)
    "int4": (WL.Workload("one_launch_int4", 1, 2, 16, 4, 64, 768, 32, 16, 4, 64, 8, 0.30, 0.70, prompt_len_min=600,
                         n_outlier=2, n_topics=3, topic_period=12), B.QEVICT_F_INT4),
    "rope": (WL.Workload("one_launch_rope", 1, 2, 16, 4, 64, 768, 32, 16, 4, 64, 8, 0.30, 0.70, prompt_len_min=600,
                         n_outlier=2, n_topics=3, topic_period=12), B.QEVICT_F_ROPE),
    "mha_d128": (WL.Workload("one_launch_mha", 1, 2, 4, 4, 128, 640, 32, 32, 4, 64, 8, 0.30, 0.70,
                             n_topics=2, topic_period=8), 0),
    "gqa8_d128_w64": (WL.Workload("one_launch_gqa8", 1, 3, 16, 2, 128, 900, 32, 64, 4, 64, 8, 0.30, 0.70,
                                  prompt_len_min=500, n_topics=2, topic_period=8), 0),
}


@pytest.mark.parametrize("case", list(SINGLE_LAUNCH_CASES))
def test_single_launch_step_variants(case):
    """One split per (sequence, KV head): the split kernel finishes the step for the INT4 and
    RoPE-faithful tiers and other head shapes, in lockstep with the oracle."""
    wl, flags = SINGLE_LAUNCH_CASES[case]
    _print(f"case: single launch {case}")
    ls = Lockstep(wl, flags=flags, n_splits=1)
    assert ls.st.info.combine_in_kernel == 1
    ls.run(32)
    _print(f"{case}: max o err {ls.max_o_err:.2e}, max score err {ls.max_s_err:.2e}, events {ls.events}")
    assert ls.st.poll_status() == 0


def test_route_timing_events_stamp_the_routing_launches():
    """qevict_time_next_route: the next routing call's kernels stamp a timing event pair (the
    routing kernel's start, the migration kernel's end); then the events are forgotten."""
    _print("case: route timing events")
    ls = Lockstep(WL.TINY.with_(budget_frac=0.25)).run(8)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    e1.record()
    torch.cuda.synchronize()
    ls.st.time_next_route(e0, e1)
    ls.st.route(-1)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3
    _print(f"route event: {us:.1f} us")
    assert 0.0 < us < 1e5
    ls.st.route(-1)   # (not timed: the pair was forgotten)
    torch.cuda.synchronize()
    assert e0.elapsed_time(e1) * 1e3 == us
    assert ls.st.poll_status() == 0


def test_determinism_bitwise():
    """Two identical runs give bit-identical state and outputs."""
    _print("case: determinism")
    outs = []
    for _ in range(2):
        ls = Lockstep(WL.TINY.with_(budget_frac=0.25)).run(16)
        ex = ls.st.export_unit(0, 0)
        outs.append((ex.score.tobytes(), b"".join(ex.ledger[w] for w in sorted(ex.ledger)), ex.state.tobytes()))
    assert outs[0] == outs[1]


def test_stream_read_calibration_reads_every_byte():
    """The streaming-read measurement aid reads every 32-bit word exactly once: the XOR of
    its per-workgroup words equals the XOR of the buffer (sizes with a ragged tail of
    pieces, and the size of one llama8b_32k layer step)."""
    dev = torch.device("cuda:0")
    g = torch.Generator().manual_seed(11)
    for kib in (1, 4097, 26593):
        _print(f"case: stream read {kib} KiB")
        host = torch.randint(-2**31, 2**31 - 1, (kib * 256,), generator=g, dtype=torch.int64).to(torch.int32)
        buf = host.to(dev)
        sink = torch.zeros(B.STREAM_READ_WGS, dtype=torch.int32, device=dev)
        B.stream_read(buf, sink)
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
        assert got == want, (kib, hex(got), hex(want))
    with pytest.raises(B.QEvictError):
        B.stream_read(torch.zeros(1000, dtype=torch.uint8, device=dev), sink)   # not a multiple of 1024 bytes


@pytest.mark.parametrize("flag", ["decay", "pnorm", "keynorm"])
def test_alternative_rankers_lockstep(flag):
    """The rankers of [QEvict] Appendix J against the oracle: routing sets, tiers, ledgers
    and pages bit-exact, rank keys within 1e-4 (cube roots for p-norm).  The tiny case
    routes every 2 steps under fast topic drift from flat initial scores, where decay and
    p-norm route differently from the cumulative score and promote windows; then a GQA-8,
    d = 128 ragged batch."""
    f = {"decay": B.QEVICT_F_RANK_DECAY, "pnorm": B.QEVICT_F_RANK_PNORM, "keynorm": B.QEVICT_F_RANK_KEYNORM}[flag]
    _print(f"case: ranker {flag}")
    wl = WL.TINY.with_(n_topics=4, topic_period=8, n_decode=96, n_outlier=2, budget_frac=0.3, omega=2)
    si = None if flag == "keynorm" else torch.zeros((1, 64), dtype=torch.float64)
    ls = Lockstep(wl, score_init=si, flags=f).run(96)
    if flag != "keynorm":     # (key-norm keys never change, so nothing is promoted)
        assert sum(e["promoted"] for e in ls.units[0].events) > 0
    _print(f"{flag} tiny: max o err {ls.max_o_err:.2e} (bf16 reading {ls.max_o_err_bf16:.2e}, gap {ls.max_reading_gap:.2e}), max score err {ls.max_s_err:.2e}, events {ls.events}")
    wl2 = WL.Workload("rank", 1, 2, 16, 2, 128, 700, 24, 32, 4, 64, 8, 0.30, 0.70, prompt_len_min=400,
                      n_outlier=2, n_topics=2, topic_period=8)
    ls2 = Lockstep(wl2, flags=f).run(24)
    _print(f"{flag} gqa8: max o err {ls2.max_o_err:.2e}, max score err {ls2.max_s_err:.2e}")


INT4_CASES = {
    # d = 64, W = 16 (one tile per chunk), G = 4, flat initial scores + topic drift: promotions
    "tiny_drift": (WL.TINY.with_(n_topics=4, topic_period=16, n_decode=64, n_outlier=2, budget_frac=0.30), True, 64),
    # d = 64, W = 32 (two tiles per chunk), G = 2, ragged batch of 2
    "d64_w32": (WL.Workload("i4a", 1, 2, 4, 2, 64, 600, 32, 32, 4, 64, 8, 0.35, 0.70, prompt_len_min=350,
                            n_outlier=2, n_topics=2, topic_period=8), False, 32),
    # d = 128, W = 32, G = 8 (one column slot), ragged batch
    "gqa8_d128": (WL.Workload("i4b", 1, 2, 16, 2, 128, 640, 24, 32, 4, 64, 8, 0.30, 0.70, prompt_len_min=300,
                              n_outlier=2, n_topics=2, topic_period=8), False, 24),
    # d = 128, W = 64 (two chunks per window), G = 8
    "w64": (WL.Workload("i4c", 1, 1, 16, 2, 128, 1200, 24, 64, 4, 128, 8, 0.30, 0.70,
                        n_outlier=2, n_topics=2, topic_period=8), False, 24),
}


@pytest.mark.parametrize("case", list(INT4_CASES))
def test_int4_tier_lockstep(case):
    """The INT4 recoverable tier ([QEvict] Appendix G.3): 16-level codes packed, promoted and
    attended; codes, parameters, ledgers and pages bit-exact, outputs within 2e-3 of ||o||."""
    wl, flat, steps = INT4_CASES[case]
    _print(f"case: int4 {case}")
    si = None
    if flat:
        n_win = math.ceil((wl.prompt_len + wl.n_decode - wl.n_sink) / wl.window)
        si = torch.zeros((wl.batch, n_win), dtype=torch.float64)
    ls = Lockstep(wl, score_init=si, flags=B.QEVICT_F_INT4).run(steps)
    assert ls.st.info.max_K_q > 0
    led = [u.win[w].ledger for u in ls.units for w in u.win if u.win[w].ledger is not None]
    assert led and max(int(l.k_codes.max()) for l in led) > 3          # codes beyond the INT2 range
    if flat:
        assert sum(e["promoted"] for u in ls.units for e in u.events) > 0
    _print(f"int4 {case}: max o err {ls.max_o_err:.2e} (bf16 reading {ls.max_o_err_bf16:.2e}, gap {ls.max_reading_gap:.2e}), max score err {ls.max_s_err:.2e}, events {ls.events}")


ROPE_CASES = {
    # d = 64, W = 16, G = 4, flat initial scores + drift: promotions re-rotate dequantized keys
    "tiny_drift": (WL.TINY.with_(n_topics=4, topic_period=16, n_decode=64, n_outlier=2, budget_frac=0.30), True, 0, 64),
    # d = 128, W = 32, G = 8, ragged batch, INT2
    "gqa8_d128": (WL.Workload("r2", 1, 2, 16, 2, 128, 640, 24, 32, 4, 64, 8, 0.30, 0.70, prompt_len_min=300,
                              n_outlier=2, n_topics=2, topic_period=8), False, 0, 24),
    # d = 128, W = 64, G = 4 (two column slots), INT4
    "w64_int4": (WL.Workload("r4", 1, 1, 8, 2, 128, 1200, 24, 64, 4, 128, 8, 0.30, 0.70,
                             n_outlier=2, n_topics=2, topic_period=8), False, B.QEVICT_F_INT4, 24),
    # d = 64, W = 32, G = 2, INT2
    "d64_w32": (WL.Workload("r5", 1, 2, 4, 2, 64, 600, 32, 32, 4, 64, 8, 0.35, 0.70, prompt_len_min=350,
                            n_outlier=2, n_topics=2, topic_period=8), False, 0, 32),
    # d = 128, W = 16 (one tile per chunk), G = 4, INT2, flat scores + drift (promotions)
    "w16_d128": (WL.Workload("r6", 1, 2, 8, 2, 128, 700, 48, 16, 4, 64, 8, 0.20, 0.70, prompt_len_min=500,
                             n_outlier=2, n_topics=4, topic_period=16), True, 0, 48),
}


@pytest.mark.parametrize("case", list(ROPE_CASES))
def test_rope_faithful_quantized_tier_lockstep(case):
    """Queries and keys handed over before RoPE ([QEvict] §4.3): cached keys rotated,
    the Quantized tier packed from keys turned back to the pre-RoPE domain and re-rotated
    inside attention and on promotion; routing, codes, ledgers and pages bit-exact,
    outputs within 2e-3 of ||o||."""
    wl, flat, extra, steps = ROPE_CASES[case]
    _print(f"case: rope {case}")
    si = None
    if flat:
        n_win = math.ceil((wl.prompt_len + wl.n_decode - wl.n_sink) / wl.window)
        si = torch.zeros((wl.batch, n_win), dtype=torch.float64)
    ls = Lockstep(wl, score_init=si, flags=B.QEVICT_F_ROPE | extra).run(steps)
    assert any(u.win[w].ledger is not None for u in ls.units for w in u.win)
    if flat:
        assert sum(e["promoted"] for u in ls.units for e in u.events) > 0
    _print(f"rope {case}: max o err {ls.max_o_err:.2e} (bf16 reading {ls.max_o_err_bf16:.2e}, gap {ls.max_reading_gap:.2e}), max score err {ls.max_s_err:.2e}, events {ls.events}")


@pytest.mark.parametrize("promote", [True, False], ids=["two-way", "one-way"])
def test_diagnostics_from_the_gpu_state_match_the_oracle(promote):
    """Appendix I diagnostics from the GPU: a policy state and an uncompressed reference
    state decode the same tokens; the per-head step masses (qevict_step_mass), tiers and
    scores they export give the same FMM, churn, tier shares, QSA / R_Q, Global LIR and
    transitions as the oracle's definitions on the oracle's own run."""
    from recoverable_kv_cache_amd import diagnostics as D
    from tests.oracle_helpers import cfg_from, oracle_trace
    from tests.test_diagnostics import DRIFT, check_library_against_oracle, oracle_summary
    _print(f"case: diagnostics promote={promote}")
    wl, steps = DRIFT, 96
    cfg = cfg_from(wl, budget_frac=0.3, promote=promote)
    events, masses, pol = oracle_trace(wl, cfg, steps, score_init=np.zeros(64))
    osum = oracle_summary(events, masses, wl, pol.caps["K_f"])
    flags = 0 if promote else B.QEVICT_F_NO_PROMOTE
    sp = B.QEvictState(B.make_config(wl, flags=flags, budget_frac=0.3), wl.prompt_lens())
    sr = B.QEvictState(B.make_config(wl, budget_frac=4.0, quant_frac=0.0), wl.prompt_lens())
    qp, kp, vp = (t.cuda() for t in WL.prompt(wl, 0))
    si = torch.zeros((1, sp.info.n_windows), dtype=torch.float64, device="cuda")
    for st in (sp, sr):
        st.prefill_init(0, qp, kp, vp, score_init=si)
    out = torch.empty((1, wl.h_q, wl.d_head), dtype=torch.float32, device="cuda")

    def run_step(j):
        q, k, v = (t.cuda() for t in WL.decode_step(wl, 0, j))
        sp.decode_attn(0, q, k, v, out)
        sr.decode_attn(0, q, k, v, out)

    tr = D.record(sp, sr, 0, 0, run_step, steps, wl.omega)
    assert len(tr.state) == len(events)
    for r, ev in enumerate(events):
        np.testing.assert_array_equal(tr.state[r], [ev["state"][w] for w in range(len(tr.state[r]))])
    err = max(float(np.abs(a - b).max()) for a, b in zip(tr.masses, masses))
    _print(f"step-mass max abs err {err:.2e}")
    assert err < 1e-5
    s = check_library_against_oracle(tr, osum, tol=1e-4)
    _print(f"diagnostics: {s}")
    with pytest.raises(B.QEvictError):      # no decode step since the last routing
        sp.step_mass(0, 0)


def test_combined_flags_int4_rope_pnorm_one_way():
    """The options together: INT4 tier, inputs before RoPE, p-norm ranker and the one-way
    variant, on the drifting tiny workload routed every 2 steps (G = 4, d = 64, W = 16)."""
    _print("case: combined flags")
    wl = WL.TINY.with_(n_topics=4, topic_period=8, n_decode=48, n_outlier=2, budget_frac=0.3, omega=2)
    si = torch.zeros((1, 64), dtype=torch.float64)
    flags = B.QEVICT_F_INT4 | B.QEVICT_F_ROPE | B.QEVICT_F_RANK_PNORM | B.QEVICT_F_NO_PROMOTE
    ls = Lockstep(wl, score_init=si, flags=flags).run(48)
    unit = ls.units[0]
    assert sum(e["promoted"] for e in unit.events) == 0
    assert any(W.ledger is not None and W.ledger.bits == 4 for W in unit.win.values())
    _print(f"combined: max o err {ls.max_o_err:.2e} (bf16 reading {ls.max_o_err_bf16:.2e}, gap {ls.max_reading_gap:.2e}), max score err {ls.max_s_err:.2e}, events {ls.events}")


def _selection_scores(kind: str, n: int) -> torch.Tensor:
    """Initial window scores that stress the router's tier selection (radix select over the
    composite key of score and window index)."""
    g = torch.Generator().manual_seed(7)
    if kind == "all_equal":          # every key ties: the window index decides
        s = torch.full((n,), 0.5, dtype=torch.float64)
    elif kind == "two_values":
        s = torch.where(torch.arange(n) % 3 == 0, 2.0, 1.0).to(torch.float64)
    elif kind == "ulp_apart":        # keys that differ only in their last mantissa bits
        s = torch.from_numpy(1.0 + (np.arange(n) % 7) * np.finfo(np.float64).eps)
        s = s[torch.randperm(n, generator=g)]
    elif kind == "signed_zeros":     # negative keys, +0 and -0 (which tie), positive keys
        v = torch.randn(n, generator=g, dtype=torch.float64)
        v[::5] = 0.0
        v[1::5] = -0.0
        s = v
    elif kind == "wide_range":       # from subnormals to 1e300
        e = torch.randint(-320, 300, (n,), generator=g).to(torch.float64)
        s = torch.pow(torch.tensor(10.0, dtype=torch.float64), e)
    else:
        raise ValueError(kind)
    return s


@pytest.mark.parametrize("kind", ["all_equal", "two_values", "ulp_apart", "signed_zeros", "wide_range"])
@pytest.mark.parametrize("one_way", [False, True], ids=["two-way", "one-way"])
def test_tier_selection_edge_cases(kind, one_way):
    """The prefill routing of 4K-token prompts (about 250 candidates per unit, more than one
    selection pass) with initial scores built to stress the radix selection: the tier sets
    bit-exact against the oracle's full sort, then two routing events."""
    _print(f"case: tier selection {kind} one_way={one_way}")
    wl = WL.Workload("selection", 1, 2, 4, 1, 64, 4096, 16, 16, 4, 64, 8, 0.40, 0.70, n_outlier=2)
    n_win = (wl.prompt_len - wl.n_sink + wl.window - 1) // wl.window
    si = torch.stack([_selection_scores(kind, n_win), _selection_scores(kind, n_win).flip(0)])
    flags = B.QEVICT_F_NO_PROMOTE if one_way else 0
    ls = Lockstep(wl, score_init=si, flags=flags)
    ls.prefill()
    # (later events depend on mass sums that the two sides round differently; where initial
    # keys tie or sit an ulp apart, only the prefill routing is a fair exact comparison)
    if kind in ("two_values", "signed_zeros", "wide_range"):
        for j in range(16):
            ls.step(j, check_every=8)
    _print(f"selection {kind}: events {ls.events}")
