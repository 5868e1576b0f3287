"""Plant plausible mistakes in the oracle (on the CPU, via monkeypatch) and check
that at least one pin catches each of them."""
import numpy as np
import pytest

from oracle import qevict_oracle as O
from tests import test_oracle_codec as TC
from tests import test_oracle_state as TS
from tests import test_oracle_rope as TR


def _fails(fn, *args):
    with pytest.raises((AssertionError, ValueError)):
        fn(*args)


def test_swapped_tier_shares_are_caught(monkeypatch):
    real = O.capacities

    def swapped(cfg, prompt_len):
        c = real(cfg, prompt_len)
        c["K_f"] = int(np.floor(cfg.quant_frac * c["B_hist"] / c["M_f"]))
        c["K_q"] = int(np.floor((1 - cfg.quant_frac) * c["B_hist"] / c["M_q"]))
        return c

    monkeypatch.setattr(O, "capacities", swapped)
    _fails(TS.test_quant_share_goes_to_quantized_tier)


def test_missing_param_bytes_are_caught(monkeypatch):
    monkeypatch.setattr(O, "quant_window_bytes", lambda cfg: cfg.window * cfg.h_kv * cfg.d // 2 + 20)
    _fails(TS.test_printed_diagnostic_capacities)


def test_wrong_logit_scale_is_caught(monkeypatch):
    real = O.softmax
    monkeypatch.setattr(O, "softmax", lambda x, axis=-1: real(x * 1.25, axis))
    _fails(TS.test_dense_equivalence_when_budget_covers_cache)


def test_reversed_tie_break_is_caught(monkeypatch):
    monkeypatch.setattr(O, "route_order", lambda cand, s: sorted(cand, key=lambda w: (-s[w], -w)))
    _fails(TS.test_route_order_equals_full_sort_and_heap_selection)


def test_nearest_offset_rounding_is_caught(monkeypatch):
    monkeypatch.setattr(O, "rd_fp16", lambda x: np.asarray(x, np.float64).astype(np.float16).astype(np.float64))
    _fails(TC.test_group_quantization_exact_definition)


def test_ties_down_code_rounding_is_caught(monkeypatch):
    real = O.quantize_groups

    def ties_down(x, axis):
        codes, off, scl = real(x, axis)
        t = 2.0 * (np.asarray(x, np.float64) - np.expand_dims(off, axis))
        s = np.expand_dims(scl, axis)
        c2 = (t > s).astype(np.uint8) + (t > 3 * s) + (t > 5 * s)
        return np.where(s == 0, 0, c2).astype(np.uint8), off, scl

    monkeypatch.setattr(O, "quantize_groups", ties_down)
    _fails(TC.test_midpoints_round_up)


def test_row_sums_instead_of_column_sums_are_caught(monkeypatch):
    real = O.prefill_column_sums

    def rows(qp, kp):
        col = real(qp, kp)
        S = col.shape[1]
        return np.ones_like(col) * (S / S)                 # every row of a softmax sums to one

    monkeypatch.setattr(O, "prefill_column_sums", rows)
    _fails(TS.test_prefill_scores_against_torch_column_sums)


def test_missing_head_average_is_caught(monkeypatch):
    real_decode = O.UnitOracle.decode

    def no_avg(self, q, k, v):
        before = dict(self.score)
        out = real_decode(self, q, k, v)
        for w, u in out["mass"].items():
            self.score[w] = before.get(w, 0.0) + u * self.cfg.h_q
            out["mass"][w] = u * self.cfg.h_q
        return out

    monkeypatch.setattr(O.UnitOracle, "decode", no_avg)
    _fails(TS.test_window_mass_against_independent_softmax)


def test_requantizing_on_redemotion_is_caught(monkeypatch):
    real_route = O.UnitOracle.route

    def requant(self, *a, **kw):
        for W in self.win.values():
            if W.state == O.FULL and W.ledger is not None:
                W.ledger = None                       # forget the write-once record
        return real_route(self, *a, **kw)

    monkeypatch.setattr(O.UnitOracle, "route", requant)
    _fails(TS.test_write_once_ledger_and_promoted_values, 2)


def test_int4_with_int2_divisor_is_caught(monkeypatch):
    real = O.quantize_groups

    def three_levels(x, axis, bits=2):
        codes, off, scl = real(x, axis, 2)                  # the 4-bit request answered with INT2
        return codes, off, scl

    monkeypatch.setattr(O, "quantize_groups", three_levels)
    _fails(TC.test_int4_exactly_recoverable_group_uses_all_sixteen_levels)


def test_int4_bytes_counted_as_int2_are_caught(monkeypatch):
    real = O.quant_window_bytes
    monkeypatch.setattr(O, "quant_window_bytes",
                        lambda cfg: real(O.OracleConfig(**{**cfg.__dict__, "quant_bits": 2})))
    _fails(TS.test_quantized_window_bytes_equal_the_stored_record, 4)


def test_quantizing_rotated_keys_is_caught(monkeypatch):
    real = O.rope_rotate

    def no_unrotate(x, pos, cs, inverse=False):
        return np.asarray(x, dtype=np.float64) if inverse else real(x, pos, cs)

    monkeypatch.setattr(O, "rope_rotate", no_unrotate)
    _fails(TR.test_quantized_in_the_pre_rope_domain_and_promoted_re_rotated)


def test_attending_unrotated_quantized_keys_is_caught(monkeypatch):
    monkeypatch.setattr(O.UnitOracle, "quant_keys", lambda self, w: self.win[w].ledger.k_hat())
    _fails(TR.test_quantized_windows_attend_with_re_rotated_keys)


def test_one_way_full_tier_left_short_is_caught(monkeypatch):
    """Planted: the one-way Full tier taken as the top K_f of all candidates with the Quantized
    winners dropped (|F| < K_f)."""
    def short(cand, scores, K_f, K_q, no_full=()):
        order = O.route_order(cand, scores)
        F = [w for w in order[:K_f] if w not in set(no_full)]
        rest = [w for w in order if w not in F]
        return F, rest[:K_q], rest[K_q:]

    monkeypatch.setattr(O, "select_tiers", short)
    _fails(TS.test_route_sets_hand_case_one_way)


def test_one_way_quantized_windows_ranked_last_are_caught(monkeypatch):
    """Planted: windows already Quantized forced behind every other candidate for the
    Quantized tier under the one-way policy."""
    def last(cand, scores, K_f, K_q, no_full=()):
        barred = set(no_full)
        order = O.route_order(cand, scores)
        F = [w for w in order if w not in barred][:K_f]
        rest = [w for w in order if w not in F and w not in barred] + [w for w in order if w in barred]
        return F, rest[:K_q], rest[K_q:]

    monkeypatch.setattr(O, "select_tiers", last)
    _fails(TS.test_route_sets_hand_case_one_way)


def test_one_way_branch_applied_to_the_bidirectional_policy_is_caught(monkeypatch):
    """Planted: the bidirectional policy barring Quantized windows from Full as well."""
    real = O.select_tiers

    def always_barred(cand, scores, K_f, K_q, no_full=()):
        return real(cand, scores, K_f, K_q, [w for w in cand if w in (0, 4)])

    monkeypatch.setattr(O, "select_tiers", always_barred)
    _fails(TS.test_route_sets_hand_case_bidirectional)


def test_bf16_execution_reading_ignored_is_caught(monkeypatch):
    """Planted: the bf16 execution reading (R2) silently falls back to the exact values."""
    real = O.UnitOracle.accessible
    monkeypatch.setattr(O.UnitOracle, "accessible", lambda self, qexec_bf16=None: real(self, False))
    _fails(TS.test_quantized_execution_readings_against_sdpa, True)


def test_bf16_execution_reading_on_keys_only_is_caught(monkeypatch):
    """Planted: only the Quantized keys rounded to bf16 in the execution reading, values exact."""
    real = O.UnitOracle.accessible

    def keys_only(self, qexec_bf16=None):
        owner, K, V = real(self, qexec_bf16)
        if qexec_bf16:
            _, _, V = real(self, False)
        return owner, K, V

    monkeypatch.setattr(O.UnitOracle, "accessible", keys_only)
    _fails(TS.test_quantized_execution_readings_against_sdpa, True)
