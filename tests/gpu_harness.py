"""Lockstep harness: run the HIP path (through the C ABI) and the fp64 oracle on the
same seeded inputs and compare after every step and every routing event.

Bars (from the decode hot path's parity contract):
* routing sets, window states, ledger flags, INT2 codes/params, the bf16
  contents of Full / recent windows and the accessible list (as a set): bit-exact;
* decode outputs: max_i |o_gpu - o_ref| / ||o_ref||_2 <= 2e-3 per (sequence, head)
  against the exact reading of the Quantized values (x_hat), and against the
  bf16(x_hat) reading wherever the two readings lie within 1e-3 of each other;
* window scores S_bar: |gpu - ref| <= 1e-4 absolute.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import qevict_oracle as O
from recoverable_kv_cache_amd import binding as B
from recoverable_kv_cache_amd import workload as WL
from tests.oracle_helpers import cfg_from, f64

O_TOL = 2e-3
S_TOL = 1e-4


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of float64 values that are exactly bf16."""
    return (np.asarray(x, np.float64).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def rel_err(o_gpu: np.ndarray, o_ref: np.ndarray) -> float:
    """max over heads of max_i |o_gpu - o_ref| / ||o_ref||_2."""
    num = np.abs(o_gpu - o_ref).max(axis=-1)
    den = np.linalg.norm(o_ref, axis=-1)
    return float((num / den).max())


def compare_accessible(ex: B.UnitExport, unit: O.UnitOracle, tag: str):
    """The accessible list ([QEvict] Algorithm 1, last step) against the oracle's accessible
    set, exactly: one sink entry, then one entry per recent / Full window (a bf16 page) and per
    Quantized window (a slot) with its first position; the device orders the entries its own
    way, so they are compared as a set.  Entries of windows that start at or after n are the
    recent windows prepared for the next positions (pages, at most omega positions ahead).
    Each entry's page or slot is the one its window record holds; no page or slot is listed
    twice; the split offsets cover the list in order."""
    cfg = unit.cfg
    acc = ex.acc
    assert acc.shape == (ex.n_acc, 4), f"{tag}: list shape {acc.shape} vs n_acc {ex.n_acc}"
    sinks = acc[acc[:, 0] == 0]
    assert sinks.shape[0] == 1 and tuple(sinks[0][2:]) == (-1, 0), f"{tag}: sink entry {sinks}"
    rows = [tuple(int(x) for x in r) for r in acc[acc[:, 0] != 0]]
    got = {(k, w, s) for k, _, w, s in rows}
    assert len(got) == len(rows), f"{tag}: an accessible window is listed twice"
    kind_of = {O.LOCAL: 1, O.FULL: 1, O.QUANT: 2}
    ref = {(kind_of[W.state], w, unit.win_start(w)) for w, W in unit.win.items() if W.state in kind_of}
    created = {e for e in got if e[2] < unit.n}
    assert created == ref, (f"{tag}: accessible set differs: missing {sorted(ref - created)[:8]}, "
                            f"extra {sorted(created - ref)[:8]}")
    for k, w, s in got - created:
        assert k == 1 and s < unit.n + cfg.omega and s == unit.win_start(w), f"{tag}: prepared entry {(k, w, s)}"
    for k, idx, w, s in rows:
        if s < unit.n:
            own = ex.win_page[w] if k == 1 else ex.win_slot[w]
            assert idx == own >= 0, f"{tag}: entry of window {w} names {idx}, its record {own}"
    for k in (1, 2):
        ids = [idx for kk, idx, _, _ in rows if kk == k]
        assert len(set(ids)) == len(ids), f"{tag}: a {'page' if k == 1 else 'slot'} is listed twice"
    sp = ex.splits
    assert sp[0] == 0 and sp[-1] == ex.n_acc and np.all(np.diff(sp) >= 0), f"{tag}: split offsets {sp}"


def compare_unit(ex: B.UnitExport, unit: O.UnitOracle, tag: str, check_scores=True):
    n_created = ex.n_windows
    assert ex.n == unit.n, f"{tag}: n {ex.n} != {unit.n}"
    assert ex.status == 0, f"{tag}: device status {ex.status}"
    assert set(range(n_created)) == set(unit.win), f"{tag}: window sets differ"
    table = unit.window_table()
    for w in range(n_created):
        st, has_led, dorm, start = table[w]
        assert ex.state[w] == st, f"{tag}: window {w} state {ex.state[w]} != {st}"
        assert bool(ex.has_ledger[w]) == has_led, f"{tag}: window {w} ledger flag"
        assert bool(ex.dormant[w]) == dorm, f"{tag}: window {w} dormant flag"
        assert ex.start_pos[w] == start
        if has_led:
            ref = O.canonical_ledger_bytes(unit.win[w].ledger)
            assert ex.ledger[w] == ref, f"{tag}: window {w} ledger bytes differ"
        if st in (O.LOCAL, O.FULL):
            k, v = ex.kv[w]
            W = unit.win[w]
            np.testing.assert_array_equal(k, bf16_bits(W.k), err_msg=f"{tag}: window {w} K page")
            np.testing.assert_array_equal(v, bf16_bits(W.v), err_msg=f"{tag}: window {w} V page")
    compare_accessible(ex, unit, tag)
    ns = min(unit.cfg.n_sink, unit.n)
    np.testing.assert_array_equal(ex.sink_k[:, :ns], bf16_bits(unit.sink_k[:, :ns]))
    np.testing.assert_array_equal(ex.sink_v[:, :ns], bf16_bits(unit.sink_v[:, :ns]))
    if check_scores:
        ref = np.array([unit.score[w] for w in range(n_created)])
        got = np.asarray(ex.score[:n_created], dtype=np.float64)
        if unit.cfg.ranker == "pnorm":   # rank key P = sum of cubed interval masses: compare P^(1/3)
            ref, got = np.cbrt(ref), np.cbrt(got)
        err = np.abs(got - ref).max() if n_created else 0.0
        assert err <= S_TOL, f"{tag}: score error {err}"
        return float(err)
    return 0.0


class Lockstep:
    def __init__(self, wl: WL.Workload, layer: int = 0, score_init=None, flags: int = 0, n_splits: int = 0,
                 ocfg_over=None, device="cuda", n_layers=1, rope_theta=WL.ROPE_THETA, sample=None):
        """``sample``: the sequences the oracle follows and the checks cover (default all)."""
        self.wl = wl
        self.layer = layer
        self.lens = wl.prompt_lens()
        cfg = B.make_config(wl, n_splits=n_splits, flags=flags, n_layers=n_layers)
        self.st = B.QEvictState(cfg, self.lens, device=device)
        ranker = ("decay" if flags & B.QEVICT_F_RANK_DECAY else "pnorm" if flags & B.QEVICT_F_RANK_PNORM
                  else "keynorm" if flags & B.QEVICT_F_RANK_KEYNORM else "cum")
        ocfg = cfg_from(wl, promote=not (flags & B.QEVICT_F_NO_PROMOTE),
                        score_every_step=not (flags & B.QEVICT_F_SCORE_ROUTE_ONLY), ranker=ranker,
                        quant_bits=4 if flags & B.QEVICT_F_INT4 else 2, rope=bool(flags & B.QEVICT_F_ROPE),
                        **(ocfg_over or {}))
        self.ocfg = ocfg
        self.rope = None
        if flags & B.QEVICT_F_ROPE:   # the rotary table: an input of both sides
            self.rope = WL.rope_table(wl.d_head, max(32, wl.prompt_len + wl.n_decode), theta=rope_theta)
            self.st.set_rope(self.rope.to(device))
        cs = None if self.rope is None else self.rope.numpy()
        self.sample = list(range(wl.batch)) if sample is None else list(sample)
        self.units = [O.UnitOracle(ocfg, self.lens[b], rope_cs=cs) for b in self.sample]
        self.score_init = score_init
        self.max_o_err = 0.0
        self.max_o_err_bf16 = 0.0     # against the bf16(x_hat) reading, where it is checked
        self.max_reading_gap = 0.0    # between the two readings of the oracle
        self.max_s_err = 0.0
        self.events = 0
        self.dev = device

    def prefill(self):
        qp, kp, vp = WL.prompt(self.wl, self.layer, with_q=self.score_init is None)
        si = None
        if self.score_init is not None:
            si = torch.zeros((self.wl.batch, self.st.info.n_windows), dtype=torch.float64)
            si[:, : self.score_init.shape[1]] = self.score_init[:, : si.shape[1]]
            si = si.to(self.dev)
        self.st.prefill_init(0, None if qp is None else qp.to(self.dev), kp.to(self.dev), vp.to(self.dev),
                             score_init=si)
        for b, unit in zip(self.sample, self.units):
            S = self.lens[b]
            init = None if self.score_init is None else self.score_init[b].numpy()
            unit.prefill(None if qp is None else f64(qp[b, :, :S]), f64(kp[b, :, :S]), f64(vp[b, :, :S]),
                         score_init=init)
        del qp, kp, vp
        self.check("prefill")

    def check(self, tag, check_scores=True):
        torch.cuda.synchronize()
        for b, unit in zip(self.sample, self.units):
            ex = self.st.export_unit(0, b)
            e = compare_unit(ex, unit, f"{tag} b={b}", check_scores)
            self.max_s_err = max(self.max_s_err, e)

    def step(self, j: int, check_every: int = 1):
        q, k, v = WL.decode_step(self.wl, self.layer, j)
        out = torch.empty((self.wl.batch, self.wl.h_q, self.wl.d_head), dtype=torch.float32, device=self.dev)
        self.st.decode_attn(0, q.to(self.dev), k.to(self.dev), v.to(self.dev), out)
        o_gpu = out.cpu().numpy().astype(np.float64)
        for b, unit in zip(self.sample, self.units):
            ref = unit.decode(f64(q[b]), f64(k[b]), f64(v[b]))
            err = rel_err(o_gpu[b], ref["o"])
            self.max_o_err = max(self.max_o_err, err)
            assert err <= O_TOL, f"step {j} b={b}: output error {err}"
            # reading R2: the bf16(x_hat) execution reading.  Where the two readings lie within
            # half the bar of each other the output must be within the bar of both; where they
            # are further apart (long contexts of Quantized outlier keys) no output can be, and
            # the gap is recorded instead.
            o16 = unit.attend(ref["q_rot"], qexec_bf16=True)[0]
            gap = rel_err(o16, ref["o"])
            err16 = rel_err(o_gpu[b], o16)
            self.max_reading_gap = max(self.max_reading_gap, gap)
            if gap <= O_TOL / 2:
                self.max_o_err_bf16 = max(self.max_o_err_bf16, err16)
                assert err16 <= O_TOL, f"step {j} b={b}: output error {err16} against the bf16 reading"
        routed = (j + 1) % self.wl.omega == 0
        if routed:
            self.st.route(0)
            for unit in self.units:
                unit.route()
            self.events += 1
        if routed or (j + 1) % check_every == 0:
            self.check(f"step {j}")

    def run(self, steps: int, check_every: int = 1):
        self.prefill()
        for j in range(steps):
            self.step(j, check_every)
        return self
