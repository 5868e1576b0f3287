"""Host-side checks of the GPU parity harness's accessible-list comparison: an export built
from an oracle state passes, and plausible list mistakes (a Quantized window dropped or listed
twice, an entry naming another window's slot, a window of the wrong kind, a missing sink
entry, split offsets that do not cover the list) are each caught.  No GPU is used."""
import numpy as np
import pytest

from oracle import qevict_oracle as O
from recoverable_kv_cache_amd import binding as B
from recoverable_kv_cache_amd import workload as WL
from tests.gpu_harness import compare_accessible
from tests.oracle_helpers import cfg_from, run_unit


def _export_of(unit: O.UnitOracle, n_splits: int = 4) -> B.UnitExport:
    """A UnitExport carrying the accessible list of the oracle's state (page / slot ids made up:
    windows in order take ids 0, 1, ...; one prepared recent page ahead of n)."""
    cfg = unit.cfg
    nw = max(unit.win) + 1
    page, slot = -np.ones(nw, np.int32), -np.ones(nw, np.int32)
    rows = [(0, 0, -1, 0)]
    np_, ns_ = 0, 0
    for w in sorted(unit.win):
        st = unit.win[w].state
        if st in (O.LOCAL, O.FULL):
            page[w] = np_
            rows.append((1, np_, w, unit.win_start(w)))
            np_ += 1
        elif st == O.QUANT:
            slot[w] = ns_
            rows.append((2, ns_, w, unit.win_start(w)))
            ns_ += 1
    nxt = nw
    if unit.win_start(nxt) < unit.n + cfg.omega:
        rows.append((1, np_, nxt, unit.win_start(nxt)))
    acc = np.array(rows[:1] + rows[1:][::-1], np.int32)      # any order
    splits = np.linspace(0, len(acc), n_splits + 1).astype(np.int32)
    z = np.zeros(0)
    return B.UnitExport(unit.n, nw, 0, 0, 0, {}, len(acc), unit.prompt_len, 0.0, z, z, z, z, z, {}, {}, z, z,
                        acc=acc, splits=splits, win_page=page, win_slot=slot)


@pytest.fixture(scope="module")
def unit():
    wl = WL.TINY.with_(n_decode=21)
    u, _ = run_unit(wl, cfg_from(wl, budget_frac=0.25), collect=False)
    assert any(W.state == O.EVICTED for W in u.win.values()) and any(W.state == O.QUANT for W in u.win.values())
    return u


def _mutated(ex: B.UnitExport, acc: np.ndarray = None, **kw) -> B.UnitExport:
    import dataclasses
    acc = ex.acc if acc is None else acc
    return dataclasses.replace(ex, acc=acc, n_acc=len(acc), **kw)


def test_oracle_list_passes(unit):
    compare_accessible(_export_of(unit), unit, "clean")


def test_list_mistakes_are_caught(unit):
    ex = _export_of(unit)
    acc = ex.acc
    q_rows = np.where(acc[:, 0] == 2)[0]
    cases = {
        "quantized window dropped": np.delete(acc, q_rows[0], axis=0),
        "window listed twice": np.vstack([acc, acc[q_rows[:1]]]),
        "sink entry missing": acc[acc[:, 0] != 0],
        "slot of another window": np.where(np.arange(len(acc))[:, None] == q_rows[0],
                                           [2, acc[q_rows[1], 1], acc[q_rows[0], 2], acc[q_rows[0], 3]], acc),
        "quantized window as a page": np.where(np.arange(len(acc))[:, None] == q_rows[0],
                                               [1, 999, acc[q_rows[0], 2], acc[q_rows[0], 3]], acc),
    }
    for name, bad in cases.items():
        splits = np.linspace(0, len(bad), len(ex.splits)).astype(np.int32)
        with pytest.raises(AssertionError):
            compare_accessible(_mutated(ex, bad, splits=splits), unit, name)
    with pytest.raises(AssertionError):
        compare_accessible(_mutated(ex, splits=ex.splits[::-1].copy()), unit, "splits reversed")
