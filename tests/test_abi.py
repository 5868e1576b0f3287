"""CPU checks of the C ABI: the library loads, exports every declared symbol, and its
host-side accounting (no GPU calls) agrees with the oracle and the printed pins."""
import ctypes
import json
import os
import re

import pytest

from oracle import qevict_oracle as O
from recoverable_kv_cache_amd import binding as B
from recoverable_kv_cache_amd import workload as WL
from tests.oracle_helpers import cfg_from

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    try:
        return B.load_library()
    except ImportError as e:
        pytest.fail(f"library not built: {e}")


def test_library_exports_every_declared_symbol():
    lib = _lib()
    header = open(os.path.join(ROOT, "include", "qevict.h")).read()
    declared = set(re.findall(r"\b(qevict_[a-z0-9_]+)\s*\(", header))
    assert declared, "no declarations found"
    assert declared == set(B.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(lib, name), name


@pytest.mark.parametrize("bits", [2, 4])
def test_capacities_match_oracle_for_all_workloads(bits):
    _lib()
    flags = B.QEVICT_F_INT4 if bits == 4 else 0
    for wl in WL.ALL_WORKLOADS:
        for S in sorted(set(wl.prompt_lens()))[:3]:
            c = B.capacities(B.make_config(wl, flags=flags), S)
            o = O.capacities(cfg_from(wl, quant_bits=bits), S)
            assert (c["K_f"], c["K_q"], c["M_f"], c["M_q"]) == (o["K_f"], o["K_q"], o["M_f"], o["M_q"]), wl.name
            assert c["B_total"] == o["B_total"] and c["B_hist"] == o["B_hist"]


def test_printed_diagnostic_capacities_through_the_abi():
    _lib()
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "diagnostic_capacities.json")))
    for case in g["cases"]:
        cfg = B.Config(batch=1, n_layers=32, h_q=g["h_q"], h_kv=g["h_kv"], d_head=g["d"], window=case["window"],
                       n_sink=g["n_sink"], n_local=g["n_local"], omega=case["window"], quant_frac=g["quant_frac"],
                       budget_frac=g["budget_frac"], max_prompt=g["prompt_len"], max_new=g["n_decode"])
        c = B.capacities(cfg, g["prompt_len"])
        assert (c["K_f"], c["K_q"]) == (case["K_f"], case["K_q"])


def test_budget_and_argument_errors():
    _lib()
    with pytest.raises(B.QEvictError) as ei:
        B.capacities(B.make_config(WL.TINY, budget_frac=0.10), 512)
    assert ei.value.status == -2
    for bad in (dict(d_head=96), dict(h_q=6), dict(window=24), dict(omega=0), dict(quant_frac=1.5)):
        with pytest.raises(B.QEvictError) as ei:
            B.plan(B.make_config(WL.TINY, **bad), [512])
        assert ei.value.status == -1, bad
    with pytest.raises(B.QEvictError):
        B.plan(B.make_config(WL.TINY), [513])        # prompt longer than max_prompt


@pytest.mark.parametrize("wl", WL.ALL_WORKLOADS, ids=lambda w: w.name)
def test_plan_sizes(wl):
    _lib()
    lens = wl.prompt_lens()
    info = B.plan(B.make_config(wl), lens)
    caps = [O.capacities(cfg_from(wl), S) for S in set(lens)]
    kf = max(c["K_f"] for c in caps)
    kq = max(c["K_q"] for c in caps)
    assert info.max_K_f == kf and info.max_K_q == kq
    assert info.n_slots >= kf + kq              # dormant ledgers keep their slot
    assert info.n_pages >= kf + (wl.n_local + wl.omega) // wl.window + 1
    assert info.n_windows * wl.window >= wl.prompt_len + wl.n_decode + wl.omega - wl.n_sink
    # the arena is dominated by the pools: pages + slots
    U = wl.batch * wl.n_layers
    pool = U * (info.n_pages * 4 * wl.h_kv * wl.window * wl.d_head
                + info.n_slots * wl.h_kv * (wl.window * wl.d_head // 2 + 4 * wl.d_head + 4 * wl.window))
    assert pool <= info.arena_bytes < 1.5 * pool + (64 << 20)
    assert info.arena_bytes < 64 << 30


def test_kernel_name_and_error_string():
    lib = _lib()
    assert lib.qevict_decode_kernel_name().decode().startswith("qevict_decode")
    assert isinstance(lib.qevict_last_error(), bytes)


def test_timing_hooks_refuse_a_null_state():
    lib = _lib()
    for fn in (lib.qevict_time_next_decode, lib.qevict_time_next_route):
        assert fn(None, None, None) == -1


def test_plan_reports_single_launch_steps_at_one_split():
    _lib()
    wl = WL.CHURN_4K
    assert B.plan(B.make_config(wl), wl.prompt_lens()).combine_in_kernel == 1       # B * h_kv = 512: one split
    assert B.plan(B.make_config(WL.LLAMA8B_32K), [32768]).combine_in_kernel == 0
    assert B.plan(B.make_config(wl, flags=B.QEVICT_F_SEPARATE_FINISH), wl.prompt_lens()).combine_in_kernel == 0
