"""The allocation-free prefill entry point (qevict_prefill_init_noalloc, the library's static
workspace) against the existing one (qevict_prefill_init with a caller workspace), through the
C ABI: two calls in a row, the second on a smaller input, each followed by decode steps and a
routing event.  The two paths run the same kernels, so the exported state (tiers, ledgers, pages,
the accessible list, fp64 scores) and the decode outputs must be identical bit for bit.  A
configuration whose workspace exceeds the static array is refused with QEVICT_E_CAPACITY."""
import numpy as np
import pytest
import torch

from recoverable_kv_cache_amd import binding as B
from recoverable_kv_cache_amd import workload as WL

pytestmark = pytest.mark.gpu

BIG = WL.Workload("noalloc_big", 1, 2, 16, 4, 128, 3072, 16, 32, 4, 256, 8, 0.25, 0.70, prompt_len_min=2048,
                  n_outlier=4, n_topics=4, topic_period=8)
SMALL = WL.TINY.with_(budget_frac=0.25, n_decode=16)


def _run(wl: WL.Workload, noalloc: bool):
    st = B.QEvictState(B.make_config(wl), wl.prompt_lens(), device="cuda")
    qp, kp, vp = WL.prompt(wl, 0, device="cuda")
    (st.prefill_init_noalloc if noalloc else st.prefill_init)(0, qp, kp, vp)
    del qp, kp, vp
    outs = []
    for j in range(wl.n_decode):
        q, k, v = (t.cuda() for t in WL.decode_step(wl, 0, j))
        out = torch.empty((wl.batch, wl.h_q, wl.d_head), dtype=torch.float32, device="cuda")
        st.decode_attn(0, q, k, v, out)
        outs.append(out.cpu())
        if (j + 1) % wl.omega == 0:
            st.route(0)
    exports = [st.export_unit(0, b) for b in range(wl.batch)]
    assert st.poll_status() == 0
    if noalloc:
        assert st.workspace is None     # no workspace tensor was made for this state
    return exports, outs


def _same(a: B.UnitExport, b: B.UnitExport, tag: str):
    for f in ("n", "n_windows", "K_f", "K_q", "status", "counters", "n_acc", "prompt_len", "sink_mass"):
        assert getattr(a, f) == getattr(b, f), f"{tag}: {f}"
    for f in ("state", "has_ledger", "dormant", "start_pos", "score", "acc", "splits", "win_page", "win_slot",
              "sink_k", "sink_v"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f), err_msg=f"{tag}: {f}")
    assert a.ledger == b.ledger, f"{tag}: ledgers"
    assert a.kv.keys() == b.kv.keys(), f"{tag}: pages"
    for w in a.kv:
        np.testing.assert_array_equal(a.kv[w][0], b.kv[w][0], err_msg=f"{tag}: K page {w}")
        np.testing.assert_array_equal(a.kv[w][1], b.kv[w][1], err_msg=f"{tag}: V page {w}")


@pytest.mark.parametrize("wl", [BIG, SMALL], ids=["first_call_larger", "second_call_smaller"])
def test_noalloc_prefill_equals_the_workspace_entry_point(wl):
    print(f"case: noalloc prefill {wl.name}", flush=True)
    st = B.QEvictState(B.make_config(wl), wl.prompt_lens(), device="cuda")
    assert 0 < st.info.prefill_ws_bytes <= B.NOALLOC_WS_BYTES
    del st
    ref_ex, ref_out = _run(wl, noalloc=False)
    got_ex, got_out = _run(wl, noalloc=True)
    for b in range(wl.batch):
        _same(got_ex[b], ref_ex[b], f"{wl.name} b={b}")
    for j, (g, r) in enumerate(zip(got_out, ref_out)):
        assert torch.equal(g, r), f"{wl.name}: decode output of step {j}"
    assert sum(int((e.state == 3).sum()) for e in got_ex) > 0     # Quantized windows were packed


def test_noalloc_prefill_refuses_a_workspace_beyond_the_static_array():
    print("case: noalloc capacity refusal", flush=True)
    wl = WL.Workload("noalloc_rope_4k", 1, 1, 32, 8, 128, 4096, 8, 32, 4, 256, 8, 0.25, 0.70)
    st = B.QEvictState(B.make_config(wl, flags=B.QEVICT_F_ROPE), wl.prompt_lens(), device="cuda")
    assert st.info.prefill_ws_bytes > B.NOALLOC_WS_BYTES
    qp, kp, vp = WL.prompt(wl, 0, device="cuda")
    with pytest.raises(B.QEvictError) as e:
        st.prefill_init_noalloc(0, qp, kp, vp)
    assert e.value.status == -3 and "static" in str(e.value)
