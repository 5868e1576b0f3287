"""GPU parity at the full size of the 32K Llama-3-8B-shaped workload (one layer, in
the launch configuration the benchmark times: batch 1, 8 KV heads, same split count).

* Decode + routing in lockstep with the oracle: the initial window scores are a
  synthetic seeded vector passed to both sides (the oracle cannot afford the
  ~9 TFLOP fp64 prompt column sums of a 32K prompt), so prefill routing, the 852
  INT2 packs, 8 decode steps and one routing event are all compared exactly.
* Prompt column sums at 32K: every row log-sum-exp and column sum of two query
  heads against fp64, every window score against the GPU's own column sums, and
  the row-sum invariant (every causal softmax row sums to one, so
  sum_w S_bar_0(w) + sink mass = prompt length).
"""
import math

import numpy as np
import pytest
import torch

from oracle import qevict_oracle as O
from recoverable_kv_cache_amd import binding as B
from recoverable_kv_cache_amd import workload as WL
from tests.gpu_harness import Lockstep
from tests.oracle_helpers import f64

pytestmark = pytest.mark.gpu

WL32 = WL.LLAMA8B_32K.with_(n_layers=1)


def test_llama8b_32k_decode_and_route_lockstep():
    print("case: 32K decode lockstep", flush=True)
    n_win = (WL32.prompt_len - WL32.n_sink + WL32.window - 1) // WL32.window
    si = WL.init_scores(WL32, 0, n_win)
    ls = Lockstep(WL32, score_init=si)
    ls.prefill()
    assert ls.st.info.n_splits == B.plan(B.make_config(WL.LLAMA8B_32K), [32768]).n_splits
    ex = ls.st.export_unit(0, 0)
    assert ex.counters["packed"] == ls.units[0].events[0]["packed"] > 800
    for j in range(8):
        ls.step(j)
    print(f"32K: max o err {ls.max_o_err:.2e} (bf16 reading {ls.max_o_err_bf16:.2e}, gap {ls.max_reading_gap:.2e}), max score err {ls.max_s_err:.2e}", flush=True)


def _blocked_column_sums(Q: np.ndarray, K: np.ndarray, lse: np.ndarray, rows: int = 512) -> np.ndarray:
    """Column sums sum_{u >= t} P[u, t] of one head's causal softmax P = exp(Q K^T / sqrt(d) - lse_u)
    (fp64), taken over blocks of query rows so that a 32K prompt fits in memory."""
    S, d = Q.shape
    col = np.zeros(S)
    for u0 in range(0, S, rows):
        u1 = min(S, u0 + rows)
        P = np.exp(Q[u0:u1] @ K[:u1].T / math.sqrt(d) - lse[u0:u1, None])
        P[:, u0:][np.triu_indices(u1 - u0, 1)] = 0.0          # key t > query u is masked
        col[:u1] += P.sum(axis=0)
    return col


def test_llama8b_32k_prefill_column_sums():
    """Prompt column sums at the full 32K size ([QEvict] §4.2: prompt attention initialises the
    window scores).  For two query heads of different GQA groups every row log-sum-exp and every
    one of the 32,768 column sums is compared with fp64 (the oracle's row log-sum-exp, a
    row-blocked column sum).  Bar: a window's score is the head average of its columns' sums, so
    it stays within the 1e-4 score bar when, for each head, the absolute column errors summed
    over each window (and over the sink prefix) stay below 1e-4.  Every exported window score
    equals the head average of the GPU's own column sums, and every causal row sums to one
    (fp32 probabilities: each row within 2^-20, so the total within S * 2^-20)."""
    print("case: 32K prefill column sums", flush=True)
    S, G, W, ns = WL32.prompt_len, WL32.h_q // WL32.h_kv, WL32.window, WL32.n_sink
    st = B.QEvictState(B.make_config(WL32), [S])
    qp, kp, vp = WL.prompt(WL32, 0, device="cuda")
    st.prefill_init(0, qp, kp, vp)
    torch.cuda.synchronize()
    ex = st.export_unit(0, 0, tables_only=True)
    lse_gpu, col_gpu = st.workspace_views()
    lse_gpu = lse_gpu.cpu().numpy()[0]
    col_gpu = col_gpu.cpu().numpy()[0]
    heads = (5, 30)
    Q = {h: qp[0, h].cpu().to(torch.float64).numpy() for h in heads}
    K = {g: kp[0, g].cpu().to(torch.float64).numpy() for g in {h // G for h in heads}}
    del qp, kp, vp
    total = ex.score[: ex.n_windows].sum() + ex.sink_mass
    print(f"row-sum invariant: {total} vs {S}", flush=True)
    assert abs(total - S) <= S * 2.0 ** -20
    # the window reduction: each exported score is the head average of the GPU's column sums
    nw = ex.n_windows
    win_cols = np.add.reduceat(col_gpu[:, ns:], np.arange(0, S - ns, W), axis=1)[:, :nw]
    np.testing.assert_allclose(ex.score[:nw], win_cols.mean(axis=0), rtol=1e-12, atol=1e-9)
    assert abs(ex.sink_mass - col_gpu[:, :ns].sum() / WL32.h_q) <= 1e-9
    for h in heads:
        Kg = K[h // G]
        lse = np.array([O.row_lse(Q[h][u], Kg[: u + 1]) for u in range(S)])
        lse_err = np.abs(lse_gpu[h] - lse / math.log(2)).max()
        ref = _blocked_column_sums(Q[h], Kg, lse)
        d = np.abs(col_gpu[h] - ref)
        per_win = np.add.reduceat(d[ns:], np.arange(0, S - ns, W))
        print(f"head {h}: row lse err {lse_err:.2e} (log2), max column err {d.max():.2e}, max per-window "
              f"sum {per_win.max():.2e}, sink-prefix sum {d[:ns].sum():.2e}, largest column {ref.max():.1f}",
              flush=True)
        assert lse_err < 1e-4
        assert per_win.max() <= 1e-4 and d[:ns].sum() <= 1e-4


def test_llama8b_32k_int4_decode_and_route_lockstep():
    """The same full-size lockstep with the INT4 recoverable tier."""
    print("case: 32K int4 decode lockstep", flush=True)
    n_win = (WL32.prompt_len - WL32.n_sink + WL32.window - 1) // WL32.window
    si = WL.init_scores(WL32, 0, n_win)
    ls = Lockstep(WL32, score_init=si, flags=B.QEVICT_F_INT4)
    ls.prefill()
    ex = ls.st.export_unit(0, 0)
    assert ex.counters["packed"] == ls.units[0].events[0]["packed"] > 400
    for j in range(8):
        ls.step(j)
    print(f"32K int4: max o err {ls.max_o_err:.2e} (bf16 reading {ls.max_o_err_bf16:.2e}, gap {ls.max_reading_gap:.2e}), max score err {ls.max_s_err:.2e}", flush=True)


def test_llama8b_32k_rope_decode_and_route_lockstep():
    """The full-size lockstep with pre-RoPE inputs and the RoPE-faithful Quantized tier
    (rotary base 500000, positions up to 33 279)."""
    print("case: 32K rope decode lockstep", flush=True)
    n_win = (WL32.prompt_len - WL32.n_sink + WL32.window - 1) // WL32.window
    si = WL.init_scores(WL32, 0, n_win)
    ls = Lockstep(WL32, score_init=si, flags=B.QEVICT_F_ROPE)
    ls.prefill()
    ex = ls.st.export_unit(0, 0)
    assert ex.counters["packed"] == ls.units[0].events[0]["packed"] > 800
    for j in range(8):
        ls.step(j)
    print(f"32K rope: max o err {ls.max_o_err:.2e} (bf16 reading {ls.max_o_err_bf16:.2e}, gap {ls.max_reading_gap:.2e}), max score err {ls.max_s_err:.2e}", flush=True)


def _init_scores(wl):
    n_win = (wl.prompt_len - wl.n_sink + wl.window - 1) // wl.window
    return WL.init_scores(wl, 0, n_win)


def test_batched_16k_b16_sampled_lockstep():
    """The batched mid-context shape at full size (one layer, batch 16, prompts of 8K-16K,
    the benchmark's split count for batch 16): the GPU decodes every sequence; the oracle
    follows sequences 0, 7 and 15 through 8 steps and a routing event (synthetic initial
    scores: 16 prompts' column sums are beyond the oracle)."""
    wl = WL.BATCHED_16K.with_(n_layers=1)
    print("case: batched 16K b16", flush=True)
    ls = Lockstep(wl, score_init=_init_scores(wl), sample=[0, 7, 15])
    assert ls.st.info.n_splits == B.plan(B.make_config(WL.BATCHED_16K), wl.prompt_lens()).n_splits
    ls.run(8)
    print(f"batched: max o err {ls.max_o_err:.2e} (bf16 reading {ls.max_o_err_bf16:.2e}, gap {ls.max_reading_gap:.2e}), max score err {ls.max_s_err:.2e}", flush=True)


def test_churn_4k_b64_sampled_lockstep_across_a_topic_switch():
    """The long-generation churn shape at full width (one layer, batch 64, 4K prompts, W = 16):
    264 decode steps cross the topic switch at step 256 (33 routing events); the oracle
    follows sequences 0 and 63, and windows move between the tiers."""
    wl = WL.CHURN_4K.with_(n_layers=1)
    print("case: churn 4K b64", flush=True)
    ls = Lockstep(wl, score_init=_init_scores(wl), sample=[0, 63]).run(264, check_every=8)
    moved = sum(e["promoted"] + e["demoted"] for u in ls.units for e in u.events)
    print(f"churn: max o err {ls.max_o_err:.2e} (bf16 reading {ls.max_o_err_bf16:.2e}, gap {ls.max_reading_gap:.2e}), max score err {ls.max_s_err:.2e}, events {ls.events}, "
          f"moves {moved}", flush=True)
    assert ls.events == 33 and moved > 0
    print("churn: fills after a pack of their page", [ls.st.export_unit(0, b).counters["paired_fills"] for b in (0, 63)],
          flush=True)


def test_llama70b_128k_b4_sampled_lockstep():
    """The 70B-shaped long context at full size (one layer, batch 4, 128K prompts, W = 64,
    GQA 8, 512 recent): 8 steps and a routing event, the oracle following sequences 0 and 3."""
    wl = WL.LLAMA70B_128K.with_(n_layers=1)
    print("case: 70B 128K b4", flush=True)
    ls = Lockstep(wl, score_init=_init_scores(wl), sample=[0, 3])
    assert ls.st.info.n_splits == B.plan(B.make_config(WL.LLAMA70B_128K), wl.prompt_lens()).n_splits
    ls.run(8)
    print(f"70B: max o err {ls.max_o_err:.2e} (bf16 reading {ls.max_o_err_bf16:.2e}, gap {ls.max_reading_gap:.2e}), max score err {ls.max_s_err:.2e}", flush=True)
