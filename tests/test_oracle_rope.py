"""Pins of the oracle's RoPE-faithful Quantized tier ([QEvict] §4.3: keys quantized in
the pre-RoPE domain with their absolute positions, RoPE re-applied after
dequantization).

Pinned against: an independent "rotate half" RoPE written with torch (the convention
of the Llama family) feeding torch's scaled_dot_product_attention when the budget
covers the whole cache; the identity table (cos 1, sin 0), under which the RoPE run
must reproduce the plain run exactly; orthogonality and relative-position invariance
of the rotation; and a planted channel that is constant before RoPE (so its scale in
the pre-RoPE domain collapses, which quantizing rotated keys would not give).
"""
import math

import numpy as np
import pytest
import torch

from oracle import qevict_oracle as O
from recoverable_kv_cache_amd import workload as WL
from tests.oracle_helpers import cfg_from, f64


def _torch_rope(x, pos, theta, d):
    """Independent rotate-half RoPE in float64: x [H][n][d], pos [n]."""
    inv = theta ** (-torch.arange(0, d, 2, dtype=torch.float64) / d)
    ang = torch.as_tensor(pos, dtype=torch.float64)[:, None] * inv[None, :]
    cos = torch.cat([torch.cos(ang)] * 2, dim=-1).to(torch.float32).to(torch.float64)
    sin = torch.cat([torch.sin(ang)] * 2, dim=-1).to(torch.float32).to(torch.float64)
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    return x * cos + torch.cat([-x2, x1], dim=-1) * sin


def test_rotation_is_orthogonal_and_relative():
    d, n_pos = 64, 300
    cs = WL.rope_table(d, n_pos, theta=10000.0).numpy()
    rng = np.random.default_rng(0)
    x = rng.standard_normal((2, 5, d))
    pos = np.array([0, 7, 64, 200, 299])
    back = O.rope_rotate(O.rope_rotate(x, pos, cs), pos, cs, inverse=True)
    np.testing.assert_allclose(back, x, atol=1e-6)     # fp32 table: cos^2 + sin^2 = 1 to ~1e-7
    np.testing.assert_allclose(np.linalg.norm(O.rope_rotate(x, pos, cs), axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-6)
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    dots = [float(O.rope_rotate(q[None, None], [50 + s], cs)[0, 0] @ O.rope_rotate(k[None, None], [20 + s], cs)[0, 0])
            for s in (0, 30, 200)]
    assert max(dots) - min(dots) < 1e-4


def test_rope_matches_torch_rotate_half():
    d, n_pos, theta = 64, 40, 10000.0
    cs = WL.rope_table(d, n_pos, theta=theta).numpy()
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, n_pos, d))
    ref = _torch_rope(torch.from_numpy(x), np.arange(n_pos), theta, d).numpy()
    np.testing.assert_allclose(O.rope_rotate(x, np.arange(n_pos), cs), ref, rtol=0, atol=1e-12)


def test_dense_rope_attention_against_torch():
    """Budget covering the cache, q = 0: every step is plain softmax attention of the
    rotated query over all rotated keys (bf16 of the rotation, as a bf16 model holds them)."""
    wl = WL.TINY.with_(n_decode=6, prompt_len=120)
    theta = 10000.0
    cs = WL.rope_table(wl.d_head, 200, theta=theta).numpy()
    cfg = cfg_from(wl, budget_frac=2.0, quant_frac=0.0, rope=True)
    qp, kp, vp = WL.prompt(wl, 0)
    S = wl.prompt_len
    unit = O.UnitOracle(cfg, S, rope_cs=cs)
    unit.prefill(f64(qp[0]), f64(kp[0]), f64(vp[0]), score_init=np.zeros(64))
    bf = lambda t: t.to(torch.bfloat16).to(torch.float64)
    Kall = bf(_torch_rope(kp[0].to(torch.float64), np.arange(S), theta, wl.d_head))
    Vall = vp[0].to(torch.float64)
    G = wl.h_q // wl.h_kv
    for j in range(wl.n_decode):
        q, k, v = WL.decode_step(wl, 0, j)
        out = unit.decode(f64(q[0]), f64(k[0]), f64(v[0]))
        p = S + j
        kr = bf(_torch_rope(k[0].to(torch.float64)[:, None], [p], theta, wl.d_head))
        Kall = torch.cat([Kall, kr], dim=1)
        Vall = torch.cat([Vall, v[0].to(torch.float64)[:, None]], dim=1)
        qr = bf(_torch_rope(q[0].to(torch.float64)[:, None], [p], theta, wl.d_head))
        ref = torch.nn.functional.scaled_dot_product_attention(
            qr, Kall.repeat_interleave(G, 0), Vall.repeat_interleave(G, 0))[:, 0].numpy()
        np.testing.assert_allclose(out["o"], ref, rtol=0, atol=1e-10)


def _run(wl, cfg, cs, steps, zero_init=True):
    qp, kp, vp = WL.prompt(wl, 0)
    S = wl.prompt_len
    unit = O.UnitOracle(cfg, S, rope_cs=cs)
    unit.prefill(f64(qp[0]), f64(kp[0]), f64(vp[0]), score_init=np.zeros(100) if zero_init else None)
    outs = []
    for j in range(steps):
        q, k, v = WL.decode_step(wl, 0, j)
        outs.append(unit.decode(f64(q[0]), f64(k[0]), f64(v[0]))["o"])
        if (j + 1) % wl.omega == 0:
            unit.route()
    return unit, outs


def test_identity_table_reproduces_the_plain_path():
    wl = WL.TINY.with_(n_topics=4, topic_period=16, n_decode=32, n_outlier=2)
    ident = np.zeros((600, wl.d_head // 2, 2), dtype=np.float32)
    ident[..., 0] = 1.0
    a, oa = _run(wl, cfg_from(wl, budget_frac=0.3), None, 32)
    b, ob = _run(wl, cfg_from(wl, budget_frac=0.3, rope=True), ident, 32)
    np.testing.assert_array_equal(np.array(oa), np.array(ob))
    assert a.score == b.score and [e["order"] for e in a.events] == [e["order"] for e in b.events]
    for w in a.win:
        la, lb = a.win[w].ledger, b.win[w].ledger
        assert (la is None) == (lb is None)
        if la is not None:
            assert O.canonical_ledger_bytes(la) == O.canonical_ledger_bytes(lb)


def test_quantized_in_the_pre_rope_domain_and_promoted_re_rotated():
    """A key channel that is constant before RoPE has (almost) no spread in the
    pre-RoPE domain, so its step is tiny there, while after RoPE it spans the pair's
    rotation.  A promoted window holds bf16 of the re-rotated dequantized keys."""
    wl = WL.TINY.with_(n_decode=0)
    cs = WL.rope_table(wl.d_head, 600, theta=10000.0).numpy()
    cfg = cfg_from(wl, budget_frac=0.25, rope=True)
    qp, kp, vp = WL.prompt(wl, 0)
    kp = kp.clone()
    kp[0, :, :, 5] = 3.0                                     # channel 5 constant before RoPE
    unit = O.UnitOracle(cfg, wl.prompt_len, rope_cs=cs)
    unit.prefill(f64(qp[0]), f64(kp[0]), f64(vp[0]), score_init=np.zeros(64))
    w = next(w for w, W in unit.win.items() if W.state == O.QUANT)
    led = unit.win[w].ledger
    others = np.delete(led.k_scl[0], 5)
    assert led.k_scl[0, 5] < 0.05 * np.median(others)
    pos = unit.positions(w)
    rot = O.rope_rotate(f64(kp[0])[:, pos], pos, cs)
    assert np.ptp(rot[0, :, 5]) > 1.0                        # after RoPE the channel moves
    unit.score[w] = 1e9
    unit.route(decode_event=False)
    W = unit.win[w]
    assert W.state == O.FULL
    np.testing.assert_array_equal(W.k, O.to_bf16(O.rope_rotate(led.k_hat(), pos, cs)))


def test_quantized_windows_attend_with_re_rotated_keys():
    """One decode step over sinks, recent / Full pages and Quantized windows, rebuilt
    independently: the Quantized keys are the ledger's dequantized pre-RoPE keys turned
    by the torch rotate-half RoPE at their positions, the rest the cached bf16 keys."""
    wl = WL.TINY.with_(n_decode=9)
    theta = 10000.0
    cs = WL.rope_table(wl.d_head, 700, theta=theta).numpy()
    cfg = cfg_from(wl, budget_frac=0.3, rope=True)
    qp, kp, vp = WL.prompt(wl, 0)
    unit = O.UnitOracle(cfg, wl.prompt_len, rope_cs=cs)
    unit.prefill(f64(qp[0]), f64(kp[0]), f64(vp[0]), score_init=np.arange(64, dtype=np.float64))
    for j in range(8):
        q, k, v = WL.decode_step(wl, 0, j)
        unit.decode(f64(q[0]), f64(k[0]), f64(v[0]))
    unit.route()
    assert any(W.state == O.QUANT for W in unit.win.values())
    q, k, v = WL.decode_step(wl, 0, 8)
    p = unit.n
    out = unit.decode(f64(q[0]), f64(k[0]), f64(v[0]))
    Ks, Vs = [torch.from_numpy(unit.sink_k)], [torch.from_numpy(unit.sink_v)]
    for w in sorted(unit.win):
        W = unit.win[w]
        if W.state == O.QUANT:
            pos = np.arange(unit.win_start(w), unit.win_end(w))
            Ks.append(_torch_rope(torch.from_numpy(W.ledger.k_hat()), pos, theta, wl.d_head))
            Vs.append(torch.from_numpy(W.ledger.v_hat()))
        elif W.state in (O.LOCAL, O.FULL):
            nt = min(wl.window, unit.n - unit.win_start(w))
            Ks.append(torch.from_numpy(W.k[:, :nt]))
            Vs.append(torch.from_numpy(W.v[:, :nt]))
    K, V = torch.cat(Ks, dim=1), torch.cat(Vs, dim=1)
    qr = _torch_rope(q[0].to(torch.float64)[:, None], [p], theta, wl.d_head).to(torch.bfloat16).to(torch.float64)
    G = wl.h_q // wl.h_kv
    ref = torch.nn.functional.scaled_dot_product_attention(qr, K.repeat_interleave(G, 0), V.repeat_interleave(G, 0))
    np.testing.assert_allclose(out["o"], ref[:, 0].numpy(), rtol=0, atol=1e-10)
