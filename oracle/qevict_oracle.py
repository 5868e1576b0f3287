"""Plain fp64 CPU oracle of the QEvict decode hot path.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module.  The
library under ``recoverable_kv_cache_amd/`` never calls it, and the two share
no code: this file restates the method from the pages in NumPy float64, one
(sequence, layer) unit at a time, with no blocking, fusion or reordering beyond
what the definitions state.

Sources (page titles; section / equation on each page):

* "QEvict: Recoverable Quantized KV Eviction for Attention-Drift-Robust
  Long-Context Decoding" (arXiv 2608.05326 mirror), cited below as [QEvict]:
  §4.1 accessible-set attention and the byte-budget inequality, §4.2 Eq. 1
  cumulative window score and prefill initialisation, §4.3 Eq. 2 cache state,
  Eq. 3 tier capacities, "Migration-Stable Quantization", Eqs. 4-6 candidate
  pool / TopK routing / migration, Appendix A Algorithm 1, Appendix B.4 Eqs. 7-8
  memory accounting, Appendix B.5 default configuration.
* The Chinese-language review of the same paper ("QEvict：面向注意力漂移的可恢复
  量化 KV 淘汰与长上下文解码"), cited as [review], §2.1-2.3: it restates Eqs. 1-6,
  names d_kv as the head dimension and gives R in Eq. 1 as the routing period.

Readings where the pages are silent or ambiguous (each one is listed with its
reason in the design notes of the repository):

* window size W and routing interval Omega are separate parameters; windows are
  aligned at absolute positions ``n_sink + w*W``;
* R in Eq. 1 is Omega, and the score accumulates at every decode step of the
  interval (flag ``score_every_step``; off = only the routing step's query);
* prefill initialisation = causal prompt-attention column sums over all prompt
  queries, averaged over H_q, for every window (also recent ones);
* a LOCAL window ages into the candidate pool at a routing event once its end
  position is <= n - n_local; the last partial window stays LOCAL;
* B_total = rho * (bf16 K+V bytes per token) * (prompt_len + n_decode) per
  sequence and layer, fixed for the run; B_local is the nominal n_local tokens;
* per-window bytes: M_f = W * b_tok + 8 (page entry); M_q = packed codes +
  fp16 offset/scale per (head, channel) for K and per (head, token) for V +
  4 B position + 16 B ledger record;
* quantization: off = fp16 rounded down from the group minimum, scl = fp16
  rounded up from (max - off)/L with L = 2^b - 1 levels above the offset (b = 2,
  the INT2 default, or b = 4 for the INT4 tier of [QEvict] Appendix G.3, which
  changes nothing else), code = nearest level with ties up, code 0 when
  scl == 0; Quantized-tier values inside attention are the exact
  ``off + code*scl`` (``qexec_bf16`` switches to their bf16 rounding);
* TopK ties break by ascending window index; routing is per (sequence, layer);
* alternative rankers ([QEvict] Appendix J, Eqs. 20-24): u_r(w) is the window's
  head-averaged mass summed over the decode steps since the previous routing event;
  "decay" sets S <- lambda*S + u_r and "pnorm" P <- P + u_r^p at each decode-time
  routing event (not at the prefill routing), starting from S_0 resp. P_0 = S_0^p
  with S_0 the prefill initialisation; "pnorm" ranks by P, which orders the
  windows as P^(1/p) does; "keynorm" sets S(w) = -(mean over the window's tokens
  of the L2 norm of the token's key over all KV heads' channels) when the window
  enters the candidate pool, from its bf16 keys, and needs no attention mass;
* RoPE-faithful Quantized tier ([QEvict] §4.3 "Migration-Stable Quantization" and
  "Cache Execution"; optional, ``rope=True``): queries and keys arrive before RoPE;
  the cache keeps keys rotated at their absolute positions (bf16 of the exact
  rotation), as a bf16 model's cache would; a window entering the Quantized tier
  for the first time is quantized from its stored keys rotated back to the
  pre-RoPE domain (exact fp64), and attention re-applies RoPE at the ledger's
  positions to the dequantized keys; a promotion writes bf16 of that re-rotation.
  The rotation pairs channel i with i + d/2 ("rotate half") and takes its cos/sin
  from a table given as input (fp32 values, one row per position).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# window states (the tier labels of [QEvict] §4.1 plus the protected recent region)
NONE, LOCAL, FULL, QUANT, EVICTED = 0, 1, 2, 3, 4

FP16_MAX = 65504.0


class BudgetError(ValueError):
    """The protected regions alone exceed the byte budget (B_hist < 0)."""


class RangeError(ValueError):
    """A value cannot be represented by the fp16 quantization parameters."""


# --------------------------------------------------------------------------------------
# configuration and byte accounting  ([QEvict] §4.1 inequality, Eq. 3, App. B.4 Eqs. 7-8)
# --------------------------------------------------------------------------------------
@dataclass(frozen=True)
class OracleConfig:
    h_q: int
    h_kv: int
    d: int
    window: int
    n_sink: int
    n_local: int
    omega: int
    quant_frac: float
    budget_frac: float
    n_decode: int
    promote: bool = True
    score_every_step: bool = True
    qexec_bf16: bool = False
    ranker: str = "cum"          # "cum" (Eq. 21, the default), "decay" (Eq. 22), "pnorm" (Eq. 23), "keynorm" (Eq. 24)
    decay_lambda: float = 0.99
    pnorm_p: int = 3
    quant_bits: int = 2          # 2 (INT2, the default) or 4 (INT4, [QEvict] Appendix G.3)
    rope: bool = False           # inputs before RoPE, Quantized tier in the pre-RoPE domain

    @property
    def group(self) -> int:
        return self.h_q // self.h_kv


def token_bytes(cfg: OracleConfig) -> int:
    """bf16 K and V of one token of one layer: Eq. 7 per token, 2 * H_kv * d * 2 bytes."""
    return 2 * cfg.h_kv * cfg.d * 2


def full_window_bytes(cfg: OracleConfig) -> int:
    """M_f: the window's bf16 K/V plus an 8-byte page entry ([QEvict] Eq. 3 text)."""
    return cfg.window * token_bytes(cfg) + 8


def quant_window_bytes(cfg: OracleConfig) -> int:
    """M_q: b-bit codes for K and V, fp16 offset+scale per (head, channel) for K and
    per (head, token) for V, a 4-byte start position and a 16-byte ledger record."""
    W, H, d = cfg.window, cfg.h_kv, cfg.d
    codes = 2 * (W * H * d * cfg.quant_bits) // 8
    kparams = 2 * 2 * H * d
    vparams = 2 * 2 * H * W
    return codes + kparams + vparams + 4 + 16


def capacities(cfg: OracleConfig, prompt_len: int) -> dict:
    """Eq. 3: K_f = floor((1-q) B_hist / M_f), K_q = floor(q B_hist / M_q)."""
    b_tok = token_bytes(cfg)
    B_total = cfg.budget_frac * b_tok * float(prompt_len + cfg.n_decode)
    B_hist = B_total - float((cfg.n_sink + cfg.n_local) * b_tok)
    if B_hist < 0:
        raise BudgetError(f"B_hist = {B_hist} < 0")
    M_f, M_q = full_window_bytes(cfg), quant_window_bytes(cfg)
    K_f = int(math.floor((1.0 - cfg.quant_frac) * B_hist / M_f))
    K_q = int(math.floor(cfg.quant_frac * B_hist / M_q))
    return dict(B_total=B_total, B_hist=B_hist, M_f=M_f, M_q=M_q, K_f=K_f, K_q=K_q, b_tok=b_tok)


# --------------------------------------------------------------------------------------
# exact roundings
# --------------------------------------------------------------------------------------
def to_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even), returned as float64."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m * 2**e, 0.5 <= |m| < 1
    qexp = np.maximum(e - 8, -133)          # 8 significant bits; subnormal quantum 2**-133
    r = np.rint(np.ldexp(x, -qexp))         # np.rint rounds half to even
    return np.ldexp(r, qexp)


def _fp16_quantum_exp(x: np.ndarray) -> np.ndarray:
    _, e = np.frexp(x)
    return np.maximum(e - 11, -24)          # 11 significant bits; subnormal quantum 2**-24


def rd_fp16(x) -> np.ndarray:
    """Largest fp16 value <= x (round toward -inf), as float64."""
    x = np.asarray(x, dtype=np.float64)
    q = _fp16_quantum_exp(x)
    r = np.ldexp(np.floor(np.ldexp(x, -q)), q)
    if np.any(np.abs(r) > FP16_MAX):
        raise RangeError("value outside the fp16 range")
    return r


def ru_fp16(x) -> np.ndarray:
    """Smallest fp16 value >= x (round toward +inf), as float64."""
    x = np.asarray(x, dtype=np.float64)
    q = _fp16_quantum_exp(x)
    r = np.ldexp(np.ceil(np.ldexp(x, -q)), q)
    if np.any(np.abs(r) > FP16_MAX):
        raise RangeError("value outside the fp16 range")
    return r


# --------------------------------------------------------------------------------------
# INT2 / INT4 asymmetric quantization  ([QEvict] §4.3 "Migration-Stable Quantization";
# Appendix G.3 for the 4-bit tier)
# --------------------------------------------------------------------------------------
def quantize_groups(x: np.ndarray, axis: int, bits: int = 2):
    """Quantize groups of ``x`` along ``axis`` to ``bits``-bit codes (L = 2^bits - 1).

    off = RD_fp16(min), scl = RU_fp16((max - off) / L); code = number of levels
    k in {1..L} with 2(x - off) >= (2k - 1) scl (nearest level, ties up),
    code = 0 where scl == 0.  Every operand is a bf16 or fp16 value, so the
    comparisons are exact in float64; the fp64 quotient by L rounds to the same
    fp16 upward value as the exact quotient (it cannot land on an fp16 value
    unless the exact quotient is one).
    """
    if bits not in (2, 4):
        raise ValueError("bits must be 2 or 4")
    L = (1 << bits) - 1
    x = np.asarray(x, dtype=np.float64)
    mn = x.min(axis=axis, keepdims=True)
    mx = x.max(axis=axis, keepdims=True)
    off = rd_fp16(mn)
    scl = ru_fp16((mx - off) / float(L))
    t = 2.0 * (x - off)
    codes = np.zeros(x.shape, dtype=np.uint8)
    for k in range(1, L + 1):
        codes += (t >= (2 * k - 1) * scl)
    codes = np.where(scl == 0.0, 0, codes).astype(np.uint8)
    return codes, np.squeeze(off, axis), np.squeeze(scl, axis)


def dequantize(codes: np.ndarray, off: np.ndarray, scl: np.ndarray, axis: int) -> np.ndarray:
    """x_hat = off + code * scl (exact in float64 for fp16 off/scl and 2- or 4-bit codes)."""
    off = np.expand_dims(off, axis)
    scl = np.expand_dims(scl, axis)
    return off + codes.astype(np.float64) * scl


@dataclass
class Ledger:
    """Write-once quantized record of one window (Lambda_w in [QEvict] Algorithm 1)."""

    k_codes: np.ndarray   # [H_kv][W][d] uint8, groups = channels (axis 1 = tokens)
    k_off: np.ndarray     # [H_kv][d]
    k_scl: np.ndarray
    v_codes: np.ndarray   # [H_kv][W][d] uint8, groups = tokens (axis 2 = channels)
    v_off: np.ndarray     # [H_kv][W]
    v_scl: np.ndarray
    start_pos: int
    dormant: bool = False
    bits: int = 2

    def k_hat(self) -> np.ndarray:
        return dequantize(self.k_codes, self.k_off, self.k_scl, axis=1)

    def v_hat(self) -> np.ndarray:
        return dequantize(self.v_codes, self.v_off, self.v_scl, axis=2)


def quantize_window(k: np.ndarray, v: np.ndarray, start_pos: int, bits: int = 2) -> Ledger:
    """Keys per channel across the window's tokens, values per token across channels."""
    if np.any(np.abs(k) > FP16_MAX) or np.any(np.abs(v) > FP16_MAX):
        raise RangeError("K/V value beyond the fp16 range")
    kc, ko, ks = quantize_groups(k, axis=1, bits=bits)
    vc, vo, vs = quantize_groups(v, axis=2, bits=bits)
    return Ledger(kc, ko, ks, vc, vo, vs, start_pos, bits=bits)


def pack_codes(codes: np.ndarray, bits: int = 2) -> np.ndarray:
    """Canonical packing of a [..., d] code array, 8/bits codes per byte: element c of
    a row goes to byte c // (8/bits), bits bits*(c % (8/bits)) upward."""
    per = 8 // bits
    c = codes.astype(np.uint8)
    d = c.shape[-1]
    c = c.reshape(c.shape[:-1] + (d // per, per))
    out = np.zeros(c.shape[:-1], dtype=np.uint8)
    for i in range(per):
        out |= (c[..., i] << (bits * i)).astype(np.uint8)
    return out


def canonical_ledger_bytes(led: Ledger) -> bytes:
    """Per KV head: K codes [W][d*b/8], V codes [W][d*b/8], K off [d], K scl [d],
    V off [W], V scl [W] (fp16 little endian); heads back to back."""
    out = bytearray()
    for h in range(led.k_codes.shape[0]):
        out += pack_codes(led.k_codes[h], led.bits).tobytes()
        out += pack_codes(led.v_codes[h], led.bits).tobytes()
        out += led.k_off[h].astype(np.float16).tobytes()
        out += led.k_scl[h].astype(np.float16).tobytes()
        out += led.v_off[h].astype(np.float16).tobytes()
        out += led.v_scl[h].astype(np.float16).tobytes()
    return bytes(out)


# --------------------------------------------------------------------------------------
# rotary position embedding ("rotate half" pairing), exact in float64
# --------------------------------------------------------------------------------------
def rope_rotate(x: np.ndarray, pos, cs: np.ndarray, inverse: bool = False) -> np.ndarray:
    """Rotate x [..., n, d] whose token axis -2 sits at positions ``pos`` [n]: channel
    pair (i, i + d/2) turns by the angle whose (cos, sin) is cs[pos, i]; ``inverse``
    turns it back.  No rounding beyond float64."""
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    c = cs[np.asarray(pos), :, 0].astype(np.float64)      # [n][h]
    s = cs[np.asarray(pos), :, 1].astype(np.float64)
    if inverse:
        s = -s
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


# --------------------------------------------------------------------------------------
# attention pieces
# --------------------------------------------------------------------------------------
def softmax(x: np.ndarray, axis: int = -1) -> np.ndarray:
    m = np.max(x, axis=axis, keepdims=True)
    e = np.exp(x - m)
    return e / e.sum(axis=axis, keepdims=True)


def prefill_column_sums(qp: np.ndarray, kp: np.ndarray) -> np.ndarray:
    """Column sums of the causal prompt attention, per q head: col[h][t] =
    sum_{u >= t} P_h[u, t] with P_h = softmax_causal(Q_h K_g^T / sqrt(d))."""
    H_q, S, d = qp.shape
    G = H_q // kp.shape[0]
    col = np.zeros((H_q, S))
    mask = np.triu(np.ones((S, S), dtype=bool), k=1)          # t > u is masked
    for h in range(H_q):
        logits = qp[h] @ kp[h // G].T / math.sqrt(d)
        logits[mask] = -np.inf
        col[h] = softmax(logits, axis=1).sum(axis=0)
    return col


def row_lse(q_row: np.ndarray, k_prefix: np.ndarray) -> float:
    """log sum_t exp(q . k_t / sqrt(d)) over the keys given (one causal row)."""
    z = k_prefix @ q_row / math.sqrt(q_row.shape[-1])
    m = z.max()
    return float(m + np.log(np.exp(z - m).sum()))


def route_order(cand, scores: dict) -> list:
    """Candidates sorted by descending score, ties by ascending window index."""
    return sorted(cand, key=lambda w: (-scores[w], w))


def select_tiers(cand, scores: dict, K_f: int, K_q: int, no_full=()) -> tuple[list, list, list]:
    """Eqs. 4-5 of [QEvict] §4.3: the first K_f candidates in rank order become Full, the
    next K_q Quantized, the rest Evicted.

    ``no_full`` holds the windows that may not enter the Full tier.  It is empty for the
    bidirectional policy; the one-way policy of Appendix K passes the windows that are
    Quantized before the event (they may stay Quantized or be evicted, never return to
    Full).  Both policies use the same capacities and the same rank order, so the one-way
    Full tier is the top K_f of the eligible candidates, and the Quantized tier the next
    K_q of all remaining candidates, Quantized or not, in that same order."""
    order = route_order(cand, scores)
    barred = set(no_full)
    F = [w for w in order if w not in barred][:K_f]
    chosen = set(F)
    rest = [w for w in order if w not in chosen]
    return F, rest[:K_q], rest[K_q:]


# --------------------------------------------------------------------------------------
# one (sequence, layer) unit of QEvict state: C = (S, L, F, Q, E) plus S_bar and Lambda
# --------------------------------------------------------------------------------------
@dataclass
class _Window:
    state: int
    k: Optional[np.ndarray] = None        # [H_kv][W][d] float64 (bf16 values) when LOCAL/FULL
    v: Optional[np.ndarray] = None
    ledger: Optional[Ledger] = None


class UnitOracle:
    """QEvict state and steps for one (sequence, layer) pair, in float64."""

    def __init__(self, cfg: OracleConfig, prompt_len: int, rope_cs: Optional[np.ndarray] = None):
        """``rope_cs`` [n_pos][d/2][2] (cos, sin) is required with ``cfg.rope``."""
        self.cfg = cfg
        if cfg.rope and rope_cs is None:
            raise ValueError("rope=True needs the (cos, sin) table")
        self.cs = None if rope_cs is None else np.asarray(rope_cs, dtype=np.float64)
        self.prompt_len = prompt_len
        self.caps = capacities(cfg, prompt_len)
        self.n = 0
        self.step = 0
        self.sink_k = np.zeros((cfg.h_kv, cfg.n_sink, cfg.d))
        self.sink_v = np.zeros((cfg.h_kv, cfg.n_sink, cfg.d))
        self.win: dict[int, _Window] = {}
        self.score: dict[int, float] = {}
        self.uacc: dict[int, float] = {}     # decay / pnorm: mass since the previous routing event
        self.events: list[dict] = []
        self.ever_evicted: set[int] = set()

    # --- positions ---------------------------------------------------------------
    def win_start(self, w: int) -> int:
        return self.cfg.n_sink + w * self.cfg.window

    def win_end(self, w: int) -> int:
        return self.win_start(w) + self.cfg.window

    def _store(self, p: int, k: np.ndarray, v: np.ndarray):
        cfg = self.cfg
        if p < cfg.n_sink:
            self.sink_k[:, p] = k
            self.sink_v[:, p] = v
            return
        w, i = divmod(p - cfg.n_sink, cfg.window)
        if w not in self.win:
            self.win[w] = _Window(LOCAL, np.zeros((cfg.h_kv, cfg.window, cfg.d)),
                                  np.zeros((cfg.h_kv, cfg.window, cfg.d)))
            self.score[w] = 0.0
            self.uacc[w] = 0.0
        W = self.win[w]
        assert W.state == LOCAL, "new tokens enter the recent region"
        W.k[:, i] = k
        W.v[:, i] = v

    # --- RoPE ([QEvict] §4.3) ----------------------------------------------------------
    def rotate_in(self, x: np.ndarray, pos) -> np.ndarray:
        """An input key / query [H][n][d] (or [H][d] at one position) as the cache holds
        it: bf16 of the exact rotation at ``pos``; unchanged without RoPE."""
        if not self.cfg.rope:
            return x
        if x.ndim == 2:
            return to_bf16(rope_rotate(x[:, None, :], [pos], self.cs))[:, 0, :]
        return to_bf16(rope_rotate(x, pos, self.cs))

    def positions(self, w: int) -> np.ndarray:
        return np.arange(self.win_start(w), self.win_end(w))

    def quant_keys(self, w: int) -> np.ndarray:
        """Keys of a Quantized window as attention uses them: x_hat, re-rotated at the
        ledger's positions (exact) with RoPE."""
        kh = self.win[w].ledger.k_hat()
        return rope_rotate(kh, self.positions(w), self.cs) if self.cfg.rope else kh

    # --- the accessible set (sinks, LOCAL, FULL, QUANT) ------------------------------
    def accessible(self, qexec_bf16: Optional[bool] = None):
        """Returns (owner[n_acc], K[H_kv][n_acc][d], V[H_kv][n_acc][d]) in chronological
        order; owner = -1 for sink tokens, else the window index.  Quantized values are
        x_hat, or bf16(x_hat) with ``qexec_bf16`` (default: the config's reading R2)."""
        cfg = self.cfg
        if qexec_bf16 is None:
            qexec_bf16 = cfg.qexec_bf16
        ns = min(cfg.n_sink, self.n)
        owners = [np.full(ns, -1)]
        Ks = [self.sink_k[:, :ns]]
        Vs = [self.sink_v[:, :ns]]
        for w in sorted(self.win):
            W = self.win[w]
            if W.state in (NONE, EVICTED):
                continue
            ntok = min(cfg.window, self.n - self.win_start(w))
            if W.state == QUANT:
                kh, vh = self.quant_keys(w), W.ledger.v_hat()
                if qexec_bf16:
                    kh, vh = to_bf16(kh), to_bf16(vh)
                Ks.append(kh[:, :ntok])
                Vs.append(vh[:, :ntok])
            else:
                Ks.append(W.k[:, :ntok])
                Vs.append(W.v[:, :ntok])
            owners.append(np.full(ntok, w))
        return np.concatenate(owners), np.concatenate(Ks, axis=1), np.concatenate(Vs, axis=1)

    # --- prefill ([QEvict] §4.2 last paragraph) -----------------------------------
    def prefill(self, qp: np.ndarray, kp: np.ndarray, vp: np.ndarray,
                score_init: Optional[np.ndarray] = None) -> dict:
        """qp [H_q][S][d], kp/vp [H_kv][S][d] (bf16 values).  Stores the prompt, sets
        S_bar_0 from the causal column sums (or from ``score_init`` [n_windows] when
        given; qp may then be None), then routes with the aged prompt windows as
        candidates."""
        cfg = self.cfg
        S = kp.shape[1]
        assert S == self.prompt_len
        if cfg.rope:
            kp = self.rotate_in(kp, np.arange(S))
            if qp is not None:
                qp = self.rotate_in(qp, np.arange(S))
        for p in range(S):
            self._store(p, kp[:, p], vp[:, p])
        self.n = S
        info = {}
        if cfg.ranker == "keynorm":
            pass   # the scores come from the keys when the windows enter the candidate pool
        elif score_init is not None:
            for w in self.win:
                self.score[w] = float(score_init[w])
        else:
            # an empty prompt has no attention rows and contributes no score
            col = prefill_column_sums(qp, kp) if S > 0 else np.zeros((cfg.h_q, 0))
            info["col"] = col
            for w in self.win:
                a, b = self.win_start(w), min(self.win_end(w), S)
                self.score[w] = float(col[:, a:b].sum() / cfg.h_q)
            info["sink_mass"] = float(col[:, :min(cfg.n_sink, S)].sum() / cfg.h_q)
        if cfg.ranker == "pnorm":   # P_0 = S_0^p: the initialisation is the first event-level score
            for w in self.win:
                self.score[w] = self.score[w] ** cfg.pnorm_p
        info["route"] = self.route(decode_event=False)
        return info

    # --- one decode step ([QEvict] §4.1 attention, §4.2 Eq. 1) ----------------------
    def decode(self, q: np.ndarray, k: np.ndarray, v: np.ndarray) -> dict:
        """q [H_q][d], k/v [H_kv][d].  Appends k, v at position n, attends over the
        accessible set and adds each window's head-averaged mass to S_bar."""
        cfg = self.cfg
        q, k = self.rotate_in(q, self.n), self.rotate_in(k, self.n)
        self._store(self.n, k, v)
        self.n += 1
        o, A, owner = self.attend(q)
        accumulate = (cfg.score_every_step or ((self.step + 1) % cfg.omega == 0)) and cfg.ranker != "keynorm"
        mass = {}
        for w in np.unique(owner[owner >= 0]):
            u = float(A[:, owner == w].sum() / cfg.h_q)
            mass[int(w)] = u
            if accumulate:
                if cfg.ranker == "cum":
                    self.score[int(w)] += u
                else:
                    self.uacc[int(w)] += u
        self.step += 1
        tier_mass = {z: np.zeros(cfg.h_q) for z in ("sink", LOCAL, FULL, QUANT)}
        tier_mass["sink"] = A[:, owner < 0].sum(axis=1)
        for w in np.unique(owner[owner >= 0]):
            tier_mass[self.win[int(w)].state] += A[:, owner == w].sum(axis=1)
        return dict(o=o, mass=mass, tier_mass=tier_mass, probs=A, owner=owner, q_rot=q)

    def attend(self, q: np.ndarray, qexec_bf16: Optional[bool] = None):
        """Softmax attention ([QEvict] §4.1) of the queries q [H_q][d] (as the cache holds
        them: rotated with RoPE) over the current accessible set, logits q.k / sqrt(d).
        Returns (o [H_q][d], probabilities A [H_q][n_acc], owner [n_acc]); the state is not
        changed.  ``qexec_bf16`` selects the Quantized values as in ``accessible``."""
        cfg = self.cfg
        owner, K, V = self.accessible(qexec_bf16)
        G = cfg.group
        o = np.zeros((cfg.h_q, cfg.d))
        A = np.zeros((cfg.h_q, owner.shape[0]))
        for h in range(cfg.h_q):
            a = softmax(K[h // G] @ q[h] / math.sqrt(cfg.d))
            A[h] = a
            o[h] = a @ V[h // G]
        return o, A, owner

    # --- alternative rankers ([QEvict] Appendix J) ------------------------------------
    def key_norm_score(self, w: int) -> float:
        """Eq. 24: minus the mean over the window's tokens of ||k_i||_2, the norm taken over
        every KV head's channels of the token's (bf16) key."""
        W = self.win[w]
        norms = [math.sqrt(float(np.sum(W.k[:, i, :] ** 2))) for i in range(self.cfg.window)]
        return -float(np.mean(norms))

    def fold_interval(self):
        """At a decode-time routing event: Eq. 22 (decay) or Eq. 23 (pnorm) with the
        mass u_r gathered since the previous event, which then starts again from 0."""
        cfg = self.cfg
        for w in self.win:
            if cfg.ranker == "decay":
                self.score[w] = cfg.decay_lambda * self.score[w] + self.uacc[w]
            elif cfg.ranker == "pnorm":
                self.score[w] = self.score[w] + self.uacc[w] ** cfg.pnorm_p
            self.uacc[w] = 0.0

    # --- routing ([QEvict] Eqs. 4-6 and Algorithm 1) --------------------------------
    def route(self, decode_event: bool = True) -> dict:
        """A routing event; ``decode_event`` is False only for the one at the end of prefill."""
        cfg, caps = self.cfg, self.caps
        K_f, K_q = caps["K_f"], caps["K_q"]
        if decode_event and cfg.ranker in ("decay", "pnorm"):
            self.fold_interval()
        aged = [w for w, W in self.win.items()
                if W.state == LOCAL and self.win_end(w) <= self.n - cfg.n_local]
        if cfg.ranker == "keynorm":
            for w in aged:
                self.score[w] = self.key_norm_score(w)
        prev_f = [w for w, W in self.win.items() if W.state == FULL]
        prev_q = [w for w, W in self.win.items() if W.state == QUANT]
        cand = prev_f + prev_q + aged
        # one-way variant (Appendix K): a Quantized window cannot return to the Full tier
        F, Q, E = select_tiers(cand, self.score, K_f, K_q, () if cfg.promote else prev_q)
        ctr = dict(aged=len(aged), promoted=0, packed=0, reactivated=0, demoted=0, evicted=len(E),
                   n_full=len(F), n_quant=len(Q))
        # Algorithm 1, promotion: Q -> F dequantizes the ledger and marks it dormant
        for w in F:
            W = self.win[w]
            if W.state == QUANT:
                W.k = to_bf16(self.quant_keys(w))
                W.v = to_bf16(W.ledger.v_hat())
                W.ledger.dormant = True
                ctr["promoted"] += 1
            W.state = FULL
        # Algorithm 1, demotion: first entry quantizes once; a dormant record is reactivated
        for w in Q:
            W = self.win[w]
            if W.state != QUANT:
                ctr["demoted"] += 1
                if W.ledger is None:
                    kq = rope_rotate(W.k, self.positions(w), self.cs, inverse=True) if cfg.rope else W.k
                    W.ledger = quantize_window(kq, W.v, self.win_start(w), cfg.quant_bits)
                    ctr["packed"] += 1
                else:
                    assert W.ledger.dormant
                    W.ledger.dormant = False
                    ctr["reactivated"] += 1
                W.k = W.v = None
            W.state = QUANT
        # Algorithm 1, eviction: release and delete the record
        for w in E:
            W = self.win[w]
            W.state, W.k, W.v, W.ledger = EVICTED, None, None, None
            self.ever_evicted.add(w)
        self.check_invariants()
        self.events.append(dict(n=self.n, F=list(F), Q=list(Q), E=list(E), order=F + Q + E, **ctr))
        return self.events[-1]

    def check_invariants(self):
        """Tier capacities and the §4.1 budget inequality over active tiers (nominal
        protected bytes), and Eq. 6: evicted windows never come back."""
        cfg, caps = self.cfg, self.caps
        nF = sum(W.state == FULL for W in self.win.values())
        nQ = sum(W.state == QUANT for W in self.win.values())
        assert nF <= caps["K_f"] and nQ <= caps["K_q"]
        used = (cfg.n_sink + cfg.n_local) * caps["b_tok"] + nF * caps["M_f"] + nQ * caps["M_q"]
        assert used <= caps["B_total"] + 1e-6
        for w in self.ever_evicted:
            assert self.win[w].state == EVICTED

    # --- due-routing helper -------------------------------------------------------
    def step_and_route(self, q, k, v) -> dict:
        """Decode step j, then route when (j + 1) % Omega == 0."""
        out = self.decode(q, k, v)
        if self.step % self.cfg.omega == 0:
            out["route"] = self.route()
        return out

    # --- export -------------------------------------------------------------------
    def window_table(self) -> dict:
        """Per window: (state, has_ledger, dormant, start_pos)."""
        return {w: (W.state, W.ledger is not None, bool(W.ledger.dormant) if W.ledger else False,
                    self.win_start(w)) for w, W in self.win.items()}
