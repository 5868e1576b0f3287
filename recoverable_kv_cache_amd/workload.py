"""Seeded synthetic inputs for the QEvict decode path.

This module only draws numbers: it holds none of the method's arithmetic (no
attention, no scores, no quantization, no routing).  Both the HIP path and the
fp64 oracle are fed from it, so the two always see identical bf16 bytes.

Recipe (the pages publish no inputs; these stand in for their workloads):

* Every value is a float32 ``standard_normal`` draw rounded once to bf16
  (round-to-nearest-even, as ``torch.Tensor.to(torch.bfloat16)`` does).
* Outliers: per (layer, kv-head), ``n_outlier`` key channels drawn without
  replacement are multiplied by 10 before the bf16 rounding.
* Planted topics: ``n_topics`` disjoint prompt windows outside the sinks and the
  final recent region.  Per (layer, sequence, kv-head, topic) a unit direction
  ``u`` is drawn and the keys of that window get ``beta * u`` added (beta = 8).
* Drift: decode query ``t`` of q-head ``h`` is ``cos(phi) g + sin(phi) sqrt(d) u``
  where ``g ~ N(0, I)`` and ``u`` is the direction of topic ``(t // period) mod
  n_topics`` for the head's kv group; ``phi`` ramps linearly from 0 to 60
  degrees over the first half of each period and then holds.
* Prompt queries are plain ``N(0, 1)``.

Streams are keyed by ``(seed, layer, sequence, stream-id)`` so any slice can be
regenerated on its own (``torch.Generator`` seeded from a hash of the key).
"""
from __future__ import annotations

import functools
import hashlib
import math
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence

import torch

# stream ids
_S_QP, _S_KP, _S_VP, _S_QD, _S_KD, _S_VD, _S_OUT, _S_TOPIC_WIN, _S_TOPIC_DIR, _S_LEN = range(10)


@dataclass(frozen=True)
class Workload:
    """Shape and schedule of one synthetic QEvict decode workload."""

    name: str
    n_layers: int
    batch: int
    h_q: int
    h_kv: int
    d_head: int
    prompt_len: int            # maximum prompt length
    n_decode: int              # generated tokens
    window: int
    n_sink: int
    n_local: int
    omega: int
    budget_frac: float
    quant_frac: float
    prompt_len_min: Optional[int] = None   # ragged prompts ~ U[min, max] when set
    n_outlier: int = 0
    n_topics: int = 0
    topic_period: int = 64
    beta: float = 8.0
    seed: int = 0

    def prompt_lens(self) -> list[int]:
        """Per-sequence prompt lengths (ragged when ``prompt_len_min`` is set)."""
        if self.prompt_len_min is None:
            return [self.prompt_len] * self.batch
        g = _gen(self.seed, 0, 0, _S_LEN)
        lo, hi = self.prompt_len_min, self.prompt_len
        return [int(x) for x in torch.randint(lo, hi + 1, (self.batch,), generator=g)]

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads of the decode benchmark.  Sinks / recent sizes that a
# workload does not name are taken from the 32K one (4 sinks, 256 recent).
TINY = Workload("tiny_512p64", 1, 1, 4, 1, 64, 512, 64, 16, 4, 64, 8, 0.40, 0.70)
LLAMA8B_32K = Workload("llama8b_32k", 32, 1, 32, 8, 128, 32768, 512, 32, 4, 256, 8, 0.20, 0.70,
                       n_outlier=4, n_topics=8, topic_period=64)
BATCHED_16K = Workload("batched_8k16k_b16", 32, 16, 32, 8, 128, 16384, 256, 32, 4, 256, 8, 0.25, 0.70,
                       prompt_len_min=8192, n_outlier=4, n_topics=8, topic_period=32)
CHURN_4K = Workload("churn_4k_4096gen_b64", 32, 64, 32, 8, 128, 4096, 4096, 16, 4, 256, 8, 0.15, 0.70,
                    n_outlier=4, n_topics=8, topic_period=256)
LLAMA70B_128K = Workload("llama70b_128k_b4", 80, 4, 64, 8, 128, 131072, 256, 64, 4, 512, 8, 0.10, 0.70,
                         n_outlier=4, n_topics=16, topic_period=16)

ALL_WORKLOADS = (TINY, LLAMA8B_32K, BATCHED_16K, CHURN_4K, LLAMA70B_128K)


def _gen(seed: int, layer: int, b: int, stream: int, device="cpu") -> torch.Generator:
    key = f"{seed}/{layer}/{b}/{stream}".encode()
    s = int.from_bytes(hashlib.sha256(key).digest()[:8], "little") & ((1 << 63) - 1)
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


def _normal(shape, gen, device) -> torch.Tensor:
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def _topic_windows(wl: Workload, layer: int, b: int, prompt_len: int) -> list[int]:
    """Disjoint prompt windows (indices) that carry a planted topic direction."""
    if wl.n_topics == 0:
        return []
    n_hist = (prompt_len - wl.n_local - wl.n_sink) // wl.window
    if n_hist < wl.n_topics:
        return []
    g = _gen(wl.seed, layer, b, _S_TOPIC_WIN)
    perm = torch.randperm(n_hist, generator=g)[: wl.n_topics]
    return sorted(int(x) for x in perm)


@functools.lru_cache(maxsize=4096)
def _topic_dirs(wl: Workload, layer: int, b: int, device) -> torch.Tensor:
    """Unit directions [h_kv][n_topics][d] (float32)."""
    g = _gen(wl.seed, layer, b, _S_TOPIC_DIR, "cpu")
    u = torch.randn((wl.h_kv, max(wl.n_topics, 1), wl.d_head), generator=g, dtype=torch.float64)
    u = u / u.norm(dim=-1, keepdim=True)
    return u.to(torch.float32).to(device)


@functools.lru_cache(maxsize=4096)
def _outlier_channels(wl: Workload, layer: int) -> torch.Tensor:
    g = _gen(wl.seed, layer, 0, _S_OUT)
    rows = [torch.randperm(wl.d_head, generator=g)[: wl.n_outlier] for _ in range(wl.h_kv)]
    return torch.stack(rows) if rows and wl.n_outlier > 0 else torch.zeros((wl.h_kv, 0), dtype=torch.long)


def prompt(wl: Workload, layer: int, device="cpu", with_q: bool = True, seqs: Optional[Sequence[int]] = None):
    """Prompt tensors for one layer, bf16, zero-padded past each prompt length.

    Returns ``q [B][H_q][S][d]``, ``k, v [B][H_kv][S][d]`` with ``S = wl.prompt_len``
    (``q`` is None with ``with_q=False``; the keys and values do not depend on it).
    ``seqs`` draws only those sequences of the batch, in the given order (their rows are
    the same as in the whole batch's draw).
    """
    S, d = wl.prompt_len, wl.d_head
    lens = wl.prompt_lens()
    gen_dev = device if str(device).startswith("cuda") else "cpu"
    qs, ks, vs = [], [], []
    outl = _outlier_channels(wl, layer)
    for b in (range(wl.batch) if seqs is None else seqs):
        q = _normal((wl.h_q, S, d), _gen(wl.seed, layer, b, _S_QP, gen_dev), gen_dev) if with_q else None
        k = _normal((wl.h_kv, S, d), _gen(wl.seed, layer, b, _S_KP, gen_dev), gen_dev)
        v = _normal((wl.h_kv, S, d), _gen(wl.seed, layer, b, _S_VP, gen_dev), gen_dev)
        if wl.n_outlier:
            for h in range(wl.h_kv):
                k[h][:, outl[h].to(k.device)] *= 10.0
        tw = _topic_windows(wl, layer, b, lens[b])
        if tw:
            u = _topic_dirs(wl, layer, b, str(k.device))
            for j, w in enumerate(tw):
                s0 = wl.n_sink + w * wl.window
                k[:, s0:s0 + wl.window, :] += wl.beta * u[:, j:j + 1, :]
        L = lens[b]
        if L < S:
            if with_q:
                q[:, L:, :] = 0
            k[:, L:, :] = 0
            v[:, L:, :] = 0
        if with_q:
            qs.append(q.to(torch.bfloat16))
        ks.append(k.to(torch.bfloat16))
        vs.append(v.to(torch.bfloat16))
    return (torch.stack(qs).to(device) if with_q else None, torch.stack(ks).to(device), torch.stack(vs).to(device))


def _phase(wl: Workload, step: int) -> tuple[int, float]:
    P = max(wl.topic_period, 1)
    j = (step // P) % max(wl.n_topics, 1)
    r = (step % P) / (P / 2.0)
    phi = math.radians(60.0) * min(r, 1.0)
    return j, phi


def decode_step(wl: Workload, layer: int, step: int, device="cpu") -> tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Decode inputs for one step of one layer: ``q [B][H_q][d]``, ``k, v [B][H_kv][d]`` (bf16).

    Each sequence draws from its own streams (keyed by layer, sequence and step); the
    outlier scaling and the drift are then applied to the whole batch at once."""
    d = wl.d_head
    gen_dev = device if str(device).startswith("cuda") else "cpu"
    G = wl.h_q // wl.h_kv
    qs, ks, vs = [], [], []
    for b in range(wl.batch):
        # one generator per (layer, b, step) so steps are independent slices
        key = b * 1_000_003 + step
        qs.append(_normal((wl.h_q, d), _gen(wl.seed, layer, key, _S_QD, gen_dev), gen_dev))
        ks.append(_normal((wl.h_kv, d), _gen(wl.seed, layer, key, _S_KD, gen_dev), gen_dev))
        vs.append(_normal((wl.h_kv, d), _gen(wl.seed, layer, key, _S_VD, gen_dev), gen_dev))
    q, k, v = torch.stack(qs), torch.stack(ks), torch.stack(vs)
    if wl.n_outlier:
        k *= _outlier_scale(wl, layer, str(k.device))
    if wl.n_topics:
        j, phi = _phase(wl, step)
        u = torch.stack([_topic_dirs(wl, layer, b, str(q.device))[:, j, :] for b in range(wl.batch)])
        uq = u.repeat_interleave(G, dim=1)                           # [B][h_q][d]
        q = math.cos(phi) * q + math.sin(phi) * math.sqrt(d) * uq
    return q.to(torch.bfloat16).to(device), k.to(torch.bfloat16).to(device), v.to(torch.bfloat16).to(device)


@functools.lru_cache(maxsize=4096)
def _outlier_scale(wl: Workload, layer: int, device) -> torch.Tensor:
    """[h_kv][d] float32: 10 on the layer's outlier key channels, 1 elsewhere."""
    m = torch.ones((wl.h_kv, wl.d_head), dtype=torch.float32)
    outl = _outlier_channels(wl, layer)
    for h in range(wl.h_kv):
        m[h, outl[h]] = 10.0
    return m.to(device)


def init_scores(wl: Workload, layer: int, n_windows: int, device="cpu") -> torch.Tensor:
    """Synthetic initial window scores ``[B][n_windows]`` (float64), for callers that
    supply their own prefill estimate instead of the prompt-attention column sums.

    Drawn as |N(0,1)| * 10 so ties have probability zero; planted topic windows get +100.
    """
    out = torch.empty((wl.batch, n_windows), dtype=torch.float64)
    lens = wl.prompt_lens()
    for b in range(wl.batch):
        g = _gen(wl.seed, layer, b, _S_LEN + 1)
        out[b] = torch.randn((n_windows,), generator=g, dtype=torch.float64).abs() * 10.0
        for w in _topic_windows(wl, layer, b, lens[b]):
            if w < n_windows:
                out[b, w] += 100.0
    return out.to(device)


ROPE_THETA = 500000.0     # base of the rotary frequencies of the Llama-3 family


def rope_table(d: int, n_pos: int, theta: float = ROPE_THETA, device="cpu") -> torch.Tensor:
    """Rotary (cos, sin) table ``[n_pos][d/2][2]`` (float32) for the "rotate half"
    pairing: pair i of position p turns by p * theta^(-2i/d).  Angles and their cosines
    and sines are evaluated in float64 and rounded once to float32; the table is an
    input of the model, handed unchanged to the library and to the oracle."""
    i = torch.arange(d // 2, dtype=torch.float64)
    inv = theta ** (-2.0 * i / d)
    ang = torch.arange(n_pos, dtype=torch.float64)[:, None] * inv[None, :]
    return torch.stack([torch.cos(ang), torch.sin(ang)], dim=-1).to(torch.float32).to(device)
