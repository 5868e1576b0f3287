"""ctypes binding of ``include/qevict.h``: argument marshalling only.

Every step of the QEvict decode path runs in the HIP library
``_lib/libqevict.so``; PyTorch only provides device memory and the stream.
Loading fails loudly when the library has not been built (there is no
fallback path).
"""
from __future__ import annotations

import ctypes
import os
import struct
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "_lib", "libqevict.so")

QEVICT_F_NO_PROMOTE = 1
QEVICT_F_SCORE_ROUTE_ONLY = 2
QEVICT_F_RANK_DECAY = 4      # alternative rankers ([QEvict] Appendix J); at most one
QEVICT_F_RANK_PNORM = 8
QEVICT_F_RANK_KEYNORM = 16
QEVICT_F_INT4 = 32           # INT4 recoverable tier ([QEvict] Appendix G.3) instead of INT2
QEVICT_F_ROPE = 64           # inputs before RoPE; Quantized tier in the pre-RoPE domain ([QEvict] §4.3)
QEVICT_F_SEPARATE_FINISH = 128   # keep the finish launch even with one split per (sequence, KV head)

DEV_E_POOL, DEV_E_WINDOW, DEV_E_RANGE, DEV_E_LIST, DEV_E_SELECT = 1, 2, 4, 8, 16

EXPORTED_SYMBOLS = (
    "qevict_capacities", "qevict_plan", "qevict_create", "qevict_destroy", "qevict_prefill_init",
    "qevict_decode_attn", "qevict_route", "qevict_pack_int2", "qevict_promote", "qevict_poll_status",
    "qevict_export_unit", "qevict_decode_kernel_name", "qevict_last_error", "qevict_time_next_decode",
    "qevict_time_next_route",
    "qevict_step_bytes", "qevict_stream_read", "qevict_set_rope", "qevict_step_mass",
    "qevict_prefill_init_noalloc",
)
NOALLOC_WS_BYTES = 32 << 20    # the static prefill workspace of qevict_prefill_init_noalloc


class QEvictError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"qevict status {status}: {msg}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_layers", ctypes.c_int32), ("h_q", ctypes.c_int32),
        ("h_kv", ctypes.c_int32), ("d_head", ctypes.c_int32), ("window", ctypes.c_int32),
        ("n_sink", ctypes.c_int32), ("n_local", ctypes.c_int32), ("omega", ctypes.c_int32),
        ("quant_frac", ctypes.c_double), ("budget_frac", ctypes.c_double),
        ("max_prompt", ctypes.c_int32), ("max_new", ctypes.c_int32), ("flags", ctypes.c_uint32),
        ("n_splits", ctypes.c_int32),
    ]


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("arena_bytes", ctypes.c_size_t), ("prefill_ws_bytes", ctypes.c_size_t),
        ("export_bytes", ctypes.c_size_t), ("n_windows", ctypes.c_int32), ("n_pages", ctypes.c_int32),
        ("n_slots", ctypes.c_int32), ("n_acc_max", ctypes.c_int32), ("n_splits", ctypes.c_int32),
        ("max_K_f", ctypes.c_int32), ("max_K_q", ctypes.c_int32), ("combine_in_kernel", ctypes.c_int32),
    ]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"QEvict HIP library not built: {path} is missing "
                          "(run `python -m recoverable_kv_cache_amd.build`)")
    lib = ctypes.CDLL(path)
    P, I, D, Z = ctypes.c_void_p, ctypes.c_int32, ctypes.c_double, ctypes.c_size_t
    lib.qevict_capacities.argtypes = [ctypes.POINTER(Config), I, ctypes.POINTER(I), ctypes.POINTER(I),
                                      ctypes.POINTER(D), ctypes.POINTER(D), ctypes.POINTER(ctypes.c_int64),
                                      ctypes.POINTER(ctypes.c_int64)]
    lib.qevict_plan.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(I), ctypes.POINTER(PlanInfo)]
    lib.qevict_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(I), P, Z, P, ctypes.POINTER(P)]
    lib.qevict_destroy.argtypes = [P]
    lib.qevict_destroy.restype = None
    lib.qevict_prefill_init.argtypes = [P, I, P, P, P, P, P, Z, P]
    lib.qevict_prefill_init_noalloc.argtypes = [P, I, P, P, P, P, P]
    lib.qevict_decode_attn.argtypes = [P, I, P, P, P, P, P]
    lib.qevict_route.argtypes = [P, I, P]
    lib.qevict_pack_int2.argtypes = [P, I, P, I, P]
    lib.qevict_promote.argtypes = [P, I, P, I, P]
    lib.qevict_poll_status.argtypes = [P, ctypes.POINTER(ctypes.c_uint32), P]
    lib.qevict_export_unit.argtypes = [P, I, I, P, Z, ctypes.POINTER(Z), P]
    lib.qevict_time_next_decode.argtypes = [P, P, P]
    lib.qevict_time_next_route.argtypes = [P, P, P]
    lib.qevict_step_bytes.argtypes = [P, I, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64), P]
    lib.qevict_stream_read.argtypes = [P, Z, P, P, P, P]
    lib.qevict_set_rope.argtypes = [P, P, I, P]
    lib.qevict_step_mass.argtypes = [P, I, I, P, P]
    lib.qevict_decode_kernel_name.restype = ctypes.c_char_p
    lib.qevict_last_error.restype = ctypes.c_char_p
    for name in EXPORTED_SYMBOLS:
        if name not in ("qevict_destroy", "qevict_decode_kernel_name", "qevict_last_error"):
            getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise QEvictError(status, _lib.qevict_last_error().decode())


def make_config(wl, n_splits: int = 0, flags: int = 0, **over) -> Config:
    """Config from a ``workload.Workload`` (any field can be overridden)."""
    f = dict(batch=wl.batch, n_layers=wl.n_layers, h_q=wl.h_q, h_kv=wl.h_kv, d_head=wl.d_head,
             window=wl.window, n_sink=wl.n_sink, n_local=wl.n_local, omega=wl.omega,
             quant_frac=wl.quant_frac, budget_frac=wl.budget_frac, max_prompt=wl.prompt_len,
             max_new=wl.n_decode, flags=flags, n_splits=n_splits)
    f.update(over)
    return Config(**f)


def capacities(cfg: Config, prompt_len: int) -> dict:
    lib = load_library()
    kf, kq = ctypes.c_int32(), ctypes.c_int32()
    bt, bh = ctypes.c_double(), ctypes.c_double()
    mf, mq = ctypes.c_int64(), ctypes.c_int64()
    _check(lib.qevict_capacities(ctypes.byref(cfg), prompt_len, ctypes.byref(kf), ctypes.byref(kq),
                                 ctypes.byref(bt), ctypes.byref(bh), ctypes.byref(mf), ctypes.byref(mq)))
    return dict(K_f=kf.value, K_q=kq.value, B_total=bt.value, B_hist=bh.value, M_f=mf.value, M_q=mq.value)


def plan(cfg: Config, prompt_lens: Sequence[int]) -> PlanInfo:
    lib = load_library()
    pl = (ctypes.c_int32 * cfg.batch)(*prompt_lens)
    info = PlanInfo()
    _check(lib.qevict_plan(ctypes.byref(cfg), pl, ctypes.byref(info)))
    return info


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _expect(t, shape, dtype_name: str, device, what: str):
    """Host-side check that a tensor matches what the kernels will index."""
    import torch
    dt = getattr(torch, dtype_name)
    if t is None:
        raise ValueError(f"{what}: missing tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what}: shape {tuple(t.shape)} != {tuple(shape)}")
    if t.dtype != dt:
        raise ValueError(f"{what}: dtype {t.dtype} != {dt}")
    if not t.is_contiguous():
        raise ValueError(f"{what}: must be contiguous")
    if t.device != device:
        raise ValueError(f"{what}: on {t.device}, state lives on {device}")


def _stream(stream) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


STREAM_READ_WGS = 1024   # workgroups of qevict_stream_read: one sink word each


def stream_read(buf, sink, ev_before=None, ev_after=None, stream=None):
    """One plain streaming read of the contiguous device tensor ``buf`` (a measurement aid
    beside the split-K kernel); ``sink`` is an int32 device tensor of STREAM_READ_WGS words
    that receives one XOR word per workgroup.  Optional torch.cuda.Event pair (timing
    enabled) stamped by the kernel's own dispatch."""
    import torch
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf: a contiguous device tensor")
    _expect(sink, (STREAM_READ_WGS,), "int32", buf.device, "sink")
    ev0 = None if ev_before is None else ctypes.c_void_p(ev_before.cuda_event)
    ev1 = None if ev_after is None else ctypes.c_void_p(ev_after.cuda_event)
    lib = load_library()
    _check(lib.qevict_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), ev0, ev1,
                                  _stream(stream)))


@dataclass
class UnitExport:
    """Canonical export of one (sequence, layer) unit."""
    n: int
    n_windows: int
    K_f: int
    K_q: int
    status: int
    counters: dict
    n_acc: int
    prompt_len: int
    sink_mass: float
    state: np.ndarray          # [n_windows] int32 (1 recent, 2 Full, 3 Quantized, 4 Evicted)
    has_ledger: np.ndarray
    dormant: np.ndarray
    start_pos: np.ndarray
    score: np.ndarray          # [n_windows] float64
    ledger: dict               # window -> canonical bytes
    kv: dict                   # window -> (K [h_kv][W][d], V) uint16 bf16 bits
    sink_k: np.ndarray
    sink_v: np.ndarray
    acc: np.ndarray = None     # [n_acc][4] int32: kind (0 sinks, 1 page, 2 slot), page / slot id, window, start
    splits: np.ndarray = None  # [n_splits + 1] int32 split offsets into the list
    win_page: np.ndarray = None   # [n_windows] int32 page id of each window (-1 if none)
    win_slot: np.ndarray = None   # [n_windows] int32 slot id of each window (-1 if none)


COUNTER_NAMES = ("aged", "promoted", "packed", "reactivated", "demoted", "evicted", "n_full", "n_quant")


class QEvictState:
    """A QEvict cache for ``cfg.batch`` sequences x ``cfg.n_layers`` layers on one GPU."""

    def __init__(self, cfg: Config, prompt_lens: Sequence[int], device="cuda", stream=None):
        import torch
        self.lib = load_library()
        self.cfg = cfg
        self.prompt_lens = list(prompt_lens)
        self.info = plan(cfg, prompt_lens)
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.arena = torch.empty(self.info.arena_bytes + 256, dtype=torch.uint8, device=self.device)
        base = self.arena.data_ptr()
        self._arena_ptr = (base + 255) // 256 * 256
        self.workspace = None
        handle = ctypes.c_void_p()
        pl = (ctypes.c_int32 * cfg.batch)(*prompt_lens)
        _check(self.lib.qevict_create(ctypes.byref(cfg), pl, ctypes.c_void_p(self._arena_ptr),
                                      self.info.arena_bytes, _stream(stream), ctypes.byref(handle)))
        self.handle = handle

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            self.lib.qevict_destroy(h)
            self.handle = None

    # -- helpers ---------------------------------------------------------------------
    def ensure_workspace(self):
        import torch
        if self.workspace is None and self.info.prefill_ws_bytes:
            self.workspace = torch.empty(self.info.prefill_ws_bytes, dtype=torch.uint8, device=self.device)
        return self.workspace

    def workspace_views(self):
        """(lse2 [B][h_q][S_max] fp32, col [B][h_q][S_max] fp64) views of the prefill workspace."""
        import torch
        ws = self.ensure_workspace()
        c = self.cfg
        n = c.batch * c.h_q * c.max_prompt
        lse = ws[: n * 4].view(torch.float32).view(c.batch, c.h_q, c.max_prompt)
        off = (n * 4 + 255) // 256 * 256
        col = ws[off: off + n * 8].view(torch.float64).view(c.batch, c.h_q, c.max_prompt)
        return lse, col

    # -- the C ABI -----------------------------------------------------------------------
    def prefill_init(self, layer: int, q, k, v, score_init=None, stream=None):
        c = self._expect_prompt(q, k, v, score_init)
        ws = None if (score_init is not None and not c.flags & QEVICT_F_ROPE) else self.ensure_workspace()
        _check(self.lib.qevict_prefill_init(self.handle, layer, _ptr(q), _ptr(k), _ptr(v), _ptr(score_init),
                                            _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))

    def prefill_init_noalloc(self, layer: int, q, k, v, score_init=None, stream=None):
        """``prefill_init`` through the allocation-free entry point (the library's static
        workspace; no workspace tensor is made)."""
        self._expect_prompt(q, k, v, score_init)
        _check(self.lib.qevict_prefill_init_noalloc(self.handle, layer, _ptr(q), _ptr(k), _ptr(v),
                                                    _ptr(score_init), _stream(stream)))

    def _expect_prompt(self, q, k, v, score_init):
        c = self.cfg
        _expect(k, (c.batch, c.h_kv, c.max_prompt, c.d_head), "bfloat16", self.device, "k_prompt")
        _expect(v, (c.batch, c.h_kv, c.max_prompt, c.d_head), "bfloat16", self.device, "v_prompt")
        if score_init is None:
            _expect(q, (c.batch, c.h_q, c.max_prompt, c.d_head), "bfloat16", self.device, "q_prompt")
        else:
            _expect(score_init, (c.batch, self.info.n_windows), "float64", self.device, "score_init")
        return c

    def step_mass(self, layer: int, b: int, out=None, stream=None):
        """Per-head mass of the last decode step: ``[h_q][n_windows + 1]`` float64 on the
        device (column 0 the sinks, 1 + w window w)."""
        import torch
        if out is None:
            out = torch.empty((self.cfg.h_q, self.info.n_windows + 1), dtype=torch.float64, device=self.device)
        _expect(out, (self.cfg.h_q, self.info.n_windows + 1), "float64", self.device, "step mass")
        _check(self.lib.qevict_step_mass(self.handle, layer, b, _ptr(out), _stream(stream)))
        return out

    def set_rope(self, table, stream=None):
        """RoPE mode: copy the (cos, sin) table ``[n_pos][d/2][2]`` (float32, on the device)."""
        _expect(table, (table.shape[0], self.cfg.d_head // 2, 2), "float32", self.device, "rope table")
        _check(self.lib.qevict_set_rope(self.handle, _ptr(table), table.shape[0], _stream(stream)))

    def decode_attn(self, layer: int, q, k, v, out, stream=None):
        c = self.cfg
        _expect(q, (c.batch, c.h_q, c.d_head), "bfloat16", self.device, "q")
        _expect(k, (c.batch, c.h_kv, c.d_head), "bfloat16", self.device, "k_new")
        _expect(v, (c.batch, c.h_kv, c.d_head), "bfloat16", self.device, "v_new")
        _expect(out, (c.batch, c.h_q, c.d_head), "float32", self.device, "out")
        _check(self.lib.qevict_decode_attn(self.handle, layer, _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                           _stream(stream)))

    def route(self, layer: int = -1, stream=None):
        _check(self.lib.qevict_route(self.handle, layer, _stream(stream)))

    def pack_int2(self, layer: int, win_ids, stream=None):
        _expect(win_ids, (self.cfg.batch, win_ids.shape[-1]), "int32", self.device, "win_ids")
        _check(self.lib.qevict_pack_int2(self.handle, layer, _ptr(win_ids), win_ids.shape[-1], _stream(stream)))

    def promote(self, layer: int, win_ids, stream=None):
        _expect(win_ids, (self.cfg.batch, win_ids.shape[-1]), "int32", self.device, "win_ids")
        _check(self.lib.qevict_promote(self.handle, layer, _ptr(win_ids), win_ids.shape[-1], _stream(stream)))

    def time_next_decode(self, ev_before, ev_after):
        """Have the next decode_attn stamp a torch.cuda.Event pair (timing enabled, already recorded once)
        at the start and the end of its split-K attention kernel."""
        _check(self.lib.qevict_time_next_decode(self.handle, ctypes.c_void_p(ev_before.cuda_event),
                                                ctypes.c_void_p(ev_after.cuda_event)))

    def time_next_route(self, ev_before, ev_after):
        """Have the next route stamp a torch.cuda.Event pair (timing enabled, already recorded once)
        at the start of its routing kernel and the end of its migration kernel."""
        _check(self.lib.qevict_time_next_route(self.handle, ctypes.c_void_p(ev_before.cuda_event),
                                               ctypes.c_void_p(ev_after.cuda_event)))

    def step_bytes(self, layer: int, stream=None) -> tuple[int, int]:
        kv, io = ctypes.c_int64(), ctypes.c_int64()
        _check(self.lib.qevict_step_bytes(self.handle, layer, ctypes.byref(kv), ctypes.byref(io), _stream(stream)))
        return kv.value, io.value

    def poll_status(self, stream=None) -> int:
        s = ctypes.c_uint32()
        _check(self.lib.qevict_poll_status(self.handle, ctypes.byref(s), _stream(stream)))
        return s.value

    def export_unit(self, layer: int, b: int, stream=None, tables_only: bool = False) -> UnitExport:
        """The unit's canonical export; ``tables_only`` parses the header, window records
        and scores only (ledgers, pages and sinks are left empty)."""
        buf = (ctypes.c_uint8 * self.info.export_bytes)()
        written = ctypes.c_size_t()
        _check(self.lib.qevict_export_unit(self.handle, layer, b, buf, self.info.export_bytes,
                                           ctypes.byref(written), _stream(stream)))
        return parse_export(bytes(buf)[: written.value], self.cfg, self.info.n_splits, tables_only)


def parse_export(blob: bytes, cfg: Config, n_splits: int, tables_only: bool = False) -> UnitExport:
    head = struct.unpack_from("<20i", blob, 0)
    assert head[0] == 0x58564551, "bad export magic"
    n, nw, K_f, K_q, status = head[1:6]
    ctr = dict(zip(COUNTER_NAMES, head[6:14]))
    ctr["paired_fills"] = head[18]   # promotions into a page a pack read at the same event
    n_acc, prompt_len = head[14], head[15]
    sink_mass = struct.unpack_from("<d", blob, 64)[0]
    at = 80
    rec = np.frombuffer(blob, dtype=np.dtype([("i", "<i4", 4), ("s", "<f8")]), count=nw, offset=at)
    at += 24 * nw
    state, has_led, dorm, start = (rec["i"][:, k].copy() for k in range(4))
    score = rec["s"].copy()
    acc = np.frombuffer(blob, dtype="<i4", count=4 * n_acc, offset=at).reshape(n_acc, 4).copy()
    at += 16 * n_acc
    splits = np.frombuffer(blob, dtype="<i4", count=n_splits + 1, offset=at).copy()
    at += 4 * (n_splits + 1)
    ids = np.frombuffer(blob, dtype="<i4", count=2 * nw, offset=at).reshape(nw, 2)
    win_page, win_slot = ids[:, 0].copy(), ids[:, 1].copy()
    at += 8 * nw
    lists = dict(acc=acc, splits=splits, win_page=win_page, win_slot=win_slot)
    if tables_only:
        empty = np.zeros((0,), dtype=np.uint16)
        return UnitExport(n, nw, K_f, K_q, status, ctr, n_acc, prompt_len, sink_mass, state, has_led, dorm, start,
                          score, {}, {}, empty, empty, **lists)
    H, W, d, ns = cfg.h_kv, cfg.window, cfg.d_head, cfg.n_sink
    qb = 4 if cfg.flags & QEVICT_F_INT4 else 2
    slot_bytes = H * (2 * W * d * qb // 8 + 4 * d + 4 * W)
    ledger = {}
    for w in range(nw):
        if has_led[w]:
            ledger[w] = blob[at: at + slot_bytes]
            at += slot_bytes
    kv = {}
    pe = 2 * H * W * d
    for w in range(nw):
        if state[w] in (1, 2):
            arr = np.frombuffer(blob, dtype="<u2", count=pe, offset=at).reshape(2, H, W, d)
            kv[w] = (arr[0].copy(), arr[1].copy())
            at += pe * 2
    sk = np.frombuffer(blob, dtype="<u2", count=2 * H * ns * d, offset=at).reshape(2, H, ns, d)
    return UnitExport(n, nw, K_f, K_q, status, ctr, n_acc, prompt_len, sink_mass, state, has_led, dorm, start,
                      score, ledger, kv, sk[0].copy(), sk[1].copy(), **lists)
