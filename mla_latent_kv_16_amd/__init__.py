"""Python binding of libmla (MLA decode, weight-absorbed form, gfx950).

Argument marshalling only: every step runs in libmla's HIP kernels.  torch
provides device memory and the current HIP stream; tensors are passed to the
C ABI as raw device pointers.  The binding fails loudly when libmla.so has not
been built -- there is no fallback.

Entry points mirror include/mla.h:
    absorb_q, plan_splits, decode_splitkv, combine, decode_merged, out_proj, append_kv,
    append_kv_noalloc,
    decode_splitkv_multi, combine_multi, combine_out_proj, prefill_naive
plus `decode_step`, which runs the four device steps in order, and
`check_paging`, a device check of the lengths and block-table entries.

With the environment variable MLA_DEBUG set (to anything but "" or "0"),
decode_splitkv, decode_splitkv_multi, decode_merged and prefill_naive first run
check_paging on their stream, wait for it and raise MlaError on a bad length or
block-table entry (the check runs even inside record_calls() and is not
recorded).
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np

__all__ = ["MlaError", "Dims", "load", "lib_path", "absorb_q", "plan_splits", "decode_splitkv",
           "decode_merged", "append_kv", "append_kv_noalloc", "decode_splitkv_multi", "combine_multi", "combine_out_proj",
           "prefill_naive",
           "combine", "out_proj", "decode_step", "fast_path", "version", "record_calls", "replay_calls",
           "check_paging", "exact_pass_count", "BF16", "F32"]

_HERE = os.path.dirname(os.path.abspath(__file__))
BF16, F32 = 0, 1
_STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported", -3: "capacity too small",
           -4: "HIP runtime error"}


class MlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: libmla status {status} ({_STATUS.get(status, '?')})")
        self.status = status


class _Dims(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("d_head", ctypes.c_int32),
                ("d_latent", ctypes.c_int32), ("d_rope", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("rope_base", ctypes.c_double), ("dtype", ctypes.c_int)]


@dataclass(frozen=True)
class Dims:
    n_heads: int
    d_head: int
    d_latent: int
    d_rope: int
    page_size: int = 64
    softmax_scale: Optional[float] = None   # default 1/sqrt(d_head + d_rope)
    rope_base: float = 10000.0
    dtype: int = BF16

    def c(self) -> _Dims:
        s = self.softmax_scale
        if s is None:
            s = 1.0 / float(np.sqrt(self.d_head + self.d_rope))
        return _Dims(self.n_heads, self.d_head, self.d_latent, self.d_rope, self.page_size,
                     float(s), float(self.rope_base), int(self.dtype))

    @property
    def row(self) -> int:
        return self.d_latent + self.d_rope


_lib = None


def lib_path() -> str:
    return os.path.join(_HERE, "libmla.so")


def load():
    """Load libmla.so (built in the package directory); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    p = lib_path()
    if not os.path.exists(p):
        raise RuntimeError(f"libmla.so not found at {p}; build it with "
                           "`python -m mla_latent_kv_16_amd.build`")
    # torch ships its own HIP runtime under the same soname (libamdhip64.so.7).
    # Load it first so that libmla binds to that one instance: two HIP runtimes
    # in one process do not share the device.
    import torch  # noqa: F401
    L = ctypes.CDLL(p)
    vp, i32, pi32 = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)
    pd = ctypes.POINTER(_Dims)
    sig = {
        "mla_absorb_q": (i32, [pd, i32, vp, vp, vp, vp, vp, vp]),
        "mla_plan_splits": (i32, [pd, i32, pi32, i32, i32, pi32, pi32, pi32]),
        "mla_plan_max_items": (ctypes.c_int64, [pd, i32, pi32]),
        "mla_plan_splits_ordered": (i32, [pd, i32, pi32, i32, i32, pi32, pi32, pi32, pi32]),
        "mla_decode_splitkv_ordered": (i32, [pd, i32, vp, vp, i32, vp, i32, vp, vp, i32, vp, vp, vp,
                                              vp]),
        "mla_decode_splitkv": (i32, [pd, i32, vp, vp, i32, vp, i32, vp, vp, i32, vp, vp, vp]),
        "mla_combine": (i32, [pd, i32, vp, vp, vp, vp, vp, vp]),
        "mla_decode_splitkv_multi": (i32, [pd, i32, i32, vp, vp, i32, vp, i32, vp, vp, i32, vp, vp,
                                            vp]),
        "mla_combine_multi": (i32, [pd, i32, i32, vp, vp, vp, vp, vp, vp]),
        "mla_decode_merged": (i32, [pd, i32, vp, vp, i32, vp, i32, vp, vp, i32, vp, vp, vp, vp, vp,
                                     vp, vp]),
        "mla_out_proj": (i32, [pd, i32, vp, vp, vp, vp]),
        "mla_combine_out_proj": (i32, [pd, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]),
        "mla_prefill_naive": (i32, [pd, i32, i32, vp, vp, vp, vp, vp, i32, vp, i32, vp, vp,
                                     ctypes.c_int64, vp, vp, vp]),
        "mla_prefill_workspace_bytes": (ctypes.c_int64, [pd, i32, i32]),
        "mla_append_kv": (i32, [pd, i32, i32, vp, vp, vp, vp, i32, ctypes.c_float, vp, i32, vp, i32,
                                 vp, ctypes.c_int64, vp]),
        "mla_append_kv_workspace_bytes": (ctypes.c_int64, [pd, i32, i32]),
        "mla_append_kv_noalloc": (i32, [pd, i32, i32, vp, vp, vp, vp, i32, ctypes.c_float, vp, i32, vp,
                                         i32, vp]),
        "mla_append_kv_noalloc_max_bytes": (ctypes.c_int64, []),
        "mla_check_paging": (i32, [pd, i32, i32, vp, i32, vp, i32, vp, vp]),
        "mla_decode_exact_pass_count": (i32, [i32, ctypes.POINTER(ctypes.c_uint64)]),
        "mla_status_string": (ctypes.c_char_p, [i32]),
        "mla_version": (i32, []),
        "mla_fast_path": (i32, [pd]),
        "mla_last_hip_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    _lib = L
    return L


_recording = None  # a list while record_calls() is active


def _launch(name: str, *args):
    """Issue one enqueueing library call (or, inside record_calls(), keep it)."""
    f = getattr(load(), name)
    if _recording is not None:
        _recording.append((f, args, name))
        return
    _check(f(*args), name)


@contextlib.contextmanager
def record_calls():
    """Inside the block the enqueueing functions below marshal and check their
    arguments as usual but do not call the library; the yielded list then
    holds the calls, with their arguments (device pointers, sizes and the
    stream, fixed at this point), for replay_calls().  For callers that
    enqueue the same work on the same buffers many times and want to skip
    the per-call marshalling."""
    global _recording
    if _recording is not None:
        raise RuntimeError("record_calls() does not nest")
    calls = []
    _recording = calls
    try:
        yield calls
    finally:
        _recording = None


def replay_calls(calls):
    """Issue recorded calls again, in order, checking every status."""
    for f, args, name in calls:
        _check(f(*args), name)


def _check(status: int, where: str):
    if status != 0:
        detail = ""
        if status == -4 and _lib is not None:
            detail = " [" + (_lib.mla_last_hip_error() or b"").decode(errors="replace") + "]"
        raise MlaError(status, where + detail)


def exact_pass_count(reset: bool = False) -> int:
    """Work items the 128-head decode redid against exact maxima on the current
    device since the last reset (synchronous)."""
    n = ctypes.c_uint64(0)
    _check(load().mla_decode_exact_pass_count(int(bool(reset)), ctypes.byref(n)),
           "mla_decode_exact_pass_count")
    return int(n.value)


def version() -> int:
    return load().mla_version()


def fast_path(dims: Dims) -> int:
    return load().mla_fast_path(ctypes.byref(dims.c()))


# ---------------------------------------------------------------------------
# torch marshalling
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _stream(stream) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(getattr(stream, "cuda_stream", stream))


def _store_dtype(dims: Dims):
    torch = _torch()
    return torch.bfloat16 if dims.dtype == BF16 else torch.float32


def _ptr(t, dtype=None, shape=None, name="tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def absorb_q(dims: Dims, q_nope, q_pe, positions, w_uk, q_abs=None, stream=None):
    """q_abs[b][i] = [(W^UK_i)^T q_nope[b][i] ; RoPE_{positions[b]}(q_pe[b][i])]."""
    torch = _torch()
    B = q_nope.shape[0]
    dt = _store_dtype(dims)
    H = dims.n_heads
    if q_abs is None:
        q_abs = torch.empty((B, H, dims.row), dtype=dt, device=q_nope.device)
    _launch("mla_absorb_q",
        ctypes.byref(dims.c()), B,
        _ptr(q_nope, dt, (B, H, dims.d_head), "q_nope"), _ptr(q_pe, dt, (B, H, dims.d_rope), "q_pe"),
        _ptr(positions, torch.int32, (B,), "positions"),
        _ptr(w_uk, dt, (H * dims.d_head, dims.d_latent), "w_uk"),
        _ptr(q_abs, dt, (B, H, dims.row), "q_abs"), _stream(stream))
    return q_abs


def plan_splits(dims: Dims, seq_lens_host, num_slots: int, ordered: bool = False):
    """Host planner: (items [W, 4] int32, split_offsets [B + 1] int32), and with
    `ordered` also the longest-first dispatch order [W] int32
    (mla_plan_splits_ordered) as a third element."""
    L = load()
    lens = np.ascontiguousarray(np.asarray(seq_lens_host, dtype=np.int32))
    B = int(lens.shape[0])
    pi32 = ctypes.POINTER(ctypes.c_int32)
    d = dims.c()
    cap = L.mla_plan_max_items(ctypes.byref(d), B, lens.ctypes.data_as(pi32))
    if cap < 0:
        raise MlaError(-1, "mla_plan_max_items")
    items = np.zeros((max(int(cap), 1), 4), dtype=np.int32)
    offs = np.zeros(B + 1, dtype=np.int32)
    n = ctypes.c_int32(0)
    if ordered:
        order = np.zeros(items.shape[0], dtype=np.int32)
        _check(L.mla_plan_splits_ordered(ctypes.byref(d), B, lens.ctypes.data_as(pi32), int(num_slots),
                                         items.shape[0], items.ctypes.data_as(pi32),
                                         offs.ctypes.data_as(pi32), order.ctypes.data_as(pi32),
                                         ctypes.byref(n)), "mla_plan_splits_ordered")
        return items[:n.value].copy(), offs, order[:n.value].copy()
    _check(L.mla_plan_splits(ctypes.byref(d), B, lens.ctypes.data_as(pi32), int(num_slots),
                             items.shape[0], items.ctypes.data_as(pi32),
                             offs.ctypes.data_as(pi32), ctypes.byref(n)), "mla_plan_splits")
    return items[:n.value].copy(), offs


def check_paging(dims: Dims, block_table, seq_lens, num_pages: int, min_len: int = 1,
                 result=None, stream=None):
    """Device check of seq_lens and the block-table entries they address:
    result int32 [2] = (number of bad values, first bad sequence or -1).
    Enqueued on the stream, not waited for."""
    torch = _torch()
    B = seq_lens.shape[0]
    if result is None:
        result = torch.empty(2, dtype=torch.int32, device=seq_lens.device)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table must have shape ({B}, max_pages)")
    _check(load().mla_check_paging(
        ctypes.byref(dims.c()), B, int(min_len), _ptr(seq_lens, torch.int32, (B,), "seq_lens"),
        int(num_pages), _ptr(block_table, torch.int32, None, "block_table"), block_table.shape[1],
        _ptr(result, torch.int32, (2,), "result"), _stream(stream)), "mla_check_paging")
    return result


def _debug_paging(dims: Dims, block_table, seq_lens, num_pages: int, min_len: int, stream, where):
    if os.environ.get("MLA_DEBUG", "0") in ("", "0"):
        return
    torch = _torch()
    r = check_paging(dims, block_table, seq_lens, num_pages, min_len, stream=stream)
    torch.cuda.synchronize(r.device)
    bad, first = (int(v) for v in r.cpu())
    if bad:
        raise MlaError(-1, f"{where}: MLA_DEBUG found {bad} bad length or block-table "
                           f"value(s), first in sequence {first}")


def decode_splitkv(dims: Dims, q_abs, kv_cache, block_table, seq_lens, items,
                   o_part=None, lse_part=None, stream=None, order=None):
    """Per work item: (o_part [W, H, d_c] float32, lse_part [W, H] float32).
    With `order` (device int32 [W], e.g. plan_splits(..., ordered=True)'s third
    output) workgroup slot s takes item order[s] (mla_decode_splitkv_ordered)."""
    torch = _torch()
    dt = _store_dtype(dims)
    B, H = q_abs.shape[0], dims.n_heads
    W = items.shape[0]
    dev = q_abs.device
    if o_part is None:
        o_part = torch.empty((W, H, dims.d_latent), dtype=torch.float32, device=dev)
    if lse_part is None:
        lse_part = torch.empty((W, H), dtype=torch.float32, device=dev)
    num_pages = kv_cache.shape[0]
    _debug_paging(dims, block_table, seq_lens, num_pages, 1, stream, "mla_decode_splitkv")
    head = [ctypes.byref(dims.c()), B, _ptr(q_abs, dt, (B, H, dims.row), "q_abs"),
            _ptr(kv_cache, dt, (num_pages, dims.page_size, dims.row), "kv_cache"), num_pages,
            _ptr(block_table, torch.int32, None, "block_table"), block_table.shape[1],
            _ptr(seq_lens, torch.int32, (B,), "seq_lens"), _ptr(items, torch.int32, (W, 4), "items"), W]
    tail = [_ptr(o_part, torch.float32, (W, H, dims.d_latent), "o_part"),
            _ptr(lse_part, torch.float32, (W, H), "lse_part"), _stream(stream)]
    if order is None:
        _launch("mla_decode_splitkv", *head, *tail)
    else:
        _launch("mla_decode_splitkv_ordered", *head, _ptr(order, torch.int32, (W,), "order"), *tail)
    return o_part, lse_part


def combine(dims: Dims, split_offsets, o_part, lse_part, batch: int, o_latent=None, lse=None,
            stream=None, want_lse: bool = True):
    """LSE merge: (o_latent [B, H, d_c] float32, lse [B, H] float32 or None)."""
    torch = _torch()
    H = dims.n_heads
    dev = o_part.device
    if o_latent is None:
        o_latent = torch.empty((batch, H, dims.d_latent), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((batch, H), dtype=torch.float32, device=dev)
    W = o_part.shape[0]
    _launch("mla_combine",
        ctypes.byref(dims.c()), batch, _ptr(split_offsets, torch.int32, (batch + 1,), "split_offsets"),
        _ptr(o_part, torch.float32, (W, H, dims.d_latent), "o_part"),
        _ptr(lse_part, torch.float32, (W, H), "lse_part"),
        _ptr(o_latent, torch.float32, (batch, H, dims.d_latent), "o_latent"),
        _ptr(lse, torch.float32, (batch, H), "lse"), _stream(stream))
    return o_latent, lse


def decode_splitkv_multi(dims: Dims, q_abs, kv_cache, block_table, seq_lens, items,
                         o_part=None, lse_part=None, stream=None):
    """q_len query tokens per sequence, q_abs [B, T, H, d_c + d_r]:
    (o_part [W, T, H, d_c] float32, lse_part [W, T, H] float32).  Token t of
    sequence b sees cache rows 0 .. seq_lens[b] - T + t."""
    torch = _torch()
    dt = _store_dtype(dims)
    B, T, H = q_abs.shape[0], q_abs.shape[1], dims.n_heads
    W = items.shape[0]
    dev = q_abs.device
    if o_part is None:
        o_part = torch.empty((W, T, H, dims.d_latent), dtype=torch.float32, device=dev)
    if lse_part is None:
        lse_part = torch.empty((W, T, H), dtype=torch.float32, device=dev)
    num_pages = kv_cache.shape[0]
    _debug_paging(dims, block_table, seq_lens, num_pages, T, stream, "mla_decode_splitkv_multi")
    _launch("mla_decode_splitkv_multi",
        ctypes.byref(dims.c()), B, T, _ptr(q_abs, dt, (B, T, H, dims.row), "q_abs"),
        _ptr(kv_cache, dt, (num_pages, dims.page_size, dims.row), "kv_cache"), num_pages,
        _ptr(block_table, torch.int32, None, "block_table"), block_table.shape[1],
        _ptr(seq_lens, torch.int32, (B,), "seq_lens"), _ptr(items, torch.int32, (W, 4), "items"), W,
        _ptr(o_part, torch.float32, (W, T, H, dims.d_latent), "o_part"),
        _ptr(lse_part, torch.float32, (W, T, H), "lse_part"), _stream(stream))
    return o_part, lse_part


def combine_multi(dims: Dims, split_offsets, o_part, lse_part, batch: int, o_latent=None, lse=None,
                  stream=None, want_lse: bool = True):
    """LSE merge per (sequence, query token): (o_latent [B, T, H, d_c], lse [B, T, H] or None)."""
    torch = _torch()
    H = dims.n_heads
    W, T = o_part.shape[0], o_part.shape[1]
    dev = o_part.device
    if o_latent is None:
        o_latent = torch.empty((batch, T, H, dims.d_latent), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((batch, T, H), dtype=torch.float32, device=dev)
    _launch("mla_combine_multi",
        ctypes.byref(dims.c()), batch, T,
        _ptr(split_offsets, torch.int32, (batch + 1,), "split_offsets"),
        _ptr(o_part, torch.float32, (W, T, H, dims.d_latent), "o_part"),
        _ptr(lse_part, torch.float32, (W, T, H), "lse_part"),
        _ptr(o_latent, torch.float32, (batch, T, H, dims.d_latent), "o_latent"),
        _ptr(lse, torch.float32, (batch, T, H), "lse"), _stream(stream))
    return o_latent, lse


def decode_merged(dims: Dims, q_abs, kv_cache, block_table, seq_lens, items, split_offsets,
                  tickets, o_part=None, lse_part=None, o_latent=None, lse=None, stream=None,
                  want_lse: bool = True):
    """decode_splitkv + combine in one launch: (o_latent [B, H, d_c], lse [B, H] or None).

    `tickets` is an int32 device tensor of 2 * B zeros; every call leaves it zero.
    """
    torch = _torch()
    dt = _store_dtype(dims)
    B, H = q_abs.shape[0], dims.n_heads
    W = items.shape[0]
    dev = q_abs.device
    if o_part is None:
        o_part = torch.empty((W, H, dims.d_latent), dtype=torch.float32, device=dev)
    if lse_part is None:
        lse_part = torch.empty((W, H), dtype=torch.float32, device=dev)
    if o_latent is None:
        o_latent = torch.empty((B, H, dims.d_latent), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    num_pages = kv_cache.shape[0]
    _debug_paging(dims, block_table, seq_lens, num_pages, 1, stream, "mla_decode_merged")
    _launch("mla_decode_merged",
        ctypes.byref(dims.c()), B, _ptr(q_abs, dt, (B, H, dims.row), "q_abs"),
        _ptr(kv_cache, dt, (num_pages, dims.page_size, dims.row), "kv_cache"), num_pages,
        _ptr(block_table, torch.int32, None, "block_table"), block_table.shape[1],
        _ptr(seq_lens, torch.int32, (B,), "seq_lens"), _ptr(items, torch.int32, (W, 4), "items"), W,
        _ptr(split_offsets, torch.int32, (B + 1,), "split_offsets"),
        _ptr(o_part, torch.float32, (W, H, dims.d_latent), "o_part"),
        _ptr(lse_part, torch.float32, (W, H), "lse_part"),
        _ptr(tickets, torch.int32, (2 * B,), "tickets"),
        _ptr(o_latent, torch.float32, (B, H, dims.d_latent), "o_latent"),
        _ptr(lse, torch.float32, (B, H), "lse"), _stream(stream))
    return o_latent, lse


def append_kv(dims: Dims, h, w_dkv, w_kr, positions, kv_cache, block_table, rms_norm: bool = True,
              eps: float = 1e-6, workspace=None, stream=None):
    """Write each sequence's new token row [c^KV | RoPE(k^R)] into the paged cache (in place)."""
    torch = _torch()
    dt = _store_dtype(dims)
    B, d_model = h.shape
    L = load()
    need = L.mla_append_kv_workspace_bytes(ctypes.byref(dims.c()), d_model, B)
    if need < 0:
        raise MlaError(-1, "mla_append_kv_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(need // 4, dtype=torch.float32, device=h.device)
    num_pages = kv_cache.shape[0]
    _check(L.mla_append_kv(
        ctypes.byref(dims.c()), d_model, B, _ptr(h, dt, (B, d_model), "h"),
        _ptr(w_dkv, dt, (dims.d_latent, d_model), "w_dkv"), _ptr(w_kr, dt, (dims.d_rope, d_model), "w_kr"),
        _ptr(positions, torch.int32, (B,), "positions"), int(bool(rms_norm)), float(eps),
        _ptr(kv_cache, dt, (num_pages, dims.page_size, dims.row), "kv_cache"), num_pages,
        _ptr(block_table, torch.int32, None, "block_table"), block_table.shape[1],
        _ptr(workspace, None, None, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream)), "mla_append_kv")
    return kv_cache


def append_kv_noalloc(dims: Dims, h, w_dkv, w_kr, positions, kv_cache, block_table,
                      rms_norm: bool = True, eps: float = 1e-6, stream=None):
    """append_kv with the partial sums in the library's static device buffer
    (no workspace; nothing allocated).  Calls that overlap on one device race."""
    torch = _torch()
    dt = _store_dtype(dims)
    B, d_model = h.shape
    L = load()
    need = L.mla_append_kv_workspace_bytes(ctypes.byref(dims.c()), d_model, B)
    cap = L.mla_append_kv_noalloc_max_bytes()
    if need > cap:
        raise MlaError(-3, f"mla_append_kv_noalloc: {B} tokens at d_model {d_model} need {need} "
                           f"bytes of scratch, the static buffer holds {cap}")
    num_pages = kv_cache.shape[0]
    _check(L.mla_append_kv_noalloc(
        ctypes.byref(dims.c()), d_model, B, _ptr(h, dt, (B, d_model), "h"),
        _ptr(w_dkv, dt, (dims.d_latent, d_model), "w_dkv"), _ptr(w_kr, dt, (dims.d_rope, d_model), "w_kr"),
        _ptr(positions, torch.int32, (B,), "positions"), int(bool(rms_norm)), float(eps),
        _ptr(kv_cache, dt, (num_pages, dims.page_size, dims.row), "kv_cache"), num_pages,
        _ptr(block_table, torch.int32, None, "block_table"), block_table.shape[1],
        _stream(stream)), "mla_append_kv_noalloc")
    return kv_cache


def out_proj(dims: Dims, o_latent, w_uv, out=None, stream=None):
    """out[b][i] = W^UV_i o_latent[b][i], float32 [B, H, d_h]."""
    torch = _torch()
    B, H = o_latent.shape[0], dims.n_heads
    dt = _store_dtype(dims)
    if out is None:
        out = torch.empty((B, H, dims.d_head), dtype=torch.float32, device=o_latent.device)
    _launch("mla_out_proj",
        ctypes.byref(dims.c()), B, _ptr(o_latent, torch.float32, (B, H, dims.d_latent), "o_latent"),
        _ptr(w_uv, dt, (H * dims.d_head, dims.d_latent), "w_uv"),
        _ptr(out, torch.float32, (B, H, dims.d_head), "out"), _stream(stream))
    return out


def combine_out_proj(dims: Dims, split_offsets, o_part, lse_part, w_uv, batch: int, out=None,
                     o_latent=None, lse=None, stream=None):
    """combine (or combine_multi) and out_proj in one launch.

    o_part [W, H, d_c] (one query token) or [W, T, H, d_c]; returns out
    [B, H, d_h] or [B, T, H, d_h].  o_latent and lse are written only when
    given (on shapes off the fast path o_latent is required).
    """
    torch = _torch()
    H = dims.n_heads
    dt = _store_dtype(dims)
    multi = o_part.dim() == 4
    W = o_part.shape[0]
    T = o_part.shape[1] if multi else 1
    lead = (batch, T) if multi else (batch,)
    if out is None:
        out = torch.empty((*lead, H, dims.d_head), dtype=torch.float32, device=o_part.device)
    _launch("mla_combine_out_proj",
        ctypes.byref(dims.c()), batch, T,
        _ptr(split_offsets, torch.int32, (batch + 1,), "split_offsets"),
        _ptr(o_part, torch.float32, (W, *lead[1:], H, dims.d_latent), "o_part"),
        _ptr(lse_part, torch.float32, (W, *lead[1:], H), "lse_part"),
        _ptr(w_uv, dt, (H * dims.d_head, dims.d_latent), "w_uv"),
        _ptr(out, torch.float32, (*lead, H, dims.d_head), "out"),
        _ptr(o_latent, torch.float32, (*lead, H, dims.d_latent), "o_latent"),
        _ptr(lse, torch.float32, (*lead, H), "lse"), _stream(stream))
    return out


def prefill_naive(dims: Dims, q_nope, q_pe, w_uk, w_uv, kv_cache, block_table, seq_lens,
                  out=None, lse=None, workspace=None, stream=None, want_lse: bool = True):
    """Prefill of the q_len newest tokens of each sequence through the materialised
    K/V path: q_nope [B, T, H, d_h], q_pe [B, T, H, d_r] (not yet rotated) ->
    (out [B, T, H, d_h] float32, lse [B, T, H] float32 or None)."""
    torch = _torch()
    dt = _store_dtype(dims)
    B, T, H = q_nope.shape[0], q_nope.shape[1], dims.n_heads
    dev = q_nope.device
    max_pages = block_table.shape[1]
    L = load()
    need = L.mla_prefill_workspace_bytes(ctypes.byref(dims.c()), B, max_pages)
    if need < 0:
        raise MlaError(-2, "mla_prefill_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(need // 2, dtype=torch.int16, device=dev)
    if out is None:
        out = torch.empty((B, T, H, dims.d_head), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    num_pages = kv_cache.shape[0]
    _debug_paging(dims, block_table, seq_lens, num_pages, T, stream, "mla_prefill_naive")
    _check(L.mla_prefill_naive(
        ctypes.byref(dims.c()), B, T, _ptr(q_nope, dt, (B, T, H, dims.d_head), "q_nope"),
        _ptr(q_pe, dt, (B, T, H, dims.d_rope), "q_pe"),
        _ptr(w_uk, dt, (H * dims.d_head, dims.d_latent), "w_uk"),
        _ptr(w_uv, dt, (H * dims.d_head, dims.d_latent), "w_uv"),
        _ptr(kv_cache, dt, (num_pages, dims.page_size, dims.row), "kv_cache"), num_pages,
        _ptr(block_table, torch.int32, None, "block_table"), max_pages,
        _ptr(seq_lens, torch.int32, (B,), "seq_lens"),
        _ptr(workspace, None, None, "workspace"), workspace.numel() * workspace.element_size(),
        _ptr(out, torch.float32, (B, T, H, dims.d_head), "out"),
        _ptr(lse, torch.float32, (B, T, H), "lse"), _stream(stream)), "mla_prefill_naive")
    return out, lse


def decode_step(dims: Dims, q_nope, q_pe, positions, w_uk, w_uv, kv_cache, block_table, seq_lens,
                items, split_offsets, bufs: Optional[dict] = None, stream=None, order=None) -> dict:
    """absorb_q -> decode_splitkv -> combine -> out_proj on one stream.

    `items`/`split_offsets` (and `order`, for plan_splits(..., ordered=True))
    are device copies of plan_splits' output.  `bufs` may hold preallocated
    q_abs, o_part, lse_part, o_latent, lse, out tensors.
    """
    b = {} if bufs is None else bufs
    B = q_nope.shape[0]
    b["q_abs"] = absorb_q(dims, q_nope, q_pe, positions, w_uk, b.get("q_abs"), stream)
    b["o_part"], b["lse_part"] = decode_splitkv(dims, b["q_abs"], kv_cache, block_table, seq_lens,
                                                items, b.get("o_part"), b.get("lse_part"), stream,
                                                order=order)
    b["o_latent"], b["lse"] = combine(dims, split_offsets, b["o_part"], b["lse_part"], B,
                                      b.get("o_latent"), b.get("lse"), stream)
    b["out"] = out_proj(dims, b["o_latent"], w_uv, b.get("out"), stream)
    return b
