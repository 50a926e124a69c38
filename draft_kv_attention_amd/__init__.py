"""Python binding of libmasw.so (MASW draft attention on MI355X / gfx950).

Argument marshalling only: every function below checks tensor devices, dtypes, shapes
and contiguity, builds the C structs of include/masw.h and calls the entry point of
the same name on the current HIP stream.  Every step of the computation runs in the
library's HIP kernels; there is no fallback.  Importing works without a GPU; calling
an entry point without the built library raises ``MaswLibraryMissing``.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmasw.so")

MASW_OK = 0
STATUS = {0: "MASW_OK", -1: "MASW_ERR_ARG", -2: "MASW_ERR_DTYPE", -3: "MASW_ERR_SHAPE",
          -4: "MASW_ERR_WORKSPACE", -5: "MASW_ERR_LAUNCH", -6: "MASW_ERR_UNIMPLEMENTED"}
DEV_PENDING_SLOT = 1
DEV_SLOT_CAPACITY = 2
DEV_SEQ_RANGE = 4
DEV_SLOT_MISSING = 8

OP_DRAFT_ATTN, OP_MATERIALIZE, OP_FULLKV_DECODE, OP_FULLKV_VERIFY = 0, 1, 2, 3
F32, BF16 = 0, 1
ROPE_ROTATE_HALF, ROPE_INTERLEAVED = 0, 1
_DTYPES = {torch.float32: F32, torch.bfloat16: BF16}


class MaswLibraryMissing(RuntimeError):
    pass


class MaswError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {status} ({STATUS.get(status, '?')})")
        self.status = status


class _Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("sink", ctypes.c_int32), ("window", ctypes.c_int32),
                ("interval", ctypes.c_int32), ("max_slots", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("scale", ctypes.c_float),
                ("num_splits", ctypes.c_int32), ("rollback", ctypes.c_int32),
                ("rope_theta", ctypes.c_float), ("rope_style", ctypes.c_int32)]


class _Layer(ctypes.Structure):
    _fields_ = [("k_sink", ctypes.c_void_p), ("v_sink", ctypes.c_void_p),
                ("k_ring", ctypes.c_void_p), ("v_ring", ctypes.c_void_p),
                ("k_slot", ctypes.c_void_p), ("v_slot", ctypes.c_void_p),
                ("n_slots", ctypes.c_void_p)]


class _Seq(ctypes.Structure):
    _fields_ = [("seq_len", ctypes.c_void_p), ("err", ctypes.c_void_p)]


_P = ctypes.c_void_p
_SIGS = {
    "masw_evict_append": (ctypes.c_int, [_P, _P, _P, _P, _P, ctypes.c_int32, _P]),
    "masw_materialize_slot": (ctypes.c_int, [_P, _P, _P, ctypes.c_int32, _P, _P, _P, _P, _P,
                                             ctypes.c_int32, _P, ctypes.c_size_t, _P]),
    "masw_draft_attn": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "fullkv_decode_attn": (ctypes.c_int, [_P, _P, _P, ctypes.c_int32, _P, _P, _P, _P, _P,
                                          ctypes.c_size_t, _P]),
    "fullkv_append": (ctypes.c_int, [_P, _P, _P, ctypes.c_int32, _P, _P, _P, _P,
                                     ctypes.c_int32, _P]),
    "masw_decode_step": (ctypes.c_int, [_P, _P, _P, _P, _P, ctypes.c_int32, _P, _P, _P,
                                        ctypes.c_size_t, _P]),
    "masw_decode_step_static": (ctypes.c_int, [_P, _P, _P, _P, _P, ctypes.c_int32, _P, _P, _P]),
    "fullkv_decode_step": (ctypes.c_int, [_P, _P, _P, ctypes.c_int32, _P, _P, _P, _P,
                                          ctypes.c_int32, _P, _P, _P, ctypes.c_size_t, _P]),
    "fullkv_verify_attn": (ctypes.c_int, [_P, _P, _P, ctypes.c_int32, _P, _P, ctypes.c_int32,
                                          _P, _P, _P, ctypes.c_size_t, _P]),
    "masw_workspace_bytes": (ctypes.c_size_t, [_P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]),
    "masw_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "masw_abi_version": (ctypes.c_int, []),
    "masw_debug_keylist": (ctypes.c_int, [_P, _P, ctypes.c_int32, _P, ctypes.c_int32, _P]),
    "masw_stream_read": (ctypes.c_int, [_P, ctypes.c_size_t, ctypes.c_int32, _P, _P]),
    "masw_rollback": (ctypes.c_int, [_P, _P, _P, _P, _P]),
    "masw_mfma_rate": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, _P, _P, _P]),
    "masw_prefill": (ctypes.c_int, [_P, _P, _P, ctypes.c_int32, _P, _P, _P, _P, ctypes.c_int32,
                                    ctypes.c_int32, _P, _P, _P, _P, _P, _P]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libmasw.so (raises MaswLibraryMissing when it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MaswLibraryMissing(
                f"{LIB_PATH} not found: build it with `python -m draft_kv_attention_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


# ---------------------------------------------------------------------------
# Plain-Python descriptions of the C structs
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Dims:
    """Mirror of masw_dims (see include/masw.h)."""
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    sink: int = 0
    window: int = 1
    interval: int = 1
    max_slots: int = 0
    dtype: torch.dtype = torch.bfloat16
    scale: float = 0.0
    num_splits: int = 0
    rollback: int = 0
    rope_theta: float = 0.0   # > 0: slot keys rotated to their position id (include/masw.h)
    rope_style: int = 0       # ROPE_ROTATE_HALF or ROPE_INTERLEAVED

    def c(self) -> _Dims:
        return _Dims(self.batch, self.n_q_heads, self.n_kv_heads, self.head_dim, self.sink,
                     self.window, self.interval, self.max_slots, _DTYPES[self.dtype],
                     float(self.scale), self.num_splits, self.rollback, float(self.rope_theta),
                     int(self.rope_style))

    @property
    def ring(self) -> int:
        return self.window + self.interval + self.rollback

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale > 0 else 1.0 / math.sqrt(self.head_dim)


@dataclasses.dataclass
class Layer:
    """One layer's memory tensors (device): sink, ring, slots and n_slots."""
    k_sink: torch.Tensor
    v_sink: torch.Tensor
    k_ring: torch.Tensor
    v_ring: torch.Tensor
    k_slot: torch.Tensor
    v_slot: torch.Tensor
    n_slots: torch.Tensor

    def c(self) -> _Layer:
        def p(t):
            return t.data_ptr() if t is not None and t.numel() else None
        return _Layer(p(self.k_sink), p(self.v_sink), p(self.k_ring), p(self.v_ring),
                      p(self.k_slot), p(self.v_slot), self.n_slots.data_ptr())


@dataclasses.dataclass
class Seq:
    seq_len: torch.Tensor   # [B] int32
    err: torch.Tensor       # [1] int32

    def c(self) -> _Seq:
        return _Seq(self.seq_len.data_ptr(), self.err.data_ptr())


def alloc_layer(d: Dims, device="cuda", fill: Optional[float] = 0.0) -> Layer:
    """Zero-filled memory of one layer (NaN-filled with fill=float('nan') for debug runs)."""
    def z(rows):
        t = torch.empty((d.batch, d.n_kv_heads, rows, d.head_dim), dtype=d.dtype, device=device)
        if fill is not None:
            t.fill_(fill)
        return t
    return Layer(z(d.sink), z(d.sink), z(d.ring), z(d.ring), z(d.max_slots), z(d.max_slots),
                 torch.zeros(d.batch, dtype=torch.int32, device=device))


def alloc_seq(batch: int, device="cuda") -> Seq:
    return Seq(torch.zeros(batch, dtype=torch.int32, device=device),
               torch.zeros(1, dtype=torch.int32, device=device))


def workspace_bytes(d: Dims, op: int, max_keys: int = 0, n_q: int = 0) -> int:
    dc = d.c()
    return int(lib().masw_workspace_bytes(ctypes.byref(dc), op, max_keys, n_q))


def workspace(d: Dims, op: int, max_keys: int = 0, n_q: int = 0, device="cuda") -> torch.Tensor:
    """Zero-filled workspace (the split tickets must start at zero; calls keep them so).
    It serves one plan: share it only between calls with equal Dims (and, for the
    full-KV ops, equal max_keys / n_q); zero it again before another plan uses it."""
    n = workspace_bytes(d, op, max_keys, n_q)
    if n == 0:
        raise MaswError("masw_workspace_bytes", -1)
    return torch.zeros(n, dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _check(t: torch.Tensor, name: str, shape, dtype):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _ok(fn: str, st: int):
    if st != MASW_OK:
        raise MaswError(fn, st)


def _ws(ws: Optional[torch.Tensor]):
    if ws is None:
        return None, 0
    return ws.data_ptr(), ws.numel() * ws.element_size()


def _check_layer(d: Dims, L: Layer):
    for nm, rows in (("k_sink", d.sink), ("v_sink", d.sink), ("k_ring", d.ring),
                     ("v_ring", d.ring), ("k_slot", d.max_slots), ("v_slot", d.max_slots)):
        _check(getattr(L, nm), nm, (d.batch, d.n_kv_heads, rows, d.head_dim), d.dtype)
    _check(L.n_slots, "n_slots", (d.batch,), torch.int32)


def _check_seq(d: Dims, s: Seq):
    _check(s.seq_len, "seq_len", (d.batch,), torch.int32)
    _check(s.err, "err", (1,), torch.int32)


def masw_evict_append(d: Dims, layer: Layer, seq: Seq, k_new: torch.Tensor, v_new: torch.Tensor,
                      stream=None) -> None:
    """Append raw tokens t-n+1..t ([B][n][Hkv][D]) with implicit eviction."""
    _check_layer(d, layer)
    _check_seq(d, seq)
    n = k_new.shape[1]
    for nm, t in (("k_new", k_new), ("v_new", v_new)):
        _check(t, nm, (d.batch, n, d.n_kv_heads, d.head_dim), d.dtype)
    dc, lc, sc = d.c(), layer.c(), seq.c()
    _ok("masw_evict_append", lib().masw_evict_append(
        ctypes.byref(dc), ctypes.byref(lc), ctypes.byref(sc), k_new.data_ptr(), v_new.data_ptr(),
        n, _stream(stream)))


def masw_materialize_slot(d: Dims, layer: Layer, seq: Seq, h: torch.Tensor, w_k_g: torch.Tensor,
                          w_v_g: torch.Tensor, q_slot: torch.Tensor, o_slot: torch.Tensor,
                          workspace: torch.Tensor, include_self: bool = False, stream=None) -> None:
    """Materialize slot g_m for every sequence whose step t is its boundary."""
    _check_layer(d, layer)
    _check_seq(d, seq)
    hidden = h.shape[1]
    _check(h, "h", (d.batch, hidden), d.dtype)
    for nm, t in (("w_k_g", w_k_g), ("w_v_g", w_v_g)):
        _check(t, nm, (hidden, d.n_kv_heads * d.head_dim), d.dtype)
    for nm, t in (("q_slot", q_slot), ("o_slot", o_slot)):
        _check(t, nm, (d.batch, d.n_q_heads, d.head_dim), d.dtype)
    wp, wb = _ws(workspace)
    dc, lc, sc = d.c(), layer.c(), seq.c()
    _ok("masw_materialize_slot", lib().masw_materialize_slot(
        ctypes.byref(dc), ctypes.byref(lc), ctypes.byref(sc), hidden, h.data_ptr(),
        w_k_g.data_ptr(), w_v_g.data_ptr(), q_slot.data_ptr(), o_slot.data_ptr(),
        1 if include_self else 0, wp, wb, _stream(stream)))


def masw_draft_attn(d: Dims, layer: Layer, seq: Seq, q: torch.Tensor, out: torch.Tensor,
                    workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Decode attention over sink ++ local ++ slots for q, out [B][Hq][D]."""
    _check_layer(d, layer)
    _check_seq(d, seq)
    for nm, t in (("q", q), ("out", out)):
        _check(t, nm, (d.batch, d.n_q_heads, d.head_dim), d.dtype)
    wp, wb = _ws(workspace)
    dc, lc, sc = d.c(), layer.c(), seq.c()
    _ok("masw_draft_attn", lib().masw_draft_attn(
        ctypes.byref(dc), ctypes.byref(lc), ctypes.byref(sc), q.data_ptr(), out.data_ptr(),
        wp, wb, _stream(stream)))


def masw_decode_step(d: Dims, layer: Layer, seq: Seq, k_new: torch.Tensor, v_new: torch.Tensor,
                     q: torch.Tensor, out: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                     stream=None) -> None:
    """Fused append of positions t-n+1..t ([B][n][Hkv][D]) and draft attention."""
    _check_layer(d, layer)
    _check_seq(d, seq)
    n = k_new.shape[1]
    for nm, t in (("k_new", k_new), ("v_new", v_new)):
        _check(t, nm, (d.batch, n, d.n_kv_heads, d.head_dim), d.dtype)
    for nm, t in (("q", q), ("out", out)):
        _check(t, nm, (d.batch, d.n_q_heads, d.head_dim), d.dtype)
    wp, wb = _ws(workspace)
    dc, lc, sc = d.c(), layer.c(), seq.c()
    _ok("masw_decode_step", lib().masw_decode_step(
        ctypes.byref(dc), ctypes.byref(lc), ctypes.byref(sc), k_new.data_ptr(), v_new.data_ptr(), n,
        q.data_ptr(), out.data_ptr(), wp, wb, _stream(stream)))


def masw_decode_step_static(d: Dims, layer: Layer, seq: Seq, k_new: torch.Tensor, v_new: torch.Tensor,
                            q: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    """masw_decode_step with the library's own fixed scratch instead of a workspace
    (allocates nothing; calls overlapping on one GPU race)."""
    _check_layer(d, layer)
    _check_seq(d, seq)
    n = k_new.shape[1]
    for nm, t in (("k_new", k_new), ("v_new", v_new)):
        _check(t, nm, (d.batch, n, d.n_kv_heads, d.head_dim), d.dtype)
    for nm, t in (("q", q), ("out", out)):
        _check(t, nm, (d.batch, d.n_q_heads, d.head_dim), d.dtype)
    dc, lc, sc = d.c(), layer.c(), seq.c()
    _ok("masw_decode_step_static", lib().masw_decode_step_static(
        ctypes.byref(dc), ctypes.byref(lc), ctypes.byref(sc), k_new.data_ptr(), v_new.data_ptr(), n,
        q.data_ptr(), out.data_ptr(), _stream(stream)))


def _check_full(d: Dims, k, v, seq_len, err):
    max_len = k.shape[2]
    for nm, t in (("k", k), ("v", v)):
        _check(t, nm, (d.batch, d.n_kv_heads, max_len, d.head_dim), d.dtype)
    _check(seq_len, "seq_len", (d.batch,), torch.int32)
    _check(err, "err", (1,), torch.int32)
    return max_len


def fullkv_decode_attn(d: Dims, k: torch.Tensor, v: torch.Tensor, seq_len: torch.Tensor,
                       err: torch.Tensor, q: torch.Tensor, out: torch.Tensor,
                       workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Decode attention over the full cache rows 0..t-1 (k, v [B][Hkv][max_len][D])."""
    max_len = _check_full(d, k, v, seq_len, err)
    for nm, t in (("q", q), ("out", out)):
        _check(t, nm, (d.batch, d.n_q_heads, d.head_dim), d.dtype)
    wp, wb = _ws(workspace)
    dc = d.c()
    _ok("fullkv_decode_attn", lib().fullkv_decode_attn(
        ctypes.byref(dc), k.data_ptr(), v.data_ptr(), max_len, seq_len.data_ptr(), err.data_ptr(),
        q.data_ptr(), out.data_ptr(), wp, wb, _stream(stream)))


def fullkv_append(d: Dims, k: torch.Tensor, v: torch.Tensor, seq_len: torch.Tensor,
                  err: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, stream=None) -> None:
    """Write positions t-n+1..t into rows t-n..t-1 of a full cache."""
    max_len = _check_full(d, k, v, seq_len, err)
    n = k_new.shape[1]
    for nm, t in (("k_new", k_new), ("v_new", v_new)):
        _check(t, nm, (d.batch, n, d.n_kv_heads, d.head_dim), d.dtype)
    dc = d.c()
    _ok("fullkv_append", lib().fullkv_append(
        ctypes.byref(dc), k.data_ptr(), v.data_ptr(), max_len, seq_len.data_ptr(), err.data_ptr(),
        k_new.data_ptr(), v_new.data_ptr(), n, _stream(stream)))


def fullkv_decode_step(d: Dims, k: torch.Tensor, v: torch.Tensor, seq_len: torch.Tensor,
                       err: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                       out: torch.Tensor, workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Fused full-cache append of positions t-n+1..t and decode attention."""
    max_len = _check_full(d, k, v, seq_len, err)
    n = k_new.shape[1]
    for nm, t in (("k_new", k_new), ("v_new", v_new)):
        _check(t, nm, (d.batch, n, d.n_kv_heads, d.head_dim), d.dtype)
    for nm, t in (("q", q), ("out", out)):
        _check(t, nm, (d.batch, d.n_q_heads, d.head_dim), d.dtype)
    wp, wb = _ws(workspace)
    dc = d.c()
    _ok("fullkv_decode_step", lib().fullkv_decode_step(
        ctypes.byref(dc), k.data_ptr(), v.data_ptr(), max_len, seq_len.data_ptr(), err.data_ptr(),
        k_new.data_ptr(), v_new.data_ptr(), n, q.data_ptr(), out.data_ptr(), wp, wb, _stream(stream)))


def fullkv_verify_attn(d: Dims, k: torch.Tensor, v: torch.Tensor, seq_len: torch.Tensor,
                       err: torch.Tensor, q: torch.Tensor, out: torch.Tensor,
                       workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Verifier attention for q, out [B][n_q][Hq][D]; query j sees keys 1..t-n_q+1+j."""
    max_len = _check_full(d, k, v, seq_len, err)
    n_q = q.shape[1]
    for nm, t in (("q", q), ("out", out)):
        _check(t, nm, (d.batch, n_q, d.n_q_heads, d.head_dim), d.dtype)
    wp, wb = _ws(workspace)
    dc = d.c()
    _ok("fullkv_verify_attn", lib().fullkv_verify_attn(
        ctypes.byref(dc), k.data_ptr(), v.data_ptr(), max_len, seq_len.data_ptr(), err.data_ptr(),
        n_q, q.data_ptr(), out.data_ptr(), wp, wb, _stream(stream)))


def masw_debug_keylist(d: Dims, seq: Seq, back: int = 0, max_keys: Optional[int] = None,
                       stream=None) -> torch.Tensor:
    """Device key resolver dump: [B][max_keys][3] = (segment, row, id), -1 padded."""
    _check_seq(d, seq)
    if max_keys is None:
        max_keys = d.sink + d.window + d.max_slots + 1
    out = torch.empty((d.batch, max_keys, 3), dtype=torch.int32, device=seq.seq_len.device)
    dc, sc = d.c(), seq.c()
    _ok("masw_debug_keylist", lib().masw_debug_keylist(
        ctypes.byref(dc), ctypes.byref(sc), back, out.data_ptr(), max_keys, _stream(stream)))
    return out


STREAM_SUMS = 256   # MASW_STREAM_SUMS


def masw_rollback(d: Dims, layer: Layer, seq: Seq, t_spec: torch.Tensor, stream=None) -> None:
    """Undo speculation: seq.seq_len already holds the accepted lengths, t_spec [B] int32
    the lengths the memory reached while drafting (see include/masw.h)."""
    _check_seq(d, seq)
    _check(t_spec, "t_spec", (d.batch,), torch.int32)
    dc, lc, sc = d.c(), layer.c(), seq.c()
    _ok("masw_rollback", lib().masw_rollback(ctypes.byref(dc), ctypes.byref(lc), ctypes.byref(sc),
                                             t_spec.data_ptr(), _stream(stream)))


def masw_prefill(d: Dims, layer: Layer, seq: Seq, k: torch.Tensor, v: torch.Tensor,
                 q: torch.Tensor, out: torch.Tensor, h_slot: Optional[torch.Tensor] = None,
                 w_k_g: Optional[torch.Tensor] = None, w_v_g: Optional[torch.Tensor] = None,
                 q_slot: Optional[torch.Tensor] = None, o_slot: Optional[torch.Tensor] = None,
                 stream=None) -> None:
    """Draft prefill of P = seq.seq_len[b] tokens per sequence (see include/masw.h):
    k, v [B][p_max][Hkv][D], q, out [B][p_max][Hq][D]; with a slot chain also h_slot
    [B][ns_max][hidden], w_k_g, w_v_g [hidden][Hkv*D], q_slot, o_slot [B][ns_max][Hq][D]."""
    _check_layer(d, layer)
    _check_seq(d, seq)
    p_max = k.shape[1]
    for nm, t in (("k", k), ("v", v)):
        _check(t, nm, (d.batch, p_max, d.n_kv_heads, d.head_dim), d.dtype)
    for nm, t in (("q", q), ("out", out)):
        _check(t, nm, (d.batch, p_max, d.n_q_heads, d.head_dim), d.dtype)
    ns_max, hidden = 0, 0
    ptrs = [None] * 5
    if h_slot is not None:
        ns_max, hidden = h_slot.shape[1], h_slot.shape[2]
        _check(h_slot, "h_slot", (d.batch, ns_max, hidden), d.dtype)
        for nm, t in (("w_k_g", w_k_g), ("w_v_g", w_v_g)):
            if t is None:
                raise ValueError(f"{nm} is required with h_slot")
            _check(t, nm, (hidden, d.n_kv_heads * d.head_dim), d.dtype)
        for nm, t in (("q_slot", q_slot), ("o_slot", o_slot)):
            if t is None:
                raise ValueError(f"{nm} is required with h_slot")
            _check(t, nm, (d.batch, ns_max, d.n_q_heads, d.head_dim), d.dtype)
        ptrs = [h_slot.data_ptr(), w_k_g.data_ptr(), w_v_g.data_ptr(), q_slot.data_ptr(),
                o_slot.data_ptr()]
    dc, lc, sc = d.c(), layer.c(), seq.c()
    _ok("masw_prefill", lib().masw_prefill(
        ctypes.byref(dc), ctypes.byref(lc), ctypes.byref(sc), p_max, k.data_ptr(), v.data_ptr(),
        q.data_ptr(), out.data_ptr(), ns_max, hidden, *ptrs, _stream(stream)))


def stream_read(buf: torch.Tensor, sums: torch.Tensor, work_groups: int = 0, stream=None) -> None:
    """Measurement helper: adds every 32-bit word of buf (contiguous, a multiple of 16
    bytes) modulo 2^32 into sums ([STREAM_SUMS] int32 on the same device, zeroed by the
    caller); the wrapping total of sums is the wrapping sum of buf's words."""
    if not buf.is_contiguous() or buf.numel() * buf.element_size() % 16:
        raise ValueError("buf must be contiguous and a multiple of 16 bytes")
    _check(sums, "sums", (STREAM_SUMS,), torch.int32)
    _ok("masw_stream_read", lib().masw_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(),
                                                   work_groups, sums.data_ptr(), _stream(stream)))


def mfma_rate(work_groups: int, iters: int, out: torch.Tensor, clocks: torch.Tensor, stream=None) -> None:
    """Measurement helper: matrix-core rate probe (see include/masw.h).  out float32
    [work_groups * 256], clocks int64 [2] (shader-clock and 100 MHz real-time ticks of
    work-group 0's first wave), both on the device."""
    _check(out, "out", (work_groups * 256,), torch.float32)
    _check(clocks, "clocks", (2,), torch.int64)
    _ok("masw_mfma_rate", lib().masw_mfma_rate(work_groups, iters, out.data_ptr(), clocks.data_ptr(),
                                               _stream(stream)))


def status_string(st: int) -> str:
    return lib().masw_status_string(st).decode()


def abi_version() -> int:
    return int(lib().masw_abi_version())
