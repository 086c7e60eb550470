"""Python binding of librkv.so (position-split decode attention for MI355X).

Argument marshalling only: every step runs in the library's HIP kernels.
The functions carry the names of the C entry points in include/rkv.h and
take torch tensors (device memory, or pinned host memory for streamed
tails) plus an optional torch stream.  There is no fallback: if the library
is not built, importing a function raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("RKV_LIB") or os.path.join(_HERE, "librkv.so")

RKV_F32, RKV_F16, RKV_Q8_0, RKV_Q4_0, RKV_TBQ3 = 0, 1, 2, 3, 4
RKV_OK, RKV_E_INVAL, RKV_E_UNSUPPORTED, RKV_E_HIP, RKV_E_NOMEM, RKV_E_STATE = 0, -1, -2, -3, -4, -5

# every symbol include/rkv.h declares
EXPORTS = (
    "rkv_status_string", "rkv_last_error", "rkv_row_bytes", "rkv_attend_workspace_bytes", "rkv_attend_segment",
    "rkv_lse_combine", "rkv_dequant_q8_0", "rkv_dequant_q4_0", "rkv_dequant_tbq3", "rkv_ring_create", "rkv_ring_destroy",
    "rkv_ring_begin_step", "rkv_stream_tail_workspace_bytes", "rkv_stream_tail", "rkv_ring_end_step",
    "rkv_ring_schedule", "rkv_attend_split", "rkv_attend_split_workspace_bytes", "rkv_append_kv",
    "rkv_plan_residency", "rkv_plan_last_error", "rkv_attend_split_partials", "rkv_attend_split_merge",
    "rkv_attend_split_noalloc",
)
# bytes of partials rkv_attend_split_noalloc can hold (RKV_NOALLOC_MAX_BYTES)
RKV_NOALLOC_MAX_BYTES = 32 << 20
RKV_RESIDENT, RKV_STREAM, RKV_QUANTIZE = 0, 1, 2
RKV_LINK_BOUND, RKV_HOST_RAM_BOUND = 0, 1


class RkvError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_status_name(code)}: {msg}")
        self.code = code


class rkv_kv_view(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("k_type", ctypes.c_int32), ("v_type", ctypes.c_int32),
        ("n_keys", ctypes.c_int64),
        ("k_pos_stride", ctypes.c_int64), ("v_pos_stride", ctypes.c_int64),
        ("k_head_stride", ctypes.c_int64), ("v_head_stride", ctypes.c_int64),
        ("k_seq_stride", ctypes.c_int64), ("v_seq_stride", ctypes.c_int64),
        ("pos0", ctypes.c_int64),
    ]


class rkv_attn_desc(ctypes.Structure):
    _fields_ = [
        ("n_seq", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("scale", ctypes.c_float), ("softcap", ctypes.c_float),
        ("q_to_kv", ctypes.POINTER(ctypes.c_int32)),
        ("q_pos", ctypes.POINTER(ctypes.c_int64)),
    ]


class rkv_residency_in(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32), ("n_kv", ctypes.c_int64), ("bytes_per_key", ctypes.c_int64),
        ("kv_budget_bytes", ctypes.c_int64), ("weights_bytes", ctypes.c_int64),
        ("vram_bw", ctypes.c_double), ("link_bw", ctypes.c_double), ("host_ram_bw", ctypes.c_double),
        ("c_engage_s", ctypes.c_double), ("compute_s_per_layer", ctypes.c_double),
        ("target_drop", ctypes.c_double), ("safety", ctypes.c_double),
    ]


class rkv_residency_plan(ctypes.Structure):
    _fields_ = [
        ("tactic", ctypes.c_int32), ("binding", ctypes.c_int32),
        ("window_keys", ctypes.c_int64), ("tail_keys", ctypes.c_int64), ("tile_keys", ctypes.c_int64),
        ("n_slots", ctypes.c_int32),
        ("bw_eff", ctypes.c_double), ("t_resident_s", ctypes.c_double), ("t_star_bytes", ctypes.c_double),
        ("drop", ctypes.c_double), ("free_zone_bytes", ctypes.c_double), ("predicted_step_s", ctypes.c_double),
        ("predicted_hidden", ctypes.c_double),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with position_split_kv_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.rkv_status_string.restype = ctypes.c_char_p
        L.rkv_status_string.argtypes = [ctypes.c_int]
        L.rkv_last_error.restype = ctypes.c_char_p
        L.rkv_last_error.argtypes = []
        L.rkv_row_bytes.restype = i64
        L.rkv_row_bytes.argtypes = [i32, i32]
        L.rkv_attend_workspace_bytes.argtypes = [ctypes.POINTER(rkv_attn_desc), ctypes.POINTER(rkv_kv_view),
                                                 ctypes.POINTER(sz)]
        L.rkv_attend_segment.argtypes = [ctypes.POINTER(rkv_attn_desc), vp, ctypes.POINTER(rkv_kv_view), vp, vp, vp,
                                         sz, vp]
        L.rkv_attend_split_workspace_bytes.argtypes = [ctypes.POINTER(rkv_attn_desc), ctypes.c_int,
                                                       ctypes.POINTER(rkv_kv_view), ctypes.POINTER(sz)]
        L.rkv_attend_split.argtypes = [ctypes.POINTER(rkv_attn_desc), vp, ctypes.c_int, ctypes.POINTER(rkv_kv_view),
                                       vp, vp, vp, sz, vp]
        L.rkv_attend_split_partials.argtypes = [ctypes.POINTER(rkv_attn_desc), vp, ctypes.c_int,
                                                ctypes.POINTER(rkv_kv_view), vp, vp, vp, sz, vp]
        L.rkv_attend_split_noalloc.argtypes = [ctypes.POINTER(rkv_attn_desc), vp, ctypes.c_int,
                                               ctypes.POINTER(rkv_kv_view), vp, vp, vp]
        L.rkv_attend_split_merge.argtypes = [ctypes.POINTER(rkv_attn_desc), ctypes.c_int, ctypes.POINTER(rkv_kv_view),
                                             vp, vp, vp, sz, vp]
        L.rkv_lse_combine.argtypes = [ctypes.c_int, ctypes.POINTER(vp), ctypes.POINTER(vp), i64, i32, vp, vp, vp]
        L.rkv_dequant_q8_0.argtypes = [vp, i64, vp, vp]
        L.rkv_dequant_q4_0.argtypes = [vp, i64, vp, vp]
        L.rkv_dequant_tbq3.argtypes = [vp, i64, vp, vp]
        L.rkv_ring_create.argtypes = [ctypes.c_int, sz, sz, vp, ctypes.POINTER(vp)]
        L.rkv_ring_destroy.argtypes = [vp]
        L.rkv_ring_begin_step.argtypes = [vp, ctypes.c_int, ctypes.POINTER(rkv_kv_view), i64]
        L.rkv_stream_tail_workspace_bytes.argtypes = [vp, ctypes.c_int, ctypes.POINTER(rkv_attn_desc),
                                                      ctypes.POINTER(sz)]
        L.rkv_stream_tail.argtypes = [vp, ctypes.c_int, ctypes.POINTER(rkv_attn_desc), vp, vp, vp, vp, vp, vp, sz, vp]
        L.rkv_ring_end_step.argtypes = [vp]
        L.rkv_append_kv.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, i64, ctypes.c_int, vp, vp,
                                    ctypes.POINTER(rkv_kv_view), ctypes.POINTER(rkv_kv_view),
                                    ctypes.POINTER(rkv_kv_view), vp, ctypes.c_int, vp]
        L.rkv_plan_residency.argtypes = [ctypes.POINTER(rkv_residency_in), ctypes.POINTER(rkv_residency_plan)]
        L.rkv_plan_last_error.restype = ctypes.c_char_p
        L.rkv_plan_last_error.argtypes = []
        L.rkv_ring_schedule.restype = i64
        L.rkv_ring_schedule.argtypes = [ctypes.c_int, ctypes.POINTER(i64), ctypes.c_int, i64, vp, vp, vp, vp]
        for name in EXPORTS:
            if name not in ("rkv_status_string", "rkv_last_error", "rkv_row_bytes", "rkv_ring_schedule",
                            "rkv_plan_last_error"):
                getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _status_name(code: int) -> str:
    try:
        return lib().rkv_status_string(code).decode()
    except Exception:
        return str(code)


def _check(code: int) -> None:
    if code != RKV_OK:
        raise RkvError(code, lib().rkv_last_error().decode())


# The current device's current stream as a raw handle. torch's private
# accessors skip building a Stream object (≈ 2.8 µs per call through
# torch.cuda.current_stream(), more than the library's own checks and launch
# preparation for a one-token append); the public route stays the fallback.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_cur_dev = getattr(torch._C, "_cuda_getDevice", None)


def _stream(stream) -> int | None:
    if stream is None:
        if _raw_stream is not None and _cur_dev is not None:
            return _raw_stream(_cur_dev())
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _addr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def row_bytes(dtype: int, head_dim: int) -> int:
    return lib().rkv_row_bytes(dtype, head_dim)


def make_view(k, v, k_type: int, v_type: int, n_keys: int, k_pos_stride: int, v_pos_stride: int,
              k_head_stride: int, v_head_stride: int, k_seq_stride: int = 0, v_seq_stride: int = 0,
              pos0: int = 0) -> rkv_kv_view:
    """A segment view; k / v are tensors or raw addresses (bytes); pos0 is the
    absolute position of its first key (used by masked calls)."""
    return rkv_kv_view(_addr(k), _addr(v), k_type, v_type, n_keys, k_pos_stride, v_pos_stride,
                       k_head_stride, v_head_stride, k_seq_stride, v_seq_stride, pos0)


class Desc:
    """rkv_attn_desc plus the storage of its head map."""

    def __init__(self, n_seq: int, n_q_heads: int, n_kv_heads: int, head_dim: int, scale: float,
                 softcap: float = 0.0, q_to_kv=None, q_pos=None):
        self._map = self._pos = None
        mp = pp = None
        if q_to_kv is not None:
            self._map = (ctypes.c_int32 * n_q_heads)(*[int(x) for x in q_to_kv])
            mp = ctypes.cast(self._map, ctypes.POINTER(ctypes.c_int32))
        if q_pos is not None:
            self._pos = (ctypes.c_int64 * n_seq)(*[int(x) for x in q_pos])
            pp = ctypes.cast(self._pos, ctypes.POINTER(ctypes.c_int64))
        self.c = rkv_attn_desc(n_seq, n_q_heads, n_kv_heads, head_dim, scale, softcap, mp, pp)

    @property
    def n_rows(self) -> int:
        return self.c.n_seq * self.c.n_q_heads


def rkv_attend_workspace_bytes(desc: Desc, seg: rkv_kv_view) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().rkv_attend_workspace_bytes(ctypes.byref(desc.c), ctypes.byref(seg), ctypes.byref(out)))
    return out.value


def rkv_attend_segment(desc: Desc, q: torch.Tensor, seg: rkv_kv_view, o: torch.Tensor, lse: torch.Tensor,
                       ws: torch.Tensor | None, stream=None) -> None:
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().rkv_attend_segment(ctypes.byref(desc.c), _addr(q), ctypes.byref(seg), _addr(o), _addr(lse),
                                    _addr(ws), ws_bytes, _stream(stream)))


def _segs(segs):
    arr = (rkv_kv_view * len(segs))(*segs)
    return arr


def rkv_attend_split_workspace_bytes(desc: Desc, segs) -> int:
    out = ctypes.c_size_t(0)
    arr = _segs(segs)
    _check(lib().rkv_attend_split_workspace_bytes(ctypes.byref(desc.c), len(segs), arr, ctypes.byref(out)))
    return out.value


def rkv_attend_split(desc: Desc, q: torch.Tensor, segs, o: torch.Tensor, lse: torch.Tensor,
                     ws: torch.Tensor | None, stream=None) -> None:
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    arr = _segs(segs)
    _check(lib().rkv_attend_split(ctypes.byref(desc.c), _addr(q), len(segs), arr, _addr(o), _addr(lse), _addr(ws),
                                  ws_bytes, _stream(stream)))


def rkv_attend_split_noalloc(desc: Desc, q: torch.Tensor, segs, o: torch.Tensor, lse: torch.Tensor,
                             stream=None) -> None:
    _check(lib().rkv_attend_split_noalloc(ctypes.byref(desc.c), _addr(q), len(segs), _segs(segs), _addr(o),
                                          _addr(lse), _stream(stream)))


def rkv_attend_split_partials(desc: Desc, q: torch.Tensor, segs, o: torch.Tensor, lse: torch.Tensor,
                              ws: torch.Tensor | None, stream=None) -> None:
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().rkv_attend_split_partials(ctypes.byref(desc.c), _addr(q), len(segs), _segs(segs), _addr(o),
                                           _addr(lse), _addr(ws), ws_bytes, _stream(stream)))


def rkv_attend_split_merge(desc: Desc, segs, o: torch.Tensor, lse: torch.Tensor, ws: torch.Tensor | None,
                           stream=None) -> None:
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().rkv_attend_split_merge(ctypes.byref(desc.c), len(segs), _segs(segs), _addr(o), _addr(lse),
                                        _addr(ws), ws_bytes, _stream(stream)))


def rkv_lse_combine(o_parts, lse_parts, o_out: torch.Tensor, lse_out: torch.Tensor, head_dim: int,
                    stream=None) -> None:
    n = len(o_parts)
    op = (ctypes.c_void_p * n)(*[_addr(t) for t in o_parts])
    lp = (ctypes.c_void_p * n)(*[_addr(t) for t in lse_parts])
    n_rows = lse_out.numel()
    _check(lib().rkv_lse_combine(n, op, lp, n_rows, head_dim, _addr(o_out), _addr(lse_out), _stream(stream)))


def rkv_dequant_q8_0(blocks: torch.Tensor, n_values: int, out: torch.Tensor, stream=None) -> None:
    _check(lib().rkv_dequant_q8_0(_addr(blocks), n_values, _addr(out), _stream(stream)))


def rkv_dequant_q4_0(blocks: torch.Tensor, n_values: int, out: torch.Tensor, stream=None) -> None:
    _check(lib().rkv_dequant_q4_0(_addr(blocks), n_values, _addr(out), _stream(stream)))


def rkv_dequant_tbq3(blocks: torch.Tensor, n_values: int, out: torch.Tensor, stream=None) -> None:
    _check(lib().rkv_dequant_tbq3(_addr(blocks), n_values, _addr(out), _stream(stream)))


def rkv_ring_schedule(tiles_per_layer, n_slots: int):
    """Pure host schedule: lists (layer, tile, slot, waits_on) per item."""
    n = len(tiles_per_layer)
    tl = (ctypes.c_int64 * max(1, n))(*tiles_per_layer)
    total = sum(tiles_per_layer)
    lay = (ctypes.c_int32 * max(1, total))()
    til = (ctypes.c_int64 * max(1, total))()
    slo = (ctypes.c_int32 * max(1, total))()
    wai = (ctypes.c_int64 * max(1, total))()
    got = lib().rkv_ring_schedule(n, tl, n_slots, total, lay, til, slo, wai)
    if got < 0:
        raise RkvError(int(got), lib().rkv_last_error().decode())
    return [(lay[j], til[j], slo[j], wai[j]) for j in range(got)]


class Ring:
    """rkv_ring_* lifecycle: a B-slot device staging ring on a copy stream."""

    def __init__(self, n_slots: int, slot_k_bytes: int, slot_v_bytes: int, copy_stream=None):
        h = ctypes.c_void_p(0)
        cs = None if copy_stream is None else _stream(copy_stream)
        _check(lib().rkv_ring_create(n_slots, slot_k_bytes, slot_v_bytes, cs, ctypes.byref(h)))
        self.h = h
        self._tails = None

    def close(self) -> None:
        if self.h:
            _check(lib().rkv_ring_destroy(self.h))
            self.h = ctypes.c_void_p(0)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def rkv_ring_begin_step(self, tails, tile_keys: int) -> None:
        """tails: one view per layer, in pinned host memory (streamed) or in
        device memory (attended in place)."""
        arr = (rkv_kv_view * max(1, len(tails)))(*tails)
        self._tails = arr
        _check(lib().rkv_ring_begin_step(self.h, len(tails), arr, tile_keys))

    def rkv_stream_tail_workspace_bytes(self, layer: int, desc: Desc) -> int:
        out = ctypes.c_size_t(0)
        _check(lib().rkv_stream_tail_workspace_bytes(self.h, layer, ctypes.byref(desc.c), ctypes.byref(out)))
        return out.value

    def rkv_stream_tail(self, layer: int, desc: Desc, q, o_window, lse_window, o, lse, ws: torch.Tensor,
                        stream=None) -> None:
        ws_bytes = ws.numel() * ws.element_size()
        _check(lib().rkv_stream_tail(self.h, layer, ctypes.byref(desc.c), _addr(q), _addr(o_window),
                                     _addr(lse_window), _addr(o), _addr(lse), _addr(ws), ws_bytes,
                                     _stream(stream)))

    def rkv_ring_end_step(self) -> None:
        _check(lib().rkv_ring_end_step(self.h))


def rkv_append_kv(n_kv_heads: int, head_dim: int, n_tokens: int, pos0: int, seq: int, k_new: torch.Tensor,
                  v_new: torch.Tensor, window: rkv_kv_view | None, tail: rkv_kv_view | None,
                  fresh: rkv_kv_view | None = None, ring: "Ring | None" = None, layer: int = 0, stream=None) -> None:
    """Store n_tokens new K / V rows (binary32 [n_tokens][n_kv_heads][head_dim]
    on the device) at positions pos0.. of a layer's window / tail."""
    ref = lambda v: None if v is None else ctypes.byref(v)
    _check(lib().rkv_append_kv(n_kv_heads, head_dim, n_tokens, pos0, seq, _addr(k_new), _addr(v_new), ref(window),
                               ref(tail), ref(fresh), None if ring is None else ring.h, layer, _stream(stream)))


def view_of_cache(kc, vc, start: int = 0, stop: int | None = None, k_seq_stride: int = 0,
                  v_seq_stride: int = 0, pos0: int | None = None) -> rkv_kv_view:
    """View of positions [start, stop) of a pair of position-major caches
    (objects with .data, .dtype, .pos_stride, .head_stride, .n_keys); its
    first key sits at absolute position pos0 (default: start)."""
    stop = kc.n_keys if stop is None else stop
    return make_view(kc.data.data_ptr() + start * kc.pos_stride, vc.data.data_ptr() + start * vc.pos_stride,
                     kc.dtype, vc.dtype, stop - start, kc.pos_stride, vc.pos_stride, kc.head_stride,
                     vc.head_stride, k_seq_stride, v_seq_stride, start if pos0 is None else pos0)


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A device workspace of at least nbytes (torch allocations are 256-byte aligned)."""
    return torch.empty(max(16, nbytes), dtype=torch.uint8, device=device)


def attend_split(desc: Desc, q: torch.Tensor, segs, stream=None, ws: torch.Tensor | None = None):
    """Allocate outputs (and workspace if none given) and run rkv_attend_split."""
    S, Hq, D = desc.c.n_seq, desc.c.n_q_heads, desc.c.head_dim
    o = torch.empty(S, Hq, D, dtype=torch.float32, device=q.device)
    lse = torch.empty(S, Hq, dtype=torch.float32, device=q.device)
    if ws is None:
        ws = workspace(rkv_attend_split_workspace_bytes(desc, segs), q.device)
    rkv_attend_split(desc, q, segs, o, lse, ws, stream)
    return o, lse


def attend(desc: Desc, q: torch.Tensor, seg: rkv_kv_view, stream=None, ws: torch.Tensor | None = None):
    """Allocate outputs (and workspace if none given) and run rkv_attend_segment."""
    S, Hq, D = desc.c.n_seq, desc.c.n_q_heads, desc.c.head_dim
    o = torch.empty(S, Hq, D, dtype=torch.float32, device=q.device)
    lse = torch.empty(S, Hq, dtype=torch.float32, device=q.device)
    if ws is None:
        ws = workspace(rkv_attend_workspace_bytes(desc, seg), q.device)
    rkv_attend_segment(desc, q, seg, o, lse, ws, stream)
    return o, lse


def rkv_plan_residency(n_layers: int, n_kv: int, bytes_per_key: int, kv_budget_bytes: int, weights_bytes: int,
                       vram_bw: float, link_bw: float, host_ram_bw: float, c_engage_s: float,
                       compute_s_per_layer: float, target_drop: float = 0.20, safety: float = 0.8) -> dict:
    """The residency plan (host arithmetic, no GPU) as a dict of the
    rkv_residency_plan fields."""
    i = rkv_residency_in(n_layers, n_kv, bytes_per_key, kv_budget_bytes, weights_bytes, vram_bw, link_bw,
                         host_ram_bw, c_engage_s, compute_s_per_layer, target_drop, safety)
    o = rkv_residency_plan()
    code = lib().rkv_plan_residency(ctypes.byref(i), ctypes.byref(o))
    if code != RKV_OK:
        raise RkvError(code, lib().rkv_plan_last_error().decode())
    return {name: getattr(o, name) for name, _ in rkv_residency_plan._fields_}
