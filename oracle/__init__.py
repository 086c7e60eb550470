"""ctypes binding of the binary64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY.  The test-suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may use this module; the product path
(``position_split_kv_amd``) never imports it.

The oracle is plain unsplit softmax attention over the whole key set in
binary64, scalar block dequantisation, and the write path (storing binary32
rows in a cache type, routing a position to the window or the tail); see the
header of oracle.c for the passages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "oracle.c")

F32, F16, Q8_0, Q4_0, TBQ3 = 0, 1, 2, 3, 4


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (-O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
                               "-o", tmp, SRC_PATH, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


class _View(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("k_type", ctypes.c_int32), ("v_type", ctypes.c_int32),
        ("n_keys", ctypes.c_int64),
        ("k_pos_stride", ctypes.c_int64), ("v_pos_stride", ctypes.c_int64),
        ("k_head_stride", ctypes.c_int64), ("v_head_stride", ctypes.c_int64),
        ("k_seq_stride", ctypes.c_int64), ("v_seq_stride", ctypes.c_int64),
    ]


class Oracle:
    """The oracle library loaded from one built .so (the default build, or a
    deliberately mutated copy that the pin tests use to show they bite)."""

    def __init__(self, path: str):
        L = ctypes.CDLL(path)
        L.orc_f16_to_f64.restype = ctypes.c_double
        L.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_row_bytes.restype = ctypes.c_int64
        L.orc_row_bytes.argtypes = [ctypes.c_int, ctypes.c_int64]
        for name in ("orc_dequant_q8_0", "orc_dequant_q4_0"):
            f = getattr(L, name)
            f.restype = ctypes.c_int
            f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        L.orc_attend.restype = ctypes.c_int
        L.orc_attend.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_double, ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(_View),
                                 ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        L.orc_lse_combine.restype = ctypes.c_int
        L.orc_lse_combine.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_void_p),
                                      ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        L.orc_f32_to_f16.restype = ctypes.c_uint16
        L.orc_f32_to_f16.argtypes = [ctypes.c_float]
        L.orc_encode_row.restype = ctypes.c_int
        L.orc_encode_row.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        L.orc_route.restype = ctypes.c_int
        L.orc_route.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)]
        L.orc_dequant_tbq3.restype = ctypes.c_int
        L.orc_dequant_tbq3.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        L.orc_tbq3_levels.restype = None
        L.orc_tbq3_levels.argtypes = [ctypes.c_void_p]
        L.orc_tbq3_signs.restype = None
        L.orc_tbq3_signs.argtypes = [ctypes.c_void_p]
        L.orc_splitmix64.restype = None
        L.orc_splitmix64.argtypes = [ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p]
        L.orc_max_threads.restype = ctypes.c_int
        L.orc_set_threads.argtypes = [ctypes.c_int]
        self.L = L

    def f16_to_f64(self, bits: int) -> float:
        return self.L.orc_f16_to_f64(bits & 0xFFFF)

    def row_bytes(self, dtype: int, head_dim: int) -> int:
        return self.L.orc_row_bytes(dtype, head_dim)

    def dequant_q8_0(self, blocks, n_values: int) -> np.ndarray:
        out = np.empty(n_values, dtype=np.float32)
        if self.L.orc_dequant_q8_0(_ptr(blocks), n_values, out.ctypes.data) != 0:
            raise ValueError("n_values must be a multiple of 32")
        return out

    def dequant_q4_0(self, blocks, n_values: int) -> np.ndarray:
        out = np.empty(n_values, dtype=np.float32)
        if self.L.orc_dequant_q4_0(_ptr(blocks), n_values, out.ctypes.data) != 0:
            raise ValueError("n_values must be a multiple of 32")
        return out

    def dequant_tbq3(self, blocks, n_values: int) -> np.ndarray:
        """Original-space values of TBQ3 blocks (binary64 rounded to binary32)."""
        out = np.empty(n_values, dtype=np.float32)
        if self.L.orc_dequant_tbq3(_ptr(blocks), n_values, out.ctypes.data) != 0:
            raise ValueError("n_values must be a multiple of 128")
        return out

    def tbq3_levels(self) -> np.ndarray:
        """The positive half of the 8-level Lloyd-Max codebook of N(0,1)."""
        out = np.zeros(4, dtype=np.float64)
        self.L.orc_tbq3_levels(out.ctypes.data)
        return out

    def tbq3_signs(self):
        """(S1, S2): the rotation's two diagonal sign vectors (+-1, 128 each)."""
        out = np.zeros(256, dtype=np.int32)
        self.L.orc_tbq3_signs(out.ctypes.data)
        return out[:128].copy(), out[128:].copy()

    def splitmix64(self, seed: int, n: int) -> list:
        out = np.zeros(n, dtype=np.uint64)
        self.L.orc_splitmix64(seed, n, out.ctypes.data)
        return [int(x) for x in out]

    def attend(self, q, views, n_kv_heads: int, scale: float, softcap: float = 0.0, q_to_kv=None, rows=None,
               q_pos=None):
        """Unsplit binary64 attention.

        q: float32 [n_seq][n_q_heads][head_dim] (host).  views: list of View
        whose keys are attended together.  rows: optional flattened row
        indices.  q_pos: optional absolute position of each sequence's query
        (it sees keys 0 .. q_pos[b] of the concatenated views).  Returns
        (o float64 [n_rows][head_dim], lse float64 [n_rows]).
        """
        q = np.ascontiguousarray(np.asarray(q, dtype=np.float32))
        n_seq, n_q_heads, head_dim = q.shape
        arr = (_View * max(1, len(views)))(*[v.c for v in views])
        rows_arr = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n_rows = n_seq * n_q_heads if rows_arr is None else len(rows_arr)
        o = np.zeros((n_rows, head_dim), dtype=np.float64)
        lse = np.zeros(n_rows, dtype=np.float64)
        m = None
        if q_to_kv is not None:
            m = np.ascontiguousarray(np.asarray(q_to_kv, dtype=np.int32))
        qp = None
        if q_pos is not None:
            qp = np.ascontiguousarray(np.asarray(q_pos, dtype=np.int64))
            assert qp.shape == (n_seq,)
        rc = self.L.orc_attend(n_seq, n_q_heads, n_kv_heads, head_dim, float(scale), float(softcap),
                               None if m is None else m.ctypes.data, None if qp is None else qp.ctypes.data,
                               q.ctypes.data, len(views), arr,
                               None if rows_arr is None else rows_arr.ctypes.data, n_rows,
                               o.ctypes.data, lse.ctypes.data)
        if rc != 0:
            raise ValueError(f"orc_attend failed ({rc})")
        return o, lse

    def lse_combine(self, o_parts, lse_parts):
        """binary64 segment merge of normalised outputs + LSEs."""
        o_parts = [np.ascontiguousarray(np.asarray(o, dtype=np.float64)) for o in o_parts]
        lse_parts = [np.ascontiguousarray(np.asarray(x, dtype=np.float64)) for x in lse_parts]
        n_rows, head_dim = o_parts[0].shape
        op = (ctypes.c_void_p * len(o_parts))(*[o.ctypes.data for o in o_parts])
        lp = (ctypes.c_void_p * len(lse_parts))(*[x.ctypes.data for x in lse_parts])
        o = np.zeros((n_rows, head_dim), dtype=np.float64)
        lse = np.zeros(n_rows, dtype=np.float64)
        if self.L.orc_lse_combine(len(o_parts), op, lp, n_rows, head_dim, o.ctypes.data, lse.ctypes.data) != 0:
            raise ValueError("orc_lse_combine failed")
        return o, lse

    def f32_to_f16(self, x: float) -> int:
        """binary16 bits nearest (ties to even) to the binary32 value x."""
        return self.L.orc_f32_to_f16(float(np.float32(x)))

    def encode_rows(self, x, dtype: int) -> np.ndarray:
        """Store binary32 rows x [..., D] in ``dtype``: uint8 [..., row_bytes]."""
        x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
        d = x.shape[-1]
        rb = self.row_bytes(dtype, d)
        if rb == 0:
            raise ValueError("bad type or head_dim")
        flat = x.reshape(-1, d)
        out = np.zeros((flat.shape[0], rb), dtype=np.uint8)
        for i in range(flat.shape[0]):
            if self.L.orc_encode_row(dtype, flat[i].ctypes.data, d, out[i].ctypes.data) != 0:
                raise ValueError("orc_encode_row failed")
        return out.reshape(*x.shape[:-1], rb)

    def route(self, pos: int, window_cap: int, tail_cap: int):
        """("window" | "tail", row) for a new row at position pos; ValueError
        when the position fits neither region."""
        row = ctypes.c_int64(0)
        r = self.L.orc_route(pos, window_cap, tail_cap, ctypes.byref(row))
        if r < 0:
            raise ValueError(f"position {pos} outside window {window_cap} + tail {tail_cap}")
        return ("window", "tail")[r], row.value

    def max_threads(self) -> int:
        return self.L.orc_max_threads()

    def set_threads(self, n: int) -> None:
        self.L.orc_set_threads(n)


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle(build())
    return _default


def f16_to_f64(bits):
    return default().f16_to_f64(bits)


def row_bytes(dtype, head_dim):
    return default().row_bytes(dtype, head_dim)


def dequant_q8_0(blocks, n_values):
    return default().dequant_q8_0(blocks, n_values)


def dequant_q4_0(blocks, n_values):
    return default().dequant_q4_0(blocks, n_values)


def dequant_tbq3(blocks, n_values):
    return default().dequant_tbq3(blocks, n_values)


def tbq3_levels():
    return default().tbq3_levels()


def tbq3_signs():
    return default().tbq3_signs()


def splitmix64(seed, n):
    return default().splitmix64(seed, n)


def attend(q, views, n_kv_heads, scale, softcap=0.0, q_to_kv=None, rows=None, q_pos=None):
    return default().attend(q, views, n_kv_heads, scale, softcap, q_to_kv, rows, q_pos)


def lse_combine(o_parts, lse_parts):
    return default().lse_combine(o_parts, lse_parts)


def f32_to_f16(x):
    return default().f32_to_f16(x)


def encode_rows(x, dtype):
    return default().encode_rows(x, dtype)


def route(pos, window_cap, tail_cap):
    return default().route(pos, window_cap, tail_cap)


def max_threads() -> int:
    return default().max_threads()


def set_threads(n: int) -> None:
    default().set_threads(n)


def _ptr(a) -> int:
    """Address of a host buffer (numpy array or CPU torch tensor)."""
    if isinstance(a, np.ndarray):
        assert a.flags["C_CONTIGUOUS"]
        return a.ctypes.data
    if a.device.type != "cpu":
        raise ValueError("oracle inputs must be host buffers")
    assert a.is_contiguous()
    return a.data_ptr()


class View:
    """A segment: positions [0, n_keys) starting at byte addresses k / v.

    ``keep`` holds references to the buffers the addresses point into.
    """

    def __init__(self, k_addr, v_addr, k_type, v_type, n_keys, k_pos_stride, v_pos_stride,
                 k_head_stride, v_head_stride, k_seq_stride=0, v_seq_stride=0, keep=()):
        self.c = _View(k_addr, v_addr, k_type, v_type, n_keys, k_pos_stride, v_pos_stride,
                       k_head_stride, v_head_stride, k_seq_stride, v_seq_stride)
        self.keep = keep


def view_of(kc, vc, start: int = 0, stop: int | None = None, k_seq_stride: int = 0, v_seq_stride: int = 0) -> View:
    """View of positions [start, stop) of a pair of host synth.Cache objects."""
    stop = kc.n_keys if stop is None else stop
    return View(_ptr(kc.data) + start * kc.pos_stride, _ptr(vc.data) + start * vc.pos_stride,
                kc.dtype, vc.dtype, stop - start, kc.pos_stride, vc.pos_stride,
                kc.head_stride, vc.head_stride, k_seq_stride, v_seq_stride, keep=(kc, vc))
