"""CPU oracle for batched paged MLA decode -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it.

Two independent implementations live here:

* ``liboracle.so`` (``oracle.c``): the paged loop in fp64, a two-pass softmax,
  OpenMP over query rows.  This is what GPU results are compared with.
* ``brute.py``: dense numpy fp64 attention over the gathered rows, used to
  pin the C oracle on small inputs.
* ``rope.py``: the rotary embedding of the query and key rope parts, pinned by
  ``tests/test_oracle_rope.py``.
* ``kv_append.py``: the KV-cache append (scatter of new latent rows into the
  pool, with the e4m3fn quantisation of an fp8 pool), pinned by
  ``tests/test_oracle_append.py``.
* ``query_fp8.py``: the e4m3fn cast of the query in the fp8 decode, pinned by
  ``tests/test_oracle_query_fp8.py``.

Every function is pinned by the tests in ``tests/test_oracle.py`` (brute
force, closed forms, invariances, library decoders); no function is left
without a pin.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import numpy as np

from . import build as _build

ROW_DIM = 576
LATENT_DIM = 512


class _Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("q_len", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32), ("bt_stride", ctypes.c_int32),
                ("kv_is_fp8", ctypes.c_int32), ("softmax_scale", ctypes.c_double), ("k_scale", ctypes.c_double)]


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """ctypes front end of one build of oracle.c (the default build, or a planted-mistake build)."""

    def __init__(self, libpath: Optional[str] = None):
        if libpath is None:
            libpath = _build.LIB
            if not os.path.exists(libpath):
                _build.build()
        self.path = libpath
        self.lib = ctypes.CDLL(libpath)
        L = self.lib
        L.oracle_version.restype = ctypes.c_int
        L.oracle_threads.restype = ctypes.c_int
        L.oracle_bf16_to_double.restype = ctypes.c_double
        L.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_e4m3fn_to_double.restype = ctypes.c_double
        L.oracle_e4m3fn_to_double.argtypes = [ctypes.c_uint8]
        for name in ("oracle_gather_rows", "oracle_gather_bytes", "oracle_decode", "oracle_decode_rows"):
            getattr(L, name).restype = ctypes.c_int
        L.oracle_attend.restype = None
        L.oracle_attend.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p]
        L.oracle_merge.restype = None
        L.oracle_merge.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_void_p]

    def threads(self) -> int:
        """OpenMP threads the oracle's loops use."""
        return int(self.lib.oracle_threads())

    # ---- scalar decoders
    def bf16(self, bits: int) -> float:
        return self.lib.oracle_bf16_to_double(int(bits))

    def e4m3fn(self, code: int) -> float:
        return self.lib.oracle_e4m3fn_to_double(int(code))

    # ---- helpers
    @staticmethod
    def dims(inp) -> _Dims:
        return _Dims(inp.batch, inp.q_len, inp.heads, inp.page_size, inp.num_pages, inp.block_table.shape[1],
                     1 if inp.kv_fp8 else 0, float(inp.softmax_scale), float(inp.k_scale))

    @staticmethod
    def _arrays(inp):
        q = np.ascontiguousarray(inp.q, dtype=np.uint16)
        pool = np.ascontiguousarray(inp.pool)
        bt = np.ascontiguousarray(inp.block_table, dtype=np.int32)
        sl = np.ascontiguousarray(inp.seq_lens, dtype=np.int32)
        return q, pool, bt, sl

    # ---- the decode
    def decode(self, inp) -> Tuple[np.ndarray, np.ndarray]:
        """All query rows: out [B, q_len, H, 512] and lse [B, q_len, H], float64."""
        q, pool, bt, sl = self._arrays(inp)
        out = np.zeros((inp.batch, inp.q_len, inp.heads, LATENT_DIM), dtype=np.float64)
        lse = np.zeros((inp.batch, inp.q_len, inp.heads), dtype=np.float64)
        d = self.dims(inp)
        rc = self.lib.oracle_decode(ctypes.byref(d), _ptr(q), _ptr(pool), _ptr(bt), _ptr(sl), _ptr(out), _ptr(lse))
        if rc != 0:
            raise ValueError("oracle: block-table entry out of range")
        return out, lse

    def decode_rows(self, inp, sel: Sequence[Tuple[int, int, int]]) -> Tuple[np.ndarray, np.ndarray]:
        """Selected query rows (b, j, h): out [n, 512], lse [n]."""
        q, pool, bt, sl = self._arrays(inp)
        s = np.ascontiguousarray(np.asarray(sel, dtype=np.int32).reshape(-1, 3))
        out = np.zeros((s.shape[0], LATENT_DIM), dtype=np.float64)
        lse = np.zeros((s.shape[0],), dtype=np.float64)
        d = self.dims(inp)
        rc = self.lib.oracle_decode_rows(ctypes.byref(d), _ptr(q), _ptr(pool), _ptr(bt), _ptr(sl),
                                         ctypes.c_int32(s.shape[0]), _ptr(s), _ptr(out), _ptr(lse))
        if rc != 0:
            raise ValueError("oracle: block-table entry out of range")
        return out, lse

    def gather_rows(self, inp, b: int, n: int) -> np.ndarray:
        """Dequantised rows [n, 576] (float64) of request b."""
        _, pool, bt, _ = self._arrays(inp)
        rows = np.zeros((max(n, 1), ROW_DIM), dtype=np.float64)
        d = self.dims(inp)
        rc = self.lib.oracle_gather_rows(ctypes.byref(d), _ptr(pool), _ptr(bt), ctypes.c_int32(b),
                                         ctypes.c_int32(n), _ptr(rows))
        if rc != 0:
            raise ValueError("oracle: block-table entry out of range")
        return rows[:n]

    def gather_bytes(self, inp, b: int, n: int) -> np.ndarray:
        """Stored rows [n, 576] of request b, byte for byte."""
        _, pool, bt, _ = self._arrays(inp)
        dst = np.zeros((max(n, 1), ROW_DIM), dtype=pool.dtype)
        d = self.dims(inp)
        rc = self.lib.oracle_gather_bytes(ctypes.byref(d), _ptr(pool), _ptr(bt), ctypes.c_int32(b),
                                          ctypes.c_int32(n), _ptr(dst))
        if rc != 0:
            raise ValueError("oracle: block-table entry out of range")
        return dst[:n]

    def attend(self, q_row_bits: np.ndarray, rows: np.ndarray, t0: int, t1: int, scale: float):
        """One query row (576 bf16 bit patterns) over decoded rows[t0:t1]: (o[512], lse)."""
        qr = np.ascontiguousarray(q_row_bits, dtype=np.uint16)
        assert qr.shape == (ROW_DIM,)
        r = np.ascontiguousarray(rows, dtype=np.float64)
        if r.size == 0:
            r = np.zeros((1, ROW_DIM))
        o = np.zeros(LATENT_DIM, dtype=np.float64)
        lse = np.zeros(1, dtype=np.float64)
        self.lib.oracle_attend(_ptr(qr), _ptr(r), int(t0), int(t1), float(scale), _ptr(o), _ptr(lse))
        return o, float(lse[0])

    def merge(self, o_parts: np.ndarray, lse_parts: np.ndarray):
        """LSE merge of S partials o_parts [S, width], lse_parts [S]: (o[width], lse)."""
        op = np.ascontiguousarray(o_parts, dtype=np.float64)
        lp = np.ascontiguousarray(lse_parts, dtype=np.float64)
        S, width = op.shape
        o = np.zeros(width, dtype=np.float64)
        lse = np.zeros(1, dtype=np.float64)
        self.lib.oracle_merge(S, width, _ptr(op), _ptr(lp), _ptr(o), _ptr(lse))
        return o, float(lse[0])


_default: Optional[Oracle] = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def decode(inp):
    return default().decode(inp)


def decode_rows(inp, sel):
    return default().decode_rows(inp, sel)
