"""CPU oracle for block-quantized weight x q8_1 activation products (ctypes over plain C).

TEST INFRASTRUCTURE ONLY: imported by the tests, by ``__graft_entry__.smoke()`` and by the
benchmark's CPU-baseline leg, never by the ``moe_expert_amd`` product path.  The C source
(``qmm_oracle.c``) shares no code with the HIP library.

All functions take and return numpy arrays.  Byte layouts are the raw block layouts
(Q8_0 34 B / 32 values, IQ4_NL 18 B / 32, CB3 110 B / 256, q8_1 36 B / 32).
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

Q8_0, IQ4_NL, CB3 = 1, 2, 3




def _signatures():
    P = C.c_void_p
    i64, i32 = C.c_int64, C.c_int
    return {
        "or_num_threads": (C.c_int, []),
        "or_set_num_threads": (None, [C.c_int]),
        "or_f16_to_f32": (C.c_float, [C.c_uint16]),
        "or_f32_to_f16": (C.c_uint16, [C.c_float]),
        "or_f64_to_f16": (C.c_uint16, [C.c_double]),
        "or_f16_to_f32_array": (None, [P, i64, P]),
        "or_f32_to_f16_array": (None, [P, i64, P]),
        "or_row_bytes": (i64, [i32, i64]),
        "or_dequant_f64": (i32, [i32, P, P, i64, i64, P]),
        "or_dequant_f16": (i32, [i32, P, P, i64, i64, P, i64]),
        "or_quantize_block_q8_1": (None, [P, P]),
        "or_quantize_q8_1": (i32, [P, i64, i32, i64, P]),
        "or_block_sums": (i32, [i32, P, P, i64, i64, P, i32, P]),
        "or_gemv": (i32, [i32, P, P, i64, i64, P, i32, P, P]),
        "or_silu_mul": (C.c_float, [C.c_float, C.c_float]),
        "or_silu_mul_array": (None, [P, P, i64, P]),
        "or_grouped": (i32, [i32, P, P, i64, i32, P, i64, P, i64, i64, P, P, P, i32, P, i32,
                             P, P, P, P, P, P, P, P]),
        "or_prefill_rows": (i32, [i32, P, P, i64, i32, P, i64, P, i32, i64, i64, P, i64, P, P,
                                  P, i64, P, P, P, P, P, P, P]),
        "or_moe_combine": (i32, [P, i64, i64, P, P, i64, i32, P]),
        "or_dense_rows": (i32, [i32, P, P, i64, i64, P, i64, P, i64, P, P]),
        "or_pack_planes": (i32, [i32, P, i64, i64, P]),
    }


def load_library(path: str):
    """Load an oracle shared library (the real one or a test-built variant)."""
    L = C.CDLL(path)
    for name, (res, args) in _signatures().items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _grid(grid):
    return None if grid is None else _c(grid, np.uint8)


class Oracle:
    """The oracle API bound to one loaded library."""

    def __init__(self, L):
        self.L = L

    def num_threads(self) -> int:
        return self.L.or_num_threads()

    def set_num_threads(self, n: int) -> None:
        """Threads of the oracle's parallel loops (timing only; results do not depend on it)."""
        self.L.or_set_num_threads(int(n))

    def row_bytes(self, wtype: int, k: int) -> int:
        return int(self.L.or_row_bytes(wtype, k))

    def f16_to_f32(self, h) -> np.ndarray:
        h = _c(h, np.uint16)
        out = np.empty(h.shape, np.float32)
        self.L.or_f16_to_f32_array(_p(h), h.size, _p(out))
        return out

    def f32_to_f16(self, f) -> np.ndarray:
        f = _c(f, np.float32)
        out = np.empty(f.shape, np.uint16)
        self.L.or_f32_to_f16_array(_p(f), f.size, _p(out))
        return out

    def f64_to_f16(self, x: float) -> int:
        return int(self.L.or_f64_to_f16(float(x)))

    def dequant_f64(self, wtype: int, w, k: int, grid=None) -> np.ndarray:
        """Exact dequantized values, [nrows, k] float64."""
        w = _c(w, np.uint8)
        nrows = w.size // self.row_bytes(wtype, k)
        out = np.empty((nrows, k), np.float64)
        g = _grid(grid)
        if self.L.or_dequant_f64(wtype, _p(w), _p(g), nrows, k, _p(out)):
            raise ValueError("bad dequant arguments")
        return out

    def dequant_f16(self, wtype: int, w, k: int, grid=None, ld: int | None = None) -> np.ndarray:
        """FP16 dequantization (bit patterns), [nrows, ld] uint16 (columns >= k left zero)."""
        w = _c(w, np.uint8)
        nrows = w.size // self.row_bytes(wtype, k)
        ld = k if ld is None else ld
        out = np.zeros((nrows, ld), np.uint16)
        g = _grid(grid)
        if self.L.or_dequant_f16(wtype, _p(w), _p(g), nrows, k, _p(out), ld):
            raise ValueError("bad dequant arguments")
        return out

    def quantize_q8_1(self, x) -> np.ndarray:
        """x: [ncols, k] float32 -> [ncols, k/32*36] uint8 q8_1 blocks."""
        x = _c(x, np.float32)
        if x.ndim == 1:
            x = x[None, :]
        ncols, k = x.shape
        out = np.empty((ncols, (k // 32) * 36), np.uint8)
        if self.L.or_quantize_q8_1(_p(x), k, ncols, k, _p(out)):
            raise ValueError("bad quantize arguments")
        return out

    def block_sums(self, wtype: int, w, k: int, xq, grid=None) -> np.ndarray:
        """Per-block integer sums, [ncols, nrows, k/32] int32."""
        w = _c(w, np.uint8)
        xq = _c(xq, np.uint8)
        nrows = w.size // self.row_bytes(wtype, k)
        ncols = xq.size // ((k // 32) * 36)
        out = np.empty((ncols, nrows, k // 32), np.int32)
        g = _grid(grid)
        if self.L.or_block_sums(wtype, _p(w), _p(g), nrows, k, _p(xq), ncols, _p(out)):
            raise ValueError("bad block_sums arguments")
        return out

    def gemv(self, wtype: int, w, k: int, xq, grid=None):
        """Dense GEMV: returns (y [ncols, nrows] float64, sum|terms| [ncols, nrows] float64)."""
        w = _c(w, np.uint8)
        xq = _c(xq, np.uint8)
        nrows = w.size // self.row_bytes(wtype, k)
        ncols = xq.size // ((k // 32) * 36)
        y = np.empty((ncols, nrows), np.float64)
        a = np.empty((ncols, nrows), np.float64)
        g = _grid(grid)
        if self.L.or_gemv(wtype, _p(w), _p(g), nrows, k, _p(xq), ncols, _p(y), _p(a)):
            raise ValueError("bad gemv arguments")
        return y, a

    def silu_mul(self, g, u) -> np.ndarray:
        g = _c(g, np.float32)
        u = _c(u, np.float32)
        out = np.empty(g.shape, np.float32)
        self.L.or_silu_mul_array(_p(g), _p(u), g.size, _p(out))
        return out

    def grouped(self, wtype_gu: int, w_gate, w_up, wtype_down: int, w_down, hidden: int, inter: int, xq,
                group_expert, group_off, entry_col, grid=None) -> dict:
        """Grouped MoE decode.  Weights are [nexperts, rows, row_bytes] uint8 arrays (or flat with
        the per-expert stride implied).  Returns a dict of g, u, gabs, uabs, h, hq, y, yabs."""
        w_gate = _c(w_gate, np.uint8)
        w_up = _c(w_up, np.uint8)
        w_down = _c(w_down, np.uint8)
        gu_stride = inter * self.row_bytes(wtype_gu, hidden)
        d_stride = hidden * self.row_bytes(wtype_down, inter)
        xq = _c(xq, np.uint8)
        ge = _c(group_expert, np.int32)
        go = _c(group_off, np.int32)
        ec = _c(entry_col, np.int32)
        ne = ec.size
        out = dict(g=np.empty((ne, inter)), u=np.empty((ne, inter)), gabs=np.empty((ne, inter)),
                   uabs=np.empty((ne, inter)), h=np.empty((ne, inter), np.float32),
                   hq=np.empty((ne, (inter // 32) * 36), np.uint8), y=np.empty((ne, hidden)),
                   yabs=np.empty((ne, hidden)))
        g = _grid(grid)
        rc = self.L.or_grouped(wtype_gu, _p(w_gate), _p(w_up), gu_stride, wtype_down, _p(w_down),
                              d_stride, _p(g), hidden, inter, _p(xq), _p(ge), _p(go), ge.size,
                              _p(ec), ne, _p(out["g"]), _p(out["u"]), _p(out["gabs"]),
                              _p(out["uabs"]), _p(out["h"]), _p(out["hq"]), _p(out["y"]),
                              _p(out["yabs"]))
        if rc:
            raise ValueError(f"or_grouped failed: {rc}")
        return out

    def prefill_rows(self, wtype_gu: int, w_gate, w_up, wtype_down: int, w_down, nexperts: int,
                     hidden: int, inter: int, x16, sorted_tok, expert_off, samples,
                     grid=None) -> dict:
        """Prefill expert GEMM on the sampled entry positions ``samples`` (int64).  ``x16`` is
        [ntok, hidden] fp16 (any 2-byte dtype).  Returns G, U, Gabs, Uabs, H16, Y, Yabs."""
        w_gate = _c(w_gate, np.uint8)
        w_up = _c(w_up, np.uint8)
        w_down = _c(w_down, np.uint8)
        gu_stride = inter * self.row_bytes(wtype_gu, hidden)
        d_stride = hidden * self.row_bytes(wtype_down, inter)
        x16 = np.ascontiguousarray(x16).view(np.uint16)
        ntok = x16.shape[0]
        st = _c(sorted_tok, np.int32)
        eo = _c(expert_off, np.int32)
        sm = _c(samples, np.int64)
        ns = sm.size
        out = dict(G=np.empty((ns, inter)), U=np.empty((ns, inter)), Gabs=np.empty((ns, inter)),
                   Uabs=np.empty((ns, inter)), H16=np.empty((ns, inter), np.uint16),
                   Y=np.empty((ns, hidden)), Yabs=np.empty((ns, hidden)))
        g = _grid(grid)
        rc = self.L.or_prefill_rows(wtype_gu, _p(w_gate), _p(w_up), gu_stride, wtype_down,
                                   _p(w_down), d_stride, _p(g), nexperts, hidden, inter, _p(x16),
                                   ntok, _p(st), _p(eo), _p(sm), ns, _p(out["G"]), _p(out["U"]),
                                   _p(out["Gabs"]), _p(out["Uabs"]), _p(out["H16"]), _p(out["Y"]),
                                   _p(out["Yabs"]))
        if rc:
            raise ValueError(f"or_prefill_rows failed: {rc}")
        return out


    def moe_combine(self, y, row_idx, w) -> np.ndarray:
        """out [ntok, hidden] float32: the router-weighted sum of each token's expert rows of y
        [nrows, hidden] in k order (row_idx, w: [ntok, topk])."""
        y = _c(y, np.float32)
        ri = _c(row_idx, np.int32)
        ww = _c(w, np.float32)
        ntok, topk = ri.shape
        out = np.empty((ntok, y.shape[1]), np.float32)
        if self.L.or_moe_combine(_p(y), y.shape[0], y.shape[1], _p(ri), _p(ww), ntok, topk, _p(out)):
            raise ValueError("bad combine arguments")
        return out

    def dense_rows(self, wtype: int, w, nrows: int, k: int, x16, samples, grid=None):
        """Dense projection of the sampled prompt tokens on FP16 weights: returns (Y, Yabs), each
        [ns, nrows] float64.  wtype 0: w is binary16 [nrows, k] already."""
        w = np.ascontiguousarray(w)
        x16 = np.ascontiguousarray(x16).view(np.uint16)
        sm = _c(samples, np.int64)
        Y = np.empty((sm.size, nrows))
        A = np.empty((sm.size, nrows))
        g = _grid(grid)
        if self.L.or_dense_rows(wtype, _p(w), _p(g), nrows, k, _p(x16), x16.shape[0], _p(sm), sm.size, _p(Y), _p(A)):
            raise ValueError("bad dense_rows arguments")
        return Y, A

    def pack_planes(self, wtype: int, w, k: int) -> np.ndarray:
        """Planes of Q8_0 / IQ4_NL rows (same shape and size as the blocks)."""
        w = _c(w, np.uint8)
        nrows = w.size // self.row_bytes(wtype, k)
        out = np.empty_like(w)
        if self.L.or_pack_planes(wtype, _p(w), nrows, k, _p(out)):
            raise ValueError("bad pack_planes arguments")
        return out


_default = None


def default() -> Oracle:
    """The oracle built from ``qmm_oracle.c`` (built with gcc on first use)."""
    global _default
    if _default is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _default = Oracle(load_library(_build.LIB))
    return _default


def __getattr__(name):
    if name in _API:
        return getattr(default(), name)
    raise AttributeError(name)


_API = set(['num_threads', 'set_num_threads', 'row_bytes', 'f16_to_f32', 'f32_to_f16', 'f64_to_f16', 'dequant_f64', 'dequant_f16', 'quantize_q8_1', 'block_sums', 'gemv', 'silu_mul', 'grouped', 'prefill_rows', 'moe_combine', 'dense_rows', 'pack_planes'])
