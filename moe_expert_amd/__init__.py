"""moe_expert_amd -- block-quantized weight x q8_1 activation products on MI355X (gfx950).

A thin ctypes binding over ``libqmm.so`` (the C ABI declared in include/qmm.h).  Every entry
point below only marshals arguments: it takes torch tensors that already live on the GPU,
passes their device pointers and the current HIP stream to the library and raises
``QmmError`` on a non-zero status.  All arithmetic runs in the library's HIP kernels; there is
no CPU fallback, and a missing library raises at first use.

Names follow the C ABI: ``qmm_quantize_q8_1``, ``qmm_dequant_f16``, ``qgemv_dense``,
``qgemv_dense_f32``, ``qmm_debug_block_sums``, ``qgemv_grouped_experts``,
``qgemm_prefill_experts`` (and the measurement hooks ``qmm_debug_stream_read``,
``qmm_debug_mfma_loop``).
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqmm.so")

QMM_Q8_0, QMM_IQ4_NL, QMM_CB3 = 1, 2, 3
QMM_FLAG_DEBUG_INTERMEDIATES = 1
BLOCK_VALUES = {QMM_Q8_0: 32, QMM_IQ4_NL: 32, QMM_CB3: 256}
BLOCK_BYTES = {QMM_Q8_0: 34, QMM_IQ4_NL: 18, QMM_CB3: 110}

_P, _I64, _I32, _U32, _U64, _SZ = C.c_void_p, C.c_int64, C.c_int, C.c_uint, C.c_uint64, C.c_size_t
SIGNATURES = {
    "qmm_version": (_I32, []),
    "qmm_status_str": (C.c_char_p, [_I32]),
    "qmm_row_bytes": (_I64, [_I32, _I64]),
    "qmm_quantize_q8_1": (_I32, [_P, _I64, _I32, _I64, _P, _P]),
    "qmm_dequant_f16": (_I32, [_I32, _P, _P, _I64, _I64, _P, _I64, _P]),
    "qgemv_dense": (_I32, [_I32, _P, _P, _I64, _I64, _P, _I32, _P, _I64, _P]),
    "qgemv_dense_f32": (_I32, [_I32, _P, _P, _I64, _I64, _P, _I32, _P, _I64, _P]),
    "qmm_debug_block_sums": (_I32, [_I32, _P, _P, _I64, _I64, _P, _I32, _P, _P]),
    "qmm_debug_stream_read": (_I32, [_P, _U64, _P, _I32, _P]),
    "qmm_debug_mfma_loop": (_I32, [_P, _I32, _I32, _P]),
    "qgemv_grouped_experts_workspace": (_SZ, [_I64, _I32, _U32]),
    "qgemv_grouped_experts": (_I32, [_I32, _P, _P, _I64, _I32, _P, _I64, _I32, _P, _I64, _I64, _P, _I32,
                                     _P, _P, _I32, _P, _I32, _P, _P, _SZ, _U32, _P]),
    "qgemm_prefill_experts_workspace": (_SZ, [_I32, _I64, _I64, _U32]),
    "qgemm_prefill_experts": (_I32, [_I32, _P, _P, _I64, _I32, _P, _I64, _I32, _I64, _I64, _P, _I64,
                                     _P, _P, _I64, _P, _P, _SZ, _U32, _P]),
}

_lib = None


class QmmError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status} ({status_str(status)})")
        self.status = status


def lib():
    """Load libqmm.so from the package directory (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m moe_expert_amd.build`")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().qmm_status_str(status).decode()


def row_bytes(wtype: int, k: int) -> int:
    return int(lib().qmm_row_bytes(wtype, k))


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return C.c_void_p(stream)
    import torch
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(fn, rc):
    if rc != 0:
        raise QmmError(fn, rc)


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def qmm_quantize_q8_1(x, out=None, stream=None):
    """x: float32 [ncols, k] (GPU) -> uint8 [ncols, k/32*36] q8_1 blocks."""
    import torch
    _dev(x, "x")
    if x.dim() == 1:
        x = x.view(1, -1)
    ncols, k = x.shape
    if out is None:
        out = torch.empty((ncols, (k // 32) * 36), dtype=torch.uint8, device=x.device)
    _check("qmm_quantize_q8_1", lib().qmm_quantize_q8_1(_ptr(x), k, ncols, k, _ptr(out), _stream(stream)))
    return out


def qmm_dequant_f16(wtype, w, nrows, k, grid=None, out=None, ld=None, stream=None):
    """Weight blocks -> binary16 [nrows, ld] (returned as torch.float16)."""
    import torch
    _dev(w, "w")
    ld = k if ld is None else ld
    if out is None:
        out = torch.empty((nrows, ld), dtype=torch.float16, device=w.device)
    _check("qmm_dequant_f16", lib().qmm_dequant_f16(wtype, _ptr(w), _ptr(grid), nrows, k, _ptr(out), ld,
                                                   _stream(stream)))
    return out


def qgemv_dense(wtype, w, nrows, k, xq, ncols, grid=None, y=None, ldy=None, stream=None):
    """y[c, r] for c < ncols: float32 [ncols, ldy] (ldy defaults to nrows)."""
    import torch
    _dev(w, "w"); _dev(xq, "xq")
    ldy = nrows if ldy is None else ldy
    if y is None:
        y = torch.empty((ncols, ldy), dtype=torch.float32, device=w.device)
    _check("qgemv_dense", lib().qgemv_dense(wtype, _ptr(w), _ptr(grid), nrows, k, _ptr(xq), ncols, _ptr(y), ldy,
                                           _stream(stream)))
    return y


def qgemv_dense_f32(wtype, w, nrows, k, x, ncols=1, grid=None, y=None, ldy=None, stream=None):
    """1, 2 or 4 fp32 columns x [ncols, k] quantized to q8_1 inside the kernel: y float32
    [ncols, ldy], bitwise qgemv_dense of qmm_quantize_q8_1(x) (k at most 3072)."""
    import torch
    _dev(w, "w"); _dev(x, "x")
    ldy = nrows if ldy is None else ldy
    if y is None:
        y = torch.empty((ncols, ldy), dtype=torch.float32, device=w.device)
    _check("qgemv_dense_f32", lib().qgemv_dense_f32(wtype, _ptr(w), _ptr(grid), nrows, k, _ptr(x), ncols, _ptr(y),
                                                   ldy, _stream(stream)))
    return y


def qmm_debug_block_sums(wtype, w, nrows, k, xq, ncols, grid=None, out=None, stream=None):
    """Per-block integer sums int32 [ncols, nrows, k/32]."""
    import torch
    _dev(w, "w"); _dev(xq, "xq")
    if out is None:
        out = torch.empty((ncols, nrows, k // 32), dtype=torch.int32, device=w.device)
    _check("qmm_debug_block_sums", lib().qmm_debug_block_sums(wtype, _ptr(w), _ptr(grid), nrows, k, _ptr(xq), ncols,
                                                             _ptr(out), _stream(stream)))
    return out


def qmm_debug_stream_read(p, nbytes, grid, out=None, stream=None):
    """Plain streaming read of the first nbytes of device tensor p in one launch of `grid`
    256-thread workgroups (the HBM reference); returns out (uint32 [grid * 256])."""
    import torch
    _dev(p, "p")
    if out is None:
        out = torch.empty(grid * 256, dtype=torch.int32, device=p.device)
    _check("qmm_debug_stream_read", lib().qmm_debug_stream_read(_ptr(p), nbytes, _ptr(out), grid, _stream(stream)))
    return out


def qmm_debug_mfma_loop(grid, iters, out=None, device="cuda", stream=None):
    """Register-only fp16 MFMA loop (grid * 4 * 8 * iters * 32768 FLOP); returns out (float
    [grid * 256])."""
    import torch
    if out is None:
        out = torch.empty(grid * 256, dtype=torch.float32, device=device)
    _check("qmm_debug_mfma_loop", lib().qmm_debug_mfma_loop(_ptr(out), grid, iters, _stream(stream)))
    return out


def qgemv_grouped_experts_workspace(inter, nentries, flags=0):
    return int(lib().qgemv_grouped_experts_workspace(inter, nentries, flags))


def qgemv_grouped_experts(wtype_gu, w_gate, w_up, wtype_down, w_down, hidden, inter, xq, group_expert,
                          group_entry_off, entry_col, grid=None, y=None, ws=None, flags=0, stream=None):
    """Grouped MoE decode.  w_gate / w_up: [nexperts, inter * row_bytes(gu, hidden)] bytes,
    w_down: [nexperts, hidden * row_bytes(down, inter)] bytes, xq: [xq_cols, hidden/32*36] q8_1;
    returns (y [nentries, hidden] float32, ws)."""
    import torch
    for t, n in ((w_gate, "w_gate"), (w_up, "w_up"), (w_down, "w_down"), (xq, "xq"), (group_expert, "group_expert"),
                 (group_entry_off, "group_entry_off"), (entry_col, "entry_col")):
        _dev(t, n)
    nentries = entry_col.numel()
    ngroups = group_expert.numel()
    nexperts = w_gate.shape[0]
    xq_cols = xq.numel() // ((hidden // 32) * 36)
    gu_stride = w_gate[0].numel()
    d_stride = w_down[0].numel()
    if y is None:
        y = torch.empty((nentries, hidden), dtype=torch.float32, device=w_gate.device)
    need = qgemv_grouped_experts_workspace(inter, nentries, flags)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=w_gate.device)
    _check("qgemv_grouped_experts", lib().qgemv_grouped_experts(
        wtype_gu, _ptr(w_gate), _ptr(w_up), gu_stride, wtype_down, _ptr(w_down), d_stride, nexperts, _ptr(grid),
        hidden, inter, _ptr(xq), xq_cols, _ptr(group_expert), _ptr(group_entry_off), ngroups, _ptr(entry_col),
        nentries, _ptr(y), _ptr(ws), ws.numel(), flags, _stream(stream)))
    return y, ws


def qgemm_prefill_experts_workspace(nexperts, inter, nentries, flags=0):
    return int(lib().qgemm_prefill_experts_workspace(nexperts, inter, nentries, flags))


def qgemm_prefill_experts(wtype_gu, w_gate, w_up, wtype_down, w_down, nexperts, hidden, inter, x_f16, sorted_tok,
                          expert_off, y=None, ws=None, flags=0, stream=None):
    """Prefill grouped expert GEMM; returns (y [nentries, hidden] float32, ws)."""
    import torch
    for t, n in ((w_gate, "w_gate"), (w_up, "w_up"), (w_down, "w_down"), (x_f16, "x_f16"),
                 (sorted_tok, "sorted_tok"), (expert_off, "expert_off")):
        _dev(t, n)
    nentries = sorted_tok.numel()
    ntok = x_f16.shape[0]
    gu_stride = inter * row_bytes(wtype_gu, hidden)
    d_stride = hidden * row_bytes(wtype_down, inter)
    if y is None:
        y = torch.empty((nentries, hidden), dtype=torch.float32, device=w_gate.device)
    need = qgemm_prefill_experts_workspace(nexperts, inter, nentries, flags)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=w_gate.device)
    _check("qgemm_prefill_experts", lib().qgemm_prefill_experts(
        wtype_gu, _ptr(w_gate), _ptr(w_up), gu_stride, wtype_down, _ptr(w_down), d_stride, nexperts, hidden, inter,
        _ptr(x_f16), ntok, _ptr(sorted_tok), _ptr(expert_off), nentries, _ptr(y), _ptr(ws), ws.numel(), flags,
        _stream(stream)))
    return y, ws
