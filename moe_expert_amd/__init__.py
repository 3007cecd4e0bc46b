"""moe_expert_amd -- block-quantized weight x q8_1 activation products on MI355X (gfx950).

A thin ctypes binding over ``libqmm.so`` (the C ABI declared in include/qmm.h).  Every entry
point below only marshals arguments: it takes torch tensors that already live on the GPU,
checks that each one is a contiguous tensor of the expected dtype on the same GPU and holds at
least the bytes the call reads or writes (``ValueError`` otherwise, before anything is launched:
the library trusts the sizes it is given), passes the device pointers and the current HIP stream
to the library and raises ``QmmError`` on a non-zero status.  All arithmetic runs in the
library's HIP kernels; there is no CPU fallback, and a missing library raises at first use.

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

QMM_Q8_0, QMM_IQ4_NL, QMM_CB3, QMM_F16 = 1, 2, 3, 4
QMM_FLAG_DEBUG_INTERMEDIATES = 1
BLOCK_VALUES = {QMM_Q8_0: 32, QMM_IQ4_NL: 32, QMM_CB3: 256, QMM_F16: 1}
BLOCK_BYTES = {QMM_Q8_0: 34, QMM_IQ4_NL: 18, QMM_CB3: 110, QMM_F16: 2}
Q8_1_BYTES = 36
GRID_BYTES = 2048

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
    "qmm_debug_stream_read": (_I32, [_P, _U64, _P, _I32, _I32, _I32, _P]),
    "qmm_debug_mfma_loop": (_I32, [_P, _I32, _I32, _P]),
    "qgemv_grouped_experts_workspace": (_SZ, [_I64, _I32, _U32]),
    "qgemv_grouped_experts": (_I32, [_I32, _P, _P, _I64, _I32, _P, _I64, _I32, _P, _I64, _I64, _P, _I32,
                                     _P, _P, _I32, _P, _I32, _P, _P, _SZ, _U32, _P]),
    "qgemv_grouped_experts_noalloc_max_bytes": (_SZ, []),
    "qgemv_grouped_experts_noalloc": (_I32, [_I32, _P, _P, _I64, _I32, _P, _I64, _I32, _P, _I64, _I64, _P, _I32,
                                             _P, _P, _I32, _P, _I32, _P, _P]),
    "qmm_moe_combine": (_I32, [_P, _I64, _I64, _P, _P, _I64, _I32, _P, _I64, _P]),
    "qmm_pack_planes": (_I32, [_I32, _P, _I64, _I64, _P, _P]),
    "qmm_planes_alloc": (_I32, [_I32, _P, _I64, _I64, C.POINTER(C.c_void_p), _P]),
    "qmm_planes_release": (_I32, [_P]),
    "qgemv_planes": (_I32, [_I32, _P, _I64, _I64, _P, _I32, _P, _I64, _P]),
    "qgemm_dense": (_I32, [_I32, _P, _I64, _I64, _P, _I64, _P, _I64, _P]),
    "qgemm_prefill_experts_q8_workspace": (_SZ, [_I32, _I64, _I64, _I64, _I64, _U32]),
    "qgemm_prefill_experts_q8": (_I32, [_I32, _P, _P, _I64, _I32, _P, _I64, _I32, _I64, _I64, _P, _I64,
                                        _P, _P, _I64, _P, _P, _SZ, _U32, _P]),
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


def _stream(stream, device=None):
    if stream is not None:
        return C.c_void_p(stream)
    import torch
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(fn, rc):
    if rc != 0:
        raise QmmError(fn, rc)


# ------------------------------------------------------------------ argument checks
#
# The C library takes plain pointers and sizes and cannot see the allocations behind them, so
# every tensor is checked here against what the call will touch.

def _dtypes(kind):
    import torch
    return {"u8": (torch.uint8,), "f32": (torch.float32,), "i32": (torch.int32,),
            "f16": tuple(d for d in (torch.float16, torch.int16, getattr(torch, "uint16", None)) if d is not None)}[kind]


def _nbytes(t) -> int:
    return int(t.numel()) * int(t.element_size())


def _need(t, name, kind, nbytes, device=None):
    """t must be a contiguous GPU tensor of dtype `kind` (u8, f32, i32, f16: any 2-byte type), on
    `device` when given, holding at least `nbytes` bytes."""
    if t is None:
        raise ValueError(f"{name} is required")
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype not in _dtypes(kind):
        raise ValueError(f"{name} must have dtype {kind}, not {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the call runs on {device}")
    if _nbytes(t) < nbytes:
        raise ValueError(f"{name} holds {_nbytes(t)} bytes; the call touches {nbytes}")
    return t


def _block_multiple(wtype, k, name="k"):
    if wtype not in BLOCK_VALUES:
        raise ValueError(f"unknown weight format {wtype}")
    if k < 1 or k % BLOCK_VALUES[wtype]:
        raise ValueError(f"{name}={k} is not a positive multiple of {BLOCK_VALUES[wtype]}")
    return (k // BLOCK_VALUES[wtype]) * BLOCK_BYTES[wtype]


def _grid_arg(wtype, grid, device, name="grid"):
    if wtype == QMM_CB3 or grid is not None:
        _need(grid, name, "u8", GRID_BYTES, device)
    return grid


def _out(t, name, kind, nbytes, device, shape, dtype):
    """A caller-supplied output (checked) or a new one of `shape`."""
    import torch
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    return _need(t, name, kind, nbytes, device)


# ------------------------------------------------------------------ entry points

def qmm_quantize_q8_1(x, out=None, stream=None):
    """x: float32 [ncols, k] (GPU) -> uint8 [ncols, k/32*36] q8_1 blocks."""
    import torch
    if getattr(x, "dim", lambda: 0)() == 1:
        x = x.view(1, -1)
    if getattr(x, "dim", lambda: 0)() != 2:
        raise ValueError("x must be [ncols, k]")
    ncols, k = x.shape
    if k < 32 or k % 32:
        raise ValueError(f"k={k} is not a positive multiple of 32")
    _need(x, "x", "f32", ncols * k * 4)
    out = _out(out, "out", "u8", ncols * (k // 32) * Q8_1_BYTES, x.device, (ncols, (k // 32) * Q8_1_BYTES),
               torch.uint8)
    _check("qmm_quantize_q8_1", lib().qmm_quantize_q8_1(_ptr(x), k, ncols, k, _ptr(out), _stream(stream, x.device)))
    return out


def qmm_dequant_f16(wtype, w, nrows, k, grid=None, out=None, ld=None, stream=None):
    """Weight blocks -> binary16 [nrows, ld] (returned as torch.float16)."""
    import torch
    rb = _block_multiple(wtype, k)
    ld = k if ld is None else ld
    if nrows < 1 or ld < k:
        raise ValueError("nrows >= 1 and ld >= k")
    _need(w, "w", "u8", nrows * rb)
    _grid_arg(wtype, grid, w.device)
    out = _out(out, "out", "f16", ((nrows - 1) * ld + k) * 2, w.device, (nrows, ld), torch.float16)
    _check("qmm_dequant_f16", lib().qmm_dequant_f16(wtype, _ptr(w), _ptr(grid), nrows, k, _ptr(out), ld,
                                                   _stream(stream, w.device)))
    return out


def _gemv_common(wtype, w, nrows, k, ncols, grid, ldy, check_w=True):
    rb = _block_multiple(wtype, k)
    if nrows < 1 or ncols < 1:
        raise ValueError("nrows and ncols must be positive")
    ldy = nrows if ldy is None else ldy
    if ldy < nrows:
        raise ValueError("ldy < nrows")
    if check_w:
        _need(w, "w", "u8", nrows * rb)
        _grid_arg(wtype, grid, w.device)
    return ldy


def qgemv_dense(wtype, w, nrows, k, xq, ncols, grid=None, y=None, ldy=None, stream=None):
    """y[c, r] for c < ncols: float32 [ncols, ldy] (ldy defaults to nrows)."""
    import torch
    ldy = _gemv_common(wtype, w, nrows, k, ncols, grid, ldy)
    _need(xq, "xq", "u8", ncols * (k // 32) * Q8_1_BYTES, w.device)
    y = _out(y, "y", "f32", ((ncols - 1) * ldy + nrows) * 4, w.device, (ncols, ldy), torch.float32)
    _check("qgemv_dense", lib().qgemv_dense(wtype, _ptr(w), _ptr(grid), nrows, k, _ptr(xq), ncols, _ptr(y), ldy,
                                           _stream(stream, w.device)))
    return y


def qgemv_dense_f32(wtype, w, nrows, k, x, ncols=1, grid=None, y=None, ldy=None, stream=None):
    """1, 2 or 4 fp32 columns x [ncols, k] quantized to q8_1 inside the kernel: y float32
    [ncols, ldy], bitwise qgemv_dense of qmm_quantize_q8_1(x) (k at most 3072)."""
    import torch
    ldy = _gemv_common(wtype, w, nrows, k, ncols, grid, ldy)
    _need(x, "x", "f32", ncols * k * 4, w.device)
    y = _out(y, "y", "f32", ((ncols - 1) * ldy + nrows) * 4, w.device, (ncols, ldy), torch.float32)
    _check("qgemv_dense_f32", lib().qgemv_dense_f32(wtype, _ptr(w), _ptr(grid), nrows, k, _ptr(x), ncols, _ptr(y),
                                                   ldy, _stream(stream, w.device)))
    return y


def qmm_debug_block_sums(wtype, w, nrows, k, xq, ncols, grid=None, out=None, stream=None):
    """Per-block integer sums int32 [ncols, nrows, k/32]."""
    import torch
    _gemv_common(wtype, w, nrows, k, ncols, grid, None)
    _need(xq, "xq", "u8", ncols * (k // 32) * Q8_1_BYTES, w.device)
    out = _out(out, "out", "i32", ncols * nrows * (k // 32) * 4, w.device, (ncols, nrows, k // 32), torch.int32)
    _check("qmm_debug_block_sums", lib().qmm_debug_block_sums(wtype, _ptr(w), _ptr(grid), nrows, k, _ptr(xq), ncols,
                                                             _ptr(out), _stream(stream, w.device)))
    return out


def qmm_debug_stream_read(p, nbytes, grid, threads=256, unroll=8, out=None, stream=None):
    """Plain streaming read of the first nbytes of device tensor p in one launch of `grid`
    workgroups of `threads` threads, `unroll` 16-byte loads in flight per thread, contiguous runs
    per workgroup (the HBM reference); returns out (uint32 [grid * threads])."""
    import torch
    if grid < 1:
        raise ValueError("grid must be positive")
    _need(p, "p", "u8", nbytes)
    out = _out(out, "out", "i32", grid * threads * 4, p.device, (grid * threads,), torch.int32)
    _check("qmm_debug_stream_read", lib().qmm_debug_stream_read(_ptr(p), nbytes, _ptr(out), grid, threads, unroll,
                                                               _stream(stream, p.device)))
    return out


def qmm_debug_mfma_loop(grid, iters, out=None, device="cuda", stream=None):
    """Register-only fp16 MFMA loop (grid * 4 * 8 * iters * 32768 FLOP); returns out (float
    [grid * 256])."""
    import torch
    if grid < 1 or iters < 1:
        raise ValueError("grid and iters must be positive")
    if out is None:
        out = torch.empty(grid * 256, dtype=torch.float32, device=device)
    _need(out, "out", "f32", grid * 256 * 4)
    _check("qmm_debug_mfma_loop", lib().qmm_debug_mfma_loop(_ptr(out), grid, iters, _stream(stream, out.device)))
    return out


def qgemv_grouped_experts_workspace(inter, nentries, flags=0):
    return int(lib().qgemv_grouped_experts_workspace(inter, nentries, flags))


def _expert_weights(t, name, nexperts, matrix_bytes, device):
    """[nexperts, ...] uint8 expert matrices of at least matrix_bytes each; returns the
    per-expert stride in bytes."""
    if getattr(t, "dim", lambda: 0)() < 1 or t.shape[0] != nexperts:
        raise ValueError(f"{name} must be [{nexperts} experts, ...]")
    _need(t, name, "u8", nexperts * matrix_bytes, device)
    stride = _nbytes(t) // nexperts
    if stride < matrix_bytes:
        raise ValueError(f"{name}: {stride} bytes per expert, one matrix is {matrix_bytes}")
    return stride


def qgemv_grouped_experts(wtype_gu, w_gate, w_up, wtype_down, w_down, hidden, inter, xq, group_expert,
                          group_entry_off, entry_col, grid=None, y=None, ws=None, flags=0, stream=None):
    """Grouped MoE decode.  w_gate / w_up: [nexperts, inter * row_bytes(gu, hidden)] bytes,
    w_down: [nexperts, hidden * row_bytes(down, inter)] bytes, xq: [xq_cols, hidden/32*36] q8_1;
    returns (y [nentries, hidden] float32, ws)."""
    import torch
    if getattr(w_gate, "dim", lambda: 0)() < 1:
        raise ValueError("w_gate must be [nexperts, ...]")
    dev = w_gate.device
    nexperts = int(w_gate.shape[0])
    gu_stride = _expert_weights(w_gate, "w_gate", nexperts, inter * _block_multiple(wtype_gu, hidden, "hidden"), dev)
    if _expert_weights(w_up, "w_up", nexperts, gu_stride, dev) != gu_stride:
        raise ValueError("w_up must have w_gate's shape")
    d_stride = _expert_weights(w_down, "w_down", nexperts, hidden * _block_multiple(wtype_down, inter, "inter"), dev)
    _grid_arg(wtype_gu if wtype_gu == QMM_CB3 else wtype_down, grid, dev)
    col_bytes = (hidden // 32) * Q8_1_BYTES
    _need(xq, "xq", "u8", col_bytes, dev)
    if _nbytes(xq) % col_bytes:
        raise ValueError("xq must hold whole q8_1 columns of width hidden")
    xq_cols = _nbytes(xq) // col_bytes
    ngroups = int(group_expert.numel())
    nentries = int(entry_col.numel())
    _need(group_expert, "group_expert", "i32", 0, dev)
    _need(group_entry_off, "group_entry_off", "i32", (ngroups + 1) * 4, dev)
    _need(entry_col, "entry_col", "i32", 0, dev)
    y = _out(y, "y", "f32", nentries * hidden * 4, dev, (nentries, hidden), torch.float32)
    need = qgemv_grouped_experts_workspace(inter, nentries, flags)
    ws = _out(ws, "ws", "u8", need, dev, (max(need, 16),), torch.uint8)
    _check("qgemv_grouped_experts", lib().qgemv_grouped_experts(
        wtype_gu, _ptr(w_gate), _ptr(w_up), gu_stride, wtype_down, _ptr(w_down), d_stride, nexperts, _ptr(grid),
        hidden, inter, _ptr(xq), xq_cols, _ptr(group_expert), _ptr(group_entry_off), ngroups, _ptr(entry_col),
        nentries, _ptr(y), _ptr(ws), _nbytes(ws), flags, _stream(stream, dev)))
    return y, ws


def qgemv_grouped_experts_noalloc(wtype_gu, w_gate, w_up, wtype_down, w_down, hidden, inter, xq, group_expert,
                                  group_entry_off, entry_col, grid=None, y=None, stream=None):
    """The grouped MoE decode without a workspace: H lives in the library's fixed device array
    (qgemv_grouped_experts_noalloc_max_bytes() bytes per GPU; calls that overlap on one GPU race).
    Arguments as qgemv_grouped_experts; returns y [nentries, hidden] float32."""
    import torch
    if getattr(w_gate, "dim", lambda: 0)() < 1:
        raise ValueError("w_gate must be [nexperts, ...]")
    dev = w_gate.device
    nexperts = int(w_gate.shape[0])
    gu_stride = _expert_weights(w_gate, "w_gate", nexperts, inter * _block_multiple(wtype_gu, hidden, "hidden"), dev)
    if _expert_weights(w_up, "w_up", nexperts, gu_stride, dev) != gu_stride:
        raise ValueError("w_up must have w_gate's shape")
    d_stride = _expert_weights(w_down, "w_down", nexperts, hidden * _block_multiple(wtype_down, inter, "inter"), dev)
    _grid_arg(wtype_gu if wtype_gu == QMM_CB3 else wtype_down, grid, dev)
    col_bytes = (hidden // 32) * Q8_1_BYTES
    _need(xq, "xq", "u8", col_bytes, dev)
    if _nbytes(xq) % col_bytes:
        raise ValueError("xq must hold whole q8_1 columns of width hidden")
    ngroups = int(group_expert.numel())
    nentries = int(entry_col.numel())
    _need(group_expert, "group_expert", "i32", 0, dev)
    _need(group_entry_off, "group_entry_off", "i32", (ngroups + 1) * 4, dev)
    _need(entry_col, "entry_col", "i32", 0, dev)
    y = _out(y, "y", "f32", nentries * hidden * 4, dev, (nentries, hidden), torch.float32)
    _check("qgemv_grouped_experts_noalloc", lib().qgemv_grouped_experts_noalloc(
        wtype_gu, _ptr(w_gate), _ptr(w_up), gu_stride, wtype_down, _ptr(w_down), d_stride, nexperts, _ptr(grid),
        hidden, inter, _ptr(xq), _nbytes(xq) // col_bytes, _ptr(group_expert), _ptr(group_entry_off), ngroups,
        _ptr(entry_col), nentries, _ptr(y), _stream(stream, dev)))
    return y


def qgemm_prefill_experts_workspace(nexperts, inter, nentries, flags=0):
    return int(lib().qgemm_prefill_experts_workspace(nexperts, inter, nentries, flags))


def qgemm_prefill_experts(wtype_gu, w_gate, w_up, wtype_down, w_down, nexperts, hidden, inter, x_f16, sorted_tok,
                          expert_off, y=None, ws=None, flags=0, stream=None):
    """Prefill grouped expert GEMM; returns (y [nentries, hidden] float32, ws)."""
    import torch
    if getattr(x_f16, "dim", lambda: 0)() != 2 or x_f16.shape[1] != hidden:
        raise ValueError("x_f16 must be [ntok, hidden]")
    dev = x_f16.device
    ntok = int(x_f16.shape[0])
    _need(x_f16, "x_f16", "f16", ntok * hidden * 2, dev)
    gu_stride = inter * _block_multiple(wtype_gu, hidden, "hidden")
    d_stride = hidden * _block_multiple(wtype_down, inter, "inter")
    for t, n, s in ((w_gate, "w_gate", gu_stride), (w_up, "w_up", gu_stride), (w_down, "w_down", d_stride)):
        if t is None or int(t.numel()) * int(t.element_size()) != nexperts * s:
            raise ValueError(f"{n} must hold {nexperts} expert matrices of {s} bytes")
        _need(t, n, "u8", nexperts * s, dev)
    nentries = int(sorted_tok.numel())
    _need(sorted_tok, "sorted_tok", "i32", 0, dev)
    _need(expert_off, "expert_off", "i32", (nexperts + 1) * 4, dev)
    y = _out(y, "y", "f32", nentries * hidden * 4, dev, (nentries, hidden), torch.float32)
    need = qgemm_prefill_experts_workspace(nexperts, inter, nentries, flags)
    ws = _out(ws, "ws", "u8", need, dev, (max(need, 16),), torch.uint8)
    _check("qgemm_prefill_experts", lib().qgemm_prefill_experts(
        wtype_gu, _ptr(w_gate), _ptr(w_up), gu_stride, wtype_down, _ptr(w_down), d_stride, nexperts, hidden, inter,
        _ptr(x_f16), ntok, _ptr(sorted_tok), _ptr(expert_off), nentries, _ptr(y), _ptr(ws), _nbytes(ws), flags,
        _stream(stream, dev)))
    return y, ws


def qmm_moe_combine(y, row_idx, weights, out=None, ldo=None, stream=None):
    """Router-weighted sum of each token's expert rows in k order: y float32 [nrows, hidden],
    row_idx int32 [ntok, topk], weights float32 [ntok, topk] -> out float32 [ntok, ldo]."""
    import torch
    if getattr(y, "dim", lambda: 0)() != 2 or getattr(row_idx, "dim", lambda: 0)() != 2:
        raise ValueError("y must be [nrows, hidden] and row_idx [ntok, topk]")
    nrows, hidden = int(y.shape[0]), int(y.shape[1])
    ntok, topk = int(row_idx.shape[0]), int(row_idx.shape[1])
    dev = y.device
    _need(y, "y", "f32", nrows * hidden * 4, dev)
    _need(row_idx, "row_idx", "i32", ntok * topk * 4, dev)
    _need(weights, "weights", "f32", ntok * topk * 4, dev)
    ldo = hidden if ldo is None else ldo
    if ldo < hidden:
        raise ValueError("ldo < hidden")
    out = _out(out, "out", "f32", (max(ntok, 1) - 1) * ldo * 4 + hidden * 4, dev, (ntok, ldo), torch.float32)
    _check("qmm_moe_combine", lib().qmm_moe_combine(_ptr(y), nrows, hidden, _ptr(row_idx), _ptr(weights), ntok, topk,
                                                   _ptr(out), ldo, _stream(stream, dev)))
    return out


def qmm_pack_planes(wtype, w, nrows, k, out=None, stream=None):
    """Q8_0 / IQ4_NL rows repacked into planes (16-block tiles: factor bytes, then scales) in a
    caller-owned uint8 buffer of the blocks' size; returns it."""
    import torch
    if wtype not in (QMM_Q8_0, QMM_IQ4_NL):
        raise ValueError("planes are Q8_0 or IQ4_NL")
    rb = _block_multiple(wtype, k)
    _need(w, "w", "u8", nrows * rb)
    out = _out(out, "out", "u8", nrows * rb, w.device, (nrows, rb), torch.uint8)
    _check("qmm_pack_planes", lib().qmm_pack_planes(wtype, _ptr(w), nrows, k, _ptr(out), _stream(stream, w.device)))
    return out


class Planes:
    """A packed copy owned by the library's allocation (qmm_planes_alloc), freed by release()
    (qmm_planes_release) or when the object is collected."""

    def __init__(self, wtype, w, nrows, k, stream=None):
        if wtype not in (QMM_Q8_0, QMM_IQ4_NL):
            raise ValueError("planes are Q8_0 or IQ4_NL")
        rb = _block_multiple(wtype, k)
        _need(w, "w", "u8", nrows * rb)
        self.wtype, self.nrows, self.k, self.device, self.nbytes = wtype, nrows, k, w.device, nrows * rb
        self.ptr = C.c_void_p()
        _check("qmm_planes_alloc", lib().qmm_planes_alloc(wtype, _ptr(w), nrows, k, C.byref(self.ptr),
                                                          _stream(stream, w.device)))

    def release(self):
        if self.ptr:
            _check("qmm_planes_release", lib().qmm_planes_release(self.ptr))
            self.ptr = C.c_void_p()

    def __del__(self):
        try:
            self.release()
        except Exception:
            pass


def qgemv_planes(wtype, planes, nrows, k, xq, ncols, y=None, ldy=None, stream=None):
    """qgemv_dense on planes (a uint8 tensor from qmm_pack_planes, or a Planes object): y
    float32 [ncols, ldy], bitwise qgemv_dense on the original blocks."""
    import torch
    if isinstance(planes, Planes):
        if (planes.wtype, planes.nrows, planes.k) != (wtype, nrows, k) or not planes.ptr:
            raise ValueError("the packed copy holds another matrix (or was released)")
        dev, ptr = planes.device, planes.ptr
        ldy = _gemv_common(wtype, None, nrows, k, ncols, None, ldy, check_w=False)
    else:
        ldy = _gemv_common(wtype, planes, nrows, k, ncols, None, ldy)
        dev, ptr = planes.device, _ptr(planes)
    _need(xq, "xq", "u8", ncols * (k // 32) * Q8_1_BYTES, dev)
    y = _out(y, "y", "f32", ((ncols - 1) * ldy + nrows) * 4, dev, (ncols, ldy), torch.float32)
    _check("qgemv_planes", lib().qgemv_planes(wtype, ptr, nrows, k, _ptr(xq), ncols, _ptr(y), ldy,
                                             _stream(stream, dev)))
    return y


def qgemm_dense(wtype, w, nrows, k, x_f16, y=None, ldy=None, stream=None):
    """Dense prompt projection y [ntok, ldy] float32 = X16 . W16^T: w Q8_0 / IQ4_NL blocks
    (converted to FP16 in the GEMM) or binary16 [nrows, k] (QMM_F16); x_f16 [ntok, k]."""
    import torch
    if wtype not in (QMM_Q8_0, QMM_IQ4_NL, QMM_F16):
        raise ValueError("dense projections take Q8_0, IQ4_NL or F16 weights")
    rb = _block_multiple(wtype, k)
    if getattr(x_f16, "dim", lambda: 0)() != 2 or x_f16.shape[1] != k:
        raise ValueError("x_f16 must be [ntok, k]")
    ntok = int(x_f16.shape[0])
    ldy = nrows if ldy is None else ldy
    if nrows < 1 or ldy < nrows:
        raise ValueError("nrows >= 1 and ldy >= nrows")
    _need(w, "w", "f16" if wtype == QMM_F16 else "u8", nrows * rb)
    _need(x_f16, "x_f16", "f16", ntok * k * 2, w.device)
    y = _out(y, "y", "f32", (max(ntok, 1) - 1) * ldy * 4 + nrows * 4, w.device, (ntok, ldy), torch.float32)
    _check("qgemm_dense", lib().qgemm_dense(wtype, _ptr(w), nrows, k, _ptr(x_f16), ntok, _ptr(y), ldy,
                                           _stream(stream, w.device)))
    return y


def qgemm_prefill_experts_q8_workspace(nexperts, hidden, inter, ntok, nentries, flags=0):
    return int(lib().qgemm_prefill_experts_q8_workspace(nexperts, hidden, inter, ntok, nentries, flags))


def qgemm_prefill_experts_q8(wtype_gu, w_gate, w_up, wtype_down, w_down, nexperts, hidden, inter, x_f16, sorted_tok,
                             expert_off, y=None, ws=None, flags=0, stream=None):
    """MMQ-style prefill (int8 MFMA, q8_1 activations, SwiGLU + q8_1 of H fused); arguments as
    qgemm_prefill_experts; returns (y [nentries, hidden] float32, ws)."""
    import torch
    if getattr(x_f16, "dim", lambda: 0)() != 2 or x_f16.shape[1] != hidden:
        raise ValueError("x_f16 must be [ntok, hidden]")
    dev = x_f16.device
    ntok = int(x_f16.shape[0])
    _need(x_f16, "x_f16", "f16", ntok * hidden * 2, dev)
    gu_stride = inter * _block_multiple(wtype_gu, hidden, "hidden")
    d_stride = hidden * _block_multiple(wtype_down, inter, "inter")
    for t, n, s in ((w_gate, "w_gate", gu_stride), (w_up, "w_up", gu_stride), (w_down, "w_down", d_stride)):
        if t is None or int(t.numel()) * int(t.element_size()) != nexperts * s:
            raise ValueError(f"{n} must hold {nexperts} expert matrices of {s} bytes")
        _need(t, n, "u8", nexperts * s, dev)
    nentries = int(sorted_tok.numel())
    _need(sorted_tok, "sorted_tok", "i32", 0, dev)
    _need(expert_off, "expert_off", "i32", (nexperts + 1) * 4, dev)
    y = _out(y, "y", "f32", nentries * hidden * 4, dev, (nentries, hidden), torch.float32)
    need = qgemm_prefill_experts_q8_workspace(nexperts, hidden, inter, ntok, nentries, flags)
    ws = _out(ws, "ws", "u8", need, dev, (max(need, 16),), torch.uint8)
    _check("qgemm_prefill_experts_q8", lib().qgemm_prefill_experts_q8(
        wtype_gu, _ptr(w_gate), _ptr(w_up), gu_stride, wtype_down, _ptr(w_down), d_stride, nexperts, hidden, inter,
        _ptr(x_f16), ntok, _ptr(sorted_tok), _ptr(expert_off), nentries, _ptr(y), _ptr(ws), _nbytes(ws), flags,
        _stream(stream, dev)))
    return y, ws
