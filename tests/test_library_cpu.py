"""The C-ABI library loads, exports every entry point include/qmm.h declares, and rejects bad
arguments before launching anything.  CPU only: no call here reaches a kernel launch."""
import ctypes as C
import os
import re

import pytest

import moe_expert_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmm.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", src)) - {"defined"})


def test_every_declared_symbol_is_exported():
    L = M.lib()
    names = declared_functions()
    assert "qgemv_dense" in names and "qgemm_prefill_experts" in names
    for n in names:
        assert hasattr(L, n), n
        assert n in M.SIGNATURES, f"binding lacks {n}"


def test_binding_names_are_declared():
    assert set(M.SIGNATURES) == set(declared_functions())


def test_row_bytes_and_status():
    assert M.row_bytes(M.QMM_Q8_0, 2560) == 2720
    assert M.row_bytes(M.QMM_IQ4_NL, 2560) == 1440
    assert M.row_bytes(M.QMM_CB3, 2560) == 1100
    assert M.row_bytes(M.QMM_CB3, 2560 + 32) == 0
    assert M.row_bytes(M.QMM_Q8_0, 33) == 0
    assert M.row_bytes(9, 64) == 0
    assert M.lib().qmm_version() >= 100
    for s in (0, -1, -2, -3, -4, -5, 7):
        assert isinstance(M.status_str(s), str)


FAKE = C.c_void_p(0x100000)      # never dereferenced: every call below fails validation first
ODD = C.c_void_p(0x100002)


@pytest.mark.parametrize("args,expect", [
    ((M.QMM_Q8_0, None, None, 64, 2560, FAKE, 1, FAKE, 64, None), -1),       # null weights
    ((7, FAKE, None, 64, 2560, FAKE, 1, FAKE, 64, None), -1),                # unknown format
    ((M.QMM_Q8_0, FAKE, None, 64, 2560, FAKE, 0, FAKE, 64, None), -1),       # no columns
    ((M.QMM_Q8_0, FAKE, None, 64, 2561, FAKE, 1, FAKE, 64, None), -1),       # k not a block multiple
    ((M.QMM_Q8_0, FAKE, None, 0, 2592, FAKE, 1, FAKE, 64, None), -1),        # no rows
    ((M.QMM_CB3, FAKE, FAKE, 64, 2560 + 64, FAKE, 1, FAKE, 64, None), -1),   # CB3 needs 256-multiples
    ((M.QMM_CB3, FAKE, None, 64, 2560, FAKE, 1, FAKE, 64, None), -1),        # CB3 without a grid
    ((M.QMM_Q8_0, ODD, None, 64, 2560, FAKE, 1, FAKE, 64, None), -3),        # misaligned weights
    ((M.QMM_Q8_0, FAKE, None, 64, 2560, FAKE, 1, FAKE, 63, None), -1),       # ldy < nrows
    ((M.QMM_Q8_0, FAKE, None, 64, 65536, FAKE, 1, FAKE, 64, None), -2),      # k beyond the limit
])
def test_qgemv_dense_rejects(args, expect):
    assert M.lib().qgemv_dense(*args) == expect


@pytest.mark.parametrize("args,expect", [
    ((M.QMM_Q8_0, FAKE, None, 64, 2560, None, 1, FAKE, 64, None), -1),      # null activations
    ((M.QMM_Q8_0, FAKE, None, 64, 2561, FAKE, 1, FAKE, 64, None), -1),      # k not a block multiple
    ((M.QMM_CB3, FAKE, None, 64, 2560, FAKE, 1, FAKE, 64, None), -1),       # CB3 without a grid
    ((M.QMM_Q8_0, FAKE, None, 64, 2560, ODD, 1, FAKE, 64, None), -3),       # misaligned activations
    ((M.QMM_Q8_0, FAKE, None, 64, 2560, FAKE, 2, FAKE, 63, None), -1),      # ldy < nrows
    ((M.QMM_Q8_0, FAKE, None, 64, 3104, FAKE, 1, FAKE, 64, None), -2),      # rows of more than 96 blocks
    ((M.QMM_Q8_0, FAKE, None, 64, 2560, FAKE, 3, FAKE, 64, None), -2),      # 3 columns
    ((M.QMM_Q8_0, FAKE, None, 64, 2560, FAKE, 8, FAKE, 64, None), -2),      # 8 columns
])
def test_qgemv_dense_f32_rejects(args, expect):
    assert M.lib().qgemv_dense_f32(*args) == expect


def test_quantize_and_dequant_reject():
    L = M.lib()
    assert L.qmm_quantize_q8_1(None, 64, 1, 64, FAKE, None) == -1
    assert L.qmm_quantize_q8_1(FAKE, 48, 1, 48, FAKE, None) == -1
    assert L.qmm_quantize_q8_1(FAKE, 64, 1, 32, FAKE, None) == -1
    assert L.qmm_quantize_q8_1(ODD, 64, 1, 64, FAKE, None) == -3
    assert L.qmm_dequant_f16(M.QMM_IQ4_NL, FAKE, None, 4, 64, FAKE, 32, None) == -1
    assert L.qmm_dequant_f16(M.QMM_CB3, FAKE, None, 4, 256, FAKE, 256, None) == -1
    assert L.qmm_dequant_f16(M.QMM_Q8_0, C.c_void_p(0x100001), None, 4, 64, FAKE, 64, None) == -3


def _gu_args(**kw):
    """qgemv_grouped_experts arguments for 4 experts 2560 -> 1024 (IQ4_NL / Q8_0), valid apart
    from what `kw` changes."""
    a = dict(wtype_gu=M.QMM_IQ4_NL, w_gate=FAKE, w_up=FAKE, gu_stride=1024 * 1440, wtype_down=M.QMM_Q8_0,
             w_down=FAKE, d_stride=2560 * 1088, nexperts=4, grid=None, hidden=2560, inter=1024, xq=FAKE,
             xq_cols=2, ge=FAKE, go=FAKE, ngroups=2, ec=FAKE, nentries=4, y=FAKE, ws=FAKE,
             ws_bytes=1 << 30, flags=0, stream=None)
    a.update(kw)
    return tuple(a.values())


@pytest.mark.parametrize("kw,expect", [
    (dict(w_up=None), -1),
    (dict(wtype_gu=M.QMM_CB3), -1),                            # CB3 without a grid
    (dict(gu_stride=1024 * 1440 - 4), -1),                     # stride below one matrix
    (dict(gu_stride=1024 * 1440 + 2), -3),                     # stride not a multiple of 4
    (dict(hidden=2560 + 16), -1),                              # not a block multiple
    (dict(inter=65536), -2),                                   # beyond the K limit
    (dict(ngroups=70000), -2),
    (dict(ws=ODD), -3),
    (dict(ws_bytes=16), -5),
    (dict(ngroups=0), 0),                                      # nothing to do: no launch
])
def test_grouped_rejects(kw, expect):
    assert M.lib().qgemv_grouped_experts(*_gu_args(**kw)) == expect


def _pf_args(**kw):
    """qgemm_prefill_experts arguments for 4 experts 2560 -> 1024 (IQ4_NL / Q8_0), valid apart
    from what `kw` changes."""
    a = dict(wtype_gu=M.QMM_IQ4_NL, w_gate=FAKE, w_up=FAKE, gu_stride=1024 * 1440, wtype_down=M.QMM_Q8_0,
             w_down=FAKE, d_stride=2560 * 1088, nexperts=4, hidden=2560, inter=1024, x=FAKE, ntok=64,
             st=FAKE, off=FAKE, nentries=128, y=FAKE, ws=FAKE, ws_bytes=1 << 30, flags=0, stream=None)
    a.update(kw)
    return tuple(a.values())


@pytest.mark.parametrize("kw,expect", [
    (dict(wtype_down=9), -1),
    (dict(x=None), -1),
    (dict(wtype_gu=M.QMM_CB3, gu_stride=1024 * 1100), -2),    # no codebook argument
    (dict(hidden=2560 + 32), -2),                              # K steps of 64
    (dict(inter=1024 + 32, d_stride=2560 * 1122), -2),
    (dict(d_stride=2560 * 1088 - 4), -1),
    (dict(x=C.c_void_p(0x100008)), -3),                        # x_f16 must be 16-byte aligned
    (dict(ws_bytes=64), -5),
    (dict(nentries=0, ws_bytes=4096), 0),                      # nothing to do: no launch
    (dict(ntok=1 << 20), -2),                                  # x_f16 of 4 GiB or more
])
def test_prefill_rejects(kw, expect):
    assert M.lib().qgemm_prefill_experts(*_pf_args(**kw)) == expect
    assert M.lib().qgemm_prefill_experts_workspace(4, 1024, 128, 0) >= 128 * 1024 * 2


def test_prefill_rejects_offsets_that_would_wrap():
    """x_f16 whose size plus the zero-read headroom (2 hidden + 128 bytes) passes 4 GiB."""
    assert M.lib().qgemm_prefill_experts(*_pf_args(ntok=838860)) == -2
    assert M.lib().qgemm_prefill_experts(*_pf_args(ntok=838859, ws_bytes=64)) == -5   # passes that check


# ------------------------------------------------------------------ binding checks (no GPU)

class FakeGpuTensor:
    """Duck-typed stand-in for a contiguous GPU tensor: the binding's checks read only these
    attributes, and every case below is refused before its pointer would be used."""

    def __init__(self, shape, dtype, device="cuda:0", contiguous=True):
        import torch
        self.shape = tuple(shape)
        self.dtype = dtype
        self.device = torch.device(device)
        self.is_cuda = self.device.type == "cuda"
        self._contiguous = contiguous

    def numel(self):
        n = 1
        for s in self.shape:
            n *= s
        return n

    def element_size(self):
        import torch
        return torch.empty((), dtype=self.dtype).element_size()

    def dim(self):
        return len(self.shape)

    def is_contiguous(self):
        return self._contiguous

    def data_ptr(self):
        raise AssertionError("the binding must refuse this call before reading a pointer")

    def __getitem__(self, i):
        return FakeGpuTensor(self.shape[1:], self.dtype, str(self.device))

    def view(self, *shape):
        return FakeGpuTensor(shape, self.dtype, str(self.device))


def _gemv_tensors(**kw):
    import torch
    t = dict(w=FakeGpuTensor((64, 1440), torch.uint8), xq=FakeGpuTensor((2, 2880), torch.uint8),
             y=FakeGpuTensor((2, 64), torch.float32))
    t.update(kw)
    return t


@pytest.mark.parametrize("change", [
    "y_short", "y_dtype", "xq_short", "xq_dtype", "w_short", "w_cpu", "w_strided", "xq_other_gpu", "k_ragged"])
def test_binding_refuses_bad_gemv_tensors(change):
    import torch
    F = FakeGpuTensor
    kw = {"y_short": dict(y=F((2, 63), torch.float32)), "y_dtype": dict(y=F((2, 64), torch.float16)),
          "xq_short": dict(xq=F((1, 2880), torch.uint8)), "xq_dtype": dict(xq=F((2, 720), torch.float32)),
          "w_short": dict(w=F((63, 1440), torch.uint8)), "w_cpu": dict(w=F((64, 1440), torch.uint8, "cpu")),
          "w_strided": dict(w=F((64, 1440), torch.uint8, contiguous=False)),
          "xq_other_gpu": dict(xq=F((2, 2880), torch.uint8, "cuda:1")), "k_ragged": {}}[change]
    t = _gemv_tensors(**kw)
    k = 2576 if change == "k_ragged" else 2560
    with pytest.raises(ValueError):
        M.qgemv_dense(M.QMM_IQ4_NL, t["w"], 64, k, t["xq"], 2, y=t["y"])


def test_binding_refuses_bad_grouped_and_prefill_tensors():
    import torch
    F = FakeGpuTensor
    u8, i32 = torch.uint8, torch.int32
    wg, wd = F((4, 1024 * 1440), u8), F((4, 2560 * 1088), u8)
    xq, ge, go, ec = F((2, 2880), u8), F((2,), i32), F((3,), i32), F((4,), i32)
    # w_up with fewer experts than w_gate
    with pytest.raises(ValueError):
        M.qgemv_grouped_experts(M.QMM_IQ4_NL, wg, F((3, 1024 * 1440), u8), M.QMM_Q8_0, wd, 2560, 1024, xq, ge, go, ec)
    # a short entry-offset array
    with pytest.raises(ValueError):
        M.qgemv_grouped_experts(M.QMM_IQ4_NL, wg, wg, M.QMM_Q8_0, wd, 2560, 1024, xq, ge, F((2,), i32), ec)
    # a float16 x for the prefill is fine, a half-width one is not; int64 token ids are not
    x16 = F((64, 1280), torch.float16)
    st, off = F((128,), i32), F((5,), i32)
    with pytest.raises(ValueError):
        M.qgemm_prefill_experts(M.QMM_IQ4_NL, wg, wg, M.QMM_Q8_0, wd, 4, 2560, 1024, x16, st, off)
    with pytest.raises(ValueError):
        M.qgemm_prefill_experts(M.QMM_IQ4_NL, wg, wg, M.QMM_Q8_0, wd, 4, 2560, 1024, F((64, 2560), torch.float16),
                                F((128,), torch.int64), off)
    # a caller workspace below the query
    with pytest.raises(ValueError):
        M.qgemm_prefill_experts(M.QMM_IQ4_NL, wg, wg, M.QMM_Q8_0, wd, 4, 2560, 1024, F((64, 2560), torch.float16),
                                st, off, y=F((128, 2560), torch.float32), ws=F((64,), u8))


@pytest.mark.parametrize("args,expect", [
    ((None, 8, 64, FAKE, FAKE, 4, 2, FAKE, 64, None), -1),          # null rows
    ((FAKE, 8, 64, FAKE, FAKE, 4, 0, FAKE, 64, None), -1),          # topk 0
    ((FAKE, 8, 64, FAKE, FAKE, 4, 65, FAKE, 64, None), -2),         # topk above 64
    ((FAKE, 8, 66, FAKE, FAKE, 4, 2, FAKE, 68, None), -2),          # hidden not a multiple of 4
    ((FAKE, 8, 64, FAKE, FAKE, 4, 2, FAKE, 60, None), -1),          # ldo < hidden
    ((C.c_void_p(0x100004), 8, 64, FAKE, FAKE, 4, 2, FAKE, 64, None), -3),   # y not 16-byte aligned
    ((FAKE, 8, 64, FAKE, FAKE, 0, 2, FAKE, 64, None), 0),           # no tokens: no launch
])
def test_combine_rejects(args, expect):
    assert M.lib().qmm_moe_combine(*args) == expect


def test_planes_reject():
    L = M.lib()
    A16 = C.c_void_p(0x100000)
    assert L.qgemv_planes(M.QMM_CB3, A16, 64, 2560, FAKE, 1, FAKE, 64, None) == -1    # planes: Q8_0 / IQ4_NL
    assert L.qgemv_planes(M.QMM_Q8_0, A16, 64, 2592, FAKE, 1, FAKE, 64, None) == -2   # rows of whole tiles
    assert L.qgemv_planes(M.QMM_Q8_0, C.c_void_p(0x100004), 64, 2560, FAKE, 1, FAKE, 64, None) == -3
    assert L.qmm_pack_planes(M.QMM_CB3, FAKE, 4, 256, FAKE, None) == -1
    assert L.qmm_pack_planes(M.QMM_Q8_0, FAKE, 4, 48, FAKE, None) == -1
    p = C.c_void_p(123)
    assert L.qmm_planes_alloc(M.QMM_IQ4_NL, None, 4, 64, C.byref(p), None) == -1 and not p.value
    assert L.qmm_planes_release(None) == 0


def test_dense_rejects():
    L = M.lib()
    A16 = C.c_void_p(0x100000)
    assert L.qgemm_dense(M.QMM_CB3, A16, 64, 2560, A16, 8, A16, 64, None) == -1      # no CB3
    assert L.qgemm_dense(M.QMM_Q8_0, A16, 64, 2592, A16, 8, A16, 64, None) == -2     # K steps of 64
    assert L.qgemm_dense(M.QMM_Q8_0, A16, 64, 2560, C.c_void_p(0x100008), 8, A16, 64, None) == -3
    assert L.qgemm_dense(M.QMM_F16, C.c_void_p(0x100004), 64, 2560, A16, 8, A16, 64, None) == -3
    assert L.qgemm_dense(M.QMM_Q8_0, A16, 64, 2560, A16, 8, A16, 63, None) == -1     # ldy < nrows
    assert L.qgemm_dense(M.QMM_Q8_0, A16, 64, 2560, A16, 0, A16, 64, None) == 0      # no tokens
    assert M.row_bytes(M.QMM_F16, 2560) == 5120


@pytest.mark.parametrize("kw,expect", [
    (dict(wtype_down=9), -1),
    (dict(wtype_gu=M.QMM_CB3, gu_stride=1024 * 1100), -2),    # no codebook argument
    (dict(hidden=2560 + 32), -2),                              # K steps of 64
    (dict(ws_bytes=64), -5),
    (dict(nentries=0, ws_bytes=1 << 30), 0),                   # nothing to do: no launch
    (dict(ntok=1677722), -2),                                  # token planes of 4 GiB or more
])
def test_mmq_rejects(kw, expect):
    assert M.lib().qgemm_prefill_experts_q8(*_pf_args(**kw)) == expect
    assert M.lib().qgemm_prefill_experts_q8_workspace(4, 2560, 1024, 64, 128, 0) >= 64 * 2560 + 128 * 1024
