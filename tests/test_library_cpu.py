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


def test_quantize_and_dequant_reject():
    L = M.lib()
    assert L.qmm_quantize_q8_1(None, 64, 1, 64, FAKE, None) == -1
    assert L.qmm_quantize_q8_1(FAKE, 48, 1, 48, FAKE, None) == -1
    assert L.qmm_quantize_q8_1(FAKE, 64, 1, 32, FAKE, None) == -1
    assert L.qmm_quantize_q8_1(ODD, 64, 1, 64, FAKE, None) == -3
    assert L.qmm_dequant_f16(M.QMM_IQ4_NL, FAKE, None, 4, 64, FAKE, 32, None) == -1
    assert L.qmm_dequant_f16(M.QMM_CB3, FAKE, None, 4, 256, FAKE, 256, None) == -1
    assert L.qmm_dequant_f16(M.QMM_Q8_0, C.c_void_p(0x100001), None, 4, 64, FAKE, 64, None) == -3
