"""GPU parity: q8_1 quantization bytes and FP16 dequantization bits against the oracle
(bit-exact)."""
import numpy as np
import pytest

import moe_expert_amd as M
import oracle
import synth
from tests.gpu_util import dev, host
from tests.oracle_pins import finite_f16_patterns

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("ncols,k,seed", [(1, 32, 1), (3, 2560, 2), (8, 6144, 3), (5, 1024, 4), (2, 96, 5)])
def test_quantize_bytes(ncols, k, seed):
    print(f"quantize ncols={ncols} k={k} seed={seed}", flush=True)
    rng = synth.rng_for(seed)
    x = synth.activations(rng, ncols, k)
    x *= np.exp2(rng.uniform(-20, 12, size=(ncols, 1))).astype(np.float32)
    x[:, 64:96] = 0.0 if k >= 96 else x[:, 64:96]          # a zero block
    if k >= 64:
        x[0, 7] = 3e4                                      # an outlier
    ref = oracle.quantize_q8_1(x)
    got = host(M.qmm_quantize_q8_1(dev(x)))
    assert np.array_equal(got, ref), f"{(got != ref).sum()} bytes differ"


def test_quantize_extreme_blocks():
    print("quantize extreme blocks", flush=True)
    rng = synth.rng_for(6)
    x = (rng.standard_normal((1, 32 * 4000)) * np.exp2(rng.uniform(-140, 120, (1, 32 * 4000)))).astype(np.float32)
    x = x.reshape(4000, 32)
    x *= np.exp2(rng.uniform(-60, 60, (4000, 1))).astype(np.float32)
    x = np.nan_to_num(x, posinf=3e38, neginf=-3e38).astype(np.float32).reshape(1, -1)
    ref = oracle.quantize_q8_1(x)
    got = host(M.qmm_quantize_q8_1(dev(x)))
    assert np.array_equal(got, ref), f"{(got != ref).sum()} bytes differ"


def test_quantize_near_ties():
    """Quotients x / d within a few binary32 ulp of half-integers (and exactly on them), for
    scales d that are not powers of two, where the quotient's rounding decides the byte: the
    quantizer's bytes equal the oracle's (its division) on every value."""
    print("quantize near ties", flush=True)
    rng = synth.rng_for(7)
    nblk = 6000
    amax = np.exp2(rng.uniform(-30, 30, nblk)).astype(np.float32) * rng.uniform(1, 2, nblk).astype(np.float32)
    d = (amax / np.float32(127.0)).astype(np.float32)
    k = rng.integers(-127, 127, size=(nblk, 31)).astype(np.float64) + 0.5
    rel = rng.choice(np.array([0.0, 1e-7, -1e-7, 3e-7, -3e-7, 2e-6, -2e-6, 1.5e-5, -1.5e-5, 3e-5, -3e-5]), size=(nblk, 31))
    x = np.empty((nblk, 32), np.float32)
    x[:, 0] = amax * np.where(rng.random(nblk) < 0.5, 1, -1).astype(np.float32)
    x[:, 1:] = (k * (1.0 + rel) * d[:, None].astype(np.float64)).astype(np.float32)
    x[:, 1:] = np.clip(x[:, 1:], -amax[:, None], amax[:, None])
    x = x.reshape(1, -1)
    ref = oracle.quantize_q8_1(x)
    got = host(M.qmm_quantize_q8_1(dev(x)))
    assert np.array_equal(got, ref), f"{(got != ref).sum()} bytes differ"


def test_quantize_rejects_ldx():
    assert M.lib().qmm_quantize_q8_1(None, 64, 1, 64, None, None) == -1


@pytest.mark.parametrize("wtype", [M.QMM_Q8_0, M.QMM_IQ4_NL, M.QMM_CB3])
def test_dequant_every_scale(wtype):
    """Every finite fp16 scale, random factors (Q8_0: over all of [-128, 127]): bit-exact FP16."""
    print(f"dequant every scale wtype={wtype}", flush=True)
    rng = synth.rng_for(100 + wtype)
    d = finite_f16_patterns()
    bv = synth.BLOCK_VALUES[wtype]
    bb = synth.BLOCK_BYTES[wtype]
    nblk = d.size
    k = bv * 8
    grid = synth.cb3_grid(rng) if wtype == M.QMM_CB3 else None
    kw = dict(qlo=-128) if wtype == M.QMM_Q8_0 else {}     # every int8 factor, -128 included
    w = synth.weights(wtype, rng, nblk // 8 + 1, k, **kw).reshape(-1, bb)[:nblk].copy()
    w[:, 0:2] = d.view(np.uint8).reshape(-1, 2)
    if wtype == M.QMM_Q8_0:
        assert (w[:, 2:].view(np.int8) == -128).any() and (w[:, 2:].view(np.int8) == 127).any()
    w = w[: (nblk // 8) * 8].reshape(-1, 8 * bb)
    ref = oracle.dequant_f16(wtype, w, k, grid)
    got = host(M.qmm_dequant_f16(wtype, dev(w), w.shape[0], k, grid=None if grid is None else dev(grid)))
    assert np.array_equal(got.view(np.uint16), ref)


@pytest.mark.parametrize("wtype,nrows,k,ld", [(M.QMM_Q8_0, 37, 2560, 2568), (M.QMM_IQ4_NL, 5, 1024, 1027),
                                              (M.QMM_CB3, 9, 2560, 2560), (M.QMM_IQ4_NL, 64, 2560, 2560)])
def test_dequant_strides(wtype, nrows, k, ld):
    """Padded ld (16-byte path), an odd ld (scalar path); padding left untouched."""
    print(f"dequant strides wtype={wtype} nrows={nrows} k={k} ld={ld}", flush=True)
    import torch
    rng = synth.rng_for(200 + nrows)
    grid = synth.cb3_grid(rng) if wtype == M.QMM_CB3 else None
    w = synth.weights(wtype, rng, nrows, k)
    ref = oracle.dequant_f16(wtype, w, k, grid, ld=ld)
    out = torch.zeros((nrows, ld), dtype=torch.float16, device="cuda")
    M.qmm_dequant_f16(wtype, dev(w), nrows, k, grid=None if grid is None else dev(grid), out=out, ld=ld)
    assert np.array_equal(host(out).view(np.uint16), ref)
