"""GPU parity of the dense prompt projection (qgemm_dense): Q8_0 / IQ4_NL weights converted to
FP16 inside the GEMM, and the two-step path (qmm_dequant_f16, then the GEMM on binary16
weights), against the oracle's FP16 product within 1e-4 * sum|w x|; the two paths bitwise equal
(the same FP16 operands summed in the same order); one-hot tokens give the FP16 weights exactly."""
import numpy as np
import pytest

import moe_expert_amd as M
import oracle
import synth
from tests.gpu_util import check_tol, dev, host

pytestmark = pytest.mark.gpu


def weights(wt, rng, nrows, k):
    return synth.weights(wt, rng, nrows, k, **(dict(qlo=-128) if wt == M.QMM_Q8_0 else {}))


def both_paths(wt, w, nrows, k, x16):
    """(fused y, two-step y) on the GPU."""
    wd = dev(w)
    xd = dev(x16.view(np.uint16))
    y = host(M.qgemm_dense(wt, wd, nrows, k, xd))
    w16 = M.qmm_dequant_f16(wt, wd, nrows, k)
    y2 = host(M.qgemm_dense(M.QMM_F16, w16, nrows, k, xd))
    return y, y2


@pytest.mark.parametrize("wt", [M.QMM_Q8_0, M.QMM_IQ4_NL])
@pytest.mark.parametrize("nrows,k,ntok", [(100, 256, 37), (256, 320, 300), (300, 2560, 257), (64, 64, 1),
                                          (513, 1024, 64)])
def test_dense_small(wt, nrows, k, ntok):
    """Partial token tiles (1, 37, 257, 300 tokens), partial column tiles (100, 300, 513 rows),
    odd numbers of 64-wide K steps (k = 64, 320)."""
    print(f"dense gemm wtype={wt} nrows={nrows} k={k} ntok={ntok}", flush=True)
    rng = synth.rng_for(2800 + nrows + ntok)
    w = weights(wt, rng, nrows, k)
    x16 = synth.prefill_tokens(rng, ntok, k)
    y, y2 = both_paths(wt, w, nrows, k, x16)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))
    ref, a = oracle.dense_rows(wt, w, nrows, k, x16, np.arange(ntok))
    check_tol(y, ref, a, what="dense")


@pytest.mark.parametrize("wt", [M.QMM_Q8_0, M.QMM_IQ4_NL])
def test_dense_onehot_tokens_give_the_weights(wt):
    """X16 = I (token t = e_t): every product but one is a zero, so y[t][r] = W16[r][t] exactly,
    for all of a 1024 x 1024 matrix."""
    print(f"dense gemm one-hot tokens wtype={wt}", flush=True)
    rng = synth.rng_for(2900 + wt)
    nrows = k = 1024
    w = weights(wt, rng, nrows, k)
    y, y2 = both_paths(wt, w, nrows, k, np.eye(k, dtype=np.float16))
    w16 = oracle.dequant_f16(wt, w, k).view(np.float16).astype(np.float32)
    assert np.array_equal(y, w16.T) and np.array_equal(y2, w16.T)


def test_dense_ldy_padding():
    import torch
    print("dense gemm ldy padding", flush=True)
    rng = synth.rng_for(2950)
    w = weights(M.QMM_IQ4_NL, rng, 90, 512)
    x16 = synth.prefill_tokens(rng, 40, 512)
    y = torch.full((40, 96), 7.0, device="cuda")
    M.qgemm_dense(M.QMM_IQ4_NL, dev(w), 90, 512, dev(x16.view(np.uint16)), y=y, ldy=96)
    yh = host(y)
    assert (yh[:, 90:] == 7.0).all()
    ref, a = oracle.dense_rows(M.QMM_IQ4_NL, w, 90, 512, x16, np.arange(40))
    check_tol(yh[:, :90], ref, a)


@pytest.mark.parametrize("wt,nrows,key", [(M.QMM_IQ4_NL, 8192, "iq4nl_8192x2560"), (M.QMM_Q8_0, 12288, "q8_0_12288x2560")])
def test_dense_full_size(wt, nrows, key):
    """8192 prompt tokens through the decode workloads' matrices (2560 -> 8192 IQ4_NL, 2560 ->
    12288 Q8_0): the first and the last token tile whole and 64 random tokens, every output of
    those rows against the oracle."""
    print(f"dense gemm full size: 8192 tokens x {nrows}x2560", flush=True)
    k, ntok = 2560, 8192
    w = synth.weights(wt, synth.rng_for(synth.SEEDS[key]), nrows, k)
    x16 = synth.prefill_tokens(synth.rng_for(synth.SEEDS[key] + 200), ntok, k)
    y, y2 = both_paths(wt, w, nrows, k, x16)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))
    rng = synth.rng_for(2960)
    rows = np.unique(np.concatenate([np.arange(256), np.arange(ntok - 256, ntok), rng.choice(ntok, 64, replace=False)]))
    ref, a = oracle.dense_rows(wt, w, nrows, k, x16, rows)
    check_tol(y[rows], ref, a, what="dense full size")
