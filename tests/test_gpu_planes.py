"""GPU parity of the weight planes: the packed bytes equal the oracle's planes bit for bit, and
the GEMV on planes equals qgemv_dense on the original blocks bitwise (the same arithmetic in the
same order, only the loads change) and the oracle within the fp32 tolerance."""
import numpy as np
import pytest

import moe_expert_amd as M
import oracle
import synth
from tests.gpu_util import check_tol, dev, host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wtype", [M.QMM_Q8_0, M.QMM_IQ4_NL])
@pytest.mark.parametrize("nrows,nb", [(3, 1), (5, 16), (7, 17), (64, 80), (9, 192), (2, 1030)])
def test_pack_bytes(wtype, nrows, nb):
    print(f"planes pack wtype={wtype} nrows={nrows} blocks={nb}", flush=True)
    kw = dict(qlo=-128) if wtype == M.QMM_Q8_0 else {}
    w = synth.weights(wtype, synth.rng_for(2500 + nb), nrows, 32 * nb, **kw)
    got = host(M.qmm_pack_planes(wtype, dev(w), nrows, 32 * nb))
    assert np.array_equal(got, oracle.pack_planes(wtype, w, 32 * nb))


@pytest.mark.parametrize("wtype", [M.QMM_Q8_0, M.QMM_IQ4_NL])
@pytest.mark.parametrize("nrows,k", [(37, 512), (300, 2560), (129, 6144), (33, 16384), (8192, 2560)])
def test_planes_gemv_equals_blocks(wtype, nrows, k):
    """Rows of 16 lanes (k = 512, 2560) and of one wave (6144, 16384: double-buffered chunks);
    1-8 and 11 columns: each output bitwise the direct-block GEMV's, and within the oracle's
    tolerance."""
    print(f"planes gemv wtype={wtype} nrows={nrows} k={k}", flush=True)
    rng = synth.rng_for(2600 + nrows)
    kw = dict(qlo=-128) if wtype == M.QMM_Q8_0 else {}
    w = synth.weights(wtype, rng, nrows, k, **kw)
    x = synth.activations(rng, 11, k)
    wd = dev(w)
    planes = M.qmm_pack_planes(wtype, wd, nrows, k)
    xq = M.qmm_quantize_q8_1(dev(x))
    for n in (1, 2, 3, 4, 5, 8, 11):
        xn = xq[:n].contiguous()
        yb = host(M.qgemv_dense(wtype, wd, nrows, k, xn, n))
        yp = host(M.qgemv_planes(wtype, planes, nrows, k, xn, n))
        assert np.array_equal(yp.view(np.uint32), yb.view(np.uint32)), n
    ref, a = oracle.gemv(wtype, w, k, host(xq))
    check_tol(yp, ref, a, what="planes gemv")


def test_planes_owned_copy():
    """qmm_planes_alloc packs into a buffer the library allocates; the GEMV on it equals the
    GEMV on the blocks; qmm_planes_release frees it (and accepts NULL)."""
    print("planes: alloc / gemv / release", flush=True)
    rng = synth.rng_for(2700)
    nrows, k = 2560, 6144
    w = synth.q8_0_weights(rng, nrows, k)
    wd = dev(w)
    x = synth.activations(rng, 8, k)
    xq = M.qmm_quantize_q8_1(dev(x))
    pl = M.Planes(M.QMM_Q8_0, wd, nrows, k)
    import torch
    torch.cuda.synchronize()
    yp = host(M.qgemv_planes(M.QMM_Q8_0, pl, nrows, k, xq, 8))
    yb = host(M.qgemv_dense(M.QMM_Q8_0, wd, nrows, k, xq, 8))
    assert np.array_equal(yp.view(np.uint32), yb.view(np.uint32))
    torch.cuda.synchronize()
    pl.release()
    assert M.lib().qmm_planes_release(None) == 0
    with pytest.raises(ValueError):
        M.qgemv_planes(M.QMM_Q8_0, pl, nrows, k, xq, 8)
