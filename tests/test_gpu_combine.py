"""GPU parity of the MoE combine (qmm_moe_combine) against the oracle, bit for bit: the sum runs
in k order with one binary32 rounding per product and per sum, so the result is unique."""
import numpy as np
import pytest

import moe_expert_amd as M
import oracle
import synth
from tests.gpu_util import dev, host

pytestmark = pytest.mark.gpu


def run(y, idx, w, ldo=None):
    import torch
    ntok = idx.shape[0]
    ldo = y.shape[1] if ldo is None else ldo
    out = torch.full((ntok, ldo), 7.0, dtype=torch.float32, device="cuda")
    M.qmm_moe_combine(dev(y), dev(idx), dev(w), out=out, ldo=ldo)
    return host(out)


@pytest.mark.parametrize("ntok,topk,hidden,nrows", [(1, 8, 2560, 16), (333, 8, 2560, 3000), (1000, 2, 1024, 2000),
                                                    (517, 16, 64, 9000), (40, 1, 12, 40), (37, 64, 4100, 400),
                                                    (5, 9, 8, 30)])
def test_combine_bitwise(ntok, topk, hidden, nrows):
    """Token counts of the page's test (1, 333, 1000, 517) and others; k from 1 to 64 (groups
    of 8 and a partial group); rows of 4 .. 4100 values (one to five 16-byte pieces per thread,
    partial chunks); indices drawn with repeats; values over a wide range."""
    print(f"combine ntok={ntok} topk={topk} hidden={hidden} nrows={nrows}", flush=True)
    rng = synth.rng_for(2100 + ntok + topk)
    y = (rng.standard_normal((nrows, hidden)) * np.exp2(rng.integers(-20, 20, (nrows, 1)))).astype(np.float32)
    idx = rng.integers(0, nrows, (ntok, topk)).astype(np.int32)
    w = synth.router_weights(rng, ntok, topk)
    got = run(y, idx, w)
    ref = oracle.moe_combine(y, idx, w)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"{(got != ref).sum()} outputs differ"


def test_combine_skips_rows_padded_stride_and_signs():
    """Indices outside the rows add nothing; zero weights and negative rows give +0; columns
    past hidden in a padded output row are not written."""
    print("combine: skipped rows, zero weights, padded ldo", flush=True)
    rng = synth.rng_for(2200)
    nrows, hidden, ntok, topk = 50, 96, 30, 5
    y = rng.standard_normal((nrows, hidden)).astype(np.float32)
    y[3] = -np.abs(y[3])
    idx = rng.integers(0, nrows, (ntok, topk)).astype(np.int32)
    idx[::3, 1] = -1
    idx[1::4, 4] = nrows
    idx[7] = 3
    w = synth.router_weights(rng, ntok, topk)
    w[7] = 0.0
    got = run(y, idx, w, ldo=100)
    ref = oracle.moe_combine(y, idx, w)
    assert np.array_equal(got[:, :hidden].view(np.uint32), ref.view(np.uint32))
    assert (got[:, hidden:] == 7.0).all()
    assert not np.signbit(got[7, :hidden]).any()


def test_combine_prefill_full_size():
    """The prefill workload: 8192 tokens, top-8 of 128 experts, hidden 2560, y in the sorted
    entry order of the routing (65536 rows); every output against the oracle."""
    print("combine full size: 8192 tokens x top-8, hidden 2560", flush=True)
    rng = synth.rng_for(synth.SEEDS["prefill"] + 10)
    ntok, topk, hidden = 8192, 8, 2560
    st, _ = synth.prefill_routing(rng, ntok, 128, topk)
    idx = synth.token_positions(st, ntok, topk)
    y = rng.standard_normal((st.size, hidden), dtype=np.float32)
    w = synth.router_weights(rng, ntok, topk)
    got = run(y, idx, w)
    ref = oracle.moe_combine(y, idx, w)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_combine_decode_shape():
    """The decode workload's shape: m = 8 tokens, each routed to the 16 groups of a grouped call
    (entry j of group g is token j): the k-th row of token j is entry 8 g + j."""
    print("combine decode shape: 8 tokens x 16 experts, hidden 2560", flush=True)
    rng = synth.rng_for(2300)
    m, ngroups, hidden = 8, 16, 2560
    y = rng.standard_normal((ngroups * m, hidden), dtype=np.float32)
    idx = (np.arange(ngroups)[None, :] * m + np.arange(m)[:, None]).astype(np.int32)
    w = synth.router_weights(rng, m, ngroups)
    got = run(y, idx, w)
    ref = oracle.moe_combine(y, idx, w)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
