"""GPU parity of the dense decode GEMV: per-block integer sums bit-exact, one-hot rows
bit-exact, fp32 outputs within 1e-4 * sum|terms| of the oracle, every column of an n-column
call bitwise equal to a one-column call."""
import numpy as np
import pytest

import moe_expert_amd as M
import oracle
import synth
from tests.gpu_util import check_tol, dev, host

pytestmark = pytest.mark.gpu

FORMATS = [M.QMM_Q8_0, M.QMM_IQ4_NL, M.QMM_CB3]


def case(wtype, nrows, k, ncols, seed, full_range=False):
    """Seeded weights, codebook and activations; full_range: Q8_0 factors over all of
    [-128, 127]."""
    rng = synth.rng_for(seed)
    grid = synth.cb3_grid(rng) if wtype == M.QMM_CB3 else None
    kw = dict(qlo=-128) if full_range and wtype == M.QMM_Q8_0 else {}
    w = synth.weights(wtype, rng, nrows, k, **kw)
    x = synth.activations(rng, ncols, k)
    return w, grid, x


def gpu_gemv(wtype, w, grid, x, nrows, k, ncols):
    xq = M.qmm_quantize_q8_1(dev(x))
    y = M.qgemv_dense(wtype, dev(w), nrows, k, xq, ncols, grid=None if grid is None else dev(grid))
    return host(y), host(xq)


@pytest.mark.parametrize("wtype", FORMATS)
@pytest.mark.parametrize("nrows,k,ncols", [(37, 512, 3), (64, 1024, 1), (100, 2560, 8), (33, 768, 5), (21, 2592, 2)])
def test_block_sums_exact(wtype, nrows, k, ncols):
    if wtype == M.QMM_CB3 and k % 256:
        pytest.skip("CB3 needs k % 256 == 0")
    print(f"block sums wtype={wtype} nrows={nrows} k={k} ncols={ncols}", flush=True)
    w, grid, x = case(wtype, nrows, k, ncols, 300 + nrows + wtype)
    xq = oracle.quantize_q8_1(x)
    ref = oracle.block_sums(wtype, w, k, xq, grid)
    got = host(M.qmm_debug_block_sums(wtype, dev(w), nrows, k, dev(xq), ncols, grid=None if grid is None else dev(grid)))
    assert np.array_equal(got, ref), f"{(got != ref).sum()} sums differ"


@pytest.mark.parametrize("wtype", FORMATS)
@pytest.mark.parametrize("nrows,k,ncols", [(37, 512, 3), (129, 2560, 8), (64, 1024, 2), (31, 6144, 7),
                                           (1, 256, 1), (300, 1536, 11), (45, 2592, 4), (7, 96, 2),
                                           (33, 12544, 5)])
def test_gemv_tolerance(wtype, nrows, k, ncols):
    if wtype == M.QMM_CB3 and k % 256:
        pytest.skip("CB3 rows are whole 256-value super-blocks")
    print(f"gemv wtype={wtype} nrows={nrows} k={k} ncols={ncols}", flush=True)
    w, grid, x = case(wtype, nrows, k, ncols, 400 + nrows + wtype)
    y, xq = gpu_gemv(wtype, w, grid, x, nrows, k, ncols)
    assert np.array_equal(xq, oracle.quantize_q8_1(x))
    ref, a = oracle.gemv(wtype, w, k, xq, grid)
    check_tol(y, ref, a, what=f"gemv {wtype}")


@pytest.mark.parametrize("wtype", FORMATS)
@pytest.mark.parametrize("k", [2560, 6144, 12544])
def test_column_invariance(wtype, k):
    """Each column of an n-column call equals the one-column call bitwise (n = 1..8, 11), for
    rows of 16 lanes (k = 2560), of one wave (k = 6144) and of one wave in several chunks
    (k = 12544)."""
    if wtype == M.QMM_CB3 and k % 256:
        pytest.skip("CB3 rows are whole 256-value super-blocks")
    nrows = 200
    print(f"column invariance wtype={wtype} k={k}", flush=True)
    w, grid, x = case(wtype, nrows, k, 11, 500 + wtype)
    wd = dev(w)
    gd = None if grid is None else dev(grid)
    xq = M.qmm_quantize_q8_1(dev(x))
    nb36 = (k // 32) * 36
    single = [host(M.qgemv_dense(wtype, wd, nrows, k, xq[c:c + 1].contiguous(), 1, grid=gd))[0] for c in range(11)]
    for n in list(range(1, 9)) + [11]:
        y = host(M.qgemv_dense(wtype, wd, nrows, k, xq[:n].contiguous(), n, grid=gd))
        for c in range(n):
            assert np.array_equal(y[c].view(np.uint32), single[c].view(np.uint32)), (n, c)
    assert nb36 == xq.shape[1]


@pytest.mark.parametrize("wtype", FORMATS)
def test_onehot_rows_exact(wtype):
    """Rows whose every block scale but one is 0: y equals that block's binary32 term bitwise."""
    bv, bb = synth.BLOCK_VALUES[wtype], synth.BLOCK_BYTES[wtype]
    k = 2560
    nb = k // bv
    print(f"one-hot rows wtype={wtype}", flush=True)
    w, grid, x = case(wtype, nb, k, 3, 600 + wtype)
    w = w.reshape(nb, nb, bb).copy()
    for r in range(nb):
        for b in range(nb):
            if b != r:
                w[r, b, 0:2] = 0
    w = w.reshape(nb, nb * bb)
    if wtype == M.QMM_CB3:
        # a super-block holds 8 sub-block terms: zero the activations outside sub-block 0 of
        # every super-block so each row keeps a single non-zero term
        x = x.copy()
        x[:, (np.arange(k) % 256) >= 32] = 0.0
    y, xq = gpu_gemv(wtype, w, grid, x, nb, k, 3)
    ref, _ = oracle.gemv(wtype, w, k, xq, grid)
    assert np.array_equal(y, ref.astype(np.float32)), np.abs(y - ref).max()


@pytest.mark.parametrize("wtype,nrows,k,cols,key", [
    (M.QMM_Q8_0, 512, 2560, (1,), "q8_0_tiny"),
    (M.QMM_IQ4_NL, 8192, 2560, (1, 2, 4, 8), "iq4nl_8192x2560"),
    (M.QMM_Q8_0, 12288, 2560, (1, 2, 3, 4), "q8_0_12288x2560"),
    (M.QMM_Q8_0, 2560, 6144, (7, 8), "q8_0_2560x6144"),
])
def test_gemv_full_sizes(wtype, nrows, k, cols, key):
    """The benchmark's GEMV workloads at their full sizes and column counts, with the benchmark's
    first weight copy and activations: every output within the fp32 tolerance of the oracle."""
    print(f"gemv full size {key}: {nrows}x{k} at {cols} columns", flush=True)
    seed = synth.SEEDS[key]
    w = synth.weights(wtype, synth.rng_for(seed), nrows, k)
    x = synth.activations(synth.rng_for(seed + 100), max(cols), k)
    wd = dev(w)
    for n in cols:
        xq = M.qmm_quantize_q8_1(dev(x[:n]))
        y = host(M.qgemv_dense(wtype, wd, nrows, k, xq, n))
        xq_h = host(xq)
        assert np.array_equal(xq_h, oracle.quantize_q8_1(x[:n]))
        ref, a = oracle.gemv(wtype, w, k, xq_h)
        check_tol(y, ref, a, what=f"gemv {key} n={n}")


@pytest.mark.parametrize("wtype", FORMATS)
@pytest.mark.parametrize("nrows,k,ncols", [(37, 512, 1), (100, 2560, 1), (300, 1536, 2), (7, 96, 4), (33, 3072, 4),
                                           (8192, 2560, 1), (8192, 2560, 4), (45, 2592, 2)])
def test_gemv_f32_fused(wtype, nrows, k, ncols):
    """The call on 1, 2 or 4 fp32 columns (q8_1 formed inside the kernel) equals the quantizer
    followed by the q8_1 GEMV bitwise, and the oracle within the fp32 tolerance.  Each column
    holds an all-zero block, a block whose scale underflows to 0, a block of magnitude 1e6 and a
    block with d = 1 exactly whose other values are halves (ties, rounded away from 0), at
    column-dependent positions."""
    if wtype == M.QMM_CB3 and k % 256:
        pytest.skip("CB3 rows are whole 256-value super-blocks")
    print(f"fused f32 gemv wtype={wtype} nrows={nrows} k={k} ncols={ncols}", flush=True)
    w, grid, x = case(wtype, nrows, k, ncols, 800 + nrows + wtype + ncols)
    x = x.copy()
    nb = k // 32
    for c in range(ncols):
        if nb >= 4 + c:
            o = 32 * c
            x[c, o:o + 32] = 0.0
            x[c, o + 32:o + 64] = np.float32(1e-45)
            x[c, o + 64:o + 96] = np.float32(1e6) * x[c, o + 64:o + 96]
            x[c, o + 96:o + 128] = np.arange(-15.5, 16.5, 1.0, dtype=np.float32)
            x[c, o + 96] = 127.0
    gd = None if grid is None else dev(grid)
    y_two, xq = gpu_gemv(wtype, w, grid, x, nrows, k, ncols)
    y = host(M.qgemv_dense_f32(wtype, dev(w), nrows, k, dev(x), ncols, grid=gd))
    assert np.array_equal(y.view(np.uint32), y_two.view(np.uint32)), np.abs(y - y_two).max()
    ref, a = oracle.gemv(wtype, w, k, oracle.quantize_q8_1(x), grid)
    check_tol(y, ref, a, what=f"fused gemv {wtype}")


@pytest.mark.parametrize("wtype,nrows,k,key", [(M.QMM_IQ4_NL, 8192, 2560, "iq4nl_8192x2560"),
                                               (M.QMM_Q8_0, 12288, 2560, "q8_0_12288x2560")])
def test_gemv_f32_full_sizes(wtype, nrows, k, key):
    """The benchmark's one-column calls on fp32 activations at full size, with its first weight
    copy and activations: every output within the fp32 tolerance of the oracle, and bitwise the
    quantizer + q8_1 GEMV result."""
    print(f"fused gemv full size {key}", flush=True)
    seed = synth.SEEDS[key]
    w = synth.weights(wtype, synth.rng_for(seed), nrows, k)
    x = synth.activations(synth.rng_for(seed + 100), 1, k)
    wd = dev(w)
    y = host(M.qgemv_dense_f32(wtype, wd, nrows, k, dev(x), 1))
    y_two = host(M.qgemv_dense(wtype, wd, nrows, k, M.qmm_quantize_q8_1(dev(x)), 1))
    assert np.array_equal(y.view(np.uint32), y_two.view(np.uint32))
    ref, a = oracle.gemv(wtype, w, k, oracle.quantize_q8_1(x))
    check_tol(y, ref, a, what=f"fused gemv {key}")


def test_gemv_f32_ldy_padding():
    """Two fp32 columns into rows of ldy > nrows: the padding is not written."""
    print("fused gemv ldy padding", flush=True)
    import torch
    w, grid, x = case(M.QMM_Q8_0, 50, 512, 2, 710)
    y = torch.full((2, 64), 7.0, device="cuda")
    M.qgemv_dense_f32(M.QMM_Q8_0, dev(w), 50, 512, dev(x), 2, y=y, ldy=64)
    yh = host(y)
    assert (yh[:, 50:] == 7.0).all()
    ref, a = oracle.gemv(M.QMM_Q8_0, w, 512, oracle.quantize_q8_1(x))
    check_tol(yh[:, :50], ref, a)


def test_ldy_padding():
    print("ldy padding", flush=True)
    import torch
    w, grid, x = case(M.QMM_IQ4_NL, 50, 512, 3, 700)
    xq = M.qmm_quantize_q8_1(dev(x))
    y = torch.full((3, 64), 7.0, device="cuda")
    M.qgemv_dense(M.QMM_IQ4_NL, dev(w), 50, 512, xq, 3, y=y, ldy=64)
    yh = host(y)
    assert (yh[:, 50:] == 7.0).all()
    ref, a = oracle.gemv(M.QMM_IQ4_NL, w, 512, host(xq))
    check_tol(yh[:, :50], ref, a)


@pytest.mark.parametrize("threads,unroll", [(256, 8), (512, 4), (1024, 16)])
def test_stream_read_reference(threads, unroll):
    """The streaming-read reference kernel reads every 16-byte chunk once: thread t of workgroup
    w XORs chunks w R + t, w R + t + threads, ... of its run of R = ceil(chunks / grid)."""
    print(f"stream read reference threads={threads} unroll={unroll}", flush=True)
    rng = np.random.default_rng(5)
    nbytes, grid = 3 * 65536 + 48, 3
    buf = rng.integers(0, 256, size=nbytes, dtype=np.uint8)
    out = host(M.qmm_debug_stream_read(dev(buf), nbytes, grid, threads=threads, unroll=unroll)).view(np.uint32)
    words = buf.view(np.uint32).reshape(-1, 4)
    chunk = words[:, 0] ^ words[:, 1] ^ words[:, 2] ^ words[:, 3]
    run = -(-chunk.size // grid)
    ref = np.zeros(grid * threads, np.uint32)
    for w in range(grid):
        seg = chunk[w * run:(w + 1) * run]
        for t in range(threads):
            ref[w * threads + t] = np.bitwise_xor.reduce(seg[t::threads]) if t < seg.size else 0
    assert np.array_equal(out, ref)


def test_mfma_loop_reference():
    """The MFMA reference loop computes what its operands give: thread t (lane l = t mod 64 of
    its wave) holds A[l mod 32][8 (l div 32) + e] = (t + e) mod 8 and B[8 (l div 32) + e][l mod
    32] = (3 t + e) mod 8, and D register r is D[8 (r div 4) + 4 (l div 32) + r mod 4][l mod 32];
    out[t] = 8 chains x iters x the sum of its D registers (small integers: exact)."""
    print("mfma loop reference", flush=True)
    grid, iters = 2, 3
    out = host(M.qmm_debug_mfma_loop(grid, iters))
    ref = np.zeros(grid * 256)
    for w0 in range(0, 256, 64):
        t = np.arange(w0, w0 + 64)
        l = t % 64
        A = np.zeros((32, 16))
        B = np.zeros((16, 32))
        for e in range(8):
            A[l % 32, 8 * (l // 32) + e] = (t + e) % 8
            B[8 * (l // 32) + e, l % 32] = (3 * t + e) % 8
        D = A @ B
        for li in range(64):
            rows = [8 * (r // 4) + 4 * (li // 32) + r % 4 for r in range(16)]
            ref[w0 + li] = 8 * iters * D[rows, li % 32].sum()
    ref[256:] = ref[:256]
    assert np.array_equal(out, ref.astype(np.float32))


@pytest.mark.parametrize("nrows,k,ncols", [(64, 2560, 1), (37, 6144, 8), (100, 1024, 5)])
def test_q8_0_minus_128(nrows, k, ncols):
    """Q8_0 factors over all of [-128, 127], plus rows whose every factor is -128: block sums
    bit-exact, one-hot rows bit-exact, outputs within the fp32 tolerance."""
    print(f"Q8_0 factor -128: nrows={nrows} k={k} ncols={ncols}", flush=True)
    wt = M.QMM_Q8_0
    w, grid, x = case(wt, nrows, k, ncols, 1300 + nrows, full_range=True)
    w = w.reshape(nrows, k // 32, 34).copy()
    w[:3, :, 2:] = np.uint8(0x80)                       # three rows of -128 only
    w = w.reshape(nrows, -1)
    assert (w.reshape(nrows, -1, 34)[3:, :, 2:].view(np.int8) == -128).any()
    xq = oracle.quantize_q8_1(x)
    got = host(M.qmm_debug_block_sums(wt, dev(w), nrows, k, dev(xq), ncols))
    assert np.array_equal(got, oracle.block_sums(wt, w, k, xq))
    y, _ = gpu_gemv(wt, w, grid, x, nrows, k, ncols)
    ref, a = oracle.gemv(wt, w, k, xq)
    check_tol(y, ref, a, what="Q8_0 -128")
    # one-hot rows: only block r of row r keeps its scale
    nb = k // 32
    w1 = w[:min(nrows, nb)].reshape(-1, nb, 34).copy()
    for r in range(w1.shape[0]):
        w1[r, np.arange(nb) != r, 0:2] = 0
    w1 = w1.reshape(w1.shape[0], -1)
    y1, _ = gpu_gemv(wt, w1, grid, x, w1.shape[0], k, ncols)
    ref1, _ = oracle.gemv(wt, w1, k, xq)
    assert np.array_equal(y1, ref1.astype(np.float32))


def test_gemv_activation_blocks_beyond_2_24():
    """A q8_1 buffer of more than 2^24 blocks (k = 32768, 16392 columns, 604 MB): the blocks of
    the last 8 columns lie at and past block 2^24, and their outputs equal an 8-column call on a
    copy of those columns, bitwise (the staging offset is a full 32-bit product; out-of-range
    reads return zeros, so a wrong offset shows as a wrong value, not a fault)."""
    import torch
    k, ncols, nrows = 32768, 16392, 16
    print(f"gemv with {ncols * k // 32} q8_1 blocks (k={k}, {ncols} columns)", flush=True)
    w, grid, x = case(M.QMM_Q8_0, nrows, k, 8, 1400)
    xq8 = M.qmm_quantize_q8_1(dev(x))
    xq = torch.zeros((ncols, (k // 32) * 36), dtype=torch.uint8, device="cuda")
    xq[ncols - 8:] = xq8
    wd = dev(w)
    y = host(M.qgemv_dense(M.QMM_Q8_0, wd, nrows, k, xq, ncols))
    y8 = host(M.qgemv_dense(M.QMM_Q8_0, wd, nrows, k, xq8, 8))
    assert np.array_equal(y[ncols - 8:].view(np.uint32), y8.view(np.uint32))
    ref, a = oracle.gemv(M.QMM_Q8_0, w, k, host(xq8))
    check_tol(y8, ref, a)
