"""GPU parity of the grouped MoE decode (gate/up + SwiGLU + q8_1 + down over groups x entries)
against the oracle, with the interval check of tests/grouped_check.py for the q8_1 decisions."""
import numpy as np
import pytest

import moe_expert_amd as M
import oracle
import synth
from tests.gpu_util import dev, host
from tests.grouped_check import check_grouped

pytestmark = pytest.mark.gpu


class Experts:
    def __init__(self, seed, nexp, hidden, inter, wt_gu=M.QMM_CB3, wt_down=M.QMM_IQ4_NL, full_range=False):
        rng = synth.rng_for(seed)
        self.grid = synth.cb3_grid(synth.rng_for(synth.SEEDS["cb3_grid"]))
        self.wt_gu, self.wt_down = wt_gu, wt_down
        self.hidden, self.inter, self.nexp = hidden, inter, nexp

        def wts(wt, nrows, k):   # full_range: Q8_0 factors over all of [-128, 127]
            return synth.weights(wt, rng, nrows, k, **(dict(qlo=-128) if full_range and wt == M.QMM_Q8_0 else {}))
        self.wg = np.stack([wts(wt_gu, inter, hidden) for _ in range(nexp)])
        self.wu = np.stack([wts(wt_gu, inter, hidden) for _ in range(nexp)])
        self.wd = np.stack([wts(wt_down, hidden, inter) for _ in range(nexp)])
        self.d = dict(wg=dev(self.wg), wu=dev(self.wu), wd=dev(self.wd), grid=dev(self.grid))
        self._wd_exact = {}

    def wd_exact(self, e):
        if e not in self._wd_exact:
            self._wd_exact[e] = oracle.dequant_f64(self.wt_down, self.wd[e], self.inter, self.grid)
        return self._wd_exact[e]

    def run_gpu(self, xq, ge, go, ec, flags=M.QMM_FLAG_DEBUG_INTERMEDIATES, y=None):
        y, ws = M.qgemv_grouped_experts(self.wt_gu, self.d["wg"], self.d["wu"], self.wt_down, self.d["wd"], self.hidden,
                                        self.inter, xq, dev(ge), dev(go), dev(ec), grid=self.d["grid"], y=y, flags=flags)
        return y, ws

    def split_ws(self, ws, nentries):
        w = host(ws)
        hbytes = nentries * (self.inter // 32) * 36
        hq = w[:hbytes].reshape(nentries, -1)
        off = (hbytes + 15) // 16 * 16
        g = w[off:off + 4 * nentries * self.inter].view(np.float32).reshape(nentries, self.inter)
        u = w[off + 4 * nentries * self.inter: off + 8 * nentries * self.inter].view(np.float32).reshape(nentries, self.inter)
        return hq, g, u

    def oracle(self, xq_h, ge, go, ec):
        return oracle.grouped(self.wt_gu, self.wg, self.wu, self.wt_down, self.wd, self.hidden, self.inter, xq_h,
                              ge, go, ec, self.grid)


def depth_of(k):
    """Roundings a block term passes through in the GPU reduction: one fma per block a lane
    holds, then four DPP additions."""
    return (k // 32 + 15) // 16 + 4


def run_case(ex, ge, go, ec, ncols, seed):
    x = synth.activations(synth.rng_for(seed), ncols, ex.hidden)
    xq = M.qmm_quantize_q8_1(dev(x))
    xq_h = host(xq)
    assert np.array_equal(xq_h, oracle.quantize_q8_1(x))
    y, ws = ex.run_gpu(xq, ge, go, ec)
    hq, g, u = ex.split_ws(ws, ec.size)
    ref = ex.oracle(xq_h, ge, go, ec)
    entry_expert = np.repeat(ge, np.diff(go))
    stats = check_grouped(ref, host(y), hq, g.astype(np.float64), u.astype(np.float64),
                          lambda k: ex.wd_exact(int(entry_expert[k])), ex.inter, depth_of(ex.hidden))
    print("grouped check:", stats, flush=True)
    return y, hq, g, u, xq


def test_grouped_small():
    print("grouped small: 5 experts 512->64, 3 groups x 3 entries", flush=True)
    ex = Experts(800, 5, 512, 64)
    ge, go, ec = synth.decode_routing(synth.rng_for(801), 5, 3, 3)
    ec = ec[::-1].copy()
    run_case(ex, ge, go, ec, 3, 802)


def test_grouped_ragged_passes():
    """Groups of 1, 11 (two passes) and 0 entries; uneven column map."""
    print("grouped ragged: groups of 1, 11, 0 entries", flush=True)
    ex = Experts(810, 6, 768, 96, wt_gu=M.QMM_CB3, wt_down=M.QMM_Q8_0)
    ge = np.array([4, 1, 2], np.int32)
    go = np.array([0, 1, 12, 12], np.int32)
    ec = synth.rng_for(811).integers(0, 5, size=12).astype(np.int32)
    run_case(ex, ge, go, ec, 5, 812)


@pytest.mark.parametrize("wt_gu,wt_down", [(M.QMM_IQ4_NL, M.QMM_Q8_0), (M.QMM_Q8_0, M.QMM_IQ4_NL)])
def test_grouped_other_formats(wt_gu, wt_down):
    """Q8_0 matrices (down, or gate/up) with factors over all of [-128, 127]."""
    print(f"grouped formats gu={wt_gu} down={wt_down}", flush=True)
    ex = Experts(820 + wt_gu, 4, 1024, 128, wt_gu=wt_gu, wt_down=wt_down, full_range=True)
    q8 = ex.wd if wt_down == M.QMM_Q8_0 else ex.wg
    assert (q8.reshape(-1, 34)[:, 2:].view(np.int8) == -128).any()
    ge, go, ec = synth.decode_routing(synth.rng_for(821), 4, 4, 2)
    run_case(ex, ge, go, ec, 2, 822)


@pytest.mark.parametrize("hidden", [3072, 4096])
def test_grouped_long_rows(hidden):
    """Long CB3 gate/up rows with 11 entries in a group (two passes): 3072 (6 blocks per lane,
    the 1024-thread workgroup with one row per lane) and 4096 (8 blocks per lane: the
    double-buffered chunks, two rows per lane)."""
    print(f"grouped long rows: 3 experts {hidden} -> 64, groups of 11 and 2 entries", flush=True)
    ex = Experts(850, 3, hidden, 64, wt_gu=M.QMM_CB3, wt_down=M.QMM_Q8_0)
    ge = np.array([2, 0], np.int32)
    go = np.array([0, 11, 13], np.int32)
    ec = synth.rng_for(851).integers(0, 6, size=13).astype(np.int32)
    run_case(ex, ge, go, ec, 6, 852)


@pytest.mark.parametrize("wt_gu,hidden", [(M.QMM_IQ4_NL, 2560), (M.QMM_Q8_0, 2560), (M.QMM_IQ4_NL, 3072),
                                          (M.QMM_Q8_0, 1536)])
def test_grouped_gate_up_rows(wt_gu, hidden):
    """IQ4_NL and Q8_0 gate/up rows of 5, 6 and 3 blocks per lane (1024-thread workgroups, one row
    per lane, the first blocks loaded before the staging and the rest after block 0), with a
    group of 9 entries (two passes) and one of 1."""
    print(f"grouped gate/up rows: gu={wt_gu}, hidden {hidden}, groups of 9 and 1 entries", flush=True)
    ex = Experts(870 + hidden + wt_gu, 3, hidden, 96, wt_gu=wt_gu, wt_down=M.QMM_IQ4_NL)
    ge = np.array([2, 0], np.int32)
    go = np.array([0, 9, 10], np.int32)
    ec = synth.rng_for(871 + hidden).integers(0, 5, size=10).astype(np.int32)
    run_case(ex, ge, go, ec, 5, 872 + hidden)


@pytest.mark.parametrize("wt_down,inter", [(M.QMM_IQ4_NL, 4096), (M.QMM_CB3, 512), (M.QMM_Q8_0, 256)])
def test_grouped_down_shapes(wt_down, inter):
    """The down kernel's instances: long rows (inter 4096, the double-buffered tile), CB3 rows
    (one row set per workgroup), short Q8_0 rows (two row sets per workgroup); IQ4_NL gate/up
    (one row per lane, 1024-thread workgroups)."""
    hidden = 288 if wt_down != M.QMM_CB3 else 512
    print(f"grouped down shapes: down {wt_down}, inter {inter}, hidden {hidden}", flush=True)
    ex = Experts(860 + inter, 3, hidden, inter, wt_gu=M.QMM_IQ4_NL, wt_down=wt_down)
    ge = np.array([1, 2, 0], np.int32)
    go = np.array([0, 3, 4, 9], np.int32)
    ec = synth.rng_for(861 + inter).integers(0, 4, size=9).astype(np.int32)
    run_case(ex, ge, go, ec, 4, 862 + inter)


@pytest.fixture(scope="module")
def full_experts():
    """The grouped decode workload: 128 experts, hidden 2560, CB3 gate/up 2560->1024, IQ4_NL
    down 1024->2560."""
    print("building 128 experts (2560 -> 1024 -> 2560)", flush=True)
    return Experts(synth.SEEDS["grouped_decode"], 128, 2560, 1024)


@pytest.mark.parametrize("m", [1, 4, 8])
def test_grouped_full_size(full_experts, m):
    print(f"grouped full size: 16 groups x {m} entries", flush=True)
    ge, go, ec = synth.decode_routing(synth.rng_for(synth.SEEDS["grouped_decode"] + m), 128, 16, m)
    run_case(full_experts, ge, go, ec, m, synth.SEEDS["grouped_decode"] + 100 + m)


def test_grouped_matches_dense_and_entry_invariance(full_experts):
    """Gate/up sums equal qgemv_dense on the same expert matrix bitwise; an entry's y does not
    depend on the other entries of its group (m = 1 vs m = 8)."""
    print("grouped vs dense / entry invariance", flush=True)
    ex = full_experts
    ge, go, ec = synth.decode_routing(synth.rng_for(830), 128, 16, 8)
    x = synth.activations(synth.rng_for(831), 8, ex.hidden)
    xq = M.qmm_quantize_q8_1(dev(x))
    y8, ws8 = ex.run_gpu(xq, ge, go, ec)
    hq8, g8, u8 = ex.split_ws(ws8, ec.size)
    for gi in (0, 7, 15):
        e = int(ge[gi])
        yd = host(M.qgemv_dense(ex.wt_gu, ex.d["wg"][e], ex.inter, ex.hidden, xq, 8, grid=ex.d["grid"]))
        for j in range(8):
            k = go[gi] + j
            assert np.array_equal(g8[k].view(np.uint32), yd[ec[k]].view(np.uint32)), (gi, j)
    # the same groups with one entry each (entry j = 0 of every group)
    go1 = np.arange(17, dtype=np.int32)
    ec1 = np.zeros(16, np.int32)
    y1, ws1 = ex.run_gpu(xq, ge, go1, ec1)
    y8h, y1h = host(y8), host(y1)
    for gi in range(16):
        k8 = go[gi] + int(np.nonzero(ec[go[gi]:go[gi + 1]] == 0)[0][0])
        assert np.array_equal(y1h[gi].view(np.uint32), y8h[k8].view(np.uint32)), gi


def test_grouped_skips_bad_groups_and_columns():
    """A group with an expert out of range is skipped (its rows untouched); an entry whose column
    is out of range reads zero activations (y = 0)."""
    print("grouped bad expert / column", flush=True)
    import torch
    ex = Experts(840, 3, 512, 64)
    ge = np.array([0, 7, 2], np.int32)            # expert 7 does not exist
    go = np.array([0, 2, 4, 6], np.int32)
    ec = np.array([0, 1, 0, 1, 1, 9], np.int32)   # column 9 does not exist (2 columns)
    x = synth.activations(synth.rng_for(841), 2, ex.hidden)
    xq = M.qmm_quantize_q8_1(dev(x))
    y = torch.full((6, ex.hidden), float("nan"), device="cuda")
    ex.run_gpu(xq, ge, go, ec, flags=0, y=y)
    yh = host(y)
    assert np.isnan(yh[2:4]).all()
    assert (yh[5] == 0).all()
    assert np.isfinite(yh[[0, 1, 4]]).all()


@pytest.mark.parametrize("ncols", [6, 12])
def test_grouped_column_maps(ncols):
    """Entry columns in any order, repeated and out of range, with at most 8 activation columns
    (all staged before the group lookup, then re-staged in LDS to the pass's entry columns) and
    with more (each pass loads its entry columns); groups of 4, 9 (two passes) and 2 entries.
    The oracle reads an out-of-range entry from an appended all-zero q8_1 column."""
    print(f"grouped column maps: {ncols} activation columns", flush=True)
    ex = Experts(860, 4, 1024, 64)
    ge = np.array([1, 3, 0], np.int32)
    go = np.array([0, 4, 13, 15], np.int32)
    ec = synth.rng_for(861 + ncols).integers(-2, ncols + 2, size=15).astype(np.int32)
    ec[0], ec[1] = ec[1], ec[1]                   # a repeated column in the first pass
    x = synth.activations(synth.rng_for(862 + ncols), ncols, ex.hidden)
    xq = M.qmm_quantize_q8_1(dev(x))
    xq_h = host(xq)
    y, ws = ex.run_gpu(xq, ge, go, ec)
    hq, g, u = ex.split_ws(ws, ec.size)
    xq_z = np.concatenate([xq_h, np.zeros((1, xq_h.shape[1]), np.uint8)])
    ec_z = np.where((ec >= 0) & (ec < ncols), ec, ncols).astype(np.int32)
    ref = ex.oracle(xq_z, ge, go, ec_z)
    entry_expert = np.repeat(ge, np.diff(go))
    stats = check_grouped(ref, host(y), hq, g.astype(np.float64), u.astype(np.float64),
                          lambda k: ex.wd_exact(int(entry_expert[k])), ex.inter, depth_of(ex.hidden))
    print("grouped check:", stats, flush=True)
    assert ((ec < 0) | (ec >= ncols)).any() and (ec[:4] != np.arange(4)).any()
