"""GPU parity of the MMQ-style prefill (qgemm_prefill_experts_q8: int8 MFMA on q8_1 activations,
SwiGLU + q8_1 of H fused) against the oracle.  The path computes what the grouped decode
computes, over the rows sorted per expert (groups = experts, entry columns = sorted tokens), so
the oracle is the grouped decode's: the tokens' q8_1 planes bit for bit against the quantizer;
g, u within the fp32 bound of a block-by-block sum; H inside the interval the q8_1 decisions
allow (its planes carry no sum field); y within 1e-4 * sum|terms| plus the validated H
differences (tests/grouped_check.py)."""
import numpy as np
import pytest

import moe_expert_amd as M
import oracle
import synth
from tests.gpu_util import dev, host
from tests.grouped_check import check_grouped

pytestmark = pytest.mark.gpu


def weights(wt, rng, nrows, k, full_range):
    return synth.weights(wt, rng, nrows, k, **(dict(qlo=-128) if full_range and wt == M.QMM_Q8_0 else {}))


class Mmq:
    def __init__(self, seed, nexp, ntok, topk, hidden, inter, wt_gu=M.QMM_IQ4_NL, wt_down=M.QMM_Q8_0, full_range=False):
        rng = synth.rng_for(seed)
        self.nexp, self.ntok, self.hidden, self.inter = nexp, ntok, hidden, inter
        self.wt_gu, self.wt_down = wt_gu, wt_down
        self.wg = np.stack([weights(wt_gu, rng, inter, hidden, full_range) for _ in range(nexp)])
        self.wu = np.stack([weights(wt_gu, rng, inter, hidden, full_range) for _ in range(nexp)])
        self.wd = np.stack([weights(wt_down, rng, hidden, inter, full_range) for _ in range(nexp)])
        self.x16 = synth.prefill_tokens(rng, ntok, hidden)
        self.st, self.off = synth.prefill_routing(rng, ntok, nexp, topk)
        self.d = dict(wg=dev(self.wg), wu=dev(self.wu), wd=dev(self.wd), x=dev(self.x16.view(np.uint16)),
                      st=dev(self.st), off=dev(self.off))
        self._wdx = {}

    def run_gpu(self, flags=M.QMM_FLAG_DEBUG_INTERMEDIATES):
        return M.qgemm_prefill_experts_q8(self.wt_gu, self.d["wg"], self.d["wu"], self.wt_down, self.d["wd"], self.nexp,
                                          self.hidden, self.inter, self.d["x"], self.d["st"], self.d["off"], flags=flags)

    def split_ws(self, ws):
        """(x planes q, d; H planes q, d; g; u) from the documented workspace layout."""
        w = host(ws)
        a16 = lambda v: (v + 15) // 16 * 16
        ne, nt, h, i = self.st.size, self.ntok, self.hidden, self.inter
        o_xd = a16(nt * h)
        o_hq = a16(o_xd + nt * (h // 32) * 2)
        o_hd = a16(o_hq + ne * i)
        o_tiles = a16(o_hd + ne * (i // 32) * 2)
        max_tiles = (ne + 127) // 128 + self.nexp
        o_g = a16(o_tiles + 4 * (1 + 3 * max_tiles))
        xq = w[:nt * h].view(np.int8).reshape(nt, h)
        xd = w[o_xd:o_xd + nt * (h // 32) * 2].view(np.uint16).reshape(nt, h // 32)
        hq = w[o_hq:o_hq + ne * i].view(np.int8).reshape(ne, i)
        hd = w[o_hd:o_hd + ne * (i // 32) * 2].view(np.uint16).reshape(ne, i // 32)
        g = w[o_g:o_g + 4 * ne * i].view(np.float32).reshape(ne, i)
        u = w[o_g + 4 * ne * i:o_g + 8 * ne * i].view(np.float32).reshape(ne, i)
        return xq, xd, hq, hd, g, u

    @staticmethod
    def blocks(q, d):
        """Planes -> q8_1 blocks (d, a zero sum field, q)."""
        rows, k = q.shape
        b = np.zeros((rows, k // 32, 36), np.uint8)
        b[:, :, 0:2] = d.view(np.uint8).reshape(rows, k // 32, 2)
        b[:, :, 4:] = q.view(np.uint8).reshape(rows, k // 32, 32)
        return b.reshape(rows, -1)

    def wd_exact(self, e):
        if e not in self._wdx:
            self._wdx[e] = oracle.dequant_f64(self.wt_down, self.wd[e], self.inter)
        return self._wdx[e]

    def check(self, samples, y, ws):
        samples = np.asarray(samples, np.int64)
        xq, xd, hq, hd, g, u = self.split_ws(ws)
        xq_ref = oracle.quantize_q8_1(self.x16.astype(np.float32))
        assert np.array_equal(self.blocks(xq, xd).reshape(self.ntok, -1, 36)[:, :, [0, 1] + list(range(4, 36))],
                              xq_ref.reshape(self.ntok, -1, 36)[:, :, [0, 1] + list(range(4, 36))]), \
            "token q8_1 planes differ from the quantizer"
        exps = (np.searchsorted(self.off, samples, side="right") - 1).astype(np.int32)
        ge = exps
        go = np.arange(samples.size + 1, dtype=np.int32)
        ref = oracle.grouped(self.wt_gu, self.wg, self.wu, self.wt_down, self.wd, self.hidden, self.inter, xq_ref,
                             ge, go, self.st[samples], None)
        depth = self.hidden // 32 + 2
        return check_grouped(ref, host(y)[samples], self.blocks(hq[samples], hd[samples]),
                             g[samples].astype(np.float64), u[samples].astype(np.float64),
                             lambda k: self.wd_exact(int(exps[k])), self.inter, depth, sum_field=False)


def test_mmq_small():
    print("mmq small: 6 experts, 40 tokens top-2, 256 -> 64 -> 256", flush=True)
    c = Mmq(3300, 6, 40, 2, 256, 64)
    y, ws = c.run_gpu()
    print(c.check(np.arange(c.st.size), y, ws), flush=True)


def test_mmq_ragged_tiles():
    """Experts of 0, 1, 31, 32, 33, 128, 129, 300 rows: no tile, partial 32-row blocks, a full
    128-row tile, experts split into 2 and 3 tiles."""
    print("mmq ragged: expert row counts 0 1 31 32 33 128 129 300", flush=True)
    counts = np.array([0, 1, 31, 32, 33, 128, 129, 300])
    c = Mmq(3310, 8, 700, 1, 512, 128)
    c.st = (np.arange(counts.sum(), dtype=np.int64) * 7 % 700).astype(np.int32)
    c.off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    c.d["st"], c.d["off"] = dev(c.st), dev(c.off)
    y, ws = c.run_gpu()
    print(c.check(np.arange(c.st.size), y, ws), flush=True)


@pytest.mark.parametrize("wt_gu,wt_down", [(M.QMM_Q8_0, M.QMM_IQ4_NL), (M.QMM_Q8_0, M.QMM_Q8_0)])
def test_mmq_formats_full_range(wt_gu, wt_down):
    """Q8_0 gate/up (factors over all of [-128, 127]), IQ4_NL or Q8_0 down; hidden 320 and inter
    192: odd numbers of 64-wide K steps, partly filled column tiles."""
    print(f"mmq formats gu={wt_gu} down={wt_down}", flush=True)
    c = Mmq(3320 + wt_down, 5, 90, 2, 320, 192, wt_gu=wt_gu, wt_down=wt_down, full_range=True)
    y, ws = c.run_gpu()
    print(c.check(np.arange(c.st.size), y, ws), flush=True)


def test_mmq_full_size():
    """8192 tokens x 2560, 128 experts, top-8, IQ4_NL gate/up 2560 -> 1024, Q8_0 down: every row
    of the largest and the smallest expert and 96 random rows."""
    print("mmq full size: 8192 x 2560, 128 experts, top-8", flush=True)
    c = Mmq(synth.SEEDS["prefill"], 128, 8192, 8, 2560, 1024)
    y, ws = c.run_gpu()
    counts = np.diff(c.off)
    rng = synth.rng_for(3330)
    samples = set()
    for e in (int(np.argmax(counts)), int(np.argmin(counts))):
        samples.update(range(int(c.off[e]), int(c.off[e + 1])))
    samples.update(rng.choice(c.st.size, size=96, replace=False).tolist())
    print(f"{len(samples)} rows", flush=True)
    print(c.check(sorted(samples), y, ws), flush=True)
    assert np.isfinite(host(y)).all()


def test_mmq_entry_independence():
    """A row's output depends only on its token and expert (bitwise)."""
    print("mmq entry independence", flush=True)
    c = Mmq(3340, 8, 96, 2, 256, 64)
    y1 = host(c.run_gpu(flags=0)[0])
    keep = np.ones(c.st.size, bool)
    keep[::3] = False
    exps = np.searchsorted(c.off, np.arange(c.st.size), side="right") - 1
    st2 = c.st[keep].astype(np.int32)
    off2 = np.zeros(c.nexp + 1, np.int32)
    off2[1:] = np.cumsum(np.bincount(exps[keep], minlength=c.nexp))
    c.st, c.off = st2, off2
    c.d["st"], c.d["off"] = dev(st2), dev(off2)
    y2 = host(c.run_gpu(flags=0)[0])
    assert np.array_equal(y2.view(np.uint32), y1[keep].view(np.uint32))
