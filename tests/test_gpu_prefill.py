"""GPU parity of the prefill grouped expert GEMM (FP16 weights + MFMA) against the oracle.

G, U: within the fp32 error of the MFMA accumulation (each product is exact in binary32 and
passes through at most K/16 + 16 additions), asserted.  H16 = fp16(silu(G) U): equal to the
oracle's where the binary16 rounding is decided by the oracle's G, U alone, otherwise inside the
interval the bound allows; the interval is widened by 8 binary32 ulp for the device's binary32
silu (expf within 1 ulp, v_rcp_f32 of 1 + e within 1 ulp, two products) against the
oracle's binary64 exp.  Y: within 1e-4 * sum|w h| plus the effect of the validated H16
differences.  Full size (8192
tokens x 2560, 128 experts, top-8) is checked on sampled entries, including every entry of
an expert split into several tiles."""
import numpy as np
import pytest

import moe_expert_amd as M
import oracle
import synth
from tests.gpu_util import dev, host
from tests.grouped_check import silu_mul_interval

pytestmark = pytest.mark.gpu
U32 = 2.0 ** -24


class Prefill:
    def __init__(self, seed, nexp, ntok, topk, hidden, inter, wt_gu=M.QMM_IQ4_NL, wt_down=M.QMM_Q8_0):
        rng = synth.rng_for(seed)
        self.nexp, self.hidden, self.inter = nexp, hidden, inter
        self.wt_gu, self.wt_down = wt_gu, wt_down
        self.wg = np.stack([synth.weights(wt_gu, rng, inter, hidden) for _ in range(nexp)])
        self.wu = np.stack([synth.weights(wt_gu, rng, inter, hidden) for _ in range(nexp)])
        self.wd = np.stack([synth.weights(wt_down, rng, hidden, inter) for _ in range(nexp)])
        self.x16 = synth.prefill_tokens(rng, ntok, hidden)
        self.st, self.off = synth.prefill_routing(rng, ntok, nexp, topk)
        self.d = dict(wg=dev(self.wg), wu=dev(self.wu), wd=dev(self.wd), x=dev(self.x16.view(np.uint16)),
                      st=dev(self.st), off=dev(self.off))

    def run_gpu(self, flags=M.QMM_FLAG_DEBUG_INTERMEDIATES):
        y, ws = M.qgemm_prefill_experts(self.wt_gu, self.d["wg"], self.d["wu"], self.wt_down, self.d["wd"], self.nexp,
                                        self.hidden, self.inter, self.d["x"], self.d["st"], self.d["off"], flags=flags)
        return y, ws

    def split_ws(self, ws):
        w = host(ws)
        ne = self.st.size
        h16 = w[: ne * self.inter * 2].view(np.uint16).reshape(ne, self.inter)
        tiles_off = (ne * self.inter * 2 + 15) // 16 * 16
        max_tiles = (ne + 255) // 256 + self.nexp
        g_off = (tiles_off + 4 * (1 + 3 * max_tiles) + 15) // 16 * 16
        g = w[g_off: g_off + 4 * ne * self.inter].view(np.float32).reshape(ne, self.inter)
        u = w[g_off + 4 * ne * self.inter: g_off + 8 * ne * self.inter].view(np.float32).reshape(ne, self.inter)
        return h16, g, u

    def check(self, samples, y, ws):
        samples = np.asarray(samples, np.int64)
        ref = oracle.prefill_rows(self.wt_gu, self.wg, self.wu, self.wt_down, self.wd, self.nexp, self.hidden,
                                  self.inter, self.x16, self.st, self.off, samples)
        h16, g, u = self.split_ws(ws)
        yh = host(y)
        depth = self.hidden // 16 + 16
        dG = 2 * depth * U32 * ref["Gabs"]
        dU = 2 * depth * U32 * ref["Uabs"]
        gs, us = g[samples].astype(np.float64), u[samples].astype(np.float64)
        assert np.all(np.abs(gs - ref["G"]) <= dG), f"G outside the fp32 bound: {np.max(np.abs(gs - ref['G']) / dG)}"
        assert np.all(np.abs(us - ref["U"]) <= dU), "U outside the fp32 bound"
        h_lo, h_hi = silu_mul_interval(ref["G"] - dG, ref["G"] + dG, ref["U"] - dU, ref["U"] + dU)
        pad = 8 * U32 * np.maximum(np.abs(h_lo), np.abs(h_hi)) + 1e-38
        with np.errstate(over="ignore"):
            lo16 = (h_lo - pad).astype(np.float16).astype(np.float64)
            hi16 = (h_hi + pad).astype(np.float16).astype(np.float64)
        hg = h16[samples].view(np.float16).astype(np.float64)
        ho = ref["H16"].view(np.float16).astype(np.float64)
        assert np.all((hg >= lo16) & (hg <= hi16)), "H16 outside its valid interval"
        unique = lo16 == hi16
        assert np.array_equal(hg[unique], ho[unique]), "H16 differs where the rounding is unique"
        dH = np.abs(hg - ho)
        # expert of each sample
        exps = np.searchsorted(self.off, samples, side="right") - 1
        wd16 = {}
        for i, p in enumerate(samples):
            extra = 0.0
            if dH[i].any():
                e = int(exps[i])
                if e not in wd16:
                    wd16[e] = oracle.dequant_f16(self.wt_down, self.wd[e], self.inter).view(np.float16).astype(np.float64)
                extra = np.abs(wd16[e]) @ dH[i]
            bound = 1e-4 * ref["Yabs"][i] + extra * (1 + 1e-6)
            err = np.abs(yh[p].astype(np.float64) - ref["Y"][i])
            assert np.all(err <= bound), f"entry {p}: Y outside tolerance, max excess {np.max(err - bound)}"
        return {"h16_ambiguous": int((~unique).sum()), "h16_differ": int((hg != ho).sum()), "rows": len(samples)}


def test_prefill_small():
    print("prefill small: 6 experts, 40 tokens top-2, 256 -> 64 -> 256", flush=True)
    pf = Prefill(900, 6, 40, 2, 256, 64)
    y, ws = pf.run_gpu()
    print(pf.check(np.arange(pf.st.size), y, ws), flush=True)


def test_prefill_ragged_tiles():
    """Experts with 0, 1, 31, 32, 33, 256, 257 and 600 rows: no tile, one partial 32-row block,
    exact blocks, a full 256-row tile, and experts split into 2 and 3 tiles of equal height."""
    print("prefill ragged: expert row counts 0 1 31 32 33 256 257 600", flush=True)
    counts = np.array([0, 1, 31, 32, 33, 256, 257, 600])
    pf = Prefill(910, 8, 1300, 1, 512, 128)
    pf.st = (np.arange(counts.sum(), dtype=np.int64) * 7 % 1300).astype(np.int32)
    pf.off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    pf.d["st"], pf.d["off"] = dev(pf.st), dev(pf.off)
    y, ws = pf.run_gpu()
    print(pf.check(np.arange(pf.st.size), y, ws), flush=True)


def test_prefill_odd_shapes():
    """hidden 320 and inter 192: an odd number of 64-wide K steps in both GEMMs, gate/up column
    tiles of 128 and down column tiles of 256 that are only partly inside the matrix."""
    print("prefill odd shapes: 5 experts, 90 tokens top-2, 320 -> 192 -> 320", flush=True)
    pf = Prefill(915, 5, 90, 2, 320, 192)
    y, ws = pf.run_gpu()
    print(pf.check(np.arange(pf.st.size), y, ws), flush=True)


def test_prefill_formats_swapped():
    print("prefill formats: Q8_0 gate/up, IQ4_NL down", flush=True)
    pf = Prefill(920, 4, 64, 2, 256, 128, wt_gu=M.QMM_Q8_0, wt_down=M.QMM_IQ4_NL)
    y, ws = pf.run_gpu()
    print(pf.check(np.arange(pf.st.size), y, ws), flush=True)


def test_prefill_full_size_sampled():
    """8192 tokens x 2560, 128 experts, top-8, gate/up IQ4_NL 2560->1024, down Q8_0 1024->2560."""
    print("prefill full size: 8192 x 2560, 128 experts, top-8", flush=True)
    pf = Prefill(synth.SEEDS["prefill"], 128, 8192, 8, 2560, 1024)
    y, ws = pf.run_gpu()
    rng = synth.rng_for(930)
    samples = set(rng.choice(pf.st.size, size=160, replace=False).tolist())
    counts = np.diff(pf.off)
    split = [e for e in range(128) if counts[e] > 256 and counts[e] % 32][:1]
    for e in split:                        # every row of one expert split into several tiles
        samples.update(range(pf.off[e], pf.off[e + 1]))
    samples.update([0, pf.st.size - 1])
    print(pf.check(sorted(samples), y, ws), flush=True)
    # rows of all other experts are finite (no unwritten output)
    assert np.isfinite(host(y)).all()


def test_prefill_entry_independence():
    """A row's output depends only on its token and expert: rerouting the other tokens changes
    nothing in it (bitwise)."""
    print("prefill entry independence", flush=True)
    pf = Prefill(940, 8, 96, 2, 256, 64)
    y1, _ = pf.run_gpu(flags=0)
    y1 = host(y1)
    # drop every second token's second expert: the remaining (token, expert) rows must not change
    keep = np.ones(pf.st.size, bool)
    exps = np.searchsorted(pf.off, np.arange(pf.st.size), side="right") - 1
    keep[::3] = False
    st2 = pf.st[keep]
    e2 = exps[keep]
    off2 = np.zeros(pf.nexp + 1, np.int32)
    off2[1:] = np.cumsum(np.bincount(e2, minlength=pf.nexp))
    pf.d["st"], pf.d["off"] = dev(st2.astype(np.int32)), dev(off2)
    pf.st = st2.astype(np.int32)
    y2, _ = pf.run_gpu(flags=0)
    assert np.array_equal(host(y2).view(np.uint32), y1[keep].view(np.uint32))
