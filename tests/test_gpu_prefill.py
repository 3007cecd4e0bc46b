"""GPU parity of the prefill grouped expert GEMM (FP16 weights + MFMA) against the oracle.

G, U: within the fp32 error of the MFMA accumulation (each product is exact in binary32 and
passes through at most K/16 + 16 additions), asserted.  H16 = fp16(silu(G) U): equal to the
oracle's where the binary16 rounding is decided by the oracle's G, U alone, otherwise inside the
interval the bound allows; the interval is widened by 8 binary32 ulp for the device's binary32
silu (expf within 1 ulp, v_rcp_f32 of 1 + e within 1 ulp, two products) against the
oracle's binary64 exp.  Y: within 1e-4 * sum|w h| plus the effect of the validated H16
differences.  Full size (8192
tokens x 2560, 128 experts, top-8) is checked on every row of 8 whole experts (each split into
several tiles) plus sampled rows.  The FP16 weights the MFMAs consume are pinned bit for bit
through one-hot tokens (G = W16 exactly) and one-hot H16 (Y = Wd16 exactly)."""
import numpy as np
import pytest

import moe_expert_amd as M
import oracle
import synth
from tests.gpu_util import dev, host
from tests.grouped_check import silu_mul_interval

pytestmark = pytest.mark.gpu
U32 = 2.0 ** -24


def weights(wt, rng, nrows, k, full_range):
    """Seeded blocks; full_range: Q8_0 factors drawn from all of [-128, 127] (the generator's
    default stops at -127)."""
    kw = dict(qlo=-128) if full_range and wt == M.QMM_Q8_0 else {}
    return synth.weights(wt, rng, nrows, k, **kw)


class Prefill:
    def __init__(self, seed, nexp, ntok, topk, hidden, inter, wt_gu=M.QMM_IQ4_NL, wt_down=M.QMM_Q8_0,
                 full_range=False):
        rng = synth.rng_for(seed)
        self.nexp, self.hidden, self.inter = nexp, hidden, inter
        self.wt_gu, self.wt_down = wt_gu, wt_down
        self.wg = np.stack([weights(wt_gu, rng, inter, hidden, full_range) for _ in range(nexp)])
        self.wu = np.stack([weights(wt_gu, rng, inter, hidden, full_range) for _ in range(nexp)])
        self.wd = np.stack([weights(wt_down, rng, hidden, inter, full_range) for _ in range(nexp)])
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


@pytest.mark.parametrize("wt_gu,wt_down", [(M.QMM_Q8_0, M.QMM_Q8_0), (M.QMM_IQ4_NL, M.QMM_Q8_0)])
def test_prefill_q8_0_full_range(wt_gu, wt_down):
    """Q8_0 factors over all of [-128, 127] (-128 is the biased byte 0x00 of the conversion)."""
    print(f"prefill Q8_0 factors -128..127: gu={wt_gu} down={wt_down}", flush=True)
    pf = Prefill(925 + wt_gu, 4, 80, 2, 320, 128, wt_gu=wt_gu, wt_down=wt_down, full_range=True)
    assert (pf.wd.reshape(-1, 34)[:, 2:].view(np.int8) == -128).any()
    y, ws = pf.run_gpu()
    print(pf.check(np.arange(pf.st.size), y, ws), flush=True)


def identity_tokens(hidden):
    """Token t is the unit row e_t (binary16 1.0 at column t): X16 = I."""
    return np.eye(hidden, dtype=np.float16)


def every_token_routing(nexp, ntok):
    """Every token to every expert; rows sorted by expert, then token."""
    st = np.tile(np.arange(ntok, dtype=np.int32), nexp)
    off = (np.arange(nexp + 1, dtype=np.int32) * ntok).astype(np.int32)
    return st, off


@pytest.mark.parametrize("wt_gu", [M.QMM_IQ4_NL, M.QMM_Q8_0])
def test_prefill_gate_up_weights_bitexact(wt_gu):
    """The FP16 weights the gate/up MFMA consumes equal the dequantized values bit for bit:
    with token t = e_t every product but one is a zero, so G[row of (e, t)][i] = Wg16[e][i][t]
    exactly (likewise U), and the debug G, U of two experts x 2560 tokens are compared with the
    oracle's FP16 dequantization of every (i, t) of both matrices."""
    hidden, inter, nexp = 2560, 1024, 2
    print(f"prefill one-hot tokens: gate/up weights bit-exact, gu={wt_gu}", flush=True)
    pf = Prefill(950 + wt_gu, nexp, 1, 1, hidden, inter, wt_gu=wt_gu, wt_down=M.QMM_Q8_0, full_range=True)
    pf.x16 = identity_tokens(hidden)
    pf.st, pf.off = every_token_routing(nexp, hidden)
    pf.d["x"], pf.d["st"], pf.d["off"] = dev(pf.x16.view(np.uint16)), dev(pf.st), dev(pf.off)
    y, ws = pf.run_gpu()
    _, g, u = pf.split_ws(ws)
    for e in range(nexp):
        rows = slice(int(pf.off[e]), int(pf.off[e + 1]))
        for got, wq, what in ((g, pf.wg, "gate"), (u, pf.wu, "up")):
            w16 = oracle.dequant_f16(wt_gu, wq[e], hidden).view(np.float16).astype(np.float32)  # [inter, hidden]
            ok = got[rows] == w16.T
            assert ok.all(), f"expert {e} {what}: {(~ok).sum()} weights differ"


def unit_gate_up(nexp, hidden, inter):
    """Q8_0 gate/up matrices for which token e_t gives h = 1.0 at intermediate index t mod inter
    and 0 elsewhere: gate value 32 (d = 1/2, q = 64) and up value 1/32 (d = 2^-10, q = 32) at
    the columns k with k mod inter = row, zero factors elsewhere; silu(32) * (1/32) = 1 in
    binary32 (e^-32 vanishes beside 1)."""
    def mat(d, q):
        m = np.zeros((inter, hidden // 32, 34), np.uint8)
        m[:, :, 0:2] = np.array([d], np.float16).view(np.uint8)
        vals = np.zeros((inter, hidden), np.int8)
        k = np.arange(hidden)
        vals[k % inter, k] = q
        m[:, :, 2:] = vals.reshape(inter, hidden // 32, 32).view(np.uint8)
        return m.reshape(inter, -1)
    g = mat(0.5, 64)
    u = mat(2.0 ** -10, 32)
    return np.stack([g] * nexp), np.stack([u] * nexp)


@pytest.mark.parametrize("wt_down", [M.QMM_Q8_0, M.QMM_IQ4_NL])
def test_prefill_down_weights_bitexact(wt_down):
    """The FP16 weights of the down MFMA equal the dequantized values bit for bit: token e_t
    through unit_gate_up gives H16 = e_(t mod inter), so Y[row of (e, t)][j] = Wd16[e][j][t mod
    inter] exactly; every (j, i) of two experts' down matrices is compared with the oracle."""
    hidden, inter, nexp = 2560, 1024, 2
    print(f"prefill one-hot H: down weights bit-exact, down={wt_down}", flush=True)
    pf = Prefill(960 + wt_down, nexp, 1, 1, hidden, inter, wt_gu=M.QMM_Q8_0, wt_down=wt_down, full_range=True)
    pf.wg, pf.wu = unit_gate_up(nexp, hidden, inter)
    pf.x16 = identity_tokens(hidden)
    pf.st, pf.off = every_token_routing(nexp, hidden)
    pf.d.update(wg=dev(pf.wg), wu=dev(pf.wu), x=dev(pf.x16.view(np.uint16)), st=dev(pf.st), off=dev(pf.off))
    y, ws = pf.run_gpu()
    h16, _, _ = pf.split_ws(ws)
    t = np.arange(hidden)
    one_hot = np.zeros((hidden, inter), np.float16)
    one_hot[t, t % inter] = 1.0
    yh = host(y)
    for e in range(nexp):
        rows = slice(int(pf.off[e]), int(pf.off[e + 1]))
        assert np.array_equal(h16[rows], one_hot.view(np.uint16)), f"expert {e}: H16 is not one-hot"
        wd16 = oracle.dequant_f16(wt_down, pf.wd[e], inter).view(np.float16).astype(np.float32)  # [hidden, inter]
        ok = yh[rows] == wd16[:, t % inter].T
        assert ok.all(), f"expert {e}: {(~ok).sum()} down weights differ"
    # and the tolerance check of the general path agrees on a few rows
    print(pf.check(np.array([0, 1, 1023, 1024, 2559, 2560, 5119]), y, ws), flush=True)


def test_prefill_full_size_whole_experts():
    """8192 tokens x 2560, 128 experts, top-8, gate/up IQ4_NL 2560->1024, down Q8_0 1024->2560:
    every row of 8 whole experts (the largest and the smallest, both split into several tiles,
    and 6 drawn at random), plus 64 random rows of the others, against the oracle."""
    print("prefill full size: 8192 x 2560, 128 experts, top-8", flush=True)
    pf = Prefill(synth.SEEDS["prefill"], 128, 8192, 8, 2560, 1024)
    y, ws = pf.run_gpu()
    counts = np.diff(pf.off)
    rng = synth.rng_for(930)
    exps = {int(np.argmax(counts)), int(np.argmin(counts))}
    exps.update(int(e) for e in rng.choice(128, size=12, replace=False) if len(exps) < 8)
    exps = sorted(exps)[:8]
    samples = set()
    for e in exps:
        samples.update(range(int(pf.off[e]), int(pf.off[e + 1])))
    samples.update(rng.choice(pf.st.size, size=64, replace=False).tolist())
    samples.update([0, pf.st.size - 1])
    print(f"experts {exps} ({counts[exps].tolist()} rows), {len(samples)} rows in all", flush=True)
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
