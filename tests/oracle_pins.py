"""Pins of the CPU oracle to things other than itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError when the oracle
disagrees with what the pages, the format definitions and mathematics fix:

* hand-worked fixtures under tests/golden/ (values derived by hand from the formats);
* numpy's IEEE binary16 conversion (a library routine) for every fp16 rounding;
* brute force: numpy float64 dequantize-then-dot on small inputs;
* closed forms and invariants (sign symmetry, power-of-two scaling, one-hot rows,
  cross-format identities, SwiGLU limits).

The same functions run against deliberately broken builds of the oracle in
test_oracle_mutations.py, which checks that each planted mistake fails at least one pin.
"""
from __future__ import annotations

import numpy as np

import synth
from tests import _golden

Q8_0, IQ4_NL, CB3 = 1, 2, 3
KV_IQ4NL = np.array([-127, -104, -83, -65, -49, -35, -22, -10, 1, 13, 25, 38, 53, 69, 89, 113])


# ------------------------------------------------------------------ helpers (independent of the oracle)

def np_f16_bits(x64: np.ndarray) -> np.ndarray:
    """numpy's correctly rounded binary16 conversion of float64 values, as bit patterns."""
    with np.errstate(over="ignore", invalid="ignore"):
        return np.asarray(x64, np.float64).astype(np.float16).view(np.uint16)


def np_q8_1_decode(xq: np.ndarray, k: int):
    """Decode q8_1 blocks with numpy: returns (x_hat float64 [ncols, k], d float64 [ncols, k/32],
    q int32 [ncols, k])."""
    xq = np.asarray(xq, np.uint8).reshape(-1, k // 32, 36)
    d = xq[:, :, 0:2].copy().view(np.float16)[:, :, 0].astype(np.float64)
    q = xq[:, :, 4:36].view(np.int8).astype(np.int32)
    xh = (q * d[:, :, None]).reshape(xq.shape[0], k)
    return xh, d, q.reshape(xq.shape[0], k)


def finite_f16_patterns() -> np.ndarray:
    p = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    return p[((p >> 10) & 31) != 31]


# ------------------------------------------------------------------ fp16

def pin_fp16_golden(orc):
    to32, from64 = _golden.fp16_cases()
    for bits, val in to32:
        got = float(orc.f16_to_f32(np.array([bits], np.uint16))[0])
        assert got == val and np.signbit(got) == np.signbit(val), (hex(bits), got, val)
    for val, bits in from64:
        assert orc.f64_to_f16(val) == bits, (val, hex(orc.f64_to_f16(val)), hex(bits))


def pin_fp16_exhaustive(orc):
    p = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.f16_to_f32(p)
    ref = p.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    # float32 -> binary16: every finite half, every midpoint between neighbours (ties), and
    # random float32 over the whole exponent range
    fin = finite_f16_patterns()
    v = np.sort(fin.view(np.float16).astype(np.float64))
    mids = ((v[1:] + v[:-1]) / 2.0).astype(np.float32)
    rng = synth.rng_for(11)
    rnd = (rng.standard_normal(400_000) * np.exp2(rng.uniform(-30, 20, 400_000))).astype(np.float32)
    xs = np.concatenate([v.astype(np.float32), mids, rnd, np.float32([65519.996, 65520, -65520, 7e4])])
    assert np.array_equal(orc.f32_to_f16(xs), np_f16_bits(xs.astype(np.float64)))


# ------------------------------------------------------------------ formats (dequantization)

def pin_formats_golden(orc):
    blk, vals, f16 = _golden.simple_block("q8_0_block.txt")
    assert np.array_equal(orc.dequant_f64(Q8_0, blk, 32)[0], vals)
    assert np.array_equal(orc.dequant_f16(Q8_0, blk, 32)[0], f16)
    blk, vals, _ = _golden.simple_block("iq4nl_block.txt")
    assert np.array_equal(orc.dequant_f64(IQ4_NL, blk, 32)[0], vals)
    blk, grid, values = _golden.cb3_superblock()
    got = orc.dequant_f64(CB3, blk, 256, grid)[0]
    for v, expect in values.items():
        assert got[v] == expect, (v, got[v], expect)


def pin_dequant_f16_exhaustive(orc):
    """FP16 dequant == numpy's binary16 rounding of the exact value, over every finite fp16
    scale and every integer factor (all 256 int8 q for Q8_0, all 16 levels for IQ4_NL, a
    sample of CB3 multiplier x magnitude x sign)."""
    d = finite_f16_patterns()
    nd = d.size
    # Q8_0: 8 blocks per scale cover the 256 int8 values
    q = np.arange(-128, 128, dtype=np.int16).astype(np.int8).view(np.uint8).reshape(8, 32)
    blk = np.empty((nd, 8, 34), np.uint8)
    blk[:, :, 0:2] = d.view(np.uint8).reshape(nd, 1, 2)
    blk[:, :, 2:] = q[None]
    w = blk.reshape(nd, 8 * 34)
    exact = orc.dequant_f64(Q8_0, w, 256)
    assert np.array_equal(orc.dequant_f16(Q8_0, w, 256), np_f16_bits(exact))
    # exact values themselves: d * q with numpy float64
    dv = d.view(np.float16).astype(np.float64)
    qv = np.arange(-128, 128, dtype=np.float64)
    assert np.array_equal(exact, dv[:, None] * qv[None, :])
    # IQ4_NL: one block per scale, bytes 0x10 0x32 ... cover all 16 indices
    blk = np.empty((nd, 18), np.uint8)
    blk[:, 0:2] = d.view(np.uint8).reshape(nd, 2)
    blk[:, 2:] = np.array([0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE] * 2, np.uint8)
    exact = orc.dequant_f64(IQ4_NL, blk, 32)
    assert np.array_equal(orc.dequant_f16(IQ4_NL, blk, 32), np_f16_bits(exact))
    idx = np.array([0, 2, 4, 6, 8, 10, 12, 14] * 2 + [1, 3, 5, 7, 9, 11, 13, 15] * 2)
    assert np.array_equal(exact, dv[:, None] * KV_IQ4NL[idx][None, :])
    # CB3: every finite scale with random codebook fields
    rng = synth.rng_for(12)
    grid = synth.cb3_grid(rng)
    w = synth.cb3_weights(rng, nd // 8, 256 * 8)
    w = w.reshape(-1, 110)
    w[:, 0:2] = d[: w.shape[0]].view(np.uint8).reshape(-1, 2)
    exact = orc.dequant_f64(CB3, w, 256, grid)
    assert np.array_equal(orc.dequant_f16(CB3, w, 256, grid), np_f16_bits(exact))


def pin_dequant_ld(orc):
    """Row stride ``ld`` > k leaves the padding untouched and rows in place."""
    rng = synth.rng_for(13)
    w = synth.q8_0_weights(rng, 5, 64)
    a = orc.dequant_f16(Q8_0, w, 64)
    b = orc.dequant_f16(Q8_0, w, 64, ld=72)
    assert np.array_equal(b[:, :64], a) and not b[:, 64:].any()


# ------------------------------------------------------------------ q8_1

def pin_q8_1_golden(orc):
    for c in _golden.q8_1_cases():
        out = orc.quantize_q8_1(c["x"][None, :])[0]
        assert int(out[0]) | (int(out[1]) << 8) == c["d"], (out[:2], hex(c["d"]))
        assert int(out[2]) | (int(out[3]) << 8) == c["s"], (out[2:4], hex(c["s"]))
        assert np.array_equal(out[4:].view(np.int8), c["q"]), (out[4:].view(np.int8), c["q"])


def _q8_1_inputs(n=20000, seed=14):
    rng = synth.rng_for(seed)
    x = rng.standard_normal((n, 32)) * np.exp2(rng.uniform(-20, 12, (n, 1)))
    x[::97, 5] *= 3e4                      # outliers
    x[::53, :] = 0.0                       # zero blocks
    x[::31, 7] = -np.abs(x[::31]).max(axis=1)  # amax carried by a negative value
    return x.astype(np.float32)


def pin_q8_1_properties(orc):
    x = _q8_1_inputs()
    n = x.shape[0]
    xq = orc.quantize_q8_1(x.reshape(1, -1)).reshape(n, 36)
    d = xq[:, 0:2].copy().view(np.float16)[:, 0]
    s = xq[:, 2:4].copy().view(np.uint16)[:, 0]
    q = xq[:, 4:].view(np.int8).astype(np.int32)
    amax = np.abs(x).max(axis=1)
    zero = amax == 0
    assert not q[zero].any() and not d[zero].view(np.uint16).any() and not s[zero].any()
    nz = ~zero
    # the element carrying amax maps to +-127 and nothing exceeds it
    assert np.all(np.abs(q[nz]).max(axis=1) == 127)
    # d = numpy's binary32 amax/127, stored as numpy's binary16 of it
    d32 = amax.astype(np.float32) / np.float32(127.0)
    assert np.array_equal(d.view(np.uint16)[nz], np_f16_bits(d32[nz].astype(np.float64)))
    # every q is a nearest integer of x/d (within the one rounding of the division)
    r = x[nz].astype(np.float64) / d32[nz, None].astype(np.float64)
    assert np.all(np.abs(q[nz] - r) <= 0.5 + 1e-6 * np.maximum(1.0, np.abs(r)))
    # s = binary16 of the binary32 product d * sum(q)
    s_ref = np_f16_bits((d32[nz] * q[nz].sum(axis=1).astype(np.float32)).astype(np.float64))
    assert np.array_equal(s[nz], s_ref)
    # sign symmetry and power-of-two scaling
    xq_neg = orc.quantize_q8_1(-x.reshape(1, -1)).reshape(n, 36)
    assert np.array_equal(xq_neg[:, 4:].view(np.int8).astype(np.int32), -q)
    assert np.array_equal(xq_neg[:, 0:2], xq[:, 0:2])
    small = nz & (amax < 1e3) & (amax > 1e-2)
    xs = (x[small] * np.float32(8.0)).astype(np.float32)
    xq8 = orc.quantize_q8_1(xs.reshape(1, -1)).reshape(-1, 36)
    assert np.array_equal(xq8[:, 4:], xq[small, 4:])
    d8 = xq8[:, 0:2].copy().view(np.float16)[:, 0].astype(np.float64)
    assert np.array_equal(d8, d[small].astype(np.float64) * 8.0)


def pin_q8_1_ties(orc):
    """x/d landing exactly on k + 1/2 rounds away from zero (d = 1 blocks)."""
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 127.0
    x[0, 1:] = np.arange(1, 32) * 2.0 - 31.5   # -29.5 ... 30.5, all halves
    q = orc.quantize_q8_1(x)[0, 4:].view(np.int8).astype(np.int32)
    expect = np.sign(x[0]) * np.floor(np.abs(x[0]) + 0.5)
    assert np.array_equal(q, expect.astype(np.int32))


# ------------------------------------------------------------------ integer dots and GEMV

def _small_case(wtype, nrows, k, ncols, seed):
    rng = synth.rng_for(seed)
    grid = synth.cb3_grid(rng) if wtype == CB3 else None
    w = synth.weights(wtype, rng, nrows, k)
    x = synth.activations(rng, ncols, k)
    return w, grid, x


def pin_block_sums(orc):
    for wtype, k in ((Q8_0, 256), (IQ4_NL, 256), (CB3, 512)):
        w, grid, x = _small_case(wtype, 7, k, 3, 20 + wtype)
        xq = orc.quantize_q8_1(x)
        _, _, q = np_q8_1_decode(xq, k)
        wx = orc.dequant_f64(wtype, w, k, grid)                    # exact values
        bv = 256 if wtype == CB3 else 32
        d_w = w.reshape(7, k // bv, -1)[:, :, 0:2].copy().view(np.float16)[:, :, 0].astype(np.float64)
        wint = wx / np.repeat(d_w, bv, axis=1)                     # integer factors
        assert np.array_equal(wint, np.round(wint)), "dequant is not d x integer"
        ref = np.einsum("rbj,cbj->crb", wint.reshape(7, k // 32, 32).astype(np.int64),
                        q.reshape(3, k // 32, 32).astype(np.int64))
        got = orc.block_sums(wtype, w, k, xq, grid)
        assert np.array_equal(got, ref)


def pin_gemv_bruteforce(orc):
    """y == float64 dequantize-then-dot, up to the one binary32 rounding of each block term."""
    for wtype, nrows, k, ncols in ((Q8_0, 33, 512, 3), (IQ4_NL, 64, 512, 5), (CB3, 17, 1024, 2)):
        w, grid, x = _small_case(wtype, nrows, k, ncols, 30 + wtype)
        xq = orc.quantize_q8_1(x)
        xh, _, _ = np_q8_1_decode(xq, k)
        wx = orc.dequant_f64(wtype, w, k, grid)
        brute = xh @ wx.T                                           # [ncols, nrows]
        y, a = orc.gemv(wtype, w, k, xq, grid)
        assert np.all(np.abs(y - brute) <= a * 2.0 ** -23 + 1e-300)
        assert np.all(a >= np.abs(y) * (1 - 1e-12))


def pin_gemv_onehot(orc):
    """Rows with a single non-zero block scale: y equals that block's binary32 term exactly."""
    for wtype, k in ((Q8_0, 256), (IQ4_NL, 256), (CB3, 512)):
        bv, bb = (256, 110) if wtype == CB3 else (32, 34 if wtype == Q8_0 else 18)
        nb = k // bv
        w, grid, x = _small_case(wtype, nb, k, 2, 40 + wtype)
        w = w.reshape(nb, nb, bb).copy()
        for r in range(nb):
            for b in range(nb):
                if b != r:
                    w[r, b, 0:2] = 0
        w = w.reshape(nb, nb * bb)
        xq = orc.quantize_q8_1(x)
        sums = orc.block_sums(wtype, w, k, xq, grid)                # [ncols, nrows, k/32]
        _, da, _ = np_q8_1_decode(xq, k)
        y, _ = orc.gemv(wtype, w, k, xq, grid)
        for r in range(nb):
            dw = np.float32(w[r, r * bb:r * bb + 2].copy().view(np.float16)[0])
            sub = range(r * bv // 32, (r + 1) * bv // 32)
            for c in range(2):
                ref = sum(float((dw * np.float32(da[c, j])) * np.float32(sums[c, r, j])) for j in sub)
                assert y[c, r] == ref, (wtype, r, c, y[c, r], ref)


def pin_cross_format(orc):
    """IQ4_NL re-encoded as Q8_0 with q = KV[idx] and the same d gives identical values, sums
    and outputs; so does CB3 with every sub-scale 0 re-encoded as Q8_0 with q = +-grid."""
    rng = synth.rng_for(50)
    nrows, k = 9, 256
    w4 = synth.iq4nl_weights(rng, nrows, k).reshape(nrows, k // 32, 18)
    lo, hi = w4[:, :, 2:] & 15, w4[:, :, 2:] >> 4
    q = KV_IQ4NL[np.concatenate([lo, hi], axis=2)].astype(np.int8)
    w8 = np.concatenate([w4[:, :, 0:2], q.view(np.uint8)], axis=2).reshape(nrows, -1)
    w4 = w4.reshape(nrows, -1)
    x = synth.activations(rng, 3, k)
    xq = orc.quantize_q8_1(x)
    assert np.array_equal(orc.dequant_f64(IQ4_NL, w4, k), orc.dequant_f64(Q8_0, w8, k))
    assert np.array_equal(orc.block_sums(IQ4_NL, w4, k, xq), orc.block_sums(Q8_0, w8, k, xq))
    assert np.array_equal(orc.gemv(IQ4_NL, w4, k, xq)[0], orc.gemv(Q8_0, w8, k, xq)[0])
    # CB3 with all sub-scales 0
    grid = synth.cb3_grid(rng)
    wc = synth.cb3_weights(rng, nrows, k).reshape(nrows, 110)
    wc[:, 106:110] = 0
    qs, qh, sg = wc[:, 2:66].astype(np.int64), wc[:, 66:74], wc[:, 74:106]
    i = np.arange(64)
    idx = qs | (((qh[:, i // 8] >> (i % 8)) & 1).astype(np.int64) << 8)
    mag = grid[idx].reshape(nrows, 256).astype(np.int64)            # value v = 4i + j
    v = np.arange(256)
    neg = (sg[:, v // 8] >> (v % 8)) & 1
    qq = (mag * (1 - 2 * neg.astype(np.int64))).astype(np.int8).reshape(nrows, 8, 32)
    d = np.repeat(wc[:, None, 0:2], 8, axis=1)
    w8 = np.concatenate([d, qq.view(np.uint8)], axis=2).reshape(nrows, -1)
    assert np.array_equal(orc.dequant_f64(CB3, wc, k, grid), orc.dequant_f64(Q8_0, w8, k))
    assert np.array_equal(orc.block_sums(CB3, wc, k, xq, grid), orc.block_sums(Q8_0, w8, k, xq))


# ------------------------------------------------------------------ SwiGLU

def pin_silu(orc):
    g = np.array([0.0, -0.0, 30.0, 100.0, -100.0, -88.0, -89.0, 1.0, -1.0, 5.0], np.float32)
    u = np.ones_like(g)
    h = orc.silu_mul(g, u)
    assert h[0] == 0 and h[1] == 0
    assert h[2] == np.float32(30.0) and h[3] == np.float32(100.0)   # e^-z below half an ulp
    assert h[4] == 0 and np.signbit(h[4])                          # e^100 overflows binary32 -> -0
    assert h[6] <= 0 and np.isfinite(h).all()
    rng = synth.rng_for(60)
    g = (rng.standard_normal(100_000) * 20).astype(np.float32)
    u = (rng.standard_normal(100_000) * 20).astype(np.float32)
    h = orc.silu_mul(g, u).astype(np.float64)
    gd, ud = g.astype(np.float64), u.astype(np.float64)
    exact = gd / (1.0 + np.exp(-gd)) * ud
    ulp = np.spacing(np.abs(exact).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(h - exact) <= 4 * ulp + 1e-38)


# ------------------------------------------------------------------ grouped decode

def _grouped_case(seed=70, nexp=5, hidden=512, inter=64, m=3, ngroups=3):
    rng = synth.rng_for(seed)
    grid = synth.cb3_grid(rng)
    wg = np.stack([synth.cb3_weights(rng, inter, hidden) for _ in range(nexp)])
    wu = np.stack([synth.cb3_weights(rng, inter, hidden) for _ in range(nexp)])
    wd = np.stack([synth.iq4nl_weights(rng, hidden, inter) for _ in range(nexp)])
    ge, go, ec = synth.decode_routing(rng, nexp, ngroups, m)
    ec = ec[::-1].copy()                                           # non-trivial column map
    x = synth.activations(rng, m, hidden)
    return grid, wg, wu, wd, ge, go, ec, x, hidden, inter


def pin_grouped(orc):
    grid, wg, wu, wd, ge, go, ec, x, hidden, inter = _grouped_case()
    xq = orc.quantize_q8_1(x)
    xh, _, _ = np_q8_1_decode(xq, hidden)
    out = orc.grouped(CB3, wg, wu, IQ4_NL, wd, hidden, inter, xq, ge, go, ec, grid)
    for gi in range(ge.size):
        e = ge[gi]
        Wg = orc.dequant_f64(CB3, wg[e], hidden, grid)
        Wu = orc.dequant_f64(CB3, wu[e], hidden, grid)
        Wd = orc.dequant_f64(IQ4_NL, wd[e], inter)
        for kk in range(go[gi], go[gi + 1]):
            xv = xh[ec[kk]]
            assert np.all(np.abs(out["g"][kk] - Wg @ xv) <= out["gabs"][kk] * 2.0 ** -23)
            assert np.all(np.abs(out["u"][kk] - Wu @ xv) <= out["uabs"][kk] * 2.0 ** -23)
            h = orc.silu_mul(out["g"][kk].astype(np.float32), out["u"][kk].astype(np.float32))
            assert np.array_equal(out["h"][kk], h)
            assert np.array_equal(out["hq"][kk], orc.quantize_q8_1(h[None, :])[0])
            hh, _, _ = np_q8_1_decode(out["hq"][kk], inter)
            assert np.all(np.abs(out["y"][kk] - Wd @ hh[0]) <= out["yabs"][kk] * 2.0 ** -23)


def pin_grouped_entry_independence(orc):
    """An entry's outputs do not depend on the other entries or groups of the call."""
    grid, wg, wu, wd, ge, go, ec, x, hidden, inter = _grouped_case(seed=71)
    xq = orc.quantize_q8_1(x)
    full = orc.grouped(CB3, wg, wu, IQ4_NL, wd, hidden, inter, xq, ge, go, ec, grid)
    for gi in range(ge.size):
        for kk in range(go[gi], go[gi + 1]):
            one = orc.grouped(CB3, wg, wu, IQ4_NL, wd, hidden, inter, xq, ge[gi:gi + 1],
                              np.array([0, 1], np.int32), ec[kk:kk + 1], grid)
            assert np.array_equal(one["y"][0], full["y"][kk])
            assert np.array_equal(one["hq"][0], full["hq"][kk])


# ------------------------------------------------------------------ prefill GEMM

def _prefill_case(seed=80, nexp=6, ntok=40, topk=2, hidden=256, inter=64):
    rng = synth.rng_for(seed)
    wg = np.stack([synth.iq4nl_weights(rng, inter, hidden) for _ in range(nexp)])
    wu = np.stack([synth.iq4nl_weights(rng, inter, hidden) for _ in range(nexp)])
    wd = np.stack([synth.q8_0_weights(rng, hidden, inter) for _ in range(nexp)])
    x16 = synth.prefill_tokens(rng, ntok, hidden)
    st, off = synth.prefill_routing(rng, ntok, nexp, topk)
    return wg, wu, wd, x16, st, off, nexp, hidden, inter


def pin_prefill(orc):
    """G, U equal float64 numpy matmuls of the FP16 weights (library routine); H16 is the
    binary16 of the SwiGLU of the binary32-rounded sums; Y equals the numpy matmul of the FP16
    down weights with H16."""
    wg, wu, wd, x16, st, off, nexp, hidden, inter = _prefill_case()
    samples = np.arange(st.size, dtype=np.int64)
    out = orc.prefill_rows(IQ4_NL, wg, wu, Q8_0, wd, nexp, hidden, inter, x16, st, off, samples)
    xf = x16.astype(np.float64)
    for e in range(nexp):
        Wg = orc.dequant_f16(IQ4_NL, wg[e], hidden).view(np.float16).astype(np.float64)
        Wu = orc.dequant_f16(IQ4_NL, wu[e], hidden).view(np.float16).astype(np.float64)
        Wd = orc.dequant_f16(Q8_0, wd[e], inter).view(np.float16).astype(np.float64)
        for p in range(off[e], off[e + 1]):
            t = st[p]
            G = Wg @ xf[t]
            U = Wu @ xf[t]
            assert np.allclose(out["G"][p], G, rtol=0, atol=1e-9) and np.allclose(out["U"][p], U, rtol=0, atol=1e-9)
            assert np.allclose(out["Gabs"][p], np.abs(Wg * xf[t]).sum(axis=1), rtol=1e-12)
            H = orc.silu_mul(G.astype(np.float32), U.astype(np.float32))
            H16 = np_f16_bits(H.astype(np.float64))
            # a G within 1e-9 of numpy's can round to another binary32 only at a tie; allow none
            assert np.array_equal(out["H16"][p], H16)
            Y = Wd @ H16.view(np.float16).astype(np.float64)
            assert np.allclose(out["Y"][p], Y, rtol=0, atol=1e-9)


def pin_prefill_entry_independence(orc):
    """A sampled entry's row depends only on its token and expert, not on which other entries
    are sampled or routed."""
    wg, wu, wd, x16, st, off, nexp, hidden, inter = _prefill_case(seed=81)
    all_s = np.arange(st.size, dtype=np.int64)
    full = orc.prefill_rows(IQ4_NL, wg, wu, Q8_0, wd, nexp, hidden, inter, x16, st, off, all_s)
    pick = all_s[::7]
    part = orc.prefill_rows(IQ4_NL, wg, wu, Q8_0, wd, nexp, hidden, inter, x16, st, off, pick)
    assert np.array_equal(part["Y"], full["Y"][pick])
    assert np.array_equal(part["H16"], full["H16"][pick])


# ------------------------------------------------------------------ MoE combine

def pin_moe_combine_golden(orc):
    """Hand-worked cases: k order, the product rounded before the sum, +0, skipped rows."""
    for name, y, idx, w, out in _golden.moe_combine_cases():
        got = orc.moe_combine(y, idx, w)[0, 0]
        assert got == out and np.signbit(got) == np.signbit(out), (name, float(got).hex(), out)


def pin_moe_combine_properties(orc):
    """Within the binary32 bound of the exact weighted sum (float64 brute force: every product
    of two binary32 values is exact in float64); one row with weight 1 copies it; moving the
    rows of y (and the indices with them) changes no bit; k order matters only by rounding."""
    rng = np.random.default_rng(90)
    nrows, hidden, ntok, topk = 64, 40, 12, 6
    y = (rng.standard_normal((nrows, hidden)) * np.exp2(rng.integers(-8, 8, (nrows, 1)))).astype(np.float32)
    idx = rng.integers(0, nrows, (ntok, topk)).astype(np.int32)
    w = rng.random((ntok, topk)).astype(np.float32)
    out = orc.moe_combine(y, idx, w).astype(np.float64)
    terms = w.astype(np.float64)[:, :, None] * y.astype(np.float64)[idx]      # [ntok, topk, hidden]
    exact = terms.sum(axis=1)
    bound = 2 * topk * 2.0 ** -24 * np.abs(terms).sum(axis=1)
    assert np.all(np.abs(out - exact) <= bound)
    one = orc.moe_combine(y, idx[:, :1], np.ones((ntok, 1), np.float32))
    assert np.array_equal(one, y[idx[:, 0]])
    perm = rng.permutation(nrows)
    inv = np.argsort(perm)
    moved = orc.moe_combine(y[perm], inv[idx].astype(np.int32), w)
    assert np.array_equal(moved.view(np.uint32), out.astype(np.float32).view(np.uint32))
    rev = orc.moe_combine(y, idx[:, ::-1].copy(), w[:, ::-1].copy()).astype(np.float64)
    assert np.all(np.abs(rev - exact) <= bound)


# ------------------------------------------------------------------ dense prompt projections

def np_dequant_f16(wtype, w, k):
    """FP16 dequantization of Q8_0 / IQ4_NL rows with numpy alone: the exact product d * factor in
    float64, rounded by numpy's binary16 conversion.  [nrows, k] float64 of the binary16 values."""
    bb = 34 if wtype == Q8_0 else 18
    blk = np.asarray(w, np.uint8).reshape(-1, k // 32, bb)
    d = blk[:, :, 0:2].copy().view(np.float16)[:, :, 0].astype(np.float64)
    if wtype == Q8_0:
        f = blk[:, :, 2:].view(np.int8).astype(np.float64)
    else:
        qs = blk[:, :, 2:].astype(np.int64)
        f = KV_IQ4NL[np.concatenate([qs & 15, qs >> 4], axis=2)].astype(np.float64)
    return (d[:, :, None] * f).astype(np.float16).astype(np.float64).reshape(blk.shape[0], k)


def pin_dense_rows(orc):
    """Y equals the float64 numpy matmul of numpy's FP16 dequantization with the tokens
    (library routines), for Q8_0 and IQ4_NL and for weights given as binary16 already; one-hot
    tokens give the weight columns exactly."""
    rng = synth.rng_for(95)
    nrows, k, ntok = 48, 192, 20
    x16 = synth.prefill_tokens(rng, ntok, k)
    samples = np.array([0, 3, 7, 19, 11], np.int64)
    for wt in (Q8_0, IQ4_NL):
        w = synth.weights(wt, rng, nrows, k, **(dict(qlo=-128) if wt == Q8_0 else {}))
        W = np_dequant_f16(wt, w, k)
        Y, A = orc.dense_rows(wt, w, nrows, k, x16, samples)
        ref = x16.astype(np.float64)[samples] @ W.T
        assert np.allclose(Y, ref, rtol=0, atol=1e-12 * np.abs(ref).max())
        assert np.allclose(A, np.abs(x16.astype(np.float64)[samples]) @ np.abs(W.T), rtol=1e-12)
        Y16, _ = orc.dense_rows(0, W.astype(np.float16).view(np.uint16), nrows, k, x16, samples)
        assert np.array_equal(Y16, Y)
        eye = np.eye(k, dtype=np.float16)
        Yi, _ = orc.dense_rows(wt, w, nrows, k, eye, np.arange(k, dtype=np.int64))
        assert np.array_equal(Yi, W.T)


# ------------------------------------------------------------------ weight planes

def pin_planes_golden(orc):
    for name, wt, k, blk, planes in _golden.planes_cases():
        assert np.array_equal(orc.pack_planes(wt, blk, k), planes), name


def pin_planes_layout(orc):
    """Rows of 1, 16, 17 and 80 blocks: each tile of n blocks holds the n blocks' factor bytes
    in order and then their n scales (numpy slicing of the blocks), rows keep their place."""
    rng = synth.rng_for(96)
    for wt in (Q8_0, IQ4_NL):
        bb, fb = (34, 32) if wt == Q8_0 else (18, 16)
        for nb in (1, 16, 17, 80):
            w = synth.weights(wt, rng, 3, 32 * nb)
            got = orc.pack_planes(wt, w, 32 * nb)
            blk = w.reshape(3, nb, bb)
            for t0 in range(0, nb, 16):
                n = min(16, nb - t0)
                tile = got[:, t0 * bb:(t0 + n) * bb]
                assert np.array_equal(tile[:, :n * fb], blk[:, t0:t0 + n, 2:].reshape(3, n * fb))
                assert np.array_equal(tile[:, n * fb:], blk[:, t0:t0 + n, 0:2].reshape(3, 2 * n))


CHEAP_PINS = [pin_fp16_golden, pin_formats_golden, pin_q8_1_golden, pin_q8_1_ties,
              pin_silu, pin_dequant_ld, pin_block_sums, pin_gemv_bruteforce, pin_gemv_onehot,
              pin_cross_format, pin_q8_1_properties, pin_grouped,
              pin_grouped_entry_independence, pin_prefill, pin_prefill_entry_independence,
              pin_moe_combine_golden, pin_moe_combine_properties, pin_dense_rows, pin_planes_golden,
              pin_planes_layout]
EXPENSIVE_PINS = [pin_fp16_exhaustive, pin_dequant_f16_exhaustive]
ALL_PINS = CHEAP_PINS + EXPENSIVE_PINS
