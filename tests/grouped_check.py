"""Checking grouped-decode outputs against the oracle where a q8_1 decision can go either way.

The GPU's gate/up sums g, u differ from the oracle's in the last bits (another summation
order), and q8_1 quantization of h = silu(g) u turns those bits into integer codes: where h/d
lies within rounding distance of a half-integer, or amax/127 of an fp16 rounding boundary, more
than one code is correct.  The check therefore

  1. bounds |g_gpu - g_oracle| and |u_gpu - u_oracle| by the fp32 error of the GPU's reduction
     (each term passes through at most `depth` roundings), and asserts it;
  2. propagates that bound through silu and the quantizer to an interval of valid d and q per
     value, using the oracle's g, u only;
  3. requires every GPU H byte to equal the oracle's where the interval holds a single value,
     and to lie in the interval elsewhere; the sum field s = fp16(d * sum q) equals the oracle's
     where the whole block is unique, and elsewhere is what a valid binary32 d gives with the
     GPU's own codes;
  4. requires |y_gpu - y_oracle| <= 1e-4 * sum|terms| + sum_j |W_down[r, j]| * |H_gpu_j - H_or_j|,
     the second term covering only the validated differences of step 3.
Every expected value comes from the oracle; the GPU's outputs are only tested.
"""
from __future__ import annotations

import numpy as np

U32 = 2.0 ** -24


def silu_mul_interval(g_lo, g_hi, u_lo, u_hi):
    """Bounds of silu(g) * u (float64) for g, u in boxes; silu(z) = z / (1 + e^-z) has one minimum
    at z* ~ -1.27846 and is monotone on either side."""
    zs = -1.2784645427610738
    def silu(z):
        with np.errstate(over="ignore"):
            return z / (1.0 + np.exp(-z))
    s_a, s_b = silu(g_lo), silu(g_hi)
    s_lo = np.minimum(s_a, s_b)
    s_hi = np.maximum(s_a, s_b)
    inside = (g_lo < zs) & (g_hi > zs)
    s_lo = np.where(inside, silu(np.float64(zs)), s_lo)
    cands = np.stack([s_lo * u_lo, s_lo * u_hi, s_hi * u_lo, s_hi * u_hi])
    return cands.min(axis=0), cands.max(axis=0)


def _round_away(v):
    return np.sign(v) * np.floor(np.abs(v) + 0.5)


def q8_1_intervals(h_lo, h_hi):
    """Valid q8_1 outcomes for 32-value blocks whose values lie in [h_lo, h_hi] (float64, shape
    [..., 32]): returns (dh_lo, dh_hi) fp16 scale bounds and (q_lo, q_hi) per value."""
    a_lo = np.where((h_lo <= 0) & (h_hi >= 0), 0.0, np.minimum(np.abs(h_lo), np.abs(h_hi)))
    a_hi = np.maximum(np.abs(h_lo), np.abs(h_hi))
    amax_lo = a_lo.max(axis=-1)
    amax_hi = a_hi.max(axis=-1)
    # binary32 amax (the value is rounded to binary32 before the division) and d = amax / 127
    d_lo = (np.float32(amax_lo) / np.float32(127.0)).astype(np.float64)
    d_hi = (np.float32(np.nextafter(np.float32(amax_hi), np.float32(np.inf))) / np.float32(127.0)).astype(np.float64)
    d_lo32 = np.float32(d_lo)
    d_hi32 = np.float32(d_hi)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        corners = []
        for h in (h_lo, h_hi):
            hf = np.float32(h)
            for d in (d_lo32, d_hi32):
                dd = np.where(d > 0, d, np.float32(np.inf))[..., None]
                corners.append(_round_away((hf / dd).astype(np.float64)))
        cs = np.clip(np.stack(corners), -127, 127)
    zero_possible = amax_lo == 0
    q_lo = cs.min(axis=0)
    q_hi = cs.max(axis=0)
    q_lo = np.where(zero_possible[..., None], np.minimum(q_lo, 0), q_lo)
    q_hi = np.where(zero_possible[..., None], np.maximum(q_hi, 0), q_hi)
    dh_lo = np.float32(d_lo).astype(np.float16).astype(np.float64)
    dh_hi = np.float32(d_hi).astype(np.float16).astype(np.float64)
    dh_lo = np.where(zero_possible, 0.0, dh_lo)
    return dh_lo, dh_hi, q_lo, q_hi, d_lo32, d_hi32, zero_possible


def s_interval(d_lo32, d_hi32, sum_q):
    """Bounds of the q8_1 sum field s = fp16(d * sum_q) (binary32 product) over binary32 scales d
    in [d_lo32, d_hi32]: the product and both roundings are monotone in d for a fixed sum."""
    sq = np.float32(sum_q)
    with np.errstate(over="ignore"):
        a = (d_lo32 * sq).astype(np.float16).astype(np.float64)
        b = (d_hi32 * sq).astype(np.float16).astype(np.float64)
    return np.minimum(a, b), np.maximum(a, b)


def decode_q8_1(hq, n):
    b = np.asarray(hq, np.uint8).reshape(-1, n // 32, 36)
    d = b[:, :, 0:2].copy().view(np.float16)[:, :, 0].astype(np.float64)
    q = b[:, :, 4:].view(np.int8).astype(np.float64)
    return d, q


def check_grouped(orc_out, y_gpu, hq_gpu, g_gpu, u_gpu, wd_exact_by_entry, inter, depth, rel=1e-4, sum_field=True):
    """orc_out: the oracle's grouped() dict; wd_exact_by_entry(k) -> exact W_down of entry k's
    expert ([hidden, inter] float64).  sum_field=False: hq_gpu carries no sum field (its bytes
    2..3 are not checked).  Returns a dict of statistics; raises AssertionError."""
    ne = y_gpu.shape[0]
    stats = {"h_blocks_differ": 0, "h_values_differ": 0, "ambiguous_values": 0}
    # 1. gate/up within the reduction bound
    dg = (depth + 2) * U32 * 2 * orc_out["gabs"]
    du = (depth + 2) * U32 * 2 * orc_out["uabs"]
    if g_gpu is not None:
        assert np.all(np.abs(g_gpu - orc_out["g"]) <= dg), "gate sums outside the fp32 reduction bound"
        assert np.all(np.abs(u_gpu - orc_out["u"]) <= du), "up sums outside the fp32 reduction bound"
        assert np.all(np.abs(g_gpu - orc_out["g"]) <= rel * orc_out["gabs"])
    # 2. intervals of h (binary32 rounding of the g, u the GPU may have, then ~4 roundings)
    g32 = orc_out["g"]
    u32 = orc_out["u"]
    h_lo, h_hi = silu_mul_interval(g32 - dg, g32 + dg, u32 - du, u32 + du)
    pad = 8 * U32 * np.maximum(np.abs(h_lo), np.abs(h_hi)) + 1e-38
    h_lo, h_hi = h_lo - pad, h_hi + pad
    dh_lo, dh_hi, q_lo, q_hi, d_lo32, d_hi32, zero_ok = q8_1_intervals(h_lo.reshape(ne, -1, 32),
                                                                        h_hi.reshape(ne, -1, 32))
    # 3. H bytes
    d_gpu, q_gpu = decode_q8_1(hq_gpu, inter)
    d_or, q_or = decode_q8_1(orc_out["hq"], inter)
    assert np.all((d_gpu >= dh_lo) & (d_gpu <= dh_hi)), "H scale outside its valid interval"
    assert np.all((q_gpu >= q_lo) & (q_gpu <= q_hi)), "H code outside its valid interval"
    unique = (q_lo == q_hi) & (dh_lo == dh_hi)[..., None]
    assert np.array_equal(q_gpu[unique], q_or[unique]), "H differs where the decision is unique"
    stats["ambiguous_values"] = int((~unique).sum())
    hb_gpu = np.asarray(hq_gpu, np.uint8).reshape(ne, -1, 36)
    hb_or = np.asarray(orc_out["hq"], np.uint8).reshape(ne, -1, 36)
    # the sum field s = fp16(d * sum q): equal to the oracle's where the block's d and codes are
    # all unique; elsewhere s is what a valid binary32 d gives with the GPU's own codes (0 for a
    # block that may be all zero)
    if sum_field:
        s_gpu = hb_gpu[:, :, 2:4].copy().view(np.float16)[:, :, 0].astype(np.float64)
        blk_unique = unique.all(axis=-1) & (d_lo32 == d_hi32)
        assert np.array_equal(hb_gpu[:, :, 2:4][blk_unique], hb_or[:, :, 2:4][blk_unique]), \
            "H sum field differs where the block is unique"
        s_lo, s_hi = s_interval(d_lo32, d_hi32, q_gpu.sum(axis=-1))
        s_ok = ((s_gpu >= s_lo) & (s_gpu <= s_hi)) | (zero_ok & (s_gpu == 0) & (d_gpu == 0))
        assert s_ok.all(), f"H sum field outside its valid interval in {(~s_ok).sum()} blocks"
        stats["s_blocks_checked"] = int(s_ok.size)
    else:
        hb_gpu = hb_gpu.copy()
        hb_gpu[:, :, 2:4] = hb_or[:, :, 2:4]    # no sum field to compare
    diff_blocks = np.any(hb_gpu != hb_or, axis=-1)
    stats["h_blocks_differ"] = int(diff_blocks.sum())
    stats["h_values_differ"] = int((q_gpu != q_or).sum())
    # 4. outputs
    Hg = (d_gpu[..., None] * q_gpu).reshape(ne, inter)
    Ho = (d_or[..., None] * q_or).reshape(ne, inter)
    dH = np.abs(Hg - Ho)
    for k in range(ne):
        extra = 0.0
        if dH[k].any():
            extra = np.abs(wd_exact_by_entry(k)) @ dH[k]
        bound = rel * orc_out["yabs"][k] + extra * (1 + 1e-6)
        err = np.abs(y_gpu[k].astype(np.float64) - orc_out["y"][k])
        assert np.all(err <= bound), f"entry {k}: y outside tolerance (max excess {np.max(err - bound)})"
    return stats
