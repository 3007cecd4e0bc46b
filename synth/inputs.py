"""Seeded generators for quantized weight blocks, activations and expert routings.

Every generator takes a ``numpy.random.Generator`` (PCG64) or a seed and returns
plain numpy arrays.  Byte layouts are the raw block layouts the library and the
oracle both consume (little-endian):

* Q8_0   : 34 bytes per 32 values  -> fp16 scale, 32 signed bytes
* IQ4_NL : 18 bytes per 32 values  -> fp16 scale, 16 bytes of 4-bit table indices
* CB3    : 110 bytes per 256 values -> fp16 scale, 64 index low bytes, 8 index high-bit
           bytes, 32 sign bytes, 4 bytes of 4-bit sub-scales

Only random numbers are produced here: a scale ``d`` is drawn as a float and
converted to IEEE half by numpy, every other field is a uniformly random integer
in the range the workload states.
"""
from __future__ import annotations

import numpy as np

Q8_0, IQ4_NL, CB3 = 1, 2, 3
BLOCK_VALUES = {Q8_0: 32, IQ4_NL: 32, CB3: 256}
BLOCK_BYTES = {Q8_0: 34, IQ4_NL: 18, CB3: 110}
Q8_1_BYTES = 36

__all__ = [
    "Q8_0", "IQ4_NL", "CB3", "BLOCK_VALUES", "BLOCK_BYTES", "Q8_1_BYTES",
    "rng_for", "row_bytes", "fp16_scales", "q8_0_weights", "iq4nl_weights",
    "cb3_weights", "cb3_grid", "weights", "activations", "decode_routing", "decode_routings",
    "prefill_routing", "prefill_tokens", "router_weights", "token_positions", "SEEDS",
]

# seed = 1000 * workload number + copy index
SEEDS = {"q8_0_tiny": 1000, "iq4nl_8192x2560": 2000, "q8_0_12288x2560": 3000,
         "q8_0_2560x6144": 3500, "grouped_decode": 4000, "cb3_grid": 4999,
         "prefill": 5000}


def rng_for(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def row_bytes(wtype: int, k: int) -> int:
    bv = BLOCK_VALUES[wtype]
    if k % bv:
        raise ValueError(f"k={k} is not a multiple of {bv}")
    return (k // bv) * BLOCK_BYTES[wtype]


def fp16_scales(rng: np.random.Generator, shape, lo: float = 1e-3, hi: float = 2e-2) -> np.ndarray:
    """Block scales d ~ U[lo, hi], stored as IEEE half (numpy's conversion)."""
    return rng.uniform(lo, hi, size=shape).astype(np.float16)


def q8_0_weights(rng: np.random.Generator, nrows: int, k: int, *, qlo: int = -127, qhi: int = 127,
                 dlo: float = 1e-3, dhi: float = 2e-2) -> np.ndarray:
    """[nrows, k/32*34] uint8: per block fp16 d ~ U[dlo, dhi], int8 q ~ U{qlo..qhi}."""
    nb = k // 32
    blk = np.empty((nrows, nb, 34), dtype=np.uint8)
    blk[:, :, 0:2] = fp16_scales(rng, (nrows, nb), dlo, dhi).view(np.uint8).reshape(nrows, nb, 2)
    blk[:, :, 2:34] = rng.integers(qlo, qhi + 1, size=(nrows, nb, 32), dtype=np.int16).astype(np.int8).view(np.uint8)
    return blk.reshape(nrows, nb * 34)


def iq4nl_weights(rng: np.random.Generator, nrows: int, k: int, *, dlo: float = 1e-3,
                  dhi: float = 2e-2) -> np.ndarray:
    """[nrows, k/32*18] uint8: per block fp16 d ~ U[dlo, dhi], 32 indices ~ U{0..15} (two per byte)."""
    nb = k // 32
    blk = np.empty((nrows, nb, 18), dtype=np.uint8)
    blk[:, :, 0:2] = fp16_scales(rng, (nrows, nb), dlo, dhi).view(np.uint8).reshape(nrows, nb, 2)
    blk[:, :, 2:18] = rng.integers(0, 256, size=(nrows, nb, 16), dtype=np.uint16).astype(np.uint8)
    return blk.reshape(nrows, nb * 18)


def cb3_weights(rng: np.random.Generator, nrows: int, k: int, *, dlo: float = 1e-3,
                dhi: float = 2e-2) -> np.ndarray:
    """[nrows, k/256*110] uint8: fp16 d, then 64 + 8 + 32 + 4 uniformly random bytes
    (9-bit grid indices ~ U{0..511}, sign bits ~ U{0,1}, 4-bit sub-scales ~ U{0..15})."""
    nb = k // 256
    blk = np.empty((nrows, nb, 110), dtype=np.uint8)
    blk[:, :, 0:2] = fp16_scales(rng, (nrows, nb), dlo, dhi).view(np.uint8).reshape(nrows, nb, 2)
    blk[:, :, 2:110] = rng.integers(0, 256, size=(nrows, nb, 108), dtype=np.uint16).astype(np.uint8)
    return blk.reshape(nrows, nb * 110)


def cb3_grid(rng: np.random.Generator | None = None) -> np.ndarray:
    """[512, 4] uint8 codebook of magnitudes ~ U{1..63} (no entry is 0)."""
    if rng is None:
        rng = rng_for(SEEDS["cb3_grid"])
    return rng.integers(1, 64, size=(512, 4), dtype=np.uint16).astype(np.uint8)


def weights(wtype: int, rng: np.random.Generator, nrows: int, k: int, **kw) -> np.ndarray:
    return {Q8_0: q8_0_weights, IQ4_NL: iq4nl_weights, CB3: cb3_weights}[wtype](rng, nrows, k, **kw)


def activations(rng: np.random.Generator, ncols: int, k: int, scale: float = 1.0) -> np.ndarray:
    """[ncols, k] float32 ~ N(0, scale^2)."""
    return (rng.standard_normal(size=(ncols, k)) * scale).astype(np.float32)


def decode_routing(rng: np.random.Generator, nexperts: int, ngroups: int, m: int):
    """Grouped decode routing: ``ngroups`` distinct experts drawn uniformly, ``m`` entries each;
    entry j of every group reads activation column j.

    Returns (group_expert[ngroups], group_entry_off[ngroups+1], entry_col[ngroups*m]) as int32.
    """
    experts = rng.choice(nexperts, size=ngroups, replace=False).astype(np.int32)
    off = (np.arange(ngroups + 1, dtype=np.int32) * m).astype(np.int32)
    cols = np.tile(np.arange(m, dtype=np.int32), ngroups)
    return experts, off, cols


def decode_routings(rng: np.random.Generator, nexperts: int, ngroups: int, m: int, count: int):
    """``count`` grouped decode routings as decode_routing, the experts of successive routings
    drawn without replacement from one permutation of all experts (disjoint while
    ``count * ngroups <= nexperts``; a fresh permutation after that)."""
    out, perm = [], np.empty(0, dtype=np.int32)
    for _ in range(count):
        if perm.size < ngroups:
            perm = rng.permutation(nexperts).astype(np.int32)
        experts, perm = perm[:ngroups].copy(), perm[ngroups:]
        off = (np.arange(ngroups + 1, dtype=np.int32) * m).astype(np.int32)
        cols = np.tile(np.arange(m, dtype=np.int32), ngroups)
        out.append((experts, off, cols))
    return out


def prefill_routing(rng: np.random.Generator, ntok: int, nexperts: int, topk: int):
    """Uniform top-k routing: every token picks ``topk`` distinct experts uniformly.
    Entries (expert, token) are sorted by expert, ties by ascending token.

    Returns (sorted_tok[ntok*topk], expert_off[nexperts+1]) as int32.
    """
    keys = rng.random(size=(ntok, nexperts))
    pick = np.argpartition(keys, topk, axis=1)[:, :topk]          # topk distinct experts per token
    tok = np.repeat(np.arange(ntok, dtype=np.int64), topk)
    exp = pick.reshape(-1).astype(np.int64)
    order = np.lexsort((tok, exp))                                # by expert, then token
    sorted_tok = tok[order].astype(np.int32)
    counts = np.bincount(exp, minlength=nexperts)
    off = np.zeros(nexperts + 1, dtype=np.int32)
    off[1:] = np.cumsum(counts)
    return sorted_tok, off


def prefill_tokens(rng: np.random.Generator, ntok: int, hidden: int) -> np.ndarray:
    """[ntok, hidden] fp16 activations ~ N(0, 1) (numpy's conversion to half)."""
    return rng.standard_normal(size=(ntok, hidden)).astype(np.float16)


def router_weights(rng: np.random.Generator, ntok: int, topk: int) -> np.ndarray:
    """[ntok, topk] float32 positive router weights, each row drawn uniformly and scaled to sum
    to 1 (in float64, then rounded to float32)."""
    w = rng.random(size=(ntok, topk)) + 1e-3
    return (w / w.sum(axis=1, keepdims=True)).astype(np.float32)


def token_positions(sorted_tok: np.ndarray, ntok: int, topk: int) -> np.ndarray:
    """[ntok, topk] int32: where each token's entries sit in an expert-sorted entry list, in the
    order of the list (ascending expert).  Every token must have exactly topk entries."""
    order = np.argsort(np.asarray(sorted_tok), kind="stable")
    return order.reshape(ntok, topk).astype(np.int32)
