"""Readers for the hand-worked fixtures under tests/golden/."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line


def simple_block(name):
    """Fixture with 'bytes:', 'values:' and optional 'f16:' lines."""
    out = {}
    for line in _lines(name):
        key, val = line.split(":", 1)
        out[key.strip()] = val.split()
    blk = np.array([int(b, 16) for b in out["bytes"]], np.uint8)
    vals = np.array([float(v) for v in out["values"]], np.float64)
    f16 = None
    if "f16" in out:
        f16 = np.array([int(b, 16) for b in out["f16"]], np.uint16)
    return blk, vals, f16


def cb3_superblock():
    grid = np.ones((512, 4), np.uint8)
    blk = np.zeros(110, np.uint8)
    values = {}
    offs = {"qs": 2, "qh": 66, "signs": 74, "scales": 106}
    for line in _lines("cb3_superblock.txt"):
        key, val = line.split(":", 1)
        key = key.strip()
        if key.startswith("grid "):
            grid[int(key.split()[1])] = [int(v) for v in val.split()]
        elif key == "d":
            d = int(val.strip(), 16)
            blk[0], blk[1] = d & 255, d >> 8
        elif key in offs:
            for item in val.split():
                i, b = item.split("=")
                blk[offs[key] + int(i)] = int(b, 16)
        elif key.startswith("value "):
            values[int(key.split()[1])] = float(val)
    return blk, grid, values


def fp16_cases():
    to_f32, from_f64 = [], []
    for line in _lines("fp16.txt"):
        kind, a, b = line.split()
        if kind == "to_f32":
            to_f32.append((int(a, 16), float(b)))
        else:
            from_f64.append((float(a), int(b, 16)))
    return to_f32, from_f64


def q8_1_cases():
    cases, cur = [], None
    for line in _lines("q8_1_blocks.txt"):
        if line.startswith("case"):
            cur = {}
            cases.append(cur)
            continue
        key, val = line.split(":", 1)
        cur[key.strip()] = val.split()
    out = []
    for c in cases:
        out.append(dict(x=np.array([float(v) for v in c["x"]], np.float32),
                        q=np.array([int(v) for v in c["q"]], np.int8),
                        d=int(c["d"][0], 16), s=int(c["s"][0], 16)))
    return out


def _cases(name):
    cases, cur = [], None
    for line in _lines(name):
        if line.startswith("case"):
            cur = {"name": line.split()[1]}
            cases.append(cur)
            continue
        key, val = line.split(":", 1)
        cur[key.strip()] = val.split()
    return cases


def _hexf(v):
    return float.fromhex(v)


def moe_combine_cases():
    """(name, y [nrows, 1] float32, idx [1, topk], w [1, topk], out float) per case."""
    out = []
    for c in _cases("moe_combine.txt"):
        y = np.array([_hexf(v) for v in c["y"]], np.float32)[:, None]
        idx = np.array([[int(v) for v in c["idx"]]], np.int32)
        w = np.array([[_hexf(v) for v in c["w"]]], np.float32)
        out.append((c["name"], y, idx, w, _hexf(c["out"][0])))
    return out


def planes_cases():
    """(name, wtype, k, blocks uint8 [1, row bytes], planes uint8 [1, row bytes]) per case."""
    out = []
    for c in _cases("planes.txt"):
        blk = np.array([int(b, 16) for b in c["blocks"]], np.uint8)[None, :]
        pl = np.array([int(b, 16) for b in c["planes"]], np.uint8)[None, :]
        out.append((c["name"], int(c["wtype"][0]), int(c["k"][0]), blk, pl))
    return out
