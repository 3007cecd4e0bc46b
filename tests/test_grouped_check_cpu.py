"""The interval check of the grouped decode (tests/grouped_check.py) on the CPU: it accepts the
oracle's own outputs (with its g, u rounded to binary32, as a GPU's would be) and rejects an H
block whose scale, code or sum field was changed, and an output moved outside the tolerance."""
import numpy as np
import pytest

import oracle
import synth
from tests.grouped_check import check_grouped


@pytest.fixture(scope="module")
def case():
    rng = synth.rng_for(5)
    nexp, hidden, inter = 4, 1024, 128
    grid = synth.cb3_grid()
    wg = np.stack([synth.cb3_weights(rng, inter, hidden) for _ in range(nexp)])
    wu = np.stack([synth.cb3_weights(rng, inter, hidden) for _ in range(nexp)])
    wd = np.stack([synth.iq4nl_weights(rng, hidden, inter) for _ in range(nexp)])
    ge, go, ec = synth.decode_routing(rng, nexp, 4, 3)
    xq = oracle.quantize_q8_1(synth.activations(rng, 3, hidden))
    ref = oracle.grouped(synth.CB3, wg, wu, synth.IQ4_NL, wd, hidden, inter, xq, ge, go, ec, grid)
    ee = np.repeat(ge, np.diff(go))
    wdx = {e: oracle.dequant_f64(synth.IQ4_NL, wd[e], inter) for e in set(ee.tolist())}
    return ref, (lambda k: wdx[int(ee[k])]), inter


def run(case, hq=None, y=None):
    ref, wd_of, inter = case
    g = ref["g"].astype(np.float32).astype(np.float64)
    u = ref["u"].astype(np.float32).astype(np.float64)
    return check_grouped(ref, ref["y"].astype(np.float32) if y is None else y, ref["hq"] if hq is None else hq,
                         g, u, wd_of, inter, 10)


def test_accepts_the_oracle(case):
    st = run(case)
    assert st["h_blocks_differ"] == 0 and st["s_blocks_checked"] > 0


@pytest.mark.parametrize("byte,what", [(1, "scale"), (2, "sum field"), (3, "sum field"), (10, "code")])
def test_rejects_a_changed_h_byte(case, byte, what):
    hq = case[0]["hq"].copy()
    hq[2, 36 * 1 + byte] ^= 0x04
    with pytest.raises(AssertionError):
        run(case, hq=hq)


def test_rejects_an_output_outside_tolerance(case):
    y = case[0]["y"].astype(np.float32).copy()
    y[1, 7] += np.float32(1e-2) * max(1.0, abs(float(y[1, 7])))
    with pytest.raises(AssertionError):
        run(case, y=y)
