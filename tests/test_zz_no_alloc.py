"""The allocation-free grouped decode (qgemv_grouped_experts_noalloc, H in the library's fixed
device array) against qgemv_grouped_experts with a caller workspace: y bitwise equal, on two
calls in a row, the second with fewer entries and experts than the first; a call whose H would
not fit the array is refused before any launch."""
import numpy as np
import pytest

import moe_expert_amd as M
import synth
from tests.gpu_util import dev, host

pytestmark = pytest.mark.gpu


def _call_pair(nexp, hidden, inter, ngroups, m, seed, wt_gu=M.QMM_CB3, wt_down=M.QMM_IQ4_NL):
    rng = synth.rng_for(seed)
    grid = dev(synth.cb3_grid(synth.rng_for(synth.SEEDS["cb3_grid"])))
    wg = dev(np.stack([synth.weights(wt_gu, rng, inter, hidden) for _ in range(nexp)]))
    wu = dev(np.stack([synth.weights(wt_gu, rng, inter, hidden) for _ in range(nexp)]))
    wd = dev(np.stack([synth.weights(wt_down, rng, hidden, inter) for _ in range(nexp)]))
    ge, go, ec = synth.decode_routing(rng, nexp, ngroups, m)
    xq = M.qmm_quantize_q8_1(dev(synth.activations(rng, m, hidden)))
    ge, go, ec = dev(ge), dev(go), dev(ec)
    y_ws, _ = M.qgemv_grouped_experts(wt_gu, wg, wu, wt_down, wd, hidden, inter, xq, ge, go, ec, grid=grid)
    y_na = M.qgemv_grouped_experts_noalloc(wt_gu, wg, wu, wt_down, wd, hidden, inter, xq, ge, go, ec, grid=grid)
    return host(y_ws), host(y_na)


def test_noalloc_matches_workspace_call_twice():
    print("noalloc grouped decode: call 1 (16 groups x 8 entries, 2560 -> 1024)", flush=True)
    a, b = _call_pair(32, 2560, 1024, 16, 8, 3100)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    print("noalloc grouped decode: call 2 (5 groups x 3 entries, 1024 -> 256)", flush=True)
    a, b = _call_pair(6, 1024, 256, 5, 3, 3101, wt_gu=M.QMM_IQ4_NL, wt_down=M.QMM_Q8_0)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_noalloc_refuses_h_beyond_the_array():
    limit = int(M.lib().qgemv_grouped_experts_noalloc_max_bytes())
    assert limit == 4 << 20
    per_entry = (1024 // 32) * 36
    too_many = limit // per_entry + 1
    rc = M.lib().qgemv_grouped_experts_noalloc(M.QMM_IQ4_NL, 0x100000, 0x100000, 1024 * 1440, M.QMM_Q8_0, 0x100000,
                                               2560 * 1088, 4, None, 2560, 1024, 0x100000, 1, 0x100000, 0x100000, 1,
                                               0x100000, too_many, 0x100000, None)
    assert rc == -5
