"""Planted mistakes in copies of the oracle must each fail at least one pin.

Each mutation edits one expression of oracle/qmm_oracle.c (a dropped term, a wrong sign,
index or rounding, a transposed operand), builds the copy with gcc into a temporary
directory and runs the pins against it.  The real oracle is not touched.  CPU only.
"""
import os
import subprocess

import pytest

import oracle
from oracle import build as obuild
from tests import oracle_pins

MUTATIONS = {
    "iq4nl_nibble_order": ("(b[2 + jj] & 15) : (b[2 + jj - 16] >> 4)",
                           "(b[2 + jj] >> 4) : (b[2 + jj - 16] & 15)"),
    "iq4nl_level_table": ("1,    13,   25,  38,  53,  69,  89,  113};",
                          "1,    13,   25,  38,  53,  69,  89,  112};"),
    "q8_0_byte_offset": ("(int8_t)b[2 + j % 32]", "(int8_t)b[1 + j % 32]"),
    "cb3_multiplier": ("return (1 + 2 * nib) * mag", "return (1 + nib) * mag"),
    "cb3_high_bit_index": ("((qh[i / 8] >> (i % 8)) & 1) << 8", "((qh[i % 8] >> (i / 8)) & 1) << 8"),
    "cb3_sign_bit_order": ("(signs[v / 8] >> (v % 8)) & 1", "(signs[v / 8] >> (7 - v % 8)) & 1"),
    "cb3_grid_column": ("grid[idx * 4 + v % 4]", "grid[idx * 4 + 3 - v % 4]"),
    "cb3_scale_nibble": ("(scales[s / 2] >> (4 * (s % 2))) & 15", "(scales[s / 2] >> (4 * (1 - s % 2))) & 15"),
    "f16_tie_away": ("return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;", "return f + 1.0;"),
    "f16_subnormal_scale": ("v = ldexp((double)m, -24);", "v = ldexp((double)m, -25);"),
    "f16_saturates": ("if (a >= 65520.0) return sign | 0x7C00;", "if (a >= 65520.0) return sign | 0x7BFF;"),
    "q8_1_half_even": ("float r = roundf(v);", "float r = rintf(v);"),
    "q8_1_scale_128": ("float d = amax / 127.0f;", "float d = amax / 128.0f;"),
    "q8_1_sum_field": ("float s = d * (float)sum;", "float s = (float)sum;"),
    "q8_1_no_clamp_zero": ("if (amax == 0.0f || d == 0.0f) return;", "if (d == 0.0f) { out[0] = 1; return; }"),
    "term_drops_activation_scale": ("float dd = or_f16_to_f32(dw) * or_f16_to_f32(da);",
                                    "float dd = or_f16_to_f32(dw);"),
    "term_wrong_scale": ("float dd = or_f16_to_f32(dw) * or_f16_to_f32(da);",
                         "float dd = or_f16_to_f32(da) * or_f16_to_f32(da);"),
    "gemv_drops_last_block": ("for (int64_t b = 0; b < nb; ++b) {\n                const uint8_t* xb",
                              "for (int64_t b = 0; b + 1 < nb; ++b) {\n                const uint8_t* xb"),
    "silu_sign": ("float den = 1.0f + e;", "float den = 1.0f - e;"),
    "silu_exp_sign": ("float e = (float)exp(-(double)g);", "float e = (float)exp((double)g);"),
    "grouped_gate_up_swapped": ("const uint8_t* wu = w_up + (int64_t)e * gu_stride;",
                                "const uint8_t* wu = w_gate + (int64_t)e * gu_stride;"),
    "grouped_wrong_column": ("const uint8_t* x = xq + (int64_t)entry_col[kk] * nbx * 36;",
                             "const uint8_t* x = xq + (int64_t)kk % 3 * nbx * 36;"),
    "grouped_h_unrounded_g": ("hbuf[i] = or_silu_mul((float)gt[i], (float)gt[2 * inter + i]);",
                              "hbuf[i] = or_silu_mul((float)gt[2 * inter + i], (float)gt[i]);"),
    "prefill_down_transposed": ("ya += wd[j * inter + i] * hrow[i];", "ya += wd[i * hidden + j] * hrow[i];"),
    "prefill_h_not_rounded": ("hrow[i] = or_f16_to_f32(hb);",
                              "hrow[i] = or_silu_mul((float)ga, (float)ua);"),
    "combine_fused_multiply_add": ("acc = acc + prod;", "acc = fmaf(w[t * topk + k], y[r * hidden + j], acc);"),
    "combine_reverse_k_order": ("int32_t r = row_idx[t * topk + k];\n                if (r < 0",
                                "int32_t r = row_idx[t * topk + (topk - 1 - k)];\n                if (r < 0"),
    "combine_drops_last_k": ("for (int k = 0; k < topk; ++k) {\n                int32_t r",
                             "for (int k = 0; k + 1 < topk; ++k) {\n                int32_t r"),
    "combine_weight_of_other_k": ("float prod = w[t * topk + k] * y[r * hidden + j];",
                                  "float prod = w[t * topk + (k + 1) % topk] * y[r * hidden + j];"),
    "combine_keeps_bad_rows": ("if (r < 0 || r >= nrows) continue;", "if (r < 0 || r >= nrows) r = 0;"),
    "dense_rows_transposed": ("or_f16_to_f32(w16[r * k + kk]) * (double)or_f16_to_f32(x16[t * k + kk])",
                              "or_f16_to_f32(w16[kk * nrows + r]) * (double)or_f16_to_f32(x16[t * k + kk])"),
    "dense_rows_unrounded": ("or_dequant_f16(wtype, (const uint8_t*)w, grid, nrows, k, w16, k);",
                             "{ or_dequant_f16(wtype, (const uint8_t*)w, grid, nrows, k, w16, k); "
                             "for (int64_t i = 0; i < nrows * k; ++i) w16[i] &= 0xFFFE; }"),
    "planes_scales_first": ("memcpy(tile + i * fb, blk + 2, (size_t)fb);       /* factors */",
                            "memcpy(tile + 2 * n + i * fb, blk + 2, (size_t)fb);       /* factors */"),
    "planes_whole_row_tile": ("int64_t n = nb - b0 < 16 ? nb - b0 : 16;", "int64_t n = nb - b0 < 32 ? nb - b0 : 32;"),
    "prefill_wrong_token": ("const uint16_t* xr = x16 + (int64_t)t * hidden;",
                            "const uint16_t* xr = x16 + (int64_t)(p % ntok) * hidden;"),
}


def _build_variant(tmp_path, name, old, new):
    src = open(obuild.SRC).read()
    assert src.count(old) == 1, f"mutation {name}: pattern not found exactly once"
    path = os.path.join(tmp_path, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = os.path.join(tmp_path, f"lib{name}.so")
    subprocess.run(["gcc", *obuild.CFLAGS, path, "-o", lib, "-lm"], check=True)
    return oracle.Oracle(oracle.load_library(lib))


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_fails_a_pin(name, tmp_path):
    old, new = MUTATIONS[name]
    orc = _build_variant(str(tmp_path), name, old, new)
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError):
            return
    pytest.fail(f"planted mistake {name} passed every pin")
