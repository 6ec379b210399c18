"""Planted mistakes in the oracle's C source must each fail at least one pin (CPU only).

Every mutant is a copy of w4a16_oracle.c with one plausible slip (a wrong nibble order,
sign encoding, scale index, exponent bias, a dropped term, a transposed operand ...),
compiled to a temporary library. None of them may pass every pin.
"""
import os

import pytest

import oracle
from oracle_pins import ALL_PINS

MUTANTS = {
    "nibble_order_high_first": ("(4 * (k % 8))", "(4 * (7 - k % 8))"),
    "offset_binary_sign": ("u >= 8 ? u - 16 : u", "u - 8"),
    "sign_ignored": ("u >= 8 ? u - 16 : u", "u"),
    "scale_row_stride": ("scales + n * (K / G), x, K, G, &y[r]", "scales + n, x, K, G, &y[r]"),
    "scale_group_index": ("double s = oracle_f16_to_double(srow[g]);",
                          "double s = oracle_f16_to_double(srow[(g + 1) % (K / G)]);"),
    "f16_bias": ("expo - 25", "expo - 24"),
    "f16_subnormal": ("ldexp((double)frac, -24)", "ldexp((double)frac, -25)"),
    "f16_hidden_bit": ("(double)(1024 + frac)", "(double)(frac)"),
    "bf16_bias": ("expo - 134", "expo - 133"),
    "bf16_sign": ("    return sign ? -v : v;\n}\n\n/* Signed", "    return v;\n}\n\n/* Signed"),
    "dropped_last_term": ("k < (g + 1) * G; ++k", "k < (g + 1) * G - 1; ++k"),
    "x_pair_swap": ("oracle_bf16_to_double(x[k])", "oracle_bf16_to_double(x[k ^ 1])"),
    "mag_signed": ("m += fabs(p);", "m += p;"),
    "moe_slot_not_id": ("((int64_t)e * N + n) * (K / 8)", "((int64_t)t * N + n) * (K / 8)"),
    "batched_ignores_ldx": ("X + m * ldx", "X + m * K"),
    "word_index": ("row[k / 8]", "row[k / 8 + (k >= 8 ? -1 : 0)]"),
    "swiglu_halves_swapped": ("int64_t rg = (int64_t)e * 2 * I + n, ru = rg + I;",
                              "int64_t ru = (int64_t)e * 2 * I + n, rg = ru + I;"),
    "silu_sign": ("g / (1.0 + exp(-g))", "g / (1.0 + exp(g))"),
    "silu_missing_gate_factor": ("h[o] = oracle_silu(g[o]) * u[o];",
                                 "h[o] = u[o] / (1.0 + exp(-g[o]));"),
    "bf16_truncates": ("double r = rint(ldexp(a, -qexp));", "double r = floor(ldexp(a, -qexp));"),
    "bf16_ties_away": ("double r = rint(ldexp(a, -qexp));", "double r = round(ldexp(a, -qexp));"),
    "bf16_subnormal_step": ("if (qexp < -133)\n        qexp = -133;",
                            "if (qexp < -140)\n        qexp = -140;"),
    "bf16_saturates": ("if (q >= ldexp(1.0, 128))\n        return (uint16_t)(sign | 0x7F80u);",
                       "if (q >= ldexp(1.0, 128))\n        return (uint16_t)(sign | 0x7F7Fu);"),
    "combine_ignores_weight": ("acc += (double)w[t] * y;", "acc += y;"),
    "down_slot_as_expert": ("int64_t row = (int64_t)e * H + n;", "int64_t row = (int64_t)t * H + n;"),
    "down_shared_h_row": ("h + (int64_t)t * I, I, G,", "h, I, G,"),
    "down_signed_mag": ("m += fabs((double)w[t]) * ym;", "m += (double)w[t] * ym;"),
    "quant_divides_by_8": ("amax / 7.0f", "amax / 8.0f"),
    "quant_ties_away": ("float qi = rintf(r);", "float qi = roundf(r);"),
    "quant_truncates": ("float qi = rintf(r);", "float qi = truncf(r);"),
    "quant_scale_truncated": ("double r = rint(ldexp(a, -qexp));  /* nearest, ties to even */",
                              "double r = floor(ldexp(a, -qexp));"),
    "quant_no_saturation": ("return (uint16_t)(sign | 0x7BFFu);", "return (uint16_t)(sign | 0x7C00u);"),
    "quant_nibble_order": ("int shift = 4 * (int)(k % 8);", "int shift = 4 * (7 - (int)(k % 8));"),
    "quant_amax_signed": ("float a = fabsf(bf16_to_float(row[k]));", "float a = bf16_to_float(row[k]);"),
    "moe_batched_token_row": ("X + m * ldx, K, G,\n                        &Y[o], &mag[o]);",
                              "X, K, G,\n                        &Y[o], &mag[o]);"),
    "moe_batched_id_index": ("ids[(int64_t)m * topk + t]", "ids[(int64_t)t * M + m]"),
    "moe_id_upper_bound": ("            if (e < 0 || e >= E) {\n                *yo = 0.0;",
                           "            if (e < 0 || e > E) {\n                *yo = 0.0;"),
    "swiglu_id_upper_bound": ("            if (e < 0 || e >= E) {\n                h[o] = g[o]",
                              "            if (e < 0 || e > E) {\n                h[o] = g[o]"),
    "combine_id_upper_bound": ("            if (e < 0 || e >= E)\n                continue;",
                               "            if (e < 0 || e > E)\n                continue;"),
    "moe_batched_id_upper_bound": ("                if (e < 0 || e >= E) {\n                    Y[o] = 0.0;",
                                   "                if (e < 0 || e > E) {\n                    Y[o] = 0.0;"),
    "three_bit_high_half_shift": ("int shift = r < 5 ? 3 * r : 16 + 3 * (r - 5);",
                                  "int shift = r < 5 ? 3 * r : 15 + 3 * (r - 5);"),
    "three_bit_word_order": ("u = (blk[t] >> shift) & 7u;", "u = (blk[2 - t] >> shift) & 7u;"),
    "three_bit_spare_bit_order": ("u = ((blk[0] >> bit) & 1u) | (((blk[1] >> bit) & 1u) << 1) | (((blk[2] >> bit) & 1u) << 2);",
                                  "u = ((blk[2] >> bit) & 1u) | (((blk[1] >> bit) & 1u) << 1) | (((blk[0] >> bit) & 1u) << 2);"),
    "three_bit_spare_codes_swapped": ("int bit = c == 30 ? 15 : 31;", "int bit = c == 30 ? 31 : 15;"),
    "three_bit_offset_binary": ("return u >= 4 ? (int)u - 8 : (int)u;", "return (int)u - 4;"),
    "three_bit_block_swap": ("double w = (double)code3_of_block(row + 3 * (k / 32), (int)(k % 32)) * s;",
                             "double w = (double)code3_of_block(row + 3 * ((k / 32) ^ 1), (int)(k % 32)) * s;"),
    "three_bit_id_upper_bound": ("            if (e < 0 || e >= E) {\n                *yo = 0.0;\n                *mo = 0.0;\n                continue;\n            }\n            int64_t row = (int64_t)e * N + n;\n            dot_row3",
                                 "            if (e < 0 || e > E) {\n                *yo = 0.0;\n                *mo = 0.0;\n                continue;\n            }\n            int64_t row = (int64_t)e * N + n;\n            dot_row3"),
    "quant_f16_subnormal": ("if (qexp < -24)\n        qexp = -24;", "if (qexp < -30)\n        qexp = -30;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new, 1))
    lib = oracle.compile_source(str(path), str(tmp_path / "mutant.so"))
    orc = oracle.Oracle(lib)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
