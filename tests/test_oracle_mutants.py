"""The oracle's pins must catch plausible mistakes.

Each mutant below is the oracle's C source with one planted error (a dropped
term, a wrong index, a swapped operand, a wrong rounding).  It is built with
gcc into a temporary directory and every pin of tests/oracle_pins.py is run
against it; at least one pin must fail.  CPU only; the committed oracle is not
modified.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
import oracle_pins
from oracle import core

SRC = os.path.join(os.path.dirname(oracle.__file__), "kvq_oracle.c")

MUTANTS = {
    "gqa_modulo": ("const int32_t g = h / hpk;", "const int32_t g = h % Hkv;"),
    "sink_not_in_denominator": ("if (sinks) Z += exp((double)sinks[h] - M);", ";"),
    "window_off_by_one": ("first = upto - window;", "first = upto - window + 1;"),
    "causal_off_by_one": ("const int64_t upto = len[b] - T + t + 1;", "const int64_t upto = len[b] - T + t;"),
    "scale_dropped": ("s[j - first] = (double)scale * acc;", "s[j - first] = acc;"),
    "q_index_transposed": ("acc += (double)qv[32 * kb + i] * blk[i];", "acc += (double)qv[nb * i + kb] * blk[i];"),
    "lse_without_max": ("(float)(M + log(Z))", "(float)(log(Z))"),
    "q8_unrounded_scale": ("float r = rintf(x[i] / ds);", "float r = rintf(x[i] / d);"),
    "q8_round_half_away": ("float r = rintf(x[i] / ds);", "float r = roundf(x[i] / ds);"),
    "q8_divisor_128": ("float d = amax / 127.0f;", "float d = amax / 128.0f;"),
    "q5_nibbles_swapped": ("(uint8_t)((code[j] & 15) | ((code[j + 16] & 15) << 4))",
                           "(uint8_t)((code[j + 16] & 15) | ((code[j] & 15) << 4))"),
    "q5_fifth_bits_reversed": ("qh |= (uint32_t)((code[i] >> 4) & 1) << i;",
                               "qh |= (uint32_t)((code[i] >> 4) & 1) << (31 - i);"),
    "q5_min_not_subtracted": ("float r = rintf((x[i] - ms) / ds);", "float r = rintf(x[i] / ds);"),
    "q5_decode_drops_min": ("x[i] = ds * (double)c + ms;", "x[i] = ds * (double)c;"),
    "q5_unrounded_min": ("float r = rintf((x[i] - ms) / ds);", "float r = rintf((x[i] - mn) / ds);"),
    "e4m3_bias_8": ("ldexp(1.0 + fr / 8.0, ex - 7)", "ldexp(1.0 + fr / 8.0, ex - 8)"),
    "e4m3_subnormal_exponent": ("ldexp((double)fr, -9)", "ldexp((double)fr, -10)"),
    "e4m3_ties_odd": ("else best = (lo & 1) == 0 ? lo : hi;", "else best = (lo & 1) == 1 ? lo : hi;"),
    "e4m3_ties_up": ("else best = (lo & 1) == 0 ? lo : hi;", "else best = hi;"),
    "e4m3_nearest_swapped": ("if (err_lo < err_hi) best = lo;", "if (err_lo < err_hi) best = hi;"),
    "e4m3_table_shifted": ("e4m3_pos[c] = kvqo_e4m3_value((uint8_t)c);", "e4m3_pos[c] = kvqo_e4m3_value((uint8_t)(c ? c - 1 : 0));"),
    "e4m3_sign_dropped": ("return (uint8_t)(best | (signbit(x) ? 0x80 : 0));", "return (uint8_t)best;"),
    "f8_unrounded_scale": ("kvqo_e4m3_from_f32(x[i] / ds)", "kvqo_e4m3_from_f32(x[i] / (amax / 448.0f))"),
    "f8_divisor_447": ("kvqo_f32_to_f16(amax / 448.0f)", "kvqo_f32_to_f16(amax / 447.0f)"),
    "f8_decode_drops_scale": ("x[i] = ds * kvqo_e4m3_value(blk[2 + i]);", "x[i] = kvqo_e4m3_value(blk[2 + i]);"),
    "f16_ties_away": ("if (rem > half || (rem == half && (q & 1u)))", "if (rem >= half)"),
    "f16_subnormal_shift": ("int shift = (e >= -14) ? 13 : 13 + (-14 - e);",
                            "int shift = (e >= -14) ? 13 : 13 + (-15 - e);"),
    "v_weight_unnormalised": ("o[d] = (float)(acc[d] / Z);", "o[d] = (float)(acc[d]);"),
    "imp_sink_not_in_denominator": ("double denom = sinks ? exp(sink - top) : 0.0;", "double denom = 0.0;"),
    "imp_unnormalised": ("exp(score[j - row_start] - top) / denom;", "exp(score[j - row_start] - top);"),
    "imp_causal_off_by_one": ("const int64_t row_end = len[b] - T + t + 1;",
                              "const int64_t row_end = len[b] - T + t;"),
    "imp_window_off_by_one": ("row_end > window ? row_end - window : 0;", "row_end > window ? row_end - window + 1 : 0;"),
    "imp_group_modulo": ("const int32_t kv_group = h / heads_per_group;", "const int32_t kv_group = h % Hkv;"),
    "f8_row_codes_at_block_stride": ("memcpy(row + 32 * k, blk + 2, 32);", "memcpy(row + 34 * k, blk + 2, 32);"),
    "f8_row_scales_first": ("row[row_elems + 2 * k] = blk[0];", "row[2 * k] = blk[0];"),
    "f8_read_scale_of_head_0": ("const uint8_t* scale = row + row_elems + 2 * k;",
                                "const uint8_t* scale = row + row_elems + 2 * kb;"),
    "f8_read_codes_of_head_0": ("memcpy(blk + 2, row + 32 * k, 32);", "memcpy(blk + 2, row + 32 * kb, 32);"),
    "f8_v_rows_as_q5_1": ("if (fmt == KVQO_FMT_E4M3) return (int64_t)Hkv * nb * 34;",
                          "if (fmt == KVQO_FMT_E4M3 && !v_side) return (int64_t)Hkv * nb * 34;"),
}


def _build(name, tmp):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    path = os.path.join(tmp, f"m_{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    hdr = os.path.join(os.path.dirname(SRC), "kvq_oracle.h")
    with open(os.path.join(tmp, "kvq_oracle.h"), "w") as f:
        f.write(open(hdr).read())
    so = os.path.join(tmp, f"m_{name}.so")
    subprocess.run(["gcc", *core.GCC_FLAGS, "-o", so, path, "-lm"], check=True)
    return core.load(so)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    with tempfile.TemporaryDirectory() as tmp:
        lib = _build(name, tmp)
        caught = []
        for pin, check in oracle_pins.ALL_CHECKS.items():
            try:
                check(lib)
            except AssertionError:
                caught.append(pin)
            except ValueError:
                caught.append(pin + "(error)")
        assert caught, f"no pin catches mutant {name}"


def test_unmutated_oracle_passes_every_pin():
    lib = oracle.load()
    for check in oracle_pins.ALL_CHECKS.values():
        check(lib)
