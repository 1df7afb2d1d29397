"""Planted mistakes in the oracle must each fail at least one pin.

Each mutant is a copy of oracle/q8ref.c with one plausible mistake (a dropped
term, a wrong index or sign, a transposed operand, a wrong rounding rule),
compiled with the oracle's own flags into a temporary library and run
through every pin of tests/pins.py on the CPU.
"""
import os
import subprocess

import pytest

import oracle
from oracle import build as obuild
import pins

MUTANTS = {
    "scale_divisor_128": ("float d32 = amax / 127.0f;", "float d32 = amax / 128.0f;"),
    "ties_toward_zero": ("(frac >= 0.5f) ? t + 1.0f : t", "(frac > 0.5f) ? t + 1.0f : t"),
    "divide_instead_of_reciprocal": ("float v = x[j] * id;", "float v = x[j] / d32;"),
    "f16_ties_away": ("if (rem > half || (rem == half && (q & 1u))) q += 1u;",
                      "if (rem >= half) q += 1u;"),
    "f16_subnormal_shift": ("shift_rne(sig, -(e + 1));", "shift_rne(sig, -e);"),
    "zero_test_exact": ("if (d32 < FLT_MIN) {", "if (d32 == 0.0f) {"),
    "bf16_shift": ("(uint32_t)b << 16;", "(uint32_t)b << 15;"),
    "drop_last_block": ("acc += s * (double)p;", "acc += (kb + 1 < KB) ? s * (double)p : 0.0;"),
    "weight_scale_index": ("q8ref_f16_to_f64(dw_row[kb])", "q8ref_f16_to_f64(dw_row[0])"),
    "activation_times_itself": ("int32_t p = block_dot(qa_row + kb * QK, qw_row + kb * QK);",
                                "int32_t p = block_dot(qa_row + kb * QK, qa_row + kb * QK);"),
    "reversed_weight_index": ("s += (int32_t)a[j] * (int32_t)w[j];",
                              "s += (int32_t)a[j] * (int32_t)w[QK - 1 - j];"),
    "transposed_output": ("C[m * N + n] = c;", "C[n * M + m] = c;"),
    "absdot_signed": ("mag += fabs(s) *", "mag += s *"),
    "block_endianness": ("b[0] = (uint8_t)(h & 0xff);\n            b[1] = (uint8_t)(h >> 8);",
                         "b[1] = (uint8_t)(h & 0xff);\n            b[0] = (uint8_t)(h >> 8);"),
    "pack_row_stride": ("* 1024 + r * 16 + t] =", "* 1024 + t * 64 + r] ="),
    "pack_half_order": ("b ? b[2 + 16 * h + t] : 0;", "b ? b[2 + 16 * (1 - h) + t] : 0;"),
    "sampled_wrong_row": ("one_output(q_a + rows[i] * K, d_a + rows[i] * KB,",
                          "one_output(q_a + cols[i] * K, d_a + rows[i] * KB,"),
    "swiglu_gate_up_swapped": ("double v = q8ref_silu(G[i]) * U[i];",
                               "double v = q8ref_silu(U[i]) * G[i];"),
    "silu_sign": ("return x / (1.0 + exp(-x));", "return x / (1.0 + exp(x));"),
    "swiglu_scale_index": ("d + m * (I / QK) + b);", "d + b * M + m);"),
    "kv3_threshold_is_level": ("float t = (kv3_levels[k] + kv3_levels[k + 1]) * 0.5f;",
                               "float t = kv3_levels[k + 1];"),
    "kv3_butterfly_sign": ("v[j + len] = a - b;", "v[j + len] = b - a;"),
    "kv3_scale_no_sqrt": ("float s = sqrtf(v[0] / (float)D);", "float s = v[0] / (float)D;"),
    "kv3_pack_stride": ("w |= (uint32_t)c << (3 * j);", "w |= (uint32_t)c << (3 * (7 - j));"),
    "kv3_decode_norm": ("out[r * D + i] = z[i] * (1.0f / (float)D);", "out[r * D + i] = z[i];"),
    "kv3_level_value": ("0.2451f,  0.7560f,", "0.2451f,  0.7650f,"),
    "kv3_sum_drops_term": ("for (int i = 0; i < D; i += 2 * len) v[i] = v[i] + v[i + len];",
                           "for (int i = 0; i < D; i += 2 * len) v[i] = v[i];"),
    "attn_not_causal": ("if (u > t || u >= L) continue;", "if (u >= L) continue;"),
    "attn_scale_no_sqrt": ("const double scale = 1.0 / sqrt((double)D);",
                           "const double scale = 1.0 / (double)D;"),
    "attn_gqa_mapping": ("const int64_t i = t / ATTN_BLK, g = h / group;",
                         "const int64_t i = t / ATTN_BLK, g = h % Hkv;"),
    "attn_no_sink": ("                take[0] = 1;\n", "                take[1 < i ? 1 : 0] = 1;\n"),
    "attn_ties_high": ("if (best < 0 || sc > bs) { best = j; bs = sc; }",
                       "if (best < 0 || sc >= bs) { best = j; bs = sc; }"),
    "attn_select_one_head": ("for (int64_t hq = h * group; hq < (h + 1) * group; ++hq)",
                             "for (int64_t hq = h * group; hq < h * group + 1; ++hq)"),
    "attn_pool_divisor": ("out[d] = acc / (double)(t1 - t0);", "out[d] = acc / (double)ATTN_BLK;"),
    "attn_diag_block_dropped": ("                take[i] = 1;\n", "                take[i - 1] = 1;\n"),
    "kv3_sum_sequential": ("for (int len = 1; len < D; len <<= 1)\n            for (int i = 0; i < D; i += 2 * len) v[i] = v[i] + v[i + len];",
                           "for (int i = 1; i < D; ++i) v[0] = v[0] + v[i];"),
    "kv3_sum_halving": ("for (int len = 1; len < D; len <<= 1)\n            for (int i = 0; i < D; i += 2 * len) v[i] = v[i] + v[i + len];",
                        "for (int len = D / 2; len >= 1; len >>= 1)\n            for (int i = 0; i < len; ++i) v[i] = v[i] + v[i + len];"),
    "kv3_sum_not_squared": ("for (int i = 0; i < D; ++i) v[i] = y[i] * y[i];",
                            "for (int i = 0; i < D; ++i) v[i] = y[i];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_pin(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(obuild.SRC).read()
    assert src.count(old) == 1, "mutation site not unique/not found: %s" % name
    path_c = tmp_path / ("q8ref_%s.c" % name)
    path_c.write_text(src.replace(old, new))
    lib = str(tmp_path / ("libq8ref_%s.so" % name))
    subprocess.run(["gcc", *obuild.CFLAGS, str(path_c), "-o", lib, "-lm"], check=True)
    orc = oracle.Oracle(lib)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
        except Exception as e:          # a crash or a shape error also counts
            failed.append("%s (%s)" % (pin.__name__, type(e).__name__))
    assert failed, "planted mistake %r passed every pin" % name


def test_wrong_gateup_interleave_fails_its_pin():
    """The gate/up interleave lives in the oracle's Python layer: a copy with
    the halves of each group swapped must fail pin_gateup_layout."""
    orc = oracle.default()

    class Swapped(oracle.Oracle):
        @staticmethod
        def interleave_gateup(gate_rows, up_rows):
            return oracle.Oracle.interleave_gateup(up_rows, gate_rows)

    bad = Swapped(orc.path)
    with pytest.raises(AssertionError):
        pins.pin_gateup_layout(bad)
