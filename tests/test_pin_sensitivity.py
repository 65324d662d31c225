"""The pins catch plausible mistakes: each mutant below is a copy of the C oracle
with one planted error (built on the CPU into a temporary directory); at least
one pin must fail on it. The real oracle source is never modified."""
import os
import subprocess

import pytest

import oracle
from tests import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "int4_oracle.c")

# (name, exact text in the oracle, replacement)
MUTANTS = [
    ("even_element_high_nibble",
     "if (k % 2 == 0)", "if (k % 2 == 1)"),
    ("offset_binary_nibble",
     "uint8_t nib = (uint8_t)(q & 0xF);", "uint8_t nib = (uint8_t)((q + 8) & 0xF);"),
    ("divide_by_unrounded_scale",
     "int q = quantize_one(row[k], sf);", "int q = quantize_one(row[k], sf == 0.0f ? 0.0f : s32);"),
    ("round_half_away_from_zero",
     "float r = rintf(t);", "float r = roundf(t);"),
    ("round_toward_zero",
     "float r = rintf(t);", "float r = truncf(t);"),
    ("no_clamp_low",
     "if (r < -8.0f) r = -8.0f;", ""),
    ("symmetric_clamp_minus7",
     "if (r < -8.0f) r = -8.0f;", "if (r < -7.0f) r = -7.0f;"),
    ("zero_group_scale_one",
     "uint16_t s16 = int4_oracle_half_from_float(s32);",
     "uint16_t s16 = int4_oracle_half_from_float(s32 == 0.0f ? 1.0f : s32);"),
    ("scale_absmax_over_8",
     "float s32 = amax / 7.0f;", "float s32 = amax / 8.0f;"),
    ("scale_reciprocal_multiply",
     "float s32 = amax / 7.0f;", "float s32 = amax * (1.0f / 7.0f);"),
    ("absmax_over_whole_row",
     "for (int64_t k = k0; k < k1; ++k) {\n                float a", "for (int64_t k = 0; k < K; ++k) {\n                float a"),
    ("unpack_no_sign_extension",
     "return v >= 8 ? v - 16 : v;", "return v;"),
    ("unpack_high_nibble_first",
     "return (prow[k / 2] >> (4 * (int)(k % 2))) & 0xF;",
     "return (prow[k / 2] >> (4 * (int)(1 - k % 2))) & 0xF;"),
    ("matmul_scale_ignores_row",
     "int4_oracle_float_from_half(scales[n * G + gi]);", "int4_oracle_float_from_half(scales[gi]);"),
    ("matmul_drops_partial_group",
     "for (int64_t gi = 0; gi < G; ++gi) {\n                int64_t k0", "for (int64_t gi = 0; gi < K / group; ++gi) {\n                int64_t k0"),
    ("matmul_scale_applied_twice",
     "acc += sf * part;", "acc += sf * sf * part;"),
    ("half_truncates",
     "double n = nearbyint(m);", "double n = floor(m);"),
    ("half_ties_away",
     "double n = nearbyint(m);", "double n = round(m);"),
    ("half_no_subnormals",
     "if (e < -14)\n        e = -14;", "if (e < -14)\n        return sign;"),
    ("half_overflow_threshold",
     "if (a >= 65520.0)", "if (a > 65504.0)"),
    ("dequantize_swaps_nibbles",
     "            out[n * K + k] = (float)q * sf;",
     "            out[n * K + k] = (float)weight_int(packed + n * B, k ^ 1, zeros ? zeros + n * G : NULL, group) * sf;"),
    ("dequantize_scale_of_next_group",
     "float sf = int4_oracle_float_from_half(scales[n * G + k / group]);\n            int q = weight_int(packed + n * B, k, zeros ? zeros + n * G : NULL, group);\n            out[n * K + k] = (float)q",
     "float sf = int4_oracle_float_from_half(scales[n * G + ((k + 1) / group < G ? (k + 1) / group : 0)]);\n            int q = weight_int(packed + n * B, k, zeros ? zeros + n * G : NULL, group);\n            out[n * K + k] = (float)q"),
    ("dequantize_half_from_unscaled",
     "out[n * K + k] = int4_oracle_half_from_float((float)q * sf);",
     "out[n * K + k] = int4_oracle_half_from_float((float)q);"),
    ("affine_zero_point_added_after_rounding",
     "double r = rint((double)t + (double)zp);", "double r = rint((double)t) + (double)zp;"),
    ("affine_range_excludes_zero",
     "float lo = 0.0f, hi = 0.0f;             /* the range includes zero */",
     "float lo = row[k0], hi = row[k0];"),
    ("affine_zero_point_sign",
     "float z = rintf(-lo / sf);", "float z = rintf(lo / sf);"),
    ("affine_code_ignores_zero_point",
     "    return raw_nibble(prow, k) - (int)zp[k / group];", "    return raw_nibble(prow, k);"),
    ("affine_scale_over_16",
     "float s32 = (hi - lo) / 15.0f;", "float s32 = (hi - lo) / 16.0f;"),
    ("epilogue_bias_dropped",
     "            acc += (double)bias[n];", "            acc += 0.0;"),
    ("epilogue_relu_keeps_negatives",
     "v = v > 0.0f ? v : 0.0f;", "v = v > 0.0f ? v : v;"),
    ("epilogue_bias_of_wrong_column",
     "            acc += (double)bias[n];", "            acc += (double)bias[(n + 1) % N];"),
    ("widen_subnormal_wrong",
     "v = ldexp((double)frac, -24);", "v = ldexp((double)(1024 + frac), -25);"),
]


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} must appear exactly once"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    out = tmp_path / f"lib{name}.so"
    subprocess.run(["cc", *oracle.CFLAGS, "-o", str(out), str(path), "-lm"], check=True)
    return oracle.load(str(out))


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    lib = _build_mutant(tmp_path, name, old, new)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            if pin is pins.pin_p4_round_trip:
                pin(lib, seeds=range(200))
            else:
                pin(lib)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name} passed every pin"
