"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
the pins catch every one: the pins are strong enough to trust the oracle."""
import os

import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, text in oracle.c, replacement)
MUTANTS = [
    ("drop_last_term", "for (int64_t k = 0; k < K; ++k) acc = acc + xr[k] * wr[k];",
     "for (int64_t k = 0; k + 1 < K; ++k) acc = acc + xr[k] * wr[k];"),
    ("points_drop_first_term", "        for (int64_t k = 0; k < K; ++k) {\n            float xv",
     "        for (int64_t k = 1; k < K; ++k) {\n            float xv"),
    ("transposed_weight_stride", "float acc = dot_f32(xf + m * K, wf + n * K, K);",
     "float acc = dot_f32(xf + m * K, wf + n, K);"),
    ("truncate_not_rne", "if (rem > half || (rem == half && (q & 1u))) q += 1u;",
     "if (rem > half && 0) q += 1u;"),
    ("ties_away_from_zero", "if (rem > half || (rem == half && (q & 1u))) q += 1u;",
     "if (rem >= half) q += 1u;"),
    ("bias_before_rounding", "if (y) y[m * ldy + n] = b ? bias_epilogue16(elem, p16, b[n]) : p16;",
     "if (y) y[m * ldy + n] = b ? narrow16(elem, acc + widen16(elem, b[n])) : p16;"),
    ("bias_wrong_index", "if (y) y[m * ldy + n] = b ? bias_epilogue16(elem, p16, b[n]) : p16;",
     "if (y) y[m * ldy + n] = b ? bias_epilogue16(elem, p16, b[m % N]) : p16;"),
    ("flush_subnormal_inputs", "mag = ldexpf((float)frac, -24);", "mag = 0.0f * (float)frac;"),
    ("drop_sign", "return sign ? -mag : mag;", "return mag;"),
    ("product_rounded_to_f16", "acc = acc + xr[k] * wr[k];",
     "acc = acc + oracle_f16_to_f32(oracle_f32_to_f16(xr[k] * wr[k]));"),
    ("f16_accumulator", "acc = acc + xr[k] * wr[k];",
     "acc = oracle_f16_to_f32(oracle_f32_to_f16(acc + xr[k] * wr[k]));"),
    ("no_carry_into_exponent", "if (q == 2048u) { q = 1024u; e += 1; }", "if (q == 2048u) { q = 1024u; }"),
    ("no_overflow_to_inf", "if (e >= 16) return (uint16_t)(sign | 0x7c00u);   /* >= 2^16: overflow */",
     "if (e >= 16) return (uint16_t)(sign | 0x7bffu);"),
    ("subnormal_shift_off_by_one", "shift = -e - 1;", "shift = -e;"),
    ("decode_bias_off_by_one", "mag = ldexpf((float)(1024u + frac), (int)e - 25);",
     "mag = ldexpf((float)(1024u + frac), (int)e - 24);"),
    ("epilogue_in_f16", "float s = oracle_f16_to_f32(proj16) + oracle_f16_to_f32(b16);\n    return oracle_f32_to_f16(s);",
     "float s = oracle_f16_to_f32(proj16) + oracle_f16_to_f32(b16);\n    return oracle_f32_to_f16(s + 0.0001f);"),
    ("acc_starts_nonzero", "float acc = 0.0f;\n    for (int64_t k = 0; k < K; ++k) acc = acc + xr[k] * wr[k];",
     "float acc = 1e-6f;\n    for (int64_t k = 0; k < K; ++k) acc = acc + xr[k] * wr[k];"),
    ("points_wrong_stride", "const uint16_t* xr = x + ms[i] * ldx;", "const uint16_t* xr = x + ms[i] * K;"),
    ("band_abs_missing", "                a += fabs(pd);", "                a += pd;"),
    ("bf16_truncate", "if (rem > 0x8000u || (rem == 0x8000u && (q & 1u))) q += 1u;   /* may carry into the exponent */",
     "if (rem > 0x8000u && 0) q += 1u;"),
    ("bf16_ties_away", "if (rem > 0x8000u || (rem == 0x8000u && (q & 1u))) q += 1u;   /* may carry into the exponent */",
     "if (rem >= 0x8000u) q += 1u;"),
    ("bf16_decode_shift", "float oracle_bf16_to_f32(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }",
     "float oracle_bf16_to_f32(uint16_t h) { return f32_from_bits((uint32_t)h << 15); }"),
    ("bf16_epilogue_as_f16", "return narrow16(elem, widen16(elem, proj16) + widen16(elem, b16));",
     "return narrow16(elem, widen16(elem, proj16) + widen16(0, b16));"),
    ("sums_before_accumulate", "if (y32) y32[m * ldy + n] = acc;", "if (y32) y32[m * ldy + n] = acc * 1.0000001f;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation site vanished: " + name
    mutated = src.replace(old, new, 1)
    path = str(tmp_path / ("m_%s.c" % name))
    open(path, "w").write(mutated)
    lib = oracle.build(src=path, out=str(tmp_path / ("lib_%s.so" % name)))
    orc = oracle.Oracle(lib)
    caught = []
    for pin in pins.FAST_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
            break
    assert caught, "no pin catches mutant " + name
