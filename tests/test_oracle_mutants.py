"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
the pins catch every one: the pins are strong enough to trust the oracle."""
import os

import pytest

import oracle
import pins
import pins_epilogue
import pins_grouped

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

# Mistakes in the multi-step epilogue, caught by the epilogue pins.
EPI_MUTANTS = [
    ("epi_silu_exp_sign", "uint16_t e = rd(elem, exp(wd(elem, n)));", "uint16_t e = rd(elem, exp(wd(elem, x)));"),
    ("epi_silu_unrounded_exp",
     "uint16_t d = rd(elem, wd(elem, cst(elem, 1.0)) + wd(elem, e));\n    return rd(elem, wd(elem, x) / wd(elem, d));",
     "uint16_t d = rd(elem, 1.0 + exp(-wd(elem, x))); (void)e;\n    return rd(elem, wd(elem, x) / wd(elem, d));"),
    ("epi_silu_one_rounding", "    return rd(elem, wd(elem, x) / wd(elem, d));\n}\n\nuint16_t oracle_epi_gelu_tanh",
     "    (void)d; return rd(elem, wd(elem, x) / (1.0 + exp(-wd(elem, x))));\n}\n\nuint16_t oracle_epi_gelu_tanh"),
    ("epi_gelu_cubic_coeff", "const uint16_t c1 = cst(elem, 0.044715);", "const uint16_t c1 = cst(elem, 0.44715);"),
    ("epi_gelu_square_not_cube", "uint16_t b = rd(elem, wd(elem, a) * wd(elem, x));", "uint16_t b = a;"),
    ("epi_gelu_tanh_unrounded_z", "uint16_t e = rd(elem, exp(wd(elem, z)));",
     "uint16_t e = rd(elem, exp(wd(elem, d) * -2.0 * sqrt(2.0 / 3.14159265358979323846))); (void)z;"),
    ("epi_gelu_erf_no_half", "return rd(elem, wd(elem, h) * wd(elem, cst(elem, 0.5)));", "return h;"),
    ("epi_gelu_erf_no_rsqrt2", "const uint16_t c3 = cst(elem, 0.70710678118654752440);",
     "const uint16_t c3 = cst(elem, 1.0);"),
    ("epi_gelu_erf_as_tanh", "uint16_t f = rd(elem, erf(wd(elem, s)));", "uint16_t f = rd(elem, tanh(wd(elem, s)));"),
    ("epi_residual_reads_bias", "case ORACLE_EPI_RESIDUAL: return rd(elem, wd(elem, t) + wd(elem, res));",
     "case ORACLE_EPI_RESIDUAL: return rd(elem, wd(elem, t) + wd(elem, bias));"),
    ("epi_mul_as_add", "case ORACLE_EPI_MUL: return rd(elem, wd(elem, t) * wd(elem, mul));",
     "case ORACLE_EPI_MUL: return rd(elem, wd(elem, t) + wd(elem, mul));"),
    ("epi_steps_reversed", "for (int s = 0; s < nsteps; ++s)\n            v = epi_step(elem, ops[s],",
     "for (int s = nsteps - 1; s >= 0; --s)\n            v = epi_step(elem, ops[s],"),
    ("epi_round_ties_away", "r = nearbyint(a / q) * q;", "r = round(a / q) * q;"),
    ("epi_round_no_subnormal_grid", "if (e < emin) e = emin;                  /* subnormal grid */", ""),
    # binary16-only slips that stay within the compositions' error bounds: a
    # constant one unit off, and an intermediate left unrounded
    ("epi_f16_c2_one_ulp_off", "const uint16_t c2 = cst(elem, -2.0 * sqrt(2.0 / 3.14159265358979323846));",
     "const uint16_t c2 = cst(elem, -2.0 * sqrt(2.0 / 3.14159265358979323846) * (elem ? 1.0 : 1.0005));"),
    ("epi_f16_silu_unrounded_denominator", "    return rd(elem, wd(elem, x) / wd(elem, d));\n}\n\nuint16_t oracle_epi_gelu_tanh",
     "    return rd(elem, wd(elem, x) / (elem ? wd(elem, d) : 1.0 + wd(elem, e)));\n}\n\nuint16_t oracle_epi_gelu_tanh"),
    ("epi_f16_gelu_erf_unrounded_sum", "uint16_t h = rd(elem, wd(elem, x) * wd(elem, g));",
     "uint16_t h = rd(elem, wd(elem, x) * (elem ? wd(elem, g) : 1.0 + wd(elem, f)));"),
    ("epi_f16_gelu_tanh_unrounded_inner", "uint16_t z = rd(elem, wd(elem, d) * wd(elem, c2));",
     "uint16_t z = rd(elem, (elem ? wd(elem, d) : wd(elem, x) + wd(elem, c)) * wd(elem, c2));"),
    ("epi_round_max_overflows", "if (r > maxv) bits = elem ? 0x7f80u : 0x7c00u;", "if (r >= maxv) bits = elem ? 0x7f80u : 0x7c00u;"),
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


# Mistakes in the grouped and indexed contractions, caught by their pins.
GROUPED_MUTANTS = [
    ("grouped_weight_block_stride", "int rc = oracle_linear(elem, x + g * sx, ldx, w + g * N * ldw, ldw,",
     "int rc = oracle_linear(elem, x + g * sx, ldx, w + g * ldw, ldw,"),
    ("grouped_bias_not_offset", "b ? b + g * N : NULL,", "b,"),
    ("grouped_activation_stride", "int rc = oracle_linear(elem, x + g * sx, ldx,", "int rc = oracle_linear(elem, x, ldx,"),
    ("indexed_next_expert", "const uint16_t* we = w + e * sw;\n        for (int64_t n = 0; n < N; ++n) {\n            float acc",
     "const uint16_t* we = w + ((e + 1) % E) * sw;\n        for (int64_t n = 0; n < N; ++n) {\n            float acc"),
    ("indexed_reversed_columns", "widen16(elem, we[k * ldw + n]);", "widen16(elem, we[k * ldw + (N - 1 - n)]);"),
    ("indexed_writes_rows_without_expert", "        if (e < 0 || e >= E) continue;\n        const uint16_t* we = w + e * sw;\n        for (int64_t n = 0; n < N; ++n) {\n            float acc",
     "        if (e < 0 || e >= E) { for (int64_t n = 0; n < N; ++n) if (y) y[m * ldy + n] = 0; continue; }\n        const uint16_t* we = w + e * sw;\n        for (int64_t n = 0; n < N; ++n) {\n            float acc"),
    ("indexed_drops_first_k", "for (int64_t k = 0; k < K; ++k) acc = acc + widen16(elem, x[m * ldx + k])",
     "for (int64_t k = 1; k < K; ++k) acc = acc + widen16(elem, x[m * ldx + k])"),
]


@pytest.mark.parametrize("name,old,new", GROUPED_MUTANTS, ids=[m[0] for m in GROUPED_MUTANTS])
def test_grouped_pins_catch_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation site vanished: " + name
    mutated = src.replace(old, new, 1)
    path = str(tmp_path / ("m_%s.c" % name))
    open(path, "w").write(mutated)
    lib = oracle.build(src=path, out=str(tmp_path / ("lib_%s.so" % name)))
    orc = oracle.Oracle(lib)
    caught = []
    for pin in pins_grouped.GROUPED_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
            break
    assert caught, "no grouped pin catches mutant " + name


@pytest.mark.parametrize("name,old,new", EPI_MUTANTS, ids=[m[0] for m in EPI_MUTANTS])
def test_epilogue_pins_catch_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation site vanished: " + name
    mutated = src.replace(old, new, 1)
    path = str(tmp_path / ("m_%s.c" % name))
    open(path, "w").write(mutated)
    lib = oracle.build(src=path, out=str(tmp_path / ("lib_%s.so" % name)))
    orc = oracle.Oracle(lib)
    caught = []
    for pin in pins_epilogue.EPILOGUE_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
            break
    assert caught, "no epilogue pin catches mutant " + name
