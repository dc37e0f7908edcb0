"""Planted mistakes in the oracle must be caught by the pins (CPU only).

Each mutant is a copy of oracle/oracle.c with one plausible bug written in
(a transposed operand, a dropped term, a wrong index, a wrong rounding rule,
double rounding, a lost compensation term, ...). The copy is compiled into a
temporary directory and every pin of tests/oracle_pins.py is run on it; at
least one pin has to fail. The real oracle is never modified.
"""
import os

import pytest

import oracle
import oracle_pins as P

MUTANTS = {
    "transposed_W": ("W[n * K + k]", "W[k * N + n]"),
    "dropped_residual": ("k <= K", "k < K"),
    "dropped_first_product": ("for (int64_t k = 0; k <= K; ++k)", "for (int64_t k = 1; k <= K; ++k)"),
    "residual_columns_reversed": (": bf16_bits_to_double(R[m * N + n]);", ": bf16_bits_to_double(R[m * N + (N - 1 - n)]);"),
    "X_reversed_in_k": ("X[m * K + k]", "X[m * K + (K - 1 - k)]"),
    "ties_away_from_zero": ("(fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0", "fl + 1.0"),
    "truncation": ("if (frac > 0.5) n = fl + 1.0;", "if (0) n = fl + 1.0;"),
    "nine_bit_mantissa": ("double q = ldexp(1.0, e - 7);", "double q = ldexp(1.0, e - 8);"),
    "double_rounding_via_fp32": ("uint16_t y = oracle_round_bf16(exact);",
                                 "uint16_t y = oracle_round_bf16((double)(float)exact);"),
    "no_compensation": ("double exact = s + c;", "double exact = s;"),
    "no_subnormal_clamp": ("if (e < -126) e = -126;", ""),
    "sign_dropped": ("return (uint16_t)(sign | ((u >> 16) & 0x7FFF));", "return (uint16_t)((u >> 16) & 0x7FFF);"),
    "fp32_accumulation": ("double t = s + p;", "double t = (double)(float)(s + p);"),
    "residual_scaled_twice": (": bf16_bits_to_double(R[m * N + n]);", ": 2.0 * bf16_bits_to_double(R[m * N + n]);"),
    # the shard epilogue (flags)
    "round_product_ignored": ("    if (round_product)\n        exact =", "    if (0)\n        exact ="),
    "round_product_residual_twice": ("if (k == K && round_product) break;", "if (0) break;"),
    "neg_zero_never_sanitised": ("if ((flags & ORACLE_NO_NEG_ZERO) && y == 0x8000) y = 0;", ""),
    "neg_zero_always_sanitised": ("if ((flags & ORACLE_NO_NEG_ZERO) && y == 0x8000) y = 0;",
                                  "if (y == 0x8000) y = 0;"),
    "round_product_flag_swapped": ("(flags & ORACLE_ROUND_PRODUCT) != 0", "(flags & ORACLE_NO_NEG_ZERO) != 0"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    before, after = MUTANTS[name]
    src = open(oracle.source_path()).read()
    assert src.count(before) == 1, "mutation anchor not unique/present: %r" % before
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(src.replace(before, after))
    so = oracle.build(src=str(mutated), out=str(tmp_path / ("liboracle_%s.so" % name)))
    orc = oracle.Oracle(so)
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "no pin caught the planted mistake %s" % name
