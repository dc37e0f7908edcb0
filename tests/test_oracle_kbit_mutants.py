"""Planted mistakes in the k-bit part of the oracle (oracle/kbit.c) must be caught by its
pins (CPU only). Each mutant is a copy of kbit.c with one plausible bug, compiled with the
unmodified oracle.c into a temporary library; at least one pin has to fail."""
import pytest

import oracle
import oracle_kbit_pins as P

MUTANTS = {
    "e4m4_bias_10": ("return ldexp(1.0 + (double)m / 16.0, e - 11);", "return ldexp(1.0 + (double)m / 16.0, e - 10);"),
    "e4m4_subnormal_shift": ("if (e == 0) return ldexp((double)m / 16.0, 1 - 11);",
                             "if (e == 0) return ldexp((double)m / 16.0, -11);"),
    "e4m4_mantissa_8ths": ("return ldexp(1.0 + (double)m / 16.0, e - 11);", "return ldexp(1.0 + (double)m / 8.0, e - 11);"),
    "encode_ties_odd": ("(c & 1) == 0 && (best & 1) == 1", "(c & 1) == 1 && (best & 1) == 0"),
    "encode_truncates": ("const double d = fabs(oracle_e4m4_decode((uint8_t)c) - v);",
                         "const double d = oracle_e4m4_decode((uint8_t)c) > v ? 1e300 : v - oracle_e4m4_decode((uint8_t)c);"),
    "codebook_unnormalised": ("for (int i = 0; i < L; ++i) cb[i] /= maxabs;", ""),
    "codebook_bins_shifted": ("phi_inv((double)(i + 1) / L)", "phi_inv((double)(i + 0.5) / L)"),
    "index_ties_high": ("if (d < bestd) { best = i; bestd = d; }", "if (d <= bestd) { best = i; bestd = d; }"),
    "index_unnormalised": ("const double v = x[j] / s;", "const double v = x[j];"),
    "plane_bits_reversed": ("idx |= (int)((planes[blk * k + b] >> j) & 1u) << b;",
                            "idx |= (int)((planes[blk * k + b] >> j) & 1u) << (k - 1 - b);"),
    "plane_elements_reversed": ("idx |= (int)((planes[blk * k + b] >> j) & 1u) << b;",
                                "idx |= (int)((planes[blk * k + b] >> (31 - j)) & 1u) << b;"),
    "gemv_drops_residual": ("for (int64_t kk = 0; kk <= K; ++kk) {", "for (int64_t kk = 0; kk < K; ++kk) {"),
    "gemv_scale_of_first_block": ("const int64_t blk = n * bpr + kk / 32;", "const int64_t blk = n * bpr;"),
    "gemv_unscaled": ("                                     oracle_e4m4_decode(absmax_e4m4[blk]);\n",
                      "                                     1.0;\n"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_kbit_mutant_is_caught(name, tmp_path):
    before, after = MUTANTS[name]
    src = open(oracle._KBIT_SRC).read()
    assert src.count(before) == 1, "mutation anchor not unique/present: %r" % before
    mutated = tmp_path / "kbit_mut.c"
    mutated.write_text(src.replace(before, after))
    so = oracle.build(kbit_src=str(mutated), out=str(tmp_path / ("liboracle_kbit_%s.so" % name)))
    orc = oracle.Oracle(so)
    failed = []
    for pin in P.ALL_KBIT_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "no pin caught the planted mistake %s" % name
