"""Planted mistakes in the KDA part of the oracle (oracle/kda.c) must be caught by its pins
(CPU only). Each mutant is a copy of kda.c with one plausible bug (one or more text edits),
compiled with the unmodified oracle.c and kbit.c into a temporary library; at least one pin
has to fail."""
import pytest

import oracle
import oracle_kda_pins as P

MUTANTS = {
    "window_off_by_one": [("const int64_t s = t + 1 + w;", "const int64_t s = t + w;")],
    "taps_reversed": [("oracle_bf16_to_double(conv_w[d * KDA_W + w])",
                       "oracle_bf16_to_double(conv_w[d * KDA_W + (KDA_W - 1 - w)])")],
    "state_reversed": [("const uint16_t x = s < KDA_W - 1 ? state_line[s * dim + d] : mixed[(bi * T + (s - (KDA_W - 1))) * dim + d];\n        acc",
                        "const uint16_t x = s < KDA_W - 1 ? state_line[(KDA_W - 2 - s) * dim + d] : mixed[(bi * T + (s - (KDA_W - 1))) * dim + d];\n        acc")],
    "conv_no_bias": [("double acc = oracle_bf16_to_double(conv_b[d]);", "double acc = 0.0;")],
    "softplus_threshold_2": [("return x > 20.0 ? x : log1p(exp(x));", "return x > 2.0 ? x : log1p(exp(x));")],
    "gate_without_exp": [("const double decay_a = exp((double)A_log[hv]);", "const double decay_a = (double)A_log[hv];")],
    "decay_sign": [("Sv[c] *= exp(g[c]);", "Sv[c] *= exp(-g[c]);")],
    "decay_after_update": [("Sv[c] *= exp(g[c]);\n", ""),
                           ("Sv[c] += u * k[c];", "Sv[c] = Sv[c] * exp(g[c]) + u * k[c];")],
    "gqa_modulo": [("const int64_t h = hv / group;", "const int64_t h = hv % H;")],
    "l2_eps_outside": [("const double qn = 1.0 / sqrt(qq + 1e-6), kn = 1.0 / sqrt(kk + 1e-6);",
                        "const double qn = 1.0 / (sqrt(qq) + 1e-6), kn = 1.0 / (sqrt(kk) + 1e-6);")],
    "no_scale": [("q[c] *= qn * scale;", "q[c] *= qn;")],
    "key_not_normalised": [("k[c] *= kn;", "k[c] *= 1.0;")],
    "no_beta": [("const double u = beta * (", "const double u = (")],
    "ring_position_shifted": [("const int64_t pos = t;", "const int64_t pos = t + 1;")],
    "output_before_update": [("Sv[c] += u * k[c];\n                        o += Sv[c] * q[c];",
                              "o += Sv[c] * q[c];\n                        Sv[c] += u * k[c];")],
    "snapshot_of_start_state": [("memcpy(dst, S, sizeof(double) * (size_t)(V * K));",
                                 "for (int64_t i = 0; i < V * K; ++i) dst[i] = (double)s0[i];")],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_kda_mutant_is_caught(name, tmp_path):
    src = open(oracle._KDA_SRC).read()
    for before, after in MUTANTS[name]:
        assert src.count(before) == 1, "mutation anchor not unique/present: %r" % before
        src = src.replace(before, after)
    mutated = tmp_path / "kda_mut.c"
    mutated.write_text(src)
    so = oracle.build(kda_src=str(mutated), out=str(tmp_path / ("liboracle_kda_%s.so" % name)))
    orc = oracle.Oracle(so)
    failed = []
    for pin in P.ALL_KDA_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "no pin caught the planted mistake %s" % name
