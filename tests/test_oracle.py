"""The CPU oracle against its pins (no GPU)."""
import numpy as np
import pytest

import oracle_pins as P
from decode_skinny_addmm_amd import synth


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=[p.__name__ for p in P.ALL_PINS])
def test_pin(pin, oracle_lib):
    pin(oracle_lib)


def test_threads_do_not_change_results(oracle_lib):
    X, ws, rs = synth.make_inputs(3, 57, 256, seed=12)
    a = oracle_lib.addmm_bf16(synth.bits(X), synth.bits(ws[0]), synth.bits(rs[0]), threads=1)
    b = oracle_lib.addmm_bf16(synth.bits(X), synth.bits(ws[0]), synth.bits(rs[0]), threads=7)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_points_match_full(oracle_lib):
    X, ws, rs = synth.make_inputs(5, 64, 128, seed=13)
    Xb, Wb, Rb = synth.bits(X), synth.bits(ws[0]), synth.bits(rs[0])
    Y, A = oracle_lib.addmm_bf16(Xb, Wb, Rb)
    rng = np.random.default_rng(0)
    ms = rng.integers(0, 5, 50)
    ns = rng.integers(0, 64, 50)
    y, a = oracle_lib.addmm_bf16_points(Xb, Wb, Rb, ms, ns)
    assert np.array_equal(y, Y[ms, ns]) and np.array_equal(a, A[ms, ns])


def test_empty_shapes(oracle_lib):
    z = np.zeros((0, 8), dtype=np.uint16)
    Y, A = oracle_lib.addmm_bf16(z, np.zeros((4, 8), np.uint16), np.zeros((0, 4), np.uint16))
    assert Y.shape == (0, 4)
    # K = 0: the sum is empty and Y = R
    R = synth.bits(synth.make_inputs(2, 3, 1)[2][0])
    Y, A = oracle_lib.addmm_bf16(np.zeros((2, 0), np.uint16), np.zeros((3, 0), np.uint16), R)
    assert np.array_equal(Y, R)


def test_points_reject_out_of_range(oracle_lib):
    X = np.zeros((2, 8), np.uint16)
    with pytest.raises(ValueError):
        oracle_lib.addmm_bf16_points(X, np.zeros((3, 8), np.uint16), np.zeros((2, 3), np.uint16), [2], [0])
