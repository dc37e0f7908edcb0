"""The parity rules of tests/parity.py reject corrupted results (CPU only): the oracle's output
for inputs with one flipped byte, compared as if it were the GPU's against the oracle's output
for the true inputs, must fail the check; the true output must pass it."""
import numpy as np
import pytest

import oracle
import parity as P
from decode_skinny_addmm_amd import synth


def test_flipped_weight_byte_is_caught():
    X, ws, rs = synth.make_inputs(4, 64, 256, seed=11)
    Xb, Wb, Rb = synth.bits(X), synth.bits(ws[0]), synth.bits(rs[0])
    y, exact = oracle.addmm_bf16(Xb, Wb, Rb)
    P.check_y(y, y, exact, "self")                      # the rule accepts the true result
    Wc = Wb.copy()
    Wc[17, 100] ^= 0x4000                               # flip an exponent bit of one weight
    yc, accc = oracle.addmm_bf16(Xb, Wc, Rb)
    with pytest.raises(AssertionError):
        P.check_y(yc, y, exact, "flipped W")
    with pytest.raises(AssertionError):
        P.check_acc(accc, exact, "flipped W")


def test_flipped_index_bit_is_caught():
    X, ps, As, rs, cb = synth.make_kbit_inputs(2, 48, 512, kbits=4, seed=3)
    Xb, Rb = synth.bits(X), synth.bits(rs[0])
    planes = ps[0].numpy().view(np.uint32).copy()
    y, exact = oracle.kbit_gemv_bf16(Xb, planes, As[0].numpy(), cb.numpy(), 4, Rb)
    P.check_y(y, y, exact, "self")
    planes[7, 3, 3] ^= 1 << 9                           # top index bit of one weight of row 7
    yc, accc = oracle.kbit_gemv_bf16(Xb, planes, As[0].numpy(), cb.numpy(), 4, Rb)
    with pytest.raises(AssertionError):
        P.check_acc(accc, exact, "flipped index bit")
