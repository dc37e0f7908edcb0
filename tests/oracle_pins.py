"""Pins for the CPU oracle: checks against facts that the oracle does not itself define.

Each pin takes an ``oracle.Oracle`` handle and raises AssertionError on a mismatch.
They are used twice: on the real oracle (tests/test_oracle.py), and on deliberately
broken copies of oracle.c (tests/test_oracle_mutants.py), where at least one pin
must fail for every planted mistake.

What fixes the expected values (never the oracle itself):
  * bf16 rounding: the list of all finite bf16 values, exact rational arithmetic,
    and torch's fp32 -> bf16 conversion (a library routine);
  * closed forms: X = 0 gives R; one-hot W rows select columns of X; integer inputs
    have integer sums that fp32 and fp64 hold exactly;
  * brute force: exact Fraction sums on tiny shapes;
  * numpy's fp64 matmul (within its error bound) on a mid-sized problem;
  * exact invariants (permuting K, scaling X by a power of two);
  * hand-derived single-element cases in tests/golden/closed_form_cases.txt, and for the
    shard epilogue (two roundings, -0 written as +0) in tests/golden/shard_epilogue_cases.txt;
  * integer rounding written out with Python integers (round half to even on 8 bits).
"""
from __future__ import annotations

import bisect
import os
from fractions import Fraction

import numpy as np
import torch

from decode_skinny_addmm_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "closed_form_cases.txt")
GOLDEN_SHARD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "shard_epilogue_cases.txt")
ROUND_PRODUCT, NO_NEG_ZERO = 1, 2   # the shard-epilogue flags of the oracle's *_ex entry points


# ---------------------------------------------------------------- independent helpers

def _bits_to_f64(b):
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


_POS = None


def _positive_bf16_table():
    """All finite non-negative bf16 values, ascending, with their bit patterns."""
    global _POS
    if _POS is None:
        bits = np.arange(0, 0x7F80, dtype=np.uint16)  # +0 .. largest finite
        _POS = ([Fraction(float(v)) for v in _bits_to_f64(bits)], [int(b) for b in bits])
    return _POS


def rne_by_enumeration(value: Fraction) -> int:
    """Nearest bf16 to an exact rational, ties to the even bit pattern, overflow to Inf."""
    vals, bits = _positive_bf16_table()
    sign = 0x8000 if value < 0 else 0
    a = -value if value < 0 else value
    top = vals[-1]
    half_ulp_top = Fraction(2) ** 119
    if a > top:
        # ties at top + half ulp go to the even neighbour, which is 2^128 -> Inf (0x7F7F is odd)
        return sign | (0x7F80 if a >= top + half_ulp_top else 0x7F7F)
    i = bisect.bisect_left(vals, a)
    if vals[i] == a:
        return sign | bits[i]
    lo, hi = i - 1, i
    dlo, dhi = a - vals[lo], vals[hi] - a
    if dlo < dhi:
        pick = lo
    elif dhi < dlo:
        pick = hi
    else:
        pick = lo if bits[lo] % 2 == 0 else hi
    return sign | bits[pick]


def torch_rne_from_f64(v: np.ndarray) -> np.ndarray:
    """Library rounding: float64 values that are exact in fp32 -> bf16 bits via torch."""
    f32 = v.astype(np.float32)
    assert np.array_equal(f32.astype(np.float64), v), "value not exact in fp32"
    t = torch.from_numpy(f32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _ub(t):
    return synth.bits(t)


def _same_bits_allow_signed_zero(a, b):
    a = np.asarray(a, dtype=np.uint16)
    b = np.asarray(b, dtype=np.uint16)
    za = (a & 0x7FFF) == 0
    zb = (b & 0x7FFF) == 0
    return bool(np.all((a == b) | (za & zb)))


# ---------------------------------------------------------------- pins

def pin_rounding_enumeration(orc):
    """Oracle rounding == nearest-even choice over the enumerated bf16 values."""
    rng = np.random.default_rng(1)
    vals = [0.0, -0.0, 1.0, 1 + 2**-8, 1 + 3 * 2**-8, 2.0**-133, 1.5 * 2.0**-133, 2.0**-134,
            2.0**-127 * 1.25, 3.3e38, 3.4e38, -3.39e38, 65504.5, 1e-39, -1e-40]
    vals += list(rng.standard_normal(300) * np.exp2(rng.integers(-140, 128, 300)))
    # exact midpoints between neighbouring bf16 values (the tie cases)
    b = rng.integers(0, 0x7F7F, 200).astype(np.uint16)
    lo = _bits_to_f64(b)
    hi = _bits_to_f64(b + 1)
    vals += list((lo + hi) / 2)
    vals += list(-(lo + hi) / 2)
    v = np.array(vals, dtype=np.float64)
    got = orc.round_bf16(v)
    want = np.array([(0x8000 if np.signbit(x) else 0) if x == 0 else rne_by_enumeration(Fraction(float(x)))
                     for x in v], dtype=np.uint16)
    # a zero keeps its sign
    assert np.array_equal(got, want), "rounding differs at %s" % v[got != want][:5]


def pin_rounding_vs_torch(orc):
    """For fp32-representable values the oracle rounds exactly as torch's fp32->bf16."""
    rng = np.random.default_rng(2)
    f = (rng.standard_normal(20000) * np.exp2(rng.integers(-60, 60, 20000))).astype(np.float32)
    v = f.astype(np.float64)
    assert np.array_equal(orc.round_bf16(v), torch_rne_from_f64(v))


def pin_golden_cases(orc):
    """Hand-derived single-element cases (tests/golden/closed_form_cases.txt)."""
    n_cases = 0
    with open(GOLDEN) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, xs, ws, r, want = [p.strip() for p in line.split("|")]
            x = np.array([float.fromhex(t) for t in xs.split()], dtype=np.float64)
            w = np.array([float.fromhex(t) for t in ws.split()], dtype=np.float64)
            assert x.shape == w.shape
            K = x.shape[0]
            X = _ub(torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(1, K))
            W = _ub(torch.from_numpy(w.astype(np.float32)).to(torch.bfloat16).view(1, K))
            R = _ub(torch.tensor([[float.fromhex(r)]], dtype=torch.float32).to(torch.bfloat16))
            # the fixture values are bf16 values by construction
            assert np.array_equal(_bits_to_f64(X)[0], x) and np.array_equal(_bits_to_f64(W)[0], w), name
            Y, _ = orc.addmm_bf16(X, W, R, threads=1)
            assert int(Y[0, 0]) == int(want, 16), "%s: got %04X want %s" % (name, Y[0, 0], want)
            n_cases += 1
    assert n_cases >= 10


def pin_x_zero_gives_r(orc):
    """X = 0 => Y = R bit-exactly (zeros compared without their sign)."""
    M, N, K = 3, 40, 72
    _, ws, rs = synth.make_inputs(M, N, K)
    X = np.zeros((M, K), dtype=np.uint16)
    R = _ub(rs[0])
    Y, ACC = orc.addmm_bf16(X, _ub(ws[0]), R, threads=2)
    assert _same_bits_allow_signed_zero(Y, R)
    assert np.array_equal(ACC, _bits_to_f64(R))


def pin_one_hot_rows(orc):
    """W[n,:] = e_{j(n)} => Y[m,n] = RNE(x[m,j(n)] + r[m,n]) (rounded by torch)."""
    M, N, K = 5, 48, 64
    X, _, rs = synth.make_inputs(M, N, K, seed=11)
    cols = (np.arange(N) * 7 + 3) % K
    W = synth.one_hot_rows(N, K, cols)
    Xb, Rb = _ub(X), _ub(rs[0])
    Y, ACC = orc.addmm_bf16(Xb, _ub(W), Rb, threads=3)
    exact = _bits_to_f64(Xb)[:, cols] + _bits_to_f64(Rb)  # exact in fp64 (and in fp32 here)
    assert np.array_equal(ACC, exact)
    assert np.array_equal(Y, torch_rne_from_f64(exact))


def pin_small_integers(orc):
    """Integer inputs: exact integer sums; Y = RNE of the integer (ties included)."""
    M, N, K = 4, 37, 3584
    X, W, R = synth.small_int_inputs(M, N, K)
    xi = X.to(torch.int64).numpy()
    wi = W.to(torch.int64).numpy()
    ri = R.to(torch.int64).numpy()
    closed = xi @ wi.T + ri  # integer arithmetic, exact
    Y, ACC = orc.addmm_bf16(_ub(X), _ub(W), _ub(R), threads=4)
    assert np.array_equal(ACC, closed.astype(np.float64))
    assert np.abs(closed).max() < 2**24
    assert np.array_equal(Y, torch_rne_from_f64(closed.astype(np.float64)))
    # the case must exercise bf16 rounding, ties included
    big = np.abs(closed) > 256
    assert big.any()
    ties = big & (np.abs(closed) % 2 == 1) & (np.abs(closed) < 512)
    assert ties.any(), "no rounding ties in the integer case"


def pin_bruteforce_fraction(orc):
    """Tiny shapes with mixed magnitudes: exact Fraction sums and enumerated rounding."""
    rng = np.random.default_rng(5)
    for (M, N, K) in [(1, 1, 1), (2, 3, 5), (3, 4, 17), (4, 2, 32), (1, 5, 8)]:
        mag_x = np.exp2(rng.integers(-20, 20, (M, K))).astype(np.float32)
        mag_w = np.exp2(rng.integers(-20, 20, (N, K))).astype(np.float32)
        x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32) * mag_x).to(torch.bfloat16)
        w = torch.from_numpy(rng.standard_normal((N, K)).astype(np.float32) * mag_w).to(torch.bfloat16)
        r = torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32)).to(torch.bfloat16)
        Xb, Wb, Rb = _ub(x), _ub(w), _ub(r)
        Y, ACC = orc.addmm_bf16(Xb, Wb, Rb, threads=1)
        xf, wf, rf = _bits_to_f64(Xb), _bits_to_f64(Wb), _bits_to_f64(Rb)
        for m in range(M):
            for n in range(N):
                ex = sum(Fraction(float(xf[m, k])) * Fraction(float(wf[n, k])) for k in range(K))
                ex += Fraction(float(rf[m, n]))
                want = rne_by_enumeration(ex)
                assert int(Y[m, n]) == want, (M, N, K, m, n)
                # compensated fp64 sum: within a few fp64 ulps of the exact value
                assert abs(Fraction(float(ACC[m, n])) - ex) <= abs(ex) * Fraction(1, 2**50) + Fraction(1, 2**200)


def pin_numpy_matmul(orc):
    """Random workload at full K: ACC agrees with numpy's fp64 X @ W^T + R within its bound."""
    M, N, K = 4, 96, 3584
    X, ws, rs = synth.make_inputs(M, N, K)
    Xb, Wb, Rb = _ub(X), _ub(ws[0]), _ub(rs[0])
    Y, ACC = orc.addmm_bf16(Xb, Wb, Rb, threads=4)
    xf, wf, rf = _bits_to_f64(Xb), _bits_to_f64(Wb), _bits_to_f64(Rb)
    ref = xf @ wf.T + rf
    S = np.abs(xf) @ np.abs(wf).T + np.abs(rf)
    # fp64 dot product error bound, K * 2^-53 * sum|terms| (generous, any summation order)
    assert np.all(np.abs(ACC - ref) <= (K + 2) * 2.0**-53 * S)
    # and the sums are not trivially small: the products matter
    assert np.abs(xf @ wf.T).mean() > 0.3


def pin_permute_k(orc):
    """Permuting the K columns of X and W together leaves the result unchanged."""
    M, N, K = 3, 24, 512
    X, ws, rs = synth.make_inputs(M, N, K, seed=3)
    perm = np.random.default_rng(9).permutation(K)
    Xb, Wb, Rb = _ub(X), _ub(ws[0]), _ub(rs[0])
    Y1, A1 = orc.addmm_bf16(Xb, Wb, Rb, threads=2)
    Y2, A2 = orc.addmm_bf16(Xb[:, perm], Wb[:, perm], Rb, threads=2)
    assert np.array_equal(Y1, Y2)
    S = np.abs(_bits_to_f64(Xb)) @ np.abs(_bits_to_f64(Wb)).T
    assert np.all(np.abs(A1 - A2) <= 2.0**-50 * S)
    # a permutation of X alone does change it (the pin is not vacuous)
    _, A3 = orc.addmm_bf16(Xb[:, perm], Wb, Rb, threads=2)
    assert not np.allclose(A1, A3)


def pin_scale_x(orc):
    """With R = 0, scaling X by 2^3 scales every exact sum by 8 and every output exponent by 3."""
    M, N, K = 2, 30, 256
    X, ws, _ = synth.make_inputs(M, N, K, seed=4)
    R = np.zeros((M, N), dtype=np.uint16)
    X8 = (X.float() * 8).to(torch.bfloat16)  # exact: power-of-two scale, no overflow
    Y1, A1 = orc.addmm_bf16(_ub(X), _ub(ws[0]), R, threads=1)
    Y2, A2 = orc.addmm_bf16(_ub(X8), _ub(ws[0]), R, threads=1)
    assert np.array_equal(A2, A1 * 8)
    nz = (Y1 & 0x7FFF) != 0
    assert np.array_equal(Y2[nz].astype(np.int32), Y1[nz].astype(np.int32) + (3 << 7))


def pin_rows_independent(orc):
    """Row m of the output depends only on row m of X and R (checked by recomputing one row alone)."""
    M, N, K = 4, 33, 200
    X, ws, rs = synth.make_inputs(M, N, K, seed=6)
    Xb, Wb, Rb = _ub(X), _ub(ws[0]), _ub(rs[0])
    Y, A = orc.addmm_bf16(Xb, Wb, Rb, threads=3)
    for m in range(M):
        Ym, Am = orc.addmm_bf16(Xb[m:m + 1], Wb, Rb[m:m + 1], threads=1)
        assert np.array_equal(Ym[0], Y[m]) and np.array_equal(Am[0], A[m])
    # W row n only affects column n
    W2 = Wb.copy()
    W2[5] = _ub(torch.ones(1, K, dtype=torch.bfloat16))[0]
    Y2, _ = orc.addmm_bf16(Xb, W2, Rb, threads=3)
    changed = np.any(Y2 != Y, axis=0)
    assert changed[5] and changed.sum() == 1


def rne_int_bf16(v: int) -> int:
    """Nearest bf16 value to an integer |v| < 2^24 (as an int), ties to even: the integers
    with 8 significant bits, written out with Python integer arithmetic."""
    v = int(v)
    a = abs(v)
    if a < 256:
        return v
    q = 1 << (a.bit_length() - 8)      # spacing of bf16 values in [2^e, 2^(e+1))
    n, rem = divmod(a, q)
    if 2 * rem > q or (2 * rem == q and n % 2 == 1):
        n += 1
    return (n * q) if v > 0 else -(n * q)


def pin_shard_golden_cases(orc):
    """Hand-derived cases of the shard epilogue (tests/golden/shard_epilogue_cases.txt)."""
    n_cases = 0
    with open(GOLDEN_SHARD) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, flags, xs, ws, r, want = [p.strip() for p in line.split("|")]
            x = np.array([float.fromhex(t) for t in xs.split()], dtype=np.float64)
            w = np.array([float.fromhex(t) for t in ws.split()], dtype=np.float64)
            K = x.shape[0]
            X = _ub(torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(1, K))
            W = _ub(torch.from_numpy(w.astype(np.float32)).to(torch.bfloat16).view(1, K))
            R = _ub(torch.tensor([[float.fromhex(r)]], dtype=torch.float32).to(torch.bfloat16))
            assert np.array_equal(_bits_to_f64(X)[0], x) and np.array_equal(_bits_to_f64(W)[0], w), name
            Y, _ = orc.addmm_bf16(X, W, R, threads=1, flags=int(flags))
            assert int(Y[0, 0]) == int(want, 16), "%s: got %04X want %s" % (name, Y[0, 0], want)
            n_cases += 1
    assert n_cases >= 10


def pin_round_product_small_integers(orc):
    """Integer inputs with the two-rounding epilogue: g = RNE(integer sum) and Y = RNE(g + r),
    both rounded by integer arithmetic; the second value the oracle reports is g + r."""
    M, N, K = 4, 37, 200
    X, W, R = synth.small_int_inputs(M, N, K, seed=9)
    X, W = X.abs(), W + 2              # x in {0, 1, 2}, w in {0, .., 4}: sums of ~500, exact
    xi = X.to(torch.int64).numpy()
    wi = W.to(torch.int64).numpy()
    ri = R.to(torch.int64).numpy()
    sums = xi @ wi.T
    g = np.vectorize(rne_int_bf16)(sums)
    want = np.vectorize(rne_int_bf16)(g + ri)
    Y, ACC = orc.addmm_bf16(_ub(X), _ub(W), _ub(R), threads=2, flags=ROUND_PRODUCT)
    assert np.array_equal(ACC, (g + ri).astype(np.float64))
    assert np.array_equal(_bits_to_f64(Y), want.astype(np.float64))
    # the case must separate two roundings from one
    assert np.any(np.vectorize(rne_int_bf16)(sums + ri) != want)


ALL_PINS = [
    pin_rounding_enumeration,
    pin_rounding_vs_torch,
    pin_golden_cases,
    pin_x_zero_gives_r,
    pin_one_hot_rows,
    pin_small_integers,
    pin_bruteforce_fraction,
    pin_numpy_matmul,
    pin_permute_k,
    pin_scale_x,
    pin_rows_independent,
    pin_shard_golden_cases,
    pin_round_product_small_integers,
]
