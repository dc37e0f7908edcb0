"""Pins for the k-bit quantized GEMV part of the CPU oracle (oracle/kbit.c).

Each pin takes an ``oracle.Oracle`` handle and raises AssertionError on a mismatch; they run
on the real oracle (tests/test_oracle_kbit.py) and on planted-mistake copies of kbit.c
(tests/test_oracle_kbit_mutants.py). What fixes the expected values, never the oracle itself:

  * the bitsandbytes page ("compare/main...QLORA-2.diff", agents/kbit_gemm_context.md):
    the E4M4 decoder written as IEEE-754 bit construction (section 1.5), its stated range
    (about 6.1e-5 .. 31) and relative step (1/16), the error budget and the SQNR floors of
    section 12;
  * mathematics: the codebook levels recomputed by numerical integration of z*pdf(z) over
    equiprobable bins found by bisection on erfc; symmetry of N(0,1);
  * exhaustive search over the 256 E4M4 codes;
  * the bit-plane layout unpacked with numpy shifts, exact Fraction sums, numpy fp64 matmul.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import torch

from oracle_pins import rne_by_enumeration

KS = (2, 3, 4, 5)


# ---------------------------------------------------------------- independent helpers

def e4m4_by_bits(codes) -> np.ndarray:
    """The page's decoder: for e > 0 the fp32 bit pattern (e - 11 + 127) << 23 | m << 19;
    for e == 0, m * 2^(1 - 11 - 4); 0 -> 0."""
    codes = np.asarray(codes, dtype=np.uint32)
    e = codes >> 4
    m = codes & 15
    bits = ((e.astype(np.int64) - 11 + 127).clip(0) << 23) | (m.astype(np.int64) << 19)
    normal = bits.astype(np.uint32).view(np.float32).astype(np.float64)
    sub = m.astype(np.float64) * 2.0 ** (1 - 11 - 4)
    return np.where(e > 0, normal, sub)


def _phi_inv(p: float) -> float:
    lo, hi = -40.0, 40.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if 0.5 * math.erfc(-mid / math.sqrt(2.0)) < p:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def codebook_by_integration(k: int) -> np.ndarray:
    """Centroids of 2^k equiprobable bins of N(0,1) by Simpson integration of z*pdf(z),
    scaled so that the largest magnitude is 1."""
    L = 1 << k
    edges = [-12.0] + [_phi_inv(i / L) for i in range(1, L)] + [12.0]
    out = []
    for i in range(L):
        a, b = edges[i], edges[i + 1]
        n = 4000
        z = np.linspace(a, b, n + 1)
        f = z * np.exp(-0.5 * z * z) / math.sqrt(2 * math.pi)
        h = (b - a) / n
        integral = h / 3 * (f[0] + f[-1] + 4 * f[1:-1:2].sum() + 2 * f[2:-1:2].sum())
        out.append(integral * L)
    out = np.array(out)
    return out / np.abs(out).max()


def unpack_indices(planes: np.ndarray, k: int) -> np.ndarray:
    """planes [..., B, k] uint32 -> indices [..., B*32]: bit j of word b is bit b of element j."""
    j = np.arange(32, dtype=np.uint32)
    bits = (planes[..., :, :, None] >> j) & 1            # [..., B, k, 32]
    weights = (1 << np.arange(k, dtype=np.uint32))[:, None]
    idx = (bits * weights).sum(axis=-2)                   # [..., B, 32]
    return idx.reshape(*planes.shape[:-2], planes.shape[-2] * 32)


def dequant_numpy(planes, absmax, cb, k) -> np.ndarray:
    idx = unpack_indices(np.asarray(planes, dtype=np.uint32), k)
    scale = np.repeat(e4m4_by_bits(absmax), 32, axis=-1)
    return np.asarray(cb, dtype=np.float32).astype(np.float64)[idx] * scale


def _nf32(orc, k):
    return orc.nf_codebook(k).astype(np.float32)


# ---------------------------------------------------------------- pins

def pin_e4m4_decode(orc):
    """All 256 codes against the page's bit-construction decoder and its stated range."""
    codes = np.arange(256, dtype=np.uint8)
    got = orc.e4m4_decode(codes)
    assert np.array_equal(got, e4m4_by_bits(codes))
    assert got[0] == 0.0
    assert abs(got[1] - 6.1e-5) < 1e-6          # smallest positive value, about 6.1e-5
    assert got[255] == 31.0                     # largest value
    assert got[0xB0] == 1.0                     # exponent 11 = the bias


def pin_e4m4_order_and_step(orc):
    """Strictly increasing in the code; relative step between normal neighbours <= 1/16."""
    v = orc.e4m4_decode(np.arange(256, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)
    normal = v[16:]
    assert np.all(np.diff(normal) / normal[:-1] <= 1.0 / 16 + 1e-15)


def pin_e4m4_encode_nearest(orc):
    """encode(decode(c)) = c; encode(v) is a nearest code (exhaustive search); midpoints
    between neighbours go to the even code; saturation above 31."""
    codes = np.arange(256, dtype=np.uint8)
    vals = e4m4_by_bits(codes)
    assert np.array_equal(orc.e4m4_encode(vals), codes)
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.uniform(0, 32, 3000), np.exp(rng.uniform(-12, 3.4, 3000))])
    enc = orc.e4m4_encode(v)
    dist = np.abs(vals[None, :] - v[:, None])
    assert np.allclose(np.abs(vals[enc] - v), dist.min(axis=1), rtol=0, atol=0)
    mids = 0.5 * (vals[1:] + vals[:-1])
    enc_m = orc.e4m4_encode(mids)
    assert np.all(enc_m % 2 == 0)
    assert np.all((enc_m == np.arange(255)) | (enc_m == np.arange(1, 256)))
    assert orc.e4m4_encode(np.array([40.0, 1e9]))[0] == 255


def pin_codebook(orc):
    """Sorted, symmetric, ends at -1 and +1, and equal to the integrated bin centroids."""
    for k in KS:
        cb = orc.nf_codebook(k)
        assert cb.shape == (1 << k,)
        assert np.all(np.diff(cb) > 0)
        assert cb[-1] == 1.0 and abs(cb[0] + 1.0) < 1e-12   # |max| = 1 (the lowest level by symmetry)
        assert np.allclose(cb, -cb[::-1], atol=1e-12)
        assert np.allclose(cb, codebook_by_integration(k), atol=2e-6), k


def pin_quantize_codebook_points(orc):
    """A block made of codebook values times a scale s (with +-s present) keeps its indices."""
    rng = np.random.default_rng(4)
    for k in KS:
        cb = _nf32(orc, k)
        idx = rng.integers(0, 1 << k, (6, 32 * 4))
        idx[:, ::32] = (1 << k) - 1                        # +1 * s in every block: absmax = s
        s = np.array([0.5, 1.0, 2.0, 3.0, 0.25, 7.0])[:, None]
        W = cb.astype(np.float64)[idx] * s
        planes, amax, raw = orc.kbit_quantize(W, k, cb)
        assert np.array_equal(unpack_indices(planes, k), idx), k
        assert np.allclose(raw, np.repeat(s, 4, axis=1))


def pin_quantize_ties_to_lower(orc):
    """An element exactly midway between two codebook entries takes the lower index (the
    page's search keeps the first best); the block's absmax is 1, so w / absmax is exact."""
    for k in KS:
        cb = _nf32(orc, k).astype(np.float64)
        L = 1 << k
        mids = 0.5 * (cb[1:] + cb[:-1])                    # exact in fp64
        row = np.zeros(32 * ((L - 1 + 31) // 32 + 1))
        row[0] = 1.0
        row[1:L] = mids
        planes, _, _ = orc.kbit_quantize(row[None, :], k, cb.astype(np.float32))
        idx = unpack_indices(planes, k)[0]
        assert idx[0] == L - 1
        assert np.array_equal(idx[1:L], np.arange(L - 1)), k


def pin_quantize_error_budget(orc):
    """The page's per-block budget: |w - dequant(quant(w))| <= (max_gap/2 + 1/16) absmax + eps."""
    rng = np.random.default_rng(5)
    W = rng.standard_normal((64, 32 * 64)) * np.exp(rng.uniform(-3, 2, (64, 1)))
    for k in KS:
        cb = _nf32(orc, k)
        planes, amax, raw = orc.kbit_quantize(W, k, cb)
        D = dequant_numpy(planes, amax, cb, k)
        gap = np.diff(cb.astype(np.float64)).max()
        bound = (gap / 2 + 1 / 16) * np.repeat(raw, 32, axis=1) + 1e-6
        assert np.all(np.abs(W - D) <= bound), k


def pin_quantize_sqnr(orc):
    """SQNR floors of the page (1M N(0,1) elements, E4M4 absmax): 5, 10, 15, 20 dB for k = 2..5."""
    rng = np.random.default_rng(6)
    W = rng.standard_normal((256, 4096))
    for k, floor in zip(KS, (5.0, 10.0, 15.0, 20.0)):
        cb = _nf32(orc, k)
        planes, amax, _ = orc.kbit_quantize(W, k, cb)
        D = dequant_numpy(planes, amax, cb, k)
        sqnr = 10 * np.log10((W ** 2).sum() / ((W - D) ** 2).sum())
        assert sqnr > floor, (k, sqnr)


def pin_dequant_layout(orc):
    """The oracle's dequantization equals the numpy unpacking of random planes and scales."""
    rng = np.random.default_rng(7)
    for k in KS:
        cb = _nf32(orc, k)
        planes = rng.integers(0, 2 ** 32, (5, 9, k), dtype=np.uint64).astype(np.uint32)
        amax = rng.integers(0, 256, (5, 9)).astype(np.uint8)
        assert np.array_equal(orc.kbit_dequant(planes, amax, cb, k), dequant_numpy(planes, amax, cb, k))


def _random_kbit(rng, M, N, K, k):
    X = torch.randn(M, K, generator=torch.Generator().manual_seed(int(rng.integers(1 << 30)))).to(torch.bfloat16)
    R = torch.randn(M, N, generator=torch.Generator().manual_seed(int(rng.integers(1 << 30)))).to(torch.bfloat16)
    planes = rng.integers(0, 2 ** 32, (N, K // 32, k), dtype=np.uint64).astype(np.uint32)
    amax = rng.integers(0x80, 0xC0, (N, K // 32)).astype(np.uint8)   # scales 1/8 .. 4
    Xb = X.view(torch.int16).numpy().view(np.uint16)
    Rb = R.view(torch.int16).numpy().view(np.uint16)
    return Xb, Rb, planes, amax


def _bits_to_f64(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def pin_kbit_gemv_x_zero(orc):
    """X = 0: Y = R bit for bit (up to the sign of zero)."""
    rng = np.random.default_rng(8)
    Xb, Rb, planes, amax = _random_kbit(rng, 3, 17, 96, 4)
    Y, ACC = orc.kbit_gemv_bf16(np.zeros_like(Xb), planes, amax, _nf32(orc, 4), 4, Rb)
    same = (Y == Rb) | (((Y & 0x7FFF) == 0) & ((Rb & 0x7FFF) == 0))
    assert same.all()
    assert np.array_equal(ACC, _bits_to_f64(Rb))


def pin_kbit_gemv_numpy(orc):
    """Exact sums against numpy fp64 (dequantized by the numpy route) within the fp64 bound,
    and the rounding against torch's."""
    rng = np.random.default_rng(9)
    for k in KS:
        M, N, K = 3, 40, 512
        Xb, Rb, planes, amax = _random_kbit(rng, M, N, K, k)
        cb = _nf32(orc, k)
        Wd = dequant_numpy(planes, amax, cb, k)
        x = _bits_to_f64(Xb)
        r = _bits_to_f64(Rb)
        ref = x @ Wd.T + r
        bound = (K + 2) * 2.0 ** -52 * (np.abs(x) @ np.abs(Wd).T + np.abs(r))
        Y, ACC = orc.kbit_gemv_bf16(Xb, planes, amax, cb, k, Rb)
        assert np.all(np.abs(ACC - ref) <= bound), k
        want = np.array([rne_by_enumeration(Fraction(v)) for v in ACC.reshape(-1)], dtype=np.uint16)
        assert np.array_equal(Y.reshape(-1), want), k


def pin_kbit_gemv_bruteforce(orc):
    """Tiny shapes: exact Fraction sums and rounding by enumeration of bf16 values."""
    rng = np.random.default_rng(10)
    for k in KS:
        M, N, K = 2, 3, 64
        Xb, Rb, planes, amax = _random_kbit(rng, M, N, K, k)
        cb = _nf32(orc, k)
        Wd = dequant_numpy(planes, amax, cb, k)
        x = _bits_to_f64(Xb)
        r = _bits_to_f64(Rb)
        Y, _ = orc.kbit_gemv_bf16(Xb, planes, amax, cb, k, Rb)
        for m in range(M):
            for n in range(N):
                exact = sum((Fraction(x[m, i]) * Fraction(Wd[n, i]) for i in range(K)), Fraction(r[m, n]))
                assert int(Y[m, n]) == rne_by_enumeration(exact), (k, m, n)


ALL_KBIT_PINS = [
    pin_e4m4_decode,
    pin_e4m4_order_and_step,
    pin_e4m4_encode_nearest,
    pin_codebook,
    pin_quantize_codebook_points,
    pin_quantize_ties_to_lower,
    pin_quantize_error_budget,
    pin_quantize_sqnr,
    pin_dequant_layout,
    pin_kbit_gemv_x_zero,
    pin_kbit_gemv_numpy,
    pin_kbit_gemv_bruteforce,
]
