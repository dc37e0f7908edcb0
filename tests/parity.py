"""Comparison rules between the GPU library and the CPU oracle.

Tolerances (the operation fixes fp32 accumulation and a bf16 output; any fp32 summation
order is a correct one, so results are compared within bounds, never bit-for-bit on
random data):
  * Y: at most 2 bf16 ULP from the oracle's correctly rounded value wherever
    |Y_exact| >= TAU = 2^-12; below TAU (cancellation, where an fp32 sum's absolute
    error is comparable to a bf16 ULP) |Y - Y_exact| <= 2 * ulp_bf16(TAU) = 2^-18.
  * ACC (the fp32 value before rounding): |ACC - Y_exact| <= 1e-4 * max(|Y_exact|, 0.1),
    and Y must equal RNE_bf16(ACC) exactly (the epilogue is a single rounding). The floor is
    a tenth of the unit output scale: an fp32 sum's error follows the size of its partial
    sums (unit scale here; each rounding of one is up to 6e-8), not the size of the result,
    so below the floor the bar is 1e-5 absolute. That still sits 200x below one bf16
    rounding of a partial sum (2^-9) and 1700x below one dropped product.
Exact-input cases (X = 0, one-hot W rows, small integers) are compared bit-for-bit.
"""
from __future__ import annotations

import numpy as np
import torch

TAU = 2.0 ** -12
ABS_FLOOR = 2.0 ** -18
ACC_REL = 1e-4
ACC_FLOOR = 0.1

# M values at which the GPU tests compare every output of the full N = 7168, K = 3584 problem
# with the oracle at the selected configuration; together they reach every configuration the
# table selects there for M = 1 ... 300 (checked on the CPU in test_abi_host.py).
FULL_ORACLE_SMALL_M = [1, 2, 3, 4, 5, 8, 9, 16]
FULL_ORACLE_LARGE_M = [17, 26, 32, 33, 40, 41, 48, 49, 57, 64, 65, 80, 81, 88, 96, 97, 128, 129, 152, 160, 176, 192, 208, 256]


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16).copy()


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ordered(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> integers ordered like the values (+0 and -0 both map to 0)."""
    b = np.asarray(b, dtype=np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    return np.abs(ordered(a) - ordered(b))


def check_y(y_gpu_bits: np.ndarray, y_ref_bits: np.ndarray, exact: np.ndarray, what: str = "") -> dict:
    y_gpu_bits = np.asarray(y_gpu_bits).reshape(-1)
    y_ref_bits = np.asarray(y_ref_bits).reshape(-1)
    exact = np.asarray(exact, dtype=np.float64).reshape(-1)
    big = np.abs(exact) >= TAU
    d = ulp_distance(y_gpu_bits, y_ref_bits)
    absdiff = np.abs(bf16_to_f64(y_gpu_bits) - exact)
    ok = np.where(big, d <= 2, absdiff <= ABS_FLOOR)
    stats = {"n": int(exact.size), "max_ulp": int(d[big].max()) if big.any() else 0,
             "n_exact_match": int((d == 0).sum()), "n_floor_branch": int((~big).sum()),
             "max_abs_small": float(absdiff[~big].max()) if (~big).any() else 0.0}
    if not ok.all():
        i = int(np.flatnonzero(~ok)[0])
        raise AssertionError("%s: %d of %d outputs outside tolerance; first at flat index %d: gpu %04x ref %04x "
                             "exact %.9g (%s)" % (what, int((~ok).sum()), ok.size, i, y_gpu_bits[i],
                                                   y_ref_bits[i], exact[i], stats))
    return stats


def rne_torch(acc_f32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(acc_f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def check_acc(acc_gpu: np.ndarray, exact: np.ndarray, what: str = "") -> float:
    acc_gpu = np.asarray(acc_gpu, dtype=np.float64).reshape(-1)
    exact = np.asarray(exact, dtype=np.float64).reshape(-1)
    err = np.abs(acc_gpu - exact)
    lim = ACC_REL * np.maximum(np.abs(exact), ACC_FLOOR)
    bad = err > lim
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise AssertionError("%s: %d accumulator values outside 1e-4 relative; first at %d: gpu %.9g exact %.9g"
                             % (what, int(bad.sum()), i, acc_gpu[i], exact[i]))
    return float((err / np.maximum(np.abs(exact), ACC_FLOOR)).max()) if err.size else 0.0
