"""TEST INFRASTRUCTURE ONLY -- the CPU oracle for Y = X * W^T + R.

Plain fp64 definition of the skinny residual GEMM (bf16 X[M,K], W[N,K],
R[M,N]; one round-to-nearest-even to bf16), written from the vLLM benchmark
page "benchmarks/kernels/benchmark_k3_cutedsl_residual.py" (module docstring
and its torch.addmm leg), plus the shard epilogue of the vLLM API page
"fused_add_multicast_skinny_gemm" behind two flags. The arithmetic lives in
``oracle.c``; this module only builds it with gcc and marshals numpy arrays.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It shares no code with the GPU library
and imports nothing from it.

Arrays of bf16 are passed as ``numpy.uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_KBIT_SRC = os.path.join(_HERE, "kbit.c")
_KDA_SRC = os.path.join(_HERE, "kda.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_default = None

# Epilogue options of the page-2 shard form (the vLLM API page
# "fused_add_multicast_skinny_gemm"): round the product sum to bf16 before adding the
# residual (two roundings), and write +0 for a -0 result.
ROUND_PRODUCT = 1
NO_NEG_ZERO = 2


def build(force: bool = True, src: str = _SRC, out: str = _LIB, kbit_src: str = _KBIT_SRC,
          kda_src: str = _KDA_SRC) -> str:
    """Compile oracle.c, kbit.c and kda.c into one shared library (plain gcc: no fast-math,
    no FMA contraction). A test may pass its own copy of any source."""
    if not force and os.path.exists(out):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-pthread", src, kbit_src, kda_src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _u16(a, shape=None) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("bf16 operands are passed as uint16 bit patterns, got %s" % a.dtype)
    if shape is not None and a.shape != tuple(shape):
        raise ValueError("expected shape %s, got %s" % (tuple(shape), a.shape))
    return a


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


class Oracle:
    """ctypes view of one build of oracle.c (the default build, or a test's own build)."""

    def __init__(self, path: str = _LIB):
        lib = ctypes.CDLL(path)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        f64p = ctypes.POINTER(ctypes.c_double)
        i64p = ctypes.POINTER(ctypes.c_int64)
        i64 = ctypes.c_int64
        u32 = ctypes.c_uint
        lib.oracle_addmm_bf16_ex.argtypes = [u16p, u16p, u16p, u16p, f64p, i64, i64, i64, u32, ctypes.c_int]
        lib.oracle_addmm_bf16_ex.restype = ctypes.c_int
        lib.oracle_addmm_bf16_points_ex.argtypes = [u16p, u16p, u16p, i64, i64, i64, i64p, i64p, i64,
                                                    u32, u16p, f64p]
        lib.oracle_addmm_bf16_points_ex.restype = ctypes.c_int
        lib.oracle_round_bf16_array.argtypes = [f64p, u16p, i64]
        lib.oracle_round_bf16_array.restype = None
        u8p = ctypes.POINTER(ctypes.c_uint8)
        u32p = ctypes.POINTER(ctypes.c_uint32)
        f32p = ctypes.POINTER(ctypes.c_float)
        lib.oracle_e4m4_decode.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m4_decode.restype = ctypes.c_double
        lib.oracle_e4m4_encode.argtypes = [ctypes.c_double]
        lib.oracle_e4m4_encode.restype = ctypes.c_uint8
        lib.oracle_nf_codebook.argtypes = [ctypes.c_int, f64p]
        lib.oracle_nf_codebook.restype = ctypes.c_int
        lib.oracle_kbit_quantize.argtypes = [f64p, i64, ctypes.c_int, f32p, u32p, u8p, f64p]
        lib.oracle_kbit_quantize.restype = ctypes.c_int
        lib.oracle_kbit_dequant.argtypes = [u32p, u8p, f32p, ctypes.c_int, i64, f64p]
        lib.oracle_kbit_dequant.restype = ctypes.c_int
        lib.oracle_kbit_gemv_bf16.argtypes = [u16p, u32p, u8p, f32p, ctypes.c_int, u16p, u16p, f64p,
                                              i64, i64, i64]
        lib.oracle_kbit_gemv_bf16.restype = ctypes.c_int
        i32p = ctypes.POINTER(ctypes.c_int32)
        lib.oracle_kda_verify.argtypes = [i64] * 9 + [ctypes.c_double] + [u16p, u16p, u16p, u16p, i32p, i32p, u16p,
                                                                         u16p, f32p, f32p, f32p, i32p, u16p, f64p,
                                                                         u16p, u16p, f64p, f64p, u16p, f64p, f64p]
        lib.oracle_kda_verify.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    # ---------------------------------------------------------------- KDA chain verify

    def kda_verify(self, inp: dict, T: int, H: int, HV: int, K: int, V: int, scale: float,
                   snapshots: bool = True, ring_len: int = 0) -> dict:
        """One KDA verify step (kda.c) on the page's tensors, given as numpy arrays under the
        page's names: bf16 bit patterns (uint16) for mixed [B*T, dim], w [dim, 4], bias [dim],
        conv_pool [lines, 3, dim], a [B*T, HV*K], b [B*T, HV]; float32 A_log [HV],
        dt_bias [HV*K], ssm [slots, HV, V, K]; int32 cache_indices and inter_indices [B].
        Optional starting contents of the outputs: win_pool [lines, T, 3, dim] (uint16),
        inter_ssm [lines, T, HV, V, K], rawv [slots, HV, R, V], rawk [slots, H, R, K]
        (uint16), g [slots, HV, R, K], beta [slots, HV, R] (float64); absent ones start at 0.
        Returns those outputs (snapshot ones if snapshots, ring ones if ring_len) plus o (bf16
        bits [B*T, HV, V]), o_exact and conv_exact (float64, before their bf16 rounding)."""
        c = lambda k, dt: np.ascontiguousarray(inp[k], dtype=dt)
        mixed, w, bias, pool = (c(k, np.uint16) for k in ("mixed", "w", "bias", "conv_pool"))
        a, b = c("a", np.uint16), c("b", np.uint16)
        A_log, dt_bias, ssm = c("A_log", np.float32), c("dt_bias", np.float32), c("ssm", np.float32)
        cidx, iidx = c("cache_indices", np.int32), c("inter_indices", np.int32)
        B = cidx.shape[0]
        dim = 2 * H * K + HV * V
        lines, slots = pool.shape[0], ssm.shape[0]
        if mixed.shape != (B * T, dim) or w.shape != (dim, 4) or pool.shape[1:] != (3, dim):
            raise ValueError("bad conv shapes")
        if ssm.shape[1:] != (HV, V, K) or a.shape != (B * T, HV * K) or b.shape != (B * T, HV):
            raise ValueError("bad recurrence shapes")
        def start(k, shape, dt):
            if k in inp and inp[k] is not None:
                return np.array(inp[k], dtype=dt, copy=True).reshape(shape)
            return np.zeros(shape, dtype=dt)
        res = {"win_pool": start("win_pool", (lines, T, 3, dim), np.uint16)}
        if snapshots:
            res["inter_ssm"] = start("inter_ssm", (lines, T, HV, V, K), np.float64)
        if ring_len:
            res["rawv"] = start("rawv", (slots, HV, ring_len, V), np.uint16)
            res["rawk"] = start("rawk", (slots, H, ring_len, K), np.uint16)
            res["g"] = start("g", (slots, HV, ring_len, K), np.float64)
            res["beta"] = start("beta", (slots, HV, ring_len), np.float64)
        res["o"] = np.zeros((B * T, HV, V), dtype=np.uint16)
        res["o_exact"] = np.zeros((B * T, HV, V), dtype=np.float64)
        res["conv_exact"] = np.zeros((B * T, dim), dtype=np.float64)
        P = lambda k, ct: _ptr(res[k], ct) if k in res else None
        u16, f64, f32, i32 = ctypes.c_uint16, ctypes.c_double, ctypes.c_float, ctypes.c_int32
        rc = self.lib.oracle_kda_verify(B, T, H, HV, K, V, lines, slots, ring_len, float(scale),
                                        _ptr(mixed, u16), _ptr(w, u16), _ptr(bias, u16), _ptr(pool, u16),
                                        _ptr(cidx, i32), _ptr(iidx, i32), _ptr(a, u16), _ptr(b, u16),
                                        _ptr(A_log, f32), _ptr(dt_bias, f32), _ptr(ssm, f32), _ptr(cidx, i32),
                                        P("win_pool", u16), P("inter_ssm", f64), P("rawv", u16), P("rawk", u16),
                                        P("g", f64), P("beta", f64), P("o", u16), P("o_exact", f64),
                                        P("conv_exact", f64))
        if rc != 0:
            raise ValueError("oracle_kda_verify: bad arguments (%d)" % rc)
        return res

    # ---------------------------------------------------------------- k-bit quantized GEMV

    def e4m4_decode(self, codes) -> np.ndarray:
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        return np.array([self.lib.oracle_e4m4_decode(int(c)) for c in codes.reshape(-1)],
                        dtype=np.float64).reshape(codes.shape)

    def e4m4_encode(self, values) -> np.ndarray:
        values = np.ascontiguousarray(values, dtype=np.float64)
        return np.array([self.lib.oracle_e4m4_encode(float(v)) for v in values.reshape(-1)],
                        dtype=np.uint8).reshape(values.shape)

    def nf_codebook(self, k: int) -> np.ndarray:
        cb = np.empty(1 << k, dtype=np.float64)
        if self.lib.oracle_nf_codebook(int(k), _ptr(cb, ctypes.c_double)) != 0:
            raise ValueError("bad k")
        return cb

    def kbit_quantize(self, W, k: int, cb):
        """W float64 [N, K] (K % 32 == 0) -> (planes uint32 [N, K/32, k], absmax E4M4 uint8
        [N, K/32], unencoded absmax float64 [N, K/32])."""
        W = np.ascontiguousarray(W, dtype=np.float64)
        cb = np.ascontiguousarray(cb, dtype=np.float32)
        N, K = W.shape
        planes = np.empty((N, K // 32, k), dtype=np.uint32)
        amax = np.empty((N, K // 32), dtype=np.uint8)
        raw = np.empty((N, K // 32), dtype=np.float64)
        rc = self.lib.oracle_kbit_quantize(_ptr(W, ctypes.c_double), W.size, int(k), _ptr(cb, ctypes.c_float),
                                           _ptr(planes, ctypes.c_uint32), _ptr(amax, ctypes.c_uint8),
                                           _ptr(raw, ctypes.c_double))
        if rc != 0:
            raise ValueError("oracle_kbit_quantize: bad arguments")
        return planes, amax, raw

    def kbit_dequant(self, planes, absmax, cb, k: int) -> np.ndarray:
        planes = np.ascontiguousarray(planes, dtype=np.uint32)
        absmax = np.ascontiguousarray(absmax, dtype=np.uint8)
        cb = np.ascontiguousarray(cb, dtype=np.float32)
        N, B = absmax.shape
        out = np.empty((N, B * 32), dtype=np.float64)
        rc = self.lib.oracle_kbit_dequant(_ptr(planes, ctypes.c_uint32), _ptr(absmax, ctypes.c_uint8),
                                          _ptr(cb, ctypes.c_float), int(k), out.size, _ptr(out, ctypes.c_double))
        if rc != 0:
            raise ValueError("oracle_kbit_dequant: bad arguments")
        return out

    def kbit_gemv_bf16(self, X, planes, absmax, cb, k: int, R):
        """Y = bf16(X @ What^T + R) with What the dequantized k-bit weights: (Y bits, exact sums)."""
        X = _u16(X)
        planes = np.ascontiguousarray(planes, dtype=np.uint32)
        absmax = np.ascontiguousarray(absmax, dtype=np.uint8)
        cb = np.ascontiguousarray(cb, dtype=np.float32)
        M, K = X.shape
        N = absmax.shape[0]
        if absmax.shape != (N, K // 32) or planes.shape != (N, K // 32, k):
            raise ValueError("planes [N, K/32, k] and absmax [N, K/32] expected")
        R = _u16(R, (M, N))
        Y = np.empty((M, N), dtype=np.uint16)
        ACC = np.empty((M, N), dtype=np.float64)
        rc = self.lib.oracle_kbit_gemv_bf16(_ptr(X, ctypes.c_uint16), _ptr(planes, ctypes.c_uint32),
                                            _ptr(absmax, ctypes.c_uint8), _ptr(cb, ctypes.c_float), int(k),
                                            _ptr(R, ctypes.c_uint16), _ptr(Y, ctypes.c_uint16),
                                            _ptr(ACC, ctypes.c_double), M, N, K)
        if rc != 0:
            raise ValueError("oracle_kbit_gemv_bf16: bad arguments")
        return Y, ACC

    def addmm_bf16(self, X, W, R, threads: int | None = None, want_acc: bool = True, flags: int = 0):
        """Return (Y bits uint16[M,N], exact fp64 sums float64[M,N] or None). flags: ROUND_PRODUCT
        and/or NO_NEG_ZERO (the page-2 epilogue); with ROUND_PRODUCT the second array holds
        bf16(sum) + r, the value of the second rounding."""
        X = _u16(X)
        W = _u16(W)
        if X.ndim != 2 or W.ndim != 2 or X.shape[1] != W.shape[1]:
            raise ValueError("X must be [M,K] and W [N,K]")
        M, K = X.shape
        N = W.shape[0]
        R = _u16(R, (M, N))
        Y = np.empty((M, N), dtype=np.uint16)
        ACC = np.empty((M, N), dtype=np.float64) if want_acc else None
        rc = self.lib.oracle_addmm_bf16_ex(_ptr(X, ctypes.c_uint16), _ptr(W, ctypes.c_uint16),
                                           _ptr(R, ctypes.c_uint16), _ptr(Y, ctypes.c_uint16),
                                           _ptr(ACC, ctypes.c_double) if ACC is not None else None,
                                           M, N, K, int(flags), int(threads or default_threads()))
        if rc != 0:
            raise RuntimeError("oracle_addmm_bf16 failed (%d)" % rc)
        return Y, ACC

    def addmm_bf16_points(self, X, W, R, ms, ns, flags: int = 0):
        """Oracle values at the listed (m, n): (Y bits uint16[c], fp64 sums float64[c])."""
        X = _u16(X)
        W = _u16(W)
        M, K = X.shape
        N = W.shape[0]
        R = _u16(R, (M, N))
        ms = np.ascontiguousarray(ms, dtype=np.int64)
        ns = np.ascontiguousarray(ns, dtype=np.int64)
        if ms.shape != ns.shape or ms.ndim != 1:
            raise ValueError("ms and ns must be 1-D and of equal length")
        c = ms.shape[0]
        Y = np.empty(c, dtype=np.uint16)
        ACC = np.empty(c, dtype=np.float64)
        rc = self.lib.oracle_addmm_bf16_points_ex(_ptr(X, ctypes.c_uint16), _ptr(W, ctypes.c_uint16),
                                                  _ptr(R, ctypes.c_uint16), M, N, K,
                                                  _ptr(ms, ctypes.c_int64), _ptr(ns, ctypes.c_int64), c,
                                                  int(flags), _ptr(Y, ctypes.c_uint16),
                                                  _ptr(ACC, ctypes.c_double))
        if rc != 0:
            raise ValueError("point index out of range")
        return Y, ACC

    def round_bf16(self, v) -> np.ndarray:
        """The oracle's rounding step, elementwise: float64 -> bf16 bits."""
        v = np.ascontiguousarray(v, dtype=np.float64)
        out = np.empty(v.shape, dtype=np.uint16)
        self.lib.oracle_round_bf16_array(_ptr(v, ctypes.c_double), _ptr(out, ctypes.c_uint16), v.size)
        return out


def default() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(_LIB):
            build()
        _default = Oracle(_LIB)
    return _default


def addmm_bf16(X, W, R, threads: int | None = None, want_acc: bool = True, flags: int = 0):
    return default().addmm_bf16(X, W, R, threads=threads, want_acc=want_acc, flags=flags)


def addmm_bf16_points(X, W, R, ms, ns, flags: int = 0):
    return default().addmm_bf16_points(X, W, R, ms, ns, flags=flags)


def round_bf16(v) -> np.ndarray:
    return default().round_bf16(v)


def source_path() -> str:
    return _SRC


def bf16_bits_to_f64(b) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64 (bits << 16 read as binary32)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def nf_codebook(k: int) -> np.ndarray:
    return default().nf_codebook(k)


def e4m4_decode(codes) -> np.ndarray:
    return default().e4m4_decode(codes)


def e4m4_encode(values) -> np.ndarray:
    return default().e4m4_encode(values)


def kbit_quantize(W, k: int, cb):
    return default().kbit_quantize(W, k, cb)


def kbit_dequant(planes, absmax, cb, k: int) -> np.ndarray:
    return default().kbit_dequant(planes, absmax, cb, k)


def kbit_gemv_bf16(X, planes, absmax, cb, k: int, R):
    return default().kbit_gemv_bf16(X, planes, absmax, cb, k, R)


def kda_verify(inp: dict, T: int, H: int, HV: int, K: int, V: int, scale: float, snapshots: bool = True,
               ring_len: int = 0) -> dict:
    return default().kda_verify(inp, T, H, HV, K, V, scale, snapshots=snapshots, ring_len=ring_len)
