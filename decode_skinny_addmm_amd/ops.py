"""Python binding of the skinny residual GEMM: argument marshalling over the C ABI only.

Y = bf16(X @ W^T + R) for bf16 X[M,K], W[N,K], R[M,N] on the GPU; every step runs in the
HIP kernels of libskinny.so. torch supplies device memory and the current stream.
Argument errors raise ValueError before the library is called (as the launcher of the
vLLM API page "fused_add_multicast_skinny_gemm" does); library errors raise SkinnyError.
"""
from __future__ import annotations

import ctypes

import torch

from ._lib import (CONFIG_FIELDS, FLAG_NO_NEG_ZERO, FLAG_ROUND_PRODUCT, SkinnyConfig, SkinnyError,  # noqa: F401
                   SkinnyResources, check, lib)


def _as_config(cfg) -> SkinnyConfig | None:
    if cfg is None:
        return None
    if isinstance(cfg, SkinnyConfig):
        return cfg
    if isinstance(cfg, dict):
        vals = [int(cfg.get(f, 0)) for f in CONFIG_FIELDS]
    else:
        vals = [int(v) for v in cfg] + [0] * (len(CONFIG_FIELDS) - len(cfg))
    return SkinnyConfig(*vals)


def _check_operands(X, W, R, out, out_dtype):
    for name, t in (("X", X), ("W", W), ("R", R), ("out", out)):
        if not isinstance(t, torch.Tensor):
            raise ValueError("%s must be a torch.Tensor" % name)
        if t.device.type != "cuda":
            raise ValueError("%s must be on the GPU" % name)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous (row-major)" % name)
        if t.dim() != 2:
            raise ValueError("%s must be 2-D" % name)
    for name, t in (("X", X), ("W", W), ("R", R)):
        if t.dtype != torch.bfloat16:
            raise ValueError("%s must be bfloat16" % name)
    if out.dtype != out_dtype:
        raise ValueError("out must be %s" % out_dtype)
    M, K = X.shape
    N = W.shape[0]
    if W.shape[1] != K:
        raise ValueError("W must be [N, K] with K = X.shape[1] (got %s vs %s)" % (tuple(W.shape), tuple(X.shape)))
    if tuple(R.shape) != (M, N) or tuple(out.shape) != (M, N):
        raise ValueError("R and out must be [M, N] = [%d, %d]" % (M, N))
    devs = {t.device for t in (X, W, R, out)}
    if len(devs) != 1:
        raise ValueError("all operands must be on the same device")
    return M, N, K


def _stream_ptr(stream, device) -> int:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return int(s.cuda_stream)


def addmm(X: torch.Tensor, W: torch.Tensor, R: torch.Tensor, out: torch.Tensor | None = None,
          config=None, stream=None) -> torch.Tensor:
    """Y = bf16(X @ W^T + R) via skinny_addmm_bf16_with_config. `out` may be R (in place)."""
    if out is None:
        out = torch.empty_like(R)
    M, N, K = _check_operands(X, W, R, out, torch.bfloat16)
    c = _as_config(config)
    with torch.cuda.device(X.device):
        st = lib().skinny_addmm_bf16_with_config(X.data_ptr(), W.data_ptr(), R.data_ptr(), out.data_ptr(),
                                                 M, N, K, ctypes.byref(c) if c is not None else None,
                                                 _stream_ptr(stream, X.device))
    check(st, "skinny_addmm_bf16")
    return out


def addmm_default(X, W, R, out, stream=None) -> torch.Tensor:
    """The plain entry point skinny_addmm_bf16 (configuration chosen by the library)."""
    M, N, K = _check_operands(X, W, R, out, torch.bfloat16)
    with torch.cuda.device(X.device):
        st = lib().skinny_addmm_bf16(X.data_ptr(), W.data_ptr(), R.data_ptr(), out.data_ptr(), M, N, K,
                                     _stream_ptr(stream, X.device))
    check(st, "skinny_addmm_bf16")
    return out


def addmm_acc_f32(X, W, R, out: torch.Tensor | None = None, config=None, stream=None) -> torch.Tensor:
    """fp32 value before rounding, fp32(sum) + fp32(R), from the same kernel (test entry)."""
    if out is None:
        out = torch.empty(R.shape, dtype=torch.float32, device=R.device)
    M, N, K = _check_operands(X, W, R, out, torch.float32)
    c = _as_config(config)
    with torch.cuda.device(X.device):
        st = lib().skinny_addmm_bf16_acc_f32(X.data_ptr(), W.data_ptr(), R.data_ptr(), out.data_ptr(),
                                             M, N, K, ctypes.byref(c) if c is not None else None,
                                             _stream_ptr(stream, X.device))
    check(st, "skinny_addmm_bf16_acc_f32")
    return out


def _check_shard_operands(X, W, R, out, out_dtype):
    """Like _check_operands, but R and out may be row-major views into wider matrices: each
    needs unit column stride and a row stride >= N (the leading dimension passed on)."""
    for name, t in (("X", X), ("W", W), ("R", R), ("out", out)):
        if not isinstance(t, torch.Tensor):
            raise ValueError("%s must be a torch.Tensor" % name)
        if t.device.type != "cuda":
            raise ValueError("%s must be on the GPU" % name)
        if t.dim() != 2:
            raise ValueError("%s must be 2-D" % name)
    for name, t in (("X", X), ("W", W)):
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous (row-major)" % name)
    for name, t in (("X", X), ("W", W), ("R", R)):
        if t.dtype != torch.bfloat16:
            raise ValueError("%s must be bfloat16" % name)
    if out.dtype != out_dtype:
        raise ValueError("out must be %s" % out_dtype)
    M, K = X.shape
    N = W.shape[0]
    if W.shape[1] != K:
        raise ValueError("W must be [N, K] with K = X.shape[1]")
    if tuple(R.shape) != (M, N) or tuple(out.shape) != (M, N):
        raise ValueError("R and out must be [M, N] = [%d, %d]" % (M, N))
    for name, t in (("R", R), ("out", out)):
        if N > 1 and t.stride(1) != 1:
            raise ValueError("%s must have unit column stride" % name)
        if M > 1 and t.stride(0) < N:
            raise ValueError("%s row stride must be >= N" % name)
    if len({t.device for t in (X, W, R, out)}) != 1:
        raise ValueError("all operands must be on the same device")
    return M, N, K, (R.stride(0) if M > 1 else N), (out.stride(0) if M > 1 else N)


def _shard_flags(round_product: bool, no_neg_zero: bool) -> int:
    return (FLAG_ROUND_PRODUCT if round_product else 0) | (FLAG_NO_NEG_ZERO if no_neg_zero else 0)


def addmm_shard(X, W, R, out=None, round_product=False, no_neg_zero=False, config=None,
                stream=None) -> torch.Tensor:
    """Tensor-parallel shard form via skinny_addmm_bf16_shard: R and out may be column blocks
    of wider row-major matrices (their row strides are passed as leading dimensions).
    round_product: round the product sum to bf16 before adding R (two roundings);
    no_neg_zero: write +0 for a -0 result."""
    if out is None:
        out = torch.empty(R.shape, dtype=torch.bfloat16, device=R.device)
    M, N, K, ldr, ldy = _check_shard_operands(X, W, R, out, torch.bfloat16)
    c = _as_config(config)
    with torch.cuda.device(X.device):
        st = lib().skinny_addmm_bf16_shard(X.data_ptr(), W.data_ptr(), R.data_ptr(), ldr, out.data_ptr(), ldy,
                                           M, N, K, _shard_flags(round_product, no_neg_zero),
                                           ctypes.byref(c) if c is not None else None,
                                           _stream_ptr(stream, X.device))
    check(st, "skinny_addmm_bf16_shard")
    return out


def addmm_shard_acc_f32(X, W, R, out=None, round_product=False, config=None, stream=None) -> torch.Tensor:
    """Test entry of the shard form: the fp32 value each output is rounded from."""
    if out is None:
        out = torch.empty(R.shape, dtype=torch.float32, device=R.device)
    M, N, K, ldr, lda = _check_shard_operands(X, W, R, out, torch.float32)
    c = _as_config(config)
    with torch.cuda.device(X.device):
        st = lib().skinny_addmm_bf16_shard_acc_f32(X.data_ptr(), W.data_ptr(), R.data_ptr(), ldr, out.data_ptr(),
                                                   lda, M, N, K, _shard_flags(round_product, False),
                                                   ctypes.byref(c) if c is not None else None,
                                                   _stream_ptr(stream, X.device))
    check(st, "skinny_addmm_bf16_shard_acc_f32")
    return out


def _check_kbit(X, planes, absmax, codebook, kbits, R, out, out_dtype):
    for name, t in (("X", X), ("planes", planes), ("absmax", absmax), ("codebook", codebook), ("R", R),
                    ("out", out)):
        if not isinstance(t, torch.Tensor):
            raise ValueError("%s must be a torch.Tensor" % name)
        if t.device.type != "cuda":
            raise ValueError("%s must be on the GPU" % name)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    if X.dtype != torch.bfloat16 or R.dtype != torch.bfloat16 or out.dtype != out_dtype:
        raise ValueError("X and R must be bfloat16, out %s" % out_dtype)
    if planes.dtype not in (torch.int32, torch.uint32) or absmax.dtype != torch.uint8 or codebook.dtype != torch.float32:
        raise ValueError("planes must be int32/uint32 bit words, absmax uint8, codebook float32")
    if X.dim() != 2:
        raise ValueError("X must be [M, K]")
    M, K = X.shape
    N = R.shape[0 if R.dim() == 1 else 1]
    if tuple(planes.shape) != (N, K // 32, kbits) or tuple(absmax.shape) != (N, K // 32):
        raise ValueError("planes must be [N, K/32, kbits] and absmax [N, K/32]")
    if tuple(codebook.shape) != (1 << kbits,):
        raise ValueError("codebook must have 2^kbits entries")
    if tuple(R.shape) != (M, N) or tuple(out.shape) != (M, N):
        raise ValueError("R and out must be [M, N]")
    return M, N, K


def kbit_gemv(X, planes, absmax, codebook, kbits: int, R, out=None, stream=None) -> torch.Tensor:
    """Y = bf16(X @ What^T + R) with What the k-bit quantized weights (skinny_kbit_gemv_bf16)."""
    if out is None:
        out = torch.empty_like(R)
    M, N, K = _check_kbit(X, planes, absmax, codebook, kbits, R, out, torch.bfloat16)
    with torch.cuda.device(X.device):
        st = lib().skinny_kbit_gemv_bf16(X.data_ptr(), planes.data_ptr(), absmax.data_ptr(), codebook.data_ptr(),
                                         int(kbits), R.data_ptr(), out.data_ptr(), M, N, K,
                                         _stream_ptr(stream, X.device))
    check(st, "skinny_kbit_gemv_bf16")
    return out


def kbit_gemv_acc_f32(X, planes, absmax, codebook, kbits: int, R, out=None, stream=None) -> torch.Tensor:
    """Test entry: the fp32 value each output of kbit_gemv is rounded from."""
    if out is None:
        out = torch.empty(R.shape, dtype=torch.float32, device=R.device)
    M, N, K = _check_kbit(X, planes, absmax, codebook, kbits, R, out, torch.float32)
    with torch.cuda.device(X.device):
        st = lib().skinny_kbit_gemv_bf16_acc_f32(X.data_ptr(), planes.data_ptr(), absmax.data_ptr(),
                                                 codebook.data_ptr(), int(kbits), R.data_ptr(), out.data_ptr(),
                                                 M, N, K, _stream_ptr(stream, X.device))
    check(st, "skinny_kbit_gemv_bf16_acc_f32")
    return out


def select_config(M: int, N: int = 7168, K: int = 3584) -> dict:
    c = SkinnyConfig()
    check(lib().skinny_select_config(M, N, K, ctypes.byref(c)), "skinny_select_config")
    return c.as_dict()


def configs() -> list[dict]:
    L = lib()
    out = []
    for i in range(L.skinny_num_configs()):
        c = SkinnyConfig()
        check(L.skinny_get_config(i, ctypes.byref(c)), "skinny_get_config")
        out.append(c.as_dict())
    return out


def config_resources(config) -> dict:
    c = _as_config(config)
    r = SkinnyResources()
    check(lib().skinny_config_resources(ctypes.byref(c), ctypes.byref(r)), "skinny_config_resources")
    return {f: int(getattr(r, f)) for f, _ in SkinnyResources._fields_}


def version() -> str:
    return lib().skinny_version().decode()
