"""Python binding of the skinny residual GEMM: argument marshalling over the C ABI only.

Y = bf16(X @ W^T + R) for bf16 X[M,K], W[N,K], R[M,N] on the GPU; every step runs in the
HIP kernels of libskinny.so. torch supplies device memory and the current stream.
Argument errors raise ValueError before the library is called (as the launcher of the
vLLM API page "fused_add_multicast_skinny_gemm" does); library errors raise SkinnyError.
"""
from __future__ import annotations

import ctypes

import torch

from ._lib import (CONFIG_FIELDS, FLAG_NO_NEG_ZERO, FLAG_ROUND_PRODUCT, SkinnyConfig, SkinnyError, SkinnyKdaArgs,  # noqa: F401
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


def _byte_span(t: torch.Tensor) -> tuple[int, int]:
    """[first, last) byte addresses of a tensor with non-negative strides."""
    if t.numel() == 0:
        return t.data_ptr(), t.data_ptr()
    last = sum((n - 1) * st for n, st in zip(t.shape, t.stride()))
    return t.data_ptr(), t.data_ptr() + (last + 1) * t.element_size()


def _overlaps(a: torch.Tensor, b: torch.Tensor) -> bool:
    (a0, a1), (b0, b1) = _byte_span(a), _byte_span(b)
    return a0 < b1 and b0 < a1


def _check_aliasing(inputs, R, out):
    """The output may be R itself (same address, strides and dtype: every residual is read
    before its own output is written) but must not overlap the other inputs or any other
    part of R. Overlap is judged on byte spans, so two column blocks interleaved in one wide
    matrix count as overlapping (a conservative refusal, never a missed overlap)."""
    if any(_overlaps(out, t) for t in inputs):
        raise ValueError("out must not overlap the operands other than R")
    if _overlaps(out, R) and not (out.data_ptr() == R.data_ptr() and out.stride() == R.stride()
                                  and out.dtype == R.dtype):
        raise ValueError("out may be R itself but must not partially overlap it")


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
    _check_aliasing((X, W), R, out)
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
    _check_aliasing((X, W), R, out)
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
    _check_aliasing((X, planes, absmax, codebook), R, out)
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


def kda_verify(inp: dict, T: int, H: int, HV: int, K: int, V: int, scale: float, snapshots: bool = True,
               ring: bool = False, out=None, stream=None) -> torch.Tensor:
    """One KDA chain-verify step (skinny_kda_verify_bf16) on device tensors named as on the
    sglang benchmark page: bf16 mixed [B*T, dim], w [dim, 4], bias [dim], conv_pool
    [lines, 3, dim], win_pool [lines, T, 3, dim], a [B*T, HV*K], b [B*T, HV]; float32 A_log
    [HV], dt_bias [HV*K], ssm [slots, HV, V, K], inter_ssm [lines, T, HV, V, K], ring
    buffers rawv [slots, HV, R, V], rawk [slots, H, R, K] (bf16), g [slots, HV, R, K], beta
    [slots, HV, R] (float32); int32 cache_indices, inter_indices [B]. Writes win_pool, and
    inter_ssm (snapshots) or the ring buffers (ring); returns o bf16 [B*T, HV, V]."""
    dim = 2 * H * K + HV * V
    B = int(inp["cache_indices"].shape[0])
    spec = {"mixed": (torch.bfloat16, (B * T, dim)), "w": (torch.bfloat16, (dim, 4)),
            "bias": (torch.bfloat16, (dim,)), "a": (torch.bfloat16, (B * T, HV * K)),
            "b": (torch.bfloat16, (B * T, HV)), "A_log": (torch.float32, (HV,)),
            "dt_bias": (torch.float32, (HV * K,)), "cache_indices": (torch.int32, (B,)),
            "inter_indices": (torch.int32, (B,))}
    lines = int(inp["conv_pool"].shape[0])
    slots = int(inp["ssm"].shape[0])
    spec["conv_pool"] = (torch.bfloat16, (lines, 3, dim))
    spec["win_pool"] = (torch.bfloat16, (lines, T, 3, dim))
    spec["ssm"] = (torch.float32, (slots, HV, V, K))
    R = 0
    if snapshots:
        spec["inter_ssm"] = (torch.float32, (lines, T, HV, V, K))
    if ring:
        R = int(inp["rawv"].shape[2])
        spec.update({"rawv": (torch.bfloat16, (slots, HV, R, V)), "rawk": (torch.bfloat16, (slots, H, R, K)),
                     "g": (torch.float32, (slots, HV, R, K)), "beta": (torch.float32, (slots, HV, R))})
    dev = inp["mixed"].device if isinstance(inp.get("mixed"), torch.Tensor) else None
    for name, (dt, shape) in spec.items():
        t = inp.get(name)
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or not t.is_contiguous():
            raise ValueError("%s must be a contiguous GPU tensor" % name)
        if t.device != dev:
            raise ValueError("%s is on %s, mixed on %s: all tensors must be on one GPU" % (name, t.device, dev))
        if t.dtype != dt or tuple(t.shape) != shape:
            raise ValueError("%s must be %s %s, got %s %s" % (name, dt, shape, t.dtype, tuple(t.shape)))
    if out is None:
        out = torch.empty((B * T, HV, V), dtype=torch.bfloat16, device=inp["mixed"].device)
    elif (out.dtype != torch.bfloat16 or tuple(out.shape) != (B * T, HV, V) or not out.is_contiguous()
          or out.device != dev):
        raise ValueError("out must be contiguous bf16 [B*T, HV, V] on the inputs' GPU")
    p = lambda name: inp[name].data_ptr() if name in spec else None
    args = SkinnyKdaArgs(mixed=p("mixed"), conv_w=p("w"), conv_b=p("bias"), conv_pool=p("conv_pool"),
                         cache_idx=p("cache_indices"), inter_idx=p("inter_indices"), a=p("a"), b=p("b"),
                         A_log=p("A_log"), dt_bias=p("dt_bias"), ssm=p("ssm"), conv_win=p("win_pool"),
                         snap=p("inter_ssm"), ring_v=p("rawv"), ring_k=p("rawk"), ring_g=p("g"),
                         ring_beta=p("beta"), out=out.data_ptr(), B=B, T=T, H=H, HV=HV, K=K, V=V,
                         lines=lines, slots=slots, ring_len=R, scale=float(scale))
    with torch.cuda.device(inp["mixed"].device):
        st = lib().skinny_kda_verify_bf16(ctypes.byref(args), _stream_ptr(stream, inp["mixed"].device))
    check(st, "skinny_kda_verify_bf16")
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


def config_kernel(config) -> dict:
    """The kernel a plain call with this configuration launches at the tuned shape: its name as
    the HIP runtime reports it and the hash of its machine code in this build (kernel_code.json,
    written by the build); None for the hash when the build's map lacks the name."""
    import json
    import os
    c = _as_config(config)
    buf = ctypes.create_string_buffer(4096)
    check(lib().skinny_config_kernel_name(ctypes.byref(c), buf, len(buf)), "skinny_config_kernel_name")
    name = buf.value.decode()
    try:
        code = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "kernel_code.json")))
    except (OSError, ValueError):
        code = {}
    return {"name": name, "code_sha256": code.get(name)}


def version() -> str:
    return lib().skinny_version().decode()
