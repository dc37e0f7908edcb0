"""Seeded synthetic inputs for the skinny residual GEMM.

This module only draws and lays out input tensors; it holds none of the
operation's arithmetic. Both the GPU tests/benchmark and the CPU oracle's
callers take their inputs from here, so both sides see the same bytes.

Recipe (shapes and seed base follow the vLLM benchmark page
"benchmarks/kernels/benchmark_k3_cutedsl_residual.py", its ``main``):
  * one CPU ``torch.Generator`` seeded with ``20260722 + M``;
  * draw order: X, then W copies 0..C-1, then R copies 0..C-1;
  * X ~ N(0,1), R ~ N(0,1), W ~ N(0,1)/sqrt(K), each drawn in fp32 and rounded
    to bf16 by torch's conversion (round-to-nearest-even).
The page draws W unscaled; the 1/sqrt(K) factor keeps the product term at unit
scale so that neither the product nor the residual dominates the output.
"""
from __future__ import annotations

import math

import torch

SEED_BASE = 20260722
N_DEFAULT = 7168
K_DEFAULT = 3584


def generator(M: int, seed: int | None = None) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(SEED_BASE + M if seed is None else seed)
    return g


def make_inputs(M: int, N: int = N_DEFAULT, K: int = K_DEFAULT, copies: int = 1,
                seed: int | None = None):
    """Return (X, [W_0..W_{C-1}], [R_0..R_{C-1}]) as CPU bf16 tensors."""
    g = generator(M, seed)
    X = torch.randn((M, K), generator=g, dtype=torch.float32).to(torch.bfloat16)
    ws = []
    scale = 1.0 / math.sqrt(K) if K > 0 else 1.0
    for _ in range(copies):
        ws.append((torch.randn((N, K), generator=g, dtype=torch.float32) * scale).to(torch.bfloat16))
    rs = [torch.randn((M, N), generator=g, dtype=torch.float32).to(torch.bfloat16) for _ in range(copies)]
    return X, ws, rs


def bits(t: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit patterns (a copy on the host)."""
    import numpy as np
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16).copy()


def from_bits(b) -> torch.Tensor:
    """numpy uint16 bit patterns -> CPU bf16 tensor."""
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


# ---- structured inputs for exact cases (no arithmetic of the operation) -------------

def one_hot_rows(N: int, K: int, cols) -> torch.Tensor:
    """W with row n equal to the unit vector e_{cols[n]} (bf16 1.0 at one position)."""
    W = torch.zeros((N, K), dtype=torch.bfloat16)
    W[torch.arange(N), torch.as_tensor(cols, dtype=torch.long)] = 1.0
    return W


def small_int_inputs(M: int, N: int, K: int, seed: int = 7):
    """Integer-valued X in [-2,2], W[n,k] = ((n + 3k) mod 5) - 2, R in [-8,8]."""
    g = generator(M, seed)
    X = torch.randint(-2, 3, (M, K), generator=g).to(torch.bfloat16)
    n = torch.arange(N).view(N, 1)
    k = torch.arange(K).view(1, K)
    W = (((n + 3 * k) % 5) - 2).to(torch.bfloat16)
    R = torch.randint(-8, 9, (M, N), generator=g).to(torch.bfloat16)
    return X, W, R


# ---- k-bit quantized weights (random bit patterns; no quantization arithmetic) ------

def make_kbit_inputs(M: int, N: int = N_DEFAULT, K: int = K_DEFAULT, kbits: int = 4, copies: int = 1,
                     seed: int | None = None):
    """Inputs of the k-bit quantized GEMV, drawn as raw bits (the GEMV takes any bits):
    X bf16 [M, K] ~ N(0,1); per copy, plane words int32 [N, K/32, kbits] (uniform random
    bits, i.e. uniform codebook indices), scale bytes uint8 [N, K/32] uniform in
    [0x60, 0x68) (E4M4 values 1/32 .. 1.44/32: the block maximum of N(0,1)/sqrt(3584)
    weights is about 0.04, so the product keeps the unit scale of the dense inputs),
    R bf16 [M, N] ~ N(0,1); and a codebook of
    2^kbits sorted float32 levels: -1, +1 and uniform draws in between.
    Returns (X, [planes], [absmax], [R], codebook)."""
    g = generator(M, 7919 + kbits if seed is None else seed)
    X = torch.randn((M, K), generator=g, dtype=torch.float32).to(torch.bfloat16)
    planes, scales = [], []
    for _ in range(copies):
        planes.append(torch.randint(-2 ** 31, 2 ** 31, (N, K // 32, kbits), generator=g, dtype=torch.int64)
                      .to(torch.int32))
        scales.append(torch.randint(0x60, 0x68, (N, K // 32), generator=g, dtype=torch.int64).to(torch.uint8))
    rs = [torch.randn((M, N), generator=g, dtype=torch.float32).to(torch.bfloat16) for _ in range(copies)]
    inner = torch.rand((2 ** kbits - 2,), generator=g, dtype=torch.float32) * 2 - 1
    codebook = torch.cat([torch.tensor([-1.0]), inner.sort().values, torch.tensor([1.0])])
    return X, planes, scales, rs, codebook


def make_kda_inputs(B: int, T: int = 4, H: int = 8, HV: int | None = None, K: int = 128, V: int = 128,
                    ring_len: int = 16, seed: int = 0):
    """Inputs of one KDA chain-verify step with the distributions of the sglang page
    "benchmark/kernels/bench_kda_verify_sweep.py" (make_inputs): bf16 mixed ~ 0.5 N(0,1)
    [B*T, 2HK + HV V], conv weight 0.3 N [dim, 4], conv bias 0.1 N [dim], conv_pool N
    [B+1, 3, dim], a 0.5 N [B*T, HV K], b N [B*T, HV]; float32 A_log 0.5 N [HV],
    dt_bias 0.5 N [HV K], ssm 0.2 N [B+1, HV, V, K]; outputs win_pool and inter_ssm zero;
    ring buffers rawv [B+1, HV, R, V], rawk [B+1, H, R, K] (bf16), g [B+1, HV, R, K],
    beta [B+1, HV, R] (float32) N(0,1); cache_indices = inter_indices = 0..B-1.
    Drawn on the host from a seeded generator; returns a dict of CPU tensors."""
    HV = H if HV is None else HV
    g = torch.Generator().manual_seed(20260722 + 1000 * B + seed)
    dim = 2 * H * K + HV * V
    lines = slots = B + 1
    rnd = lambda *s, dt=torch.bfloat16: torch.randn(*s, generator=g, dtype=torch.float32).to(dt)
    return {
        "mixed": (rnd(B * T, dim, dt=torch.float32) * 0.5).to(torch.bfloat16),
        "w": (rnd(dim, 4, dt=torch.float32) * 0.3).to(torch.bfloat16),
        "bias": (rnd(dim, dt=torch.float32) * 0.1).to(torch.bfloat16),
        "a": (rnd(B * T, HV * K, dt=torch.float32) * 0.5).to(torch.bfloat16),
        "b": rnd(B * T, HV),
        "A_log": rnd(HV, dt=torch.float32) * 0.5,
        "dt_bias": rnd(HV * K, dt=torch.float32) * 0.5,
        "conv_pool": rnd(lines, 3, dim),
        "ssm": rnd(slots, HV, V, K, dt=torch.float32) * 0.2,
        "win_pool": torch.zeros(lines, T, 3, dim, dtype=torch.bfloat16),
        "inter_ssm": torch.zeros(lines, T, HV, V, K, dtype=torch.float32),
        "rawv": rnd(slots, HV, ring_len, V),
        "rawk": rnd(slots, H, ring_len, K),
        "g": rnd(slots, HV, ring_len, K, dt=torch.float32),
        "beta": rnd(slots, HV, ring_len, dt=torch.float32),
        "cache_indices": torch.arange(B, dtype=torch.int32),
        "inter_indices": torch.arange(B, dtype=torch.int32),
    }


def kda_to_numpy(inp: dict) -> dict:
    """The same tensors as numpy arrays, bf16 ones as uint16 bit patterns."""
    out = {}
    for k, t in inp.items():
        out[k] = bits(t) if t.dtype == torch.bfloat16 else t.numpy().copy()
    return out
