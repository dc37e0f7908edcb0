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


def _kda_table(B: int, T: int, H: int, HV: int, K: int, V: int, ring_len: int):
    """(name, shape, standard deviation, dtype) of every random input of one KDA verify step,
    grouped as conv inputs, gate inputs, recurrent state, ring contents. Normal draws, taken
    in this order from one generator, in fp32 and then converted to the listed dtype."""
    dim = 2 * H * K + HV * V          # conv channels: q, k (H heads each) and v (HV heads)
    slots = B + 1                     # state/ring slots and conv lines: one spare
    bf, f32 = torch.bfloat16, torch.float32
    return [
        # conv1d: mixed projections of the T draft tokens, its taps and bias, the cached inputs
        ("mixed", (B * T, dim), 0.5, bf),
        ("w", (dim, 4), 0.3, bf),
        ("bias", (dim,), 0.1, bf),
        ("conv_pool", (slots, 3, dim), 1.0, bf),
        # gate: per-token a (per K channel) and b (per value head), per-head A_log and dt_bias
        ("a", (B * T, HV * K), 0.5, bf),
        ("b", (B * T, HV), 1.0, bf),
        ("A_log", (HV,), 0.5, f32),
        ("dt_bias", (HV * K,), 0.5, f32),
        # recurrent state [V, K] per slot and value head
        ("ssm", (slots, HV, V, K), 0.2, f32),
        # ring entries (overwritten by a ring-layout call; random, so unwritten ones show)
        ("rawv", (slots, HV, ring_len, V), 1.0, bf),
        ("rawk", (slots, H, ring_len, K), 1.0, bf),
        ("g", (slots, HV, ring_len, K), 1.0, f32),
        ("beta", (slots, HV, ring_len), 1.0, f32),
    ]


def make_kda_inputs(B: int, T: int = 4, H: int = 8, HV: int | None = None, K: int = 128, V: int = 128,
                    ring_len: int = 16, seed: int = 0):
    """Inputs of one KDA chain-verify step with the shapes and distributions of the sglang page
    "benchmark/kernels/bench_kda_verify_sweep.py" (its input maker): every random tensor of
    _kda_table drawn from one CPU generator seeded 20260722 + 1000 B + seed (the page draws on
    the GPU); the window and snapshot outputs zero-filled; cache and snapshot indices 0 .. B-1.
    Returns a dict of CPU tensors."""
    HV = H if HV is None else HV
    g = torch.Generator().manual_seed(SEED_BASE + 1000 * B + seed)
    out = {}
    for name, shape, std, dtype in _kda_table(B, T, H, HV, K, V, ring_len):
        out[name] = (torch.randn(shape, generator=g, dtype=torch.float32) * std).to(dtype)
    dim = 2 * H * K + HV * V
    out["win_pool"] = torch.zeros(B + 1, T, 3, dim, dtype=torch.bfloat16)
    out["inter_ssm"] = torch.zeros(B + 1, T, HV, V, K, dtype=torch.float32)
    out["cache_indices"] = torch.arange(B, dtype=torch.int32)
    out["inter_indices"] = torch.arange(B, dtype=torch.int32)
    return out


def kda_to_numpy(inp: dict) -> dict:
    """The same tensors as numpy arrays, bf16 ones as uint16 bit patterns."""
    out = {}
    for k, t in inp.items():
        out[k] = bits(t) if t.dtype == torch.bfloat16 else t.numpy().copy()
    return out
