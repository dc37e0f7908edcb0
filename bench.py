#!/usr/bin/env python3
"""Benchmark of the skinny residual GEMM  Y = bf16(X W^T + R)  on one MI355X.

Method (the vLLM benchmark page "benchmarks/kernels/benchmark_k3_cutedsl_residual.py",
functions graph_samples / summarize / rotating_buffer_count, re-done for HIP):
  * seeded synthetic inputs (decode_skinny_addmm_amd.synth), N = 7168, K = 3584;
  * W and R rotate over C copies (default 6, about 308 MB: more than the 256 MB Infinity
    Cache and the L2s), so every call streams its W from HBM;
  * one HIP graph captures `--calls` launches (default 500) cycling over the copies;
    a step is one replay of that graph; warm-up replays are untimed;
  * HIP events on the stream the graph runs on bracket every timed replay.

Default run (no flags): M = 4, 6 copies, 500 calls per graph, prints ONE JSON line with
the throughput (algorithmic HBM GB/s), the roofline fraction against 8 TB/s and the CPU
oracle timed on this host as a baseline. The same line carries `curve`: the metric at
M = 1, 2, 4, ..., 256 (each M on its own seeded inputs and rotation, the library's selected
configuration; median/p10/p90 us, GB/s, HBM and MFMA fractions, a sampled oracle check, and
the one-copy cache-warm time), and `m64_valu_vs_mfma`: the pages' SIMT GEMV at its best grid
point against the matrix-core path at M = 64.

Other modes write JSONL rows (one per configuration or M) to --out:
  --mode sweep    every built configuration at --m (default 16)
  --mode mcurve   M in {1,2,4,8,16,32,64,128,256}, library-selected configuration
  --mode shard    the tensor-parallel shard form (vLLM API page "fused_add_multicast_skinny_gemm"):
                  N = 7168/--shards columns for rank --rank, R and Y as column blocks of the
                  full-width matrices, two roundings and no -0, W rotated over >= 40 copies
  --mode shard-sweep   the same over every built configuration
  --mode kda      the KDA chain-verify step (sglang page "benchmark/kernels/bench_kda_verify_sweep.py"):
                  H = HV = 8, K = V = 128, T = 4, B in --ms (default 1,4,16,64), snapshot and ring
                  mode; states and outputs rotate over enough copies to exceed 320 MB
  --mode kbit     the k-bit quantized decode GEMV (bitsandbytes page "compare/main...QLORA-2.diff"),
                  N = 7168, K = 3584, k in --kbits, M in --ms (default 1,2,4,16); the planes and
                  scale bytes rotate over enough copies to exceed 308 MB
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

N_DIM = 7168
K_DIM = 3584
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak (published)
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak (published)


def algorithmic_bytes(M: int, N: int = None, K: int = None) -> int:
    """W read once, X read once, R read once, Y written once (bf16)."""
    N = N_DIM if N is None else N
    K = K_DIM if K is None else K
    return 2 * N * K + 2 * M * K + 2 * M * N + 2 * M * N


def kbit_algorithmic_bytes(M: int, N: int, K: int, kbits: int) -> int:
    """k bit-plane words and one scale byte per 32 weights read once, the 2^k-entry fp32
    codebook, X and R read once, Y written once (bf16)."""
    return N * (K // 32) * (4 * kbits + 1) + 4 * (1 << kbits) + 2 * M * K + 2 * M * N + 2 * M * N


def kda_algorithmic_bytes(B: int, T: int, H: int, HV: int, K: int, V: int, ring: bool) -> int:
    """Bytes one KDA verify call must move: the fp32 states read once; snapshots (T states
    written) or ring entries (v, k bf16; g, beta fp32); the conv inputs (T tokens and 3 cached
    inputs per channel, 4 taps and a bias) and windows (3 inputs per token); gates a, b,
    dt_bias, A_log; the bf16 output."""
    dim = 2 * H * K + HV * V
    state = B * HV * V * K * 4
    states_out = 0 if ring else T * state
    ring_out = (B * HV * T * V * 2 + B * H * T * K * 2 + B * HV * T * K * 4 + B * HV * T * 4) if ring else 0
    conv = B * T * dim * 2 + B * 3 * dim * 2 + dim * 5 * 2 + B * T * 3 * dim * 2
    gates = B * T * HV * K * 2 + B * T * HV * 2 + HV * K * 4 + HV * 4
    out = B * T * HV * V * 2
    return state + states_out + ring_out + conv + gates + out


def lookup_traffic(sk, cfg: dict, M: int, N: int = None, K: int = None):
    """HBM bytes per launch measured by rocprofv3 FETCH_SIZE/WRITE_SIZE runs for this exact
    kernel instance and shape (profiles/traffic.json, scaled by a copy-kernel calibration).
    Entries are keyed by the kernel's name and the hash of its machine code in the build that
    was measured, so the figure reads None as soon as that kernel's code changes."""
    N = N_DIM if N is None else N
    K = K_DIM if K is None else K
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        entries = json.load(open(path))["entries"]
        kern = sk.config_kernel(cfg)
    except (OSError, ValueError, KeyError, RuntimeError):
        return None
    for e in entries:
        if (kern["name"] in (e.get("kernel"), e.get("kernel_mangled")) and kern["code_sha256"]
                and e.get("code_sha256") == kern["code_sha256"]
                and e.get("M") == M and e.get("N") == N and e.get("K") == K):
            return {"bytes": e["traffic_bytes"], "fetch_bytes": e["fetch_bytes"], "write_bytes": e["write_bytes"],
                    "source": "profiles/" + e["summary"]}
    return None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def config_shard(args, candidates):
    """Every n-th candidate from the i-th on (--config-shard i --num-config-shards n), so a long
    sweep can be split over several runs; the shards together cover the list once."""
    return candidates[args.config_shard::args.num_config_shards]


def parse_config(s: str | None):
    if not s:
        return None
    v = [int(t) for t in s.split(",")]
    if len(v) not in (5, 6, 7, 8):
        raise argparse.ArgumentTypeError("config must be PATH,BLOCK,OUTPUTS,K_UNROLL,VECTOR_WIDTH"
                                         "[,M_TILE[,K_SPLIT[,K_STAGE]]]")
    keys = ("path", "block_size", "outputs_per_block", "k_unroll", "vector_width", "m_tile", "k_split", "k_stage")
    d = dict(zip(keys, v))
    d.setdefault("m_tile", 0)
    d.setdefault("k_split", 1)
    d.setdefault("k_stage", 0)
    return d


def percentile(ordered, frac):
    pos = frac * (len(ordered) - 1)
    lo, hi = math.floor(pos), math.ceil(pos)
    if lo == hi:
        return ordered[lo]
    w = pos - lo
    return ordered[lo] * (1 - w) + ordered[hi] * w


def summarize(samples):
    o = sorted(samples)
    mean = statistics.mean(samples)
    return {"median_us": statistics.median(samples), "p10_us": percentile(o, 0.1),
            "p90_us": percentile(o, 0.9), "mean_us": mean,
            "cv_pct": statistics.pstdev(samples) / mean * 100.0 if mean else 0.0}


class Workload:
    """Device-resident inputs: one X, C copies of W and R, C outputs."""

    def __init__(self, M: int, copies: int, N: int = N_DIM, K: int = K_DIM):
        import torch

        from decode_skinny_addmm_amd import synth
        t0 = time.time()
        X, ws, rs = synth.make_inputs(M, N, K, copies=copies)
        self.host = (X, ws[0], rs[0])
        self.M, self.N, self.K, self.copies = M, N, K, copies
        self.X = X.cuda()
        self.W = [w.cuda() for w in ws]
        self.R = [r.cuda() for r in rs]
        self.Y = [torch.empty_like(r) for r in self.R]
        del ws, rs
        torch.cuda.synchronize()
        log("inputs M=%d copies=%d ready in %.1fs (%.1f MB of W+R)" % (
            M, copies, time.time() - t0, copies * (N * K + M * N) * 2 / 1e6))


class OneCopy:
    """A Workload's first copy alone (W, R and Y of copy 0), for the cache-warm reference row."""

    def __init__(self, wl):
        self.host, self.M, self.N, self.K, self.copies = wl.host, wl.M, wl.N, wl.K, 1
        self.X, self.W, self.R, self.Y = wl.X, wl.W[:1], wl.R[:1], wl.Y[:1]


class ShardWorkload:
    """One rank's share of the N-sharded op: W holds N_total/shards rows (C seeded copies, enough
    to stream from HBM), R and Y are column blocks of [M, N_total] matrices at the rank's offset."""

    def __init__(self, M: int, copies: int, shards: int, rank: int, N_total: int = N_DIM, K: int = K_DIM):
        import torch

        from decode_skinny_addmm_amd import synth
        t0 = time.time()
        N = N_total // shards
        c0 = rank * N
        X, ws, rs = synth.make_inputs(M, N, K, copies=copies)
        self.host = (X, ws[0], rs[0])
        self.M, self.N, self.K, self.copies, self.N_total, self.c0 = M, N, K, copies, N_total, c0
        self.X = X.cuda()
        self.W = [w.cuda() for w in ws]
        self.Rwide = [torch.zeros((M, N_total), dtype=torch.bfloat16, device="cuda") for _ in rs]
        for rw, r in zip(self.Rwide, rs):
            rw[:, c0:c0 + N].copy_(r.cuda())
        self.Ywide = [torch.zeros((M, N_total), dtype=torch.bfloat16, device="cuda") for _ in rs]
        self.R = [rw[:, c0:c0 + N] for rw in self.Rwide]
        self.Y = [yw[:, c0:c0 + N] for yw in self.Ywide]
        del ws, rs
        torch.cuda.synchronize()
        log("shard inputs M=%d N=%d (rank %d of %d) copies=%d ready in %.1fs (%.1f MB of W)" % (
            M, N, rank, shards, copies, time.time() - t0, copies * N * K * 2 / 1e6))


class KbitWorkload:
    """Device-resident k-bit GEMV inputs: one X and codebook, C copies of (planes, scales) and R."""

    def __init__(self, M: int, copies: int, kbits: int, N: int = N_DIM, K: int = K_DIM):
        import torch

        from decode_skinny_addmm_amd import synth
        t0 = time.time()
        X, ps, As, rs, cb = synth.make_kbit_inputs(M, N, K, kbits=kbits, copies=copies)
        self.host = (X, ps[0], As[0], rs[0], cb)
        self.M, self.N, self.K, self.copies, self.kbits = M, N, K, copies, kbits
        self.X = X.cuda()
        self.cb = cb.cuda()
        self.W = [(p.cuda(), a.cuda()) for p, a in zip(ps, As)]
        self.R = [r.cuda() for r in rs]
        self.Y = [torch.empty_like(r) for r in self.R]
        del ps, As, rs
        torch.cuda.synchronize()
        log("kbit inputs M=%d k=%d copies=%d ready in %.1fs (%.1f MB of planes+scales)" % (
            M, kbits, copies, time.time() - t0, copies * N * (K // 32) * (4 * kbits + 1) / 1e6))


def time_graph(launch, wl, calls: int, warmup: int, steps: int):
    """Capture `calls` launches cycling over the copies into one graph; time `steps` replays.

    Returns (per-replay microseconds list, total elapsed ms, stream used)."""
    import torch
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for i in range(wl.copies):  # eager warm-up over every copy
            launch(wl.X, wl.W[i], wl.R[i], wl.Y[i])
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for c in range(calls):
            i = c % wl.copies
            launch(wl.X, wl.W[i], wl.R[i], wl.Y[i])
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            g.replay()
    stream.synchronize()
    events = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        events[0].record(stream)
        for s in range(steps):
            g.replay()
            events[s + 1].record(stream)
    events[-1].synchronize()
    torch.cuda.synchronize()
    per = [events[s].elapsed_time(events[s + 1]) * 1000.0 for s in range(steps)]  # us per replay
    total_ms = events[0].elapsed_time(events[-1])
    del g
    return per, total_ms


def secondary_correctness(wl, launch):
    """Page-1 style statistics of copy 0 against an fp32 torch product (reported, not gating)."""
    import torch
    X, W, R = wl.X, wl.W[0], wl.R[0]
    Y = torch.empty_like(R)
    launch(X, W, R, Y)
    torch.cuda.synchronize()
    ref = X.float() @ W.float().t() + R.float()
    err = (Y.float() - ref).abs()
    cos = torch.nn.functional.cosine_similarity(Y.float().flatten(), ref.flatten(), dim=0).item()
    return {"cosine": cos, "max_abs_error": err.max().item(),
            "max_scaled_error": (err / (ref.abs() + 1.0)).max().item(), "valid": cos > 0.999}


def oracle_parity_sample(wl, launch, count=512):
    """Sampled oracle check of copy 0 (2 bf16 ULP rule); returns the max ULP distance."""
    import numpy as np
    import torch

    import oracle
    from decode_skinny_addmm_amd import synth
    X, W, R = wl.host
    Y = torch.empty_like(wl.R[0])
    launch(wl.X, wl.W[0], wl.R[0], Y)
    torch.cuda.synchronize()
    yg = synth.bits(Y)
    rng = np.random.default_rng(0)
    ms = rng.integers(0, wl.M, count)
    ns = rng.integers(0, wl.N, count)
    yo, ex = oracle.addmm_bf16_points(synth.bits(X), synth.bits(W), synth.bits(R), ms, ns)

    def key(b):
        b = b.astype(np.int64)
        return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)
    d = np.abs(key(yg[ms, ns]) - key(yo))
    big = np.abs(ex) >= 2.0 ** -12
    return int(d[big].max()) if big.any() else 0


def cpu_baseline(M: int, seconds: float):
    """The CPU oracle, as it stands, on full calls of the same workload (copy 0), on the host's
    usable threads; a shorter sample on one thread is reported beside it."""
    import oracle
    from decode_skinny_addmm_amd import synth
    X, ws, rs = synth.make_inputs(M, N_DIM, K_DIM)
    Xb, Wb, Rb = synth.bits(X), synth.bits(ws[0]), synth.bits(rs[0])
    threads = oracle.default_threads()
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit():
        threads = min(threads, int(omp))

    def timed(nthreads, budget):
        calls = 0
        t0 = time.perf_counter()
        while True:
            oracle.addmm_bf16(Xb, Wb, Rb, threads=nthreads, want_acc=False)
            calls += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return calls, el

    calls, el = timed(threads, seconds)
    per_call = el / calls
    calls1, el1 = timed(1, max(1.0, seconds / 4))
    per_call1 = el1 / calls1
    return {"value": algorithmic_bytes(M) / per_call / 1e9, "unit": "GB/s", "cores": threads,
            "kind": "oracle", "us_per_call": per_call * 1e6,
            "sample": "%d full calls (M=%d, N=%d, K=%d, copy 0) in %.1f s on %d threads" % (
                calls, M, N_DIM, K_DIM, el, threads),
            "one_thread": {"value": algorithmic_bytes(M) / per_call1 / 1e9, "unit": "GB/s",
                           "us_per_call": per_call1 * 1e6,
                           "sample": "%d full calls in %.1f s on 1 thread" % (calls1, el1)}}


def probe_launches(sk):
    """Reference kernels (include/skinny_probe.h) with the operation's launch signature."""
    import torch
    L = sk.ops.lib()
    sink = torch.zeros(4, dtype=torch.float32, device="cuda")

    def cur():
        return torch.cuda.current_stream().cuda_stream

    def null(X, W, R, Y):
        sk.ops.check(L.skinny_probe_null(cur()), "skinny_probe_null")

    def read(X, W, R, Y, unroll=8):
        sk.ops.check(L.skinny_probe_read(W.data_ptr(), W.numel() * 2, sink.data_ptr(), 0, unroll, cur()),
                     "skinny_probe_read")
    return null, read


def probe_rows_and_spin(sk):
    """The GEMV-shaped read (every load issued first) and the busy-kernel launch probe."""
    import torch
    L = sk.ops.lib()
    sink = torch.zeros(4, dtype=torch.float32, device="cuda")

    def cur():
        return torch.cuda.current_stream().cuda_stream

    def read_rows(X, W, R, Y, rpb=32):
        sk.ops.check(L.skinny_probe_read_rows(W.data_ptr(), W.shape[0], rpb, sink.data_ptr(), cur()),
                     "skinny_probe_read_rows")

    def spin(X, W, R, Y, ns=4000, blocks=224, threads=448):
        sk.ops.check(L.skinny_probe_spin(ns, blocks, threads, cur()), "skinny_probe_spin")
    return read_rows, spin


def reference_rows(sk, wl, calls, warmup, steps):
    """Per-launch floor and the streaming-read rate over the same rotating W copies."""
    null, read = probe_launches(sk)
    out = {}
    per, total_ms = time_graph(null, wl, calls, warmup, steps)
    out["null_kernel_us"] = total_ms * 1000.0 / (steps * calls)
    for u in (4, 8, 16):
        per, total_ms = time_graph(lambda X, W, R, Y, u=u: read(X, W, R, Y, u), wl, calls, warmup, steps)
        us = total_ms * 1000.0 / (steps * calls)
        out["stream_read_u%d" % u] = {"us": us, "gbs": wl.N * wl.K * 2 / (us * 1e-6) / 1e9}
    read_rows, spin = probe_rows_and_spin(sk)
    if wl.K == K_DIM:
        for rpb in (32, 28, 16, 8):
            per, total_ms = time_graph(lambda X, W, R, Y, r=rpb: read_rows(X, W, R, Y, r), wl, calls, warmup, steps)
            us = total_ms * 1000.0 / (steps * calls)
            out["read_rows_rpb%d" % rpb] = {"us": us, "gbs": wl.N * wl.K * 2 / (us * 1e-6) / 1e9,
                                            "workgroups": -(-wl.N // rpb)}
    for ns in (4000, 8000):
        per, total_ms = time_graph(lambda X, W, R, Y, n=ns: spin(X, W, R, Y, n), wl, calls, warmup, steps)
        us = total_ms * 1000.0 / (steps * calls)
        out["spin_%dns_224x448" % ns] = {"us": us, "overhead_us": us - ns / 1000.0}
    best = max(v["gbs"] for k, v in out.items() if k.startswith("stream_read") or k.startswith("read_rows"))
    out["stream_read_best_gbs"] = best
    return out


def run_probe(args, sk):
    """Streaming-read reference kernel over launch shapes (JSONL rows to --out)."""
    import torch
    null, read = probe_launches(sk)
    L = sk.ops.lib()
    sink = torch.zeros(4, dtype=torch.float32, device="cuda")
    wl = Workload(1, args.copies)
    out = open(args.out, "a") if args.out else None
    nbytes = wl.N * wl.K * 2
    shapes = []
    for u in (1, 2, 4, 8, 16):
        for blocks in (256, 512, 1024, 2048, 4096, 8192):
            shapes.append((blocks, u))
        shapes.append((nbytes // (4096 * u), u))  # one pass: every thread one batch of u loads
    for blocks, u in shapes:
        def launch(X, W, R, Y, b=blocks, u=u):
            sk.ops.check(L.skinny_probe_read(W.data_ptr(), nbytes, sink.data_ptr(), b, u,
                                             torch.cuda.current_stream().cuda_stream), "probe_read")
        per, total_ms = time_graph(launch, wl, args.calls, args.warmup, args.steps)
        us = total_ms * 1000.0 / (args.steps * args.calls)
        row = {"probe": "read", "bytes": nbytes, "blocks": blocks, "unroll": u, "us": us,
               "gbs": nbytes / (us * 1e-6) / 1e9}
        log(json.dumps(row))
        if out:
            out.write(json.dumps(row) + "\n")
    # steady state: one launch over all copies at once (one large buffer)
    big = torch.empty(wl.copies * nbytes // 2, dtype=torch.bfloat16, device="cuda")
    for u in (2, 4, 8):
        for blocks in (1024, 2048, 4096):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            for rep in range(3):
                sk.ops.check(L.skinny_probe_read(big.data_ptr(), big.numel() * 2, sink.data_ptr(), blocks, u,
                                                 torch.cuda.current_stream().cuda_stream), "probe_read")
            torch.cuda.synchronize()
            ev[0].record()
            for rep in range(20):
                sk.ops.check(L.skinny_probe_read(big.data_ptr(), big.numel() * 2, sink.data_ptr(), blocks, u,
                                                 torch.cuda.current_stream().cuda_stream), "probe_read")
            ev[1].record()
            ev[1].synchronize()
            us = ev[0].elapsed_time(ev[1]) * 1000.0 / 20
            row = {"probe": "read_big", "bytes": big.numel() * 2, "blocks": blocks, "unroll": u, "us": us,
                   "gbs": big.numel() * 2 / (us * 1e-6) / 1e9}
            log(json.dumps(row))
            if out:
                out.write(json.dumps(row) + "\n")
    if out:
        out.close()


def run_calib(args, sk):
    """Plain copy of a known size (the read+write reference for byte counters)."""
    import torch
    L = sk.ops.lib()
    nbytes = N_DIM * K_DIM * 2
    src = torch.randn(nbytes // 2, dtype=torch.float32, device="cuda").view(torch.bfloat16)[: nbytes // 2]
    src = src.contiguous()
    dst = torch.empty_like(src)
    for _ in range(max(1, args.steps)):
        sk.ops.check(L.skinny_probe_copy(dst.data_ptr(), src.data_ptr(), nbytes,
                                         torch.cuda.current_stream().cuda_stream), "probe_copy")
    torch.cuda.synchronize()
    print(json.dumps({"calib": "copy", "bytes_read": nbytes, "bytes_written": nbytes,
                      "launches": max(1, args.steps)}), flush=True)


def make_launch(sk, config):
    if config is not None and config.get("reference") == "torch.addmm":
        import torch
        return lambda X, W, R, Y: torch.addmm(R, X, W.t(), out=Y)
    if config is None:
        return lambda X, W, R, Y: sk.addmm_default(X, W, R, Y)
    return lambda X, W, R, Y: sk.addmm(X, W, R, out=Y, config=config)


def measure(sk, wl, config, calls, warmup, steps):
    launch = make_launch(sk, config)
    per, total_ms = time_graph(launch, wl, calls, warmup, steps)
    us_per_call = [p / calls for p in per]
    mean_us = total_ms * 1000.0 / (steps * calls)
    gbs = algorithmic_bytes(wl.M, wl.N, wl.K) / (mean_us * 1e-6) / 1e9
    return launch, us_per_call, mean_us, gbs


CURVE_MS = (1, 2, 4, 8, 16, 32, 64, 128, 256)
# The best point of the pages' SIMT grid at M = 64 (block 64, 8 outputs per block, k-unroll 1,
# 16-byte vectors, 16-row X tile), timed beside the library's matrix-core choice.
SIMT_BEST_M64 = {"path": 4, "block_size": 64, "outputs_per_block": 8, "k_unroll": 1, "vector_width": 8,
                 "m_tile": 16, "k_split": 1}


def curve_point(sk, wl, cfg, calls, warmup, steps, one_copy=True):
    """One M of the metric's curve: rotated (the metric) and one-copy cache-warm timings."""
    M = wl.M
    launch, samples, mean_us, gbs = measure(sk, wl, cfg, calls, warmup, steps)
    st = summarize(samples)
    flops = 2.0 * M * wl.N * wl.K
    row = {"M": M, "config": cfg, "us": round(mean_us, 4),
           "median_us": round(st["median_us"], 4), "p10_us": round(st["p10_us"], 4),
           "p90_us": round(st["p90_us"], 4), "cv_pct": round(st["cv_pct"], 3),
           "gbs": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
           "frac_mfma": round(flops / (mean_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 5),
           "max_ulp_sampled": oracle_parity_sample(wl, launch, 256)}
    if one_copy:
        _, _, one_us, _ = measure(sk, OneCopy(wl), cfg, calls, warmup, steps)
        row["one_copy_cache_warm_us"] = round(one_us, 4)
    return row


def run_curve(args, sk):
    """The metric over M = 1 ... 256 at the library's selected configuration, each M on its own
    seeded inputs (6 rotating copies), plus the M = 64 comparison of the pages' SIMT GEMV with
    the matrix-core path."""
    import torch
    curve, m64 = [], None
    steps, warmup = max(5, args.steps // 2), max(2, args.warmup)
    for M in CURVE_MS:
        wl = Workload(M, args.copies)
        row = curve_point(sk, wl, sk.select_config(M), args.calls, warmup, steps)
        log("curve " + json.dumps(row))
        curve.append(row)
        if M == 64:
            simt = curve_point(sk, wl, SIMT_BEST_M64, args.calls, warmup, steps, one_copy=False)
            m64 = {"valu_simt_best": simt, "mfma_selected": row,
                   "mfma_speedup": round(simt["us"] / row["us"], 3)}
            log("m64 " + json.dumps(m64))
        del wl
        torch.cuda.empty_cache()
    return curve, m64


def run_default(args, sk):
    import torch
    M = args.m
    wl = Workload(M, args.copies)
    cfg = args.config or sk.select_config(M)
    launch, samples, mean_us, gbs = measure(sk, wl, cfg, args.calls, args.warmup, args.steps)
    st = summarize(samples)
    flops = 2.0 * M * N_DIM * K_DIM
    res = sk.config_resources(cfg) if cfg.get("m_tile") else None
    row = {
        "metric": "us/call + achieved HBM GB/s (% roofline), Y=X*W^T+R N=7168 K=3584, M=1..256",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(mean_us * args.calls / 1000.0, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "skinny residual GEMM M=%d N=%d K=%d, bf16 in/out, fp32 accumulate; "
                               "W,R rotated over %d seeded copies; HIP graph of %d calls per step"
                               % (M, N_DIM, K_DIM, args.copies, args.calls),
                   "M": M, "N": N_DIM, "K": K_DIM, "copies": args.copies, "calls_per_step": args.calls,
                   "kernel_config": cfg, "resources": res, "kernel": sk.config_kernel(cfg)},
        "us_per_call": round(mean_us, 4),
        "us_per_call_stats": {k: round(v, 4) for k, v in st.items()},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": (lambda t: t["bytes"] if t else None)(lookup_traffic(sk, cfg, M)),
                     "traffic_detail": lookup_traffic(sk, cfg, M),
                     "bytes_per_launch": algorithmic_bytes(M),
                     "mfma_frac": round(flops / (mean_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 5)},
        "device": torch.cuda.get_device_name(0),
        "device_meta": device_meta(),
    }
    if not args.no_reference:
        # the same kernel on one copy of W and R, timed right after the metric: after the first
        # call they are served from the 256 MB Infinity Cache, so the gap to the rotated figure
        # shows that the rotation defeats it
        _, _, one_us, one_gbs = measure(sk, OneCopy(wl), cfg, args.calls, args.warmup, args.steps)
        ref = {"op_one_copy_cache_warm": {"us": round(one_us, 4), "gbs": round(one_gbs, 2),
                                          "note": "one W/R copy, cache-resident after the first call; not the metric"}}
        ref.update(reference_rows(sk, wl, args.calls, max(2, args.warmup // 4), max(5, args.steps // 5)))
        ref["op_frac_of_stream_read"] = round(gbs / ref["stream_read_best_gbs"], 4)
        row["reference"] = ref
    try:
        row["parity_max_ulp_sampled"] = oracle_parity_sample(wl, launch)
        row["secondary_correctness"] = secondary_correctness(wl, launch)
    except Exception as e:  # noqa: BLE001
        row["parity_error"] = "%s: %s" % (type(e).__name__, e)
    if not args.no_curve:
        del wl
        torch.cuda.empty_cache()
        row["curve"], row["m64_valu_vs_mfma"] = run_curve(args, sk)
    if not args.no_cpu_baseline:
        row["cpu_baseline"] = cpu_baseline(M, args.cpu_seconds)
    print(json.dumps(row), flush=True)


def device_meta() -> dict:
    """What the rows are measured on: device name, gfx architecture, CU count, HIP and torch
    versions, the host's usable cores (the CPU oracle's baseline runs there), and the
    SKINNY_CONFIG override when one replaced the library's table for this run."""
    import torch
    p = torch.cuda.get_device_properties(0)
    return {"device": torch.cuda.get_device_name(0), "arch": getattr(p, "gcnArchName", None),
            "cus": p.multi_processor_count, "hip": torch.version.hip, "torch": torch.__version__,
            "host_cores": len(os.sched_getaffinity(0)), "skinny_config_env": os.environ.get("SKINNY_CONFIG")}


def done_rows(path):
    """(m, n, k, config) of the valid rows already in a JSONL file: a sweep given the same --out
    with --resume skips them, so an interrupted sweep continues where it stopped."""
    keys = set()
    if path and os.path.exists(path):
        for line in open(path):
            try:
                r = json.loads(line)
            except ValueError:
                continue
            if r.get("valid", True) and "config" in r and "m" in r:
                keys.add((r["m"], r.get("n"), r.get("k"), json.dumps(r["config"], sort_keys=True)))
    return keys


def sweep_rows(args, sk, Ms, config_lists):
    import torch
    from decode_skinny_addmm_amd._lib import PATH_SIMT
    done = done_rows(args.out) if getattr(args, "resume", False) else set()
    out = open(args.out, "a") if args.out else None
    meta = device_meta()
    for M in Ms:
        todo = [c for c in config_lists(M)
                if (M, args.n, args.k, json.dumps(c, sort_keys=True)) not in done]
        if not todo:
            continue
        wl = Workload(M, args.copies, args.n, args.k)
        for cfg in todo:
            row = {"m": M, "n": wl.N, "k": wl.K, "config": cfg, "copies": args.copies,
                   "calls": args.calls, **meta}
            if cfg.get("path") == PATH_SIMT:
                # the pages' kernels need K to be a whole number of block_size*vector_width
                # tiles, k_unroll at a time; this family takes a predicated tail instead
                tile = cfg["block_size"] * cfg["vector_width"]
                row["tail_free"] = wl.K % tile == 0 and (wl.K // tile) % cfg["k_unroll"] == 0
            try:
                launch, samples, mean_us, gbs = measure(sk, wl, cfg, args.calls, args.warmup, args.steps)
                row.update(summarize(samples))
                row.update({"mean_us_total": mean_us, "gbs": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
                            "mfma_frac": 2.0 * M * wl.N * wl.K / (mean_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                            "resources": sk.config_resources(cfg) if cfg.get("m_tile") else None,
                            "max_ulp_sampled": oracle_parity_sample(wl, launch, 256)})
            except Exception as e:  # noqa: BLE001
                row.update({"valid": False, "error": "%s: %s" % (type(e).__name__, e)})
            line = json.dumps(row, sort_keys=True)
            log(line)
            if out:
                out.write(line + "\n")
                out.flush()
        del wl
        torch.cuda.empty_cache()
    if out:
        out.close()


def run_shard(args, sk):
    """The tensor-parallel shard form: N = 7168/shards columns per rank, W rotated over enough
    copies to exceed L2 and the Infinity Cache, R read from and Y written into column blocks of
    the full-width matrices, both shard-epilogue flags on (two roundings, no -0)."""
    import numpy as np
    import torch

    import oracle
    from decode_skinny_addmm_amd import synth
    Ms = [int(x) for x in args.ms.split(",")] if args.ms else [1, 2, 4, 8]
    N = N_DIM // args.shards
    copies = args.copies if args.copies != 6 else max(40, -(-308_000_000 // (N * K_DIM * 2)))
    configs = None
    if args.paths:
        paths = {int(x) for x in args.paths.split(",")}
    out = open(args.out, "a") if args.out else None
    for M in Ms:
        wl = ShardWorkload(M, copies, args.shards, args.rank)
        if args.mode == "shard-sweep":
            configs = config_shard(args, [c for c in sk.configs()
                                          if -(-M // c["m_tile"]) <= 4 and (not args.paths or c["path"] in paths)])
        for cfg in (configs or [args.config or sk.select_config(M, N)]):
            def launch(X, W, R, Y, cfg=cfg):
                return sk.addmm_shard(X, W, R, out=Y, round_product=True, no_neg_zero=True, config=cfg)
            row = {"mode": "shard", "m": M, "n": N, "k": K_DIM, "n_total": N_DIM, "shards": args.shards,
                   "rank": args.rank, "copies": copies, "calls": args.calls, "config": cfg}
            try:
                per, total_ms = time_graph(launch, wl, args.calls, args.warmup, args.steps)
                us = [p / args.calls for p in per]
                mean_us = total_ms * 1000.0 / (args.steps * args.calls)
                nbytes = algorithmic_bytes(M, N, K_DIM)
                row.update(summarize(us))
                row.update({"mean_us_total": mean_us, "gbs": nbytes / (mean_us * 1e-6) / 1e9,
                            "frac_hbm": nbytes / (mean_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                            "bytes_per_launch": nbytes})
                # sampled parity against the oracle with the same flags (two roundings: the result
                # can sit one bf16 step of the rounded product away from the oracle's)
                X, W, R = wl.host
                Y = torch.zeros_like(wl.Rwide[0])
                Yv = Y[:, wl.c0:wl.c0 + N]
                launch(wl.X, wl.W[0], wl.R[0], Yv)
                torch.cuda.synchronize()
                rng = np.random.default_rng(0)
                ms = rng.integers(0, M, 256)
                ns = rng.integers(0, N, 256)
                yo, _ = oracle.addmm_bf16_points(synth.bits(X), synth.bits(W), synth.bits(R), ms, ns,
                                                 flags=oracle.ROUND_PRODUCT | oracle.NO_NEG_ZERO)
                yg = synth.bits(Yv.contiguous())[ms, ns]
                row["matches_oracle_frac"] = float(np.mean(yg == yo))
            except Exception as e:  # noqa: BLE001
                row.update({"valid": False, "error": "%s: %s" % (type(e).__name__, e)})
            line = json.dumps(row, sort_keys=True)
            print(line, flush=True)
            if out:
                out.write(line + "\n")
                out.flush()
        del wl
        torch.cuda.empty_cache()
    if out:
        out.close()


def run_kbit(args, sk):
    """The k-bit quantized GEMV at N = 7168, K = 3584: per (k, M) one JSON row with the mean
    launch time, algorithmic GB/s and roofline fraction, the dense bf16 kernel at the same M
    for context, and a full comparison of copy 0 against the oracle."""
    import numpy as np
    import torch

    import oracle
    Ms = [int(x) for x in args.ms.split(",")] if args.ms else [1, 2, 4, 16]
    kbs = [int(x) for x in args.kbits.split(",")]
    out = open(args.out, "a") if args.out else None
    for kb in kbs:
        per_copy = N_DIM * (K_DIM // 32) * (4 * kb + 1)
        copies = max(8, -(-308_000_000 // per_copy))
        for M in Ms:
            wl = KbitWorkload(M, copies, kb)

            def launch(X, W, R, Y, wl=wl):
                return sk.kbit_gemv(X, W[0], W[1], wl.cb, wl.kbits, R, out=Y)
            row = {"mode": "kbit", "kbits": kb, "m": M, "n": N_DIM, "k": K_DIM, "copies": copies,
                   "calls": args.calls}
            try:
                per, total_ms = time_graph(launch, wl, args.calls, args.warmup, args.steps)
                us = [p / args.calls for p in per]
                mean_us = total_ms * 1000.0 / (args.steps * args.calls)
                nbytes = kbit_algorithmic_bytes(M, N_DIM, K_DIM, kb)
                row.update(summarize(us))
                row.update({"mean_us_total": mean_us, "gbs": nbytes / (mean_us * 1e-6) / 1e9,
                            "frac_hbm": nbytes / (mean_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                            "bytes_per_launch": nbytes})
                X, pl, am, R, cb = wl.host
                Y = launch(wl.X, wl.W[0], wl.R[0], torch.empty_like(wl.R[0]))
                torch.cuda.synchronize()
                yo, _ = oracle.kbit_gemv_bf16(synth_bits(X), pl.numpy().view(np.uint32), am.numpy(), cb.numpy(),
                                              kb, synth_bits(R))
                row["matches_oracle_frac"] = float(np.mean(synth_bits(Y.cpu()) == yo))
            except Exception as e:  # noqa: BLE001
                row.update({"valid": False, "error": "%s: %s" % (type(e).__name__, e)})
            line = json.dumps(row, sort_keys=True)
            print(line, flush=True)
            if out:
                out.write(line + "\n")
                out.flush()
            del wl
            torch.cuda.empty_cache()
    if out:
        out.close()


def run_kda(args, sk):
    """The KDA verify step at the page's layer shape, per (B, mode): one JSON row with the mean
    call time (graph replays of --calls launches rotating over copies of the states and
    outputs), algorithmic GB/s and roofline fraction, and a sampled check against the oracle."""
    import numpy as np
    import torch

    import oracle
    from decode_skinny_addmm_amd import synth
    T, H, HV, K, V = 4, 8, 8, 128, 128
    Bs = [int(x) for x in args.ms.split(",")] if args.ms else [1, 4, 16, 64]
    layouts = args.layouts.split(",")
    if not layouts or any(lay not in ("snapshots", "ring") for lay in layouts):
        raise SystemExit("--layouts takes a comma-separated list of snapshots and ring")
    out = open(args.out, "a") if args.out else None
    for B in Bs:
        for ring in [lay == "ring" for lay in layouts]:
            base = synth.make_kda_inputs(B, T=T, H=H, HV=HV, K=K, V=V)
            per_copy = B * HV * V * K * 4 * (1 if ring else 1 + T)
            copies = max(2, min(256, -(-320_000_000 // per_copy)))
            shared = {k: v.cuda() for k, v in base.items() if k not in ("ssm", "inter_ssm", "rawv", "rawk", "g", "beta")}
            per = []
            for c in range(copies):
                d = dict(shared)
                d["ssm"] = base["ssm"].cuda()
                if ring:
                    for k in ("rawv", "rawk", "g", "beta"):
                        d[k] = base[k].cuda()
                else:
                    d["inter_ssm"] = torch.empty_like(base["inter_ssm"], device="cuda")
                per.append(d)
            outs = [torch.empty((B * T, HV, V), dtype=torch.bfloat16, device="cuda") for _ in range(copies)]
            scale = K ** -0.5

            class W:  # what time_graph expects: X, W[i], R[i], Y[i], copies
                pass
            wl = W()
            wl.copies, wl.X, wl.W, wl.R, wl.Y = copies, None, per, [None] * copies, outs

            def launch(X, Wc, R, Y):
                return sk.kda_verify(Wc, T, H, HV, K, V, scale, snapshots=not ring, ring=ring, out=Y)
            row = {"mode": "kda", "B": B, "T": T, "H": H, "HV": HV, "K": K, "V": V,
                   "layout": "ring" if ring else "snapshots", "copies": copies, "calls": args.calls}
            try:
                per_us, total_ms = time_graph(launch, wl, args.calls, args.warmup, args.steps)
                us = [p / args.calls for p in per_us]
                mean_us = total_ms * 1000.0 / (args.steps * args.calls)
                nbytes = kda_algorithmic_bytes(B, T, H, HV, K, V, ring)
                row.update(summarize(us))
                row.update({"mean_us_total": mean_us, "gbs": nbytes / (mean_us * 1e-6) / 1e9,
                            "frac_hbm": nbytes / (mean_us * 1e-6) / 1e9 / HBM_PEAK_GBS, "bytes_per_launch": nbytes})
                # copy 0 against the oracle: output bits within 2 bf16 steps
                o = launch(None, per[0], None, outs[0])
                torch.cuda.synchronize()
                ref = oracle.kda_verify(synth.kda_to_numpy(base), T, H, HV, K, V, scale, snapshots=not ring,
                                        ring_len=16 if ring else 0)
                g = synth.bits(o.cpu()).astype(np.int64)
                r = ref["o"].astype(np.int64)
                ordered = lambda b: np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)
                row["o_within_2ulp_frac"] = float(np.mean(np.abs(ordered(g) - ordered(r)) <= 2))
            except Exception as e:  # noqa: BLE001
                row.update({"valid": False, "error": "%s: %s" % (type(e).__name__, e)})
            line = json.dumps(row, sort_keys=True)
            print(line, flush=True)
            if out:
                out.write(line + "\n")
                out.flush()
            del per, outs, shared
            torch.cuda.empty_cache()
    if out:
        out.close()


def synth_bits(t):
    from decode_skinny_addmm_amd import synth
    return synth.bits(t)


def main():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100, help="timed graph replays")
    p.add_argument("--warmup", type=int, default=20, help="untimed graph replays")
    p.add_argument("--m", type=int, default=None)
    p.add_argument("--copies", type=int, default=6)
    p.add_argument("--calls", type=int, default=500, help="launches captured per graph (one step)")
    p.add_argument("--config", type=parse_config, default=None)
    p.add_argument("--mode", choices=("default", "sweep", "mcurve", "probe", "calib", "shard", "shard-sweep",
                                        "kbit", "kda"),
                   default="default")
    p.add_argument("--shards", type=int, default=8, help="shard/shard-sweep: ranks the 7168 columns split over")
    p.add_argument("--rank", type=int, default=3, help="shard/shard-sweep: which rank's column block")
    p.add_argument("--kbits", type=str, default="2,3,4,5", help="kbit: comma-separated bits per weight")
    p.add_argument("--layouts", type=str, default="snapshots,ring",
                   help="kda: comma-separated state layouts to time (snapshots, ring)")
    p.add_argument("--out", type=str, default=None)
    p.add_argument("--resume", action="store_true",
                   help="sweep/mcurve: skip the (M, N, K, config) rows already valid in --out")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-reference", action="store_true", help="skip the null/stream-read reference rows")
    p.add_argument("--no-curve", action="store_true", help="default mode: skip the M = 1 ... 256 curve")
    p.add_argument("--ms", type=str, default=None, help="comma-separated M list for sweep/mcurve")
    p.add_argument("--n", type=int, default=N_DIM, help="sweep/mcurve: N (rows of W); the default run uses 7168")
    p.add_argument("--k", type=int, default=K_DIM, help="sweep/mcurve: K; the default run uses 3584")
    p.add_argument("--paths", type=str, default=None, help="sweep only these kernel paths (comma-separated ids)")
    p.add_argument("--config-shard", type=int, default=0,
                   help="sweep/shard-sweep: time candidates i, i + n, i + 2n, ... of each M's list")
    p.add_argument("--num-config-shards", type=int, default=1,
                   help="sweep/shard-sweep: n, the number of shards the candidate lists are split into")
    p.add_argument("--with-torch", action="store_true",
                   help="mcurve: add torch.addmm (the vendor library) as a context row")
    args = p.parse_args()
    if args.num_config_shards < 1 or not 0 <= args.config_shard < args.num_config_shards:
        print("--config-shard must lie in [0, --num-config-shards)", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path (got --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import decode_skinny_addmm_amd as sk
    sk.ops.lib()
    if args.mode == "default":
        args.m = args.m or 4
        run_default(args, sk)
    elif args.mode == "probe":
        run_probe(args, sk)
    elif args.mode == "calib":
        run_calib(args, sk)
    elif args.mode in ("shard", "shard-sweep"):
        run_shard(args, sk)
    elif args.mode == "kbit":
        run_kbit(args, sk)
    elif args.mode == "kda":
        run_kda(args, sk)
    elif args.mode == "sweep":
        Ms = [int(x) for x in args.ms.split(",")] if args.ms else [args.m or 16]
        paths = {int(x) for x in args.paths.split(",")} if args.paths else None
        # configurations that would re-read W more than 4 times (ceil(M / m_tile) passes) are
        # skipped: they are never competitive and take long to time
        sweep_rows(args, sk, Ms, lambda m: config_shard(args, [c for c in sk.configs()
                                                               if -(-m // c["m_tile"]) <= 4
                                                               and (paths is None or c["path"] in paths)]))
    else:
        Ms = [int(x) for x in args.ms.split(",")] if args.ms else (
            [args.m] if args.m else [1, 2, 4, 8, 16, 32, 64, 128, 256])
        sweep_rows(args, sk, Ms, lambda m: [args.config or sk.select_config(m)] +
                   ([{"reference": "torch.addmm"}] if args.with_torch else []))


if __name__ == "__main__":
    main()
