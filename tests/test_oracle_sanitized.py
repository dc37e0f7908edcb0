"""The CPU oracle (oracle/*.c) built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc,
host code only) and run through every entry point on small inputs in a child process: an
out-of-bounds access, use of freed memory or undefined arithmetic in the oracle aborts the
child. CPU only."""
import os
import subprocess
import sys
import textwrap

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime():
    try:
        p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True, check=True)
    except (OSError, subprocess.CalledProcessError):
        return None
    path = p.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_under_asan_ubsan(tmp_path):
    asan = _runtime()
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    so = str(tmp_path / "liboracle_san.so")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
           oracle._SRC, oracle._KBIT_SRC, oracle._KDA_SRC, "-o", so, "-lm"]
    subprocess.run(cmd, check=True)
    script = textwrap.dedent("""
        import sys
        sys.path.insert(0, %r)
        sys.path.insert(0, %r)
        import numpy as np
        import oracle
        from decode_skinny_addmm_amd import synth
        orc = oracle.Oracle(%r)
        X, ws, rs = synth.make_inputs(3, 40, 72, seed=5)
        b = synth.bits
        orc.addmm_bf16(b(X), b(ws[0]), b(rs[0]), threads=2)
        orc.addmm_bf16(b(X), b(ws[0]), b(rs[0]), threads=1, flags=oracle.ROUND_PRODUCT | oracle.NO_NEG_ZERO)
        orc.addmm_bf16_points(b(X), b(ws[0]), b(rs[0]), np.array([0, 2]), np.array([5, 39]))
        orc.round_bf16(np.array([0.0, -1.5, 1e39, 1e-40]))
        for k in (2, 3, 4, 5):
            cb = orc.nf_codebook(k).astype(np.float32)
            W = oracle.bf16_bits_to_f64(b(ws[0]))[:, :64]
            planes, amax, _ = orc.kbit_quantize(W, k, cb)
            orc.kbit_dequant(planes, amax, cb, k)
            orc.kbit_gemv_bf16(b(X)[:, :64], planes, amax, cb, k, b(rs[0]))
        orc.e4m4_encode(np.array([0.0, 1e-6, 0.5, 40.0]))
        orc.e4m4_decode(np.arange(256, dtype=np.uint8))
        inp = synth.kda_to_numpy(synth.make_kda_inputs(2, T=3, H=1, HV=2, K=16, V=8))
        orc.kda_verify(inp, 3, 1, 2, 16, 8, 0.25, snapshots=True)
        orc.kda_verify(inp, 3, 1, 2, 16, 8, 0.25, snapshots=False, ring_len=16)
        print("sanitized oracle ok")
    """) % (ROOT, os.path.join(ROOT, "tests"), so)
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    p = subprocess.run([sys.executable, "-c", script], env=env, capture_output=True, text=True, timeout=600)
    assert p.returncode == 0 and "sanitized oracle ok" in p.stdout, (p.stdout[-2000:], p.stderr[-4000:])
