"""Host-only checks of the C ABI library: it loads, exports every declared symbol, and its
argument checks answer before anything is launched (no GPU needed)."""
import ctypes
import os
import re

import pytest

from decode_skinny_addmm_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("skinny.h", "skinny_probe.h")]


def declared_functions():
    txt = "".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"SKINNY_API\s+[\w\s\*]+?\b(skinny_\w+)\s*\(", txt)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libskinny.so not built")
    return _lib.lib()


def test_header_declares_the_boundary():
    names = declared_functions()
    for f in ("skinny_addmm_bf16", "skinny_select_config", "skinny_addmm_bf16_with_config",
              "skinny_addmm_bf16_acc_f32", "skinny_status_string"):
        assert f in names
    assert set(names) == set(_lib.EXPORTED)


def test_every_declared_symbol_is_exported(L):
    for f in declared_functions():
        assert hasattr(L, f), f


def test_only_declared_symbols_are_exported():
    out = os.popen("nm -D --defined-only %s" % _lib.LIB_PATH).read()
    syms = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert syms == set(declared_functions())


def test_select_config_covers_all_m(L):
    seen = set()
    for M in list(range(1, 300)) + [1000, 100000]:
        c = _lib.SkinnyConfig()
        assert L.skinny_select_config(M, 7168, 3584, ctypes.byref(c)) == 0
        d = c.as_dict()
        assert d["block_size"] % 64 == 0 and d["m_tile"] >= 1 and d["path"] in (0, 1, 2, 3, 4, 5, 6, 7)
        seen.add(tuple(d.values()))
    # every selected configuration is built into the library
    built = set()
    for i in range(L.skinny_num_configs()):
        c = _lib.SkinnyConfig()
        assert L.skinny_get_config(i, ctypes.byref(c)) == 0
        built.add(tuple(c.as_dict().values()))
    assert seen <= built
    assert L.skinny_select_config(1, 1, 8, None) == 1
    assert L.skinny_select_config(-1, 1, 8, ctypes.byref(_lib.SkinnyConfig())) == 1


@pytest.mark.parametrize("N", [7168, 896])
def test_table_rows_resolve_without_fallback(L, N):
    """At the tuned K every table row (full width and narrow) names a built instance: the
    general fallbacks (direct MFMA, register GEMM) are only for K the table's kernels cannot
    take, so selecting one here would mean a mistyped row."""
    for M in list(range(1, 300)) + [1000]:
        c = _lib.SkinnyConfig()
        assert L.skinny_select_config(M, N, 3584, ctypes.byref(c)) == 0
        assert c.as_dict()["path"] not in (1, 3), (M, N, c.as_dict())


def test_full_oracle_parity_reaches_every_selected_config(L):
    """Every configuration the table selects at N = 7168, K = 3584 for M = 1 ... 300 is one that
    the full-output GPU parity tests run (their M lists live in parity.py), so a new or changed
    table row cannot go without a full comparison with the oracle."""
    import parity as P

    def sel(M):
        c = _lib.SkinnyConfig()
        assert L.skinny_select_config(M, 7168, 3584, ctypes.byref(c)) == 0
        return tuple(c.as_dict().values())

    tested = {sel(M) for M in P.FULL_ORACLE_SMALL_M + P.FULL_ORACLE_LARGE_M}
    missing = {(M, sel(M)) for M in range(1, 301) if sel(M) not in tested}
    assert not missing, sorted(missing)[:5]


@pytest.mark.parametrize("M,K,path,k_stage", [
    (8, 1032, 2, 0),        # not a whole number of 128-wide stages: LDS-MFMA (any K up to 3584)
    (8, 4104, 1, 0),        # beyond the LDS-MFMA slice as well: the direct MFMA fallback
    (48, 3712, 7, 128),     # not a whole number of 256-wide stages: 128-wide ones
    (48, 1032, 3, 0),       # neither: the register GEMM fallback
])
def test_second_choice_when_the_row_cannot_take_k(L, M, K, path, k_stage):
    """A table row whose kernel cannot take K gives way to the M range's second choice before
    the general fallback."""
    c = _lib.SkinnyConfig()
    assert L.skinny_select_config(M, 7168, K, ctypes.byref(c)) == 0
    d = c.as_dict()
    assert (d["path"], d["k_stage"]) == (path, k_stage), d


ENV_PROBE = r"""
import ctypes, json, sys
sys.path.insert(0, sys.argv[1])
from decode_skinny_addmm_amd import _lib
L = _lib.lib()
c = _lib.SkinnyConfig()
sel = L.skinny_select_config(4, 7168, 3584, ctypes.byref(c))
built = []
for i in range(L.skinny_num_configs()):
    b = _lib.SkinnyConfig()
    L.skinny_get_config(i, ctypes.byref(b))
    built.append(list(b.as_dict().values()))
call = None
if sys.argv[2] == "call":
    # only for values that fail before any launch (malformed, or not built): the pointers are fake
    assert sel != 0 or list(c.as_dict().values()) not in built
    fake = ctypes.c_void_p(4096)
    call = L.skinny_addmm_bf16(fake, fake, fake, fake, 1, 64, 64, None)
print(json.dumps({"sel": sel, "cfg": list(c.as_dict().values()), "call": call}))
"""


def run_env_probe(value, mode):
    import json
    import subprocess
    import sys
    env = dict(os.environ, SKINNY_CONFIG=value)
    out = subprocess.run([sys.executable, "-c", ENV_PROBE, ROOT, mode], env=env, capture_output=True,
                         text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    return json.loads(out.stdout.strip().splitlines()[-1])


@pytest.mark.parametrize("value,cfg", [
    ("2, 256, 32, 4, 8, 4", [2, 256, 32, 4, 8, 4, 1, 0]),           # trailing fields default to 1, 0
    ("6,512,64,4,8,128,2,64", [6, 512, 64, 4, 8, 128, 2, 64]),
    ("0,448,4,7,8", [0, 448, 4, 7, 8, 0, 1, 0])])
def test_env_config_replaces_the_table(L, value, cfg):
    """SKINNY_CONFIG replaces the table for calls that name no configuration (read once per
    process, so each case runs in a child process)."""
    r = run_env_probe(value, "select")
    assert r["sel"] == 0 and r["cfg"] == cfg


@pytest.mark.parametrize("value,sel,call", [
    ("2,256,32,4", 1, 1),             # too few fields
    ("2,256,32,4,8,4,1,0,9", 1, 1),   # too many
    ("2,256,x,4,8", 1, 1),            # not a number
    ("2,256,32,4,8,", 1, 1),          # empty field
    ("2;256;32;4;8", 1, 1),           # wrong separator
    ("0,64,1,1,8", 0, 3)])            # well formed but not built: the compute call says so
def test_env_config_errors(L, value, sel, call):
    r = run_env_probe(value, "call")
    assert r["sel"] == sel and r["call"] == call


def test_get_config_range(L):
    c = _lib.SkinnyConfig()
    assert L.skinny_get_config(-1, ctypes.byref(c)) == 1
    assert L.skinny_get_config(L.skinny_num_configs(), ctypes.byref(c)) == 1


def test_probe_argument_checks(L):
    assert L.skinny_probe_read(A16, -16, A16, 0, 4, None) == 1
    assert L.skinny_probe_read(A16, 24, A16, 0, 4, None) == 2
    assert L.skinny_probe_read(A16, 32, A16, 0, 3, None) == 1
    assert L.skinny_probe_read(A16, 0, A16, 0, 4, None) == 0
    assert L.skinny_probe_copy(A16, A16 + 8, 32, None) == 2
    assert L.skinny_probe_copy(None, None, 0, None) == 0


def test_status_strings(L):
    for s in range(5):
        assert len(L.skinny_status_string(s)) > 0
    assert L.skinny_status_string(99) == b"unknown status"
    assert L.skinny_version().decode().count(".") == 2


# Fake device addresses: every call below must be refused by the argument checks, which
# run before any HIP call, so nothing is dereferenced or launched.
A16 = 0x10000
A2 = 0x20002


@pytest.mark.parametrize("args,expect", [
    ((A16, A16, A16, A16, -1, 8, 8), 1),          # negative M
    ((A16, A16, A16, A16, 1, -8, 8), 1),          # negative N
    ((A16, A16, A16, A16, 1, 8, -8), 1),          # negative K
    ((A16, A16, A16, A16, 1, 8, 12), 3),          # K % 8 != 0
    ((A16, A16, None, A16, 1, 8, 8), 1),          # NULL residual
    ((A16, A16, A16, None, 1, 8, 8), 1),          # NULL output
    ((None, A16, A16, A16, 1, 8, 8), 1),          # NULL X with K > 0
    ((A16, None, A16, A16, 1, 8, 8), 1),          # NULL W with K > 0
    ((A16 + 8, A16, A16, A16, 1, 8, 8), 2),       # X not 16-byte aligned
    ((A16, A16 + 2, A16, A16, 1, 8, 8), 2),       # W not 16-byte aligned
    ((A16, A16, A2 + 1, A16, 1, 8, 8), 2),        # R odd address
    ((A16, A16, A16, A2 + 1, 1, 8, 8), 2),        # Y odd address
    ((None, None, None, None, 0, 8, 8), 0),       # M == 0: no-op
    ((None, None, None, None, 4, 0, 8), 0),       # N == 0: no-op
])
def test_argument_checks(L, args, expect):
    X, W, R, Y, M, N, K = args
    assert L.skinny_addmm_bf16(X, W, R, Y, M, N, K, None) == expect
    assert L.skinny_addmm_bf16_with_config(X, W, R, Y, M, N, K, None, None) == expect
    if expect != 2 or Y != A2 + 1:
        assert L.skinny_addmm_bf16_acc_f32(X, W, R, Y, M, N, K, None, None) == expect


def test_acc_needs_4_byte_alignment(L):
    assert L.skinny_addmm_bf16_acc_f32(A16, A16, A16, A2, 1, 8, 8, None, None) == 2


@pytest.mark.parametrize("cfg,expect", [
    ((0, 100, 4, 7, 8, 1, 1), 1),     # block not a multiple of 64
    ((0, 256, 0, 7, 8, 1, 1), 1),     # no outputs
    ((0, 256, 4, 7, 3, 1, 1), 1),     # vector width out of range
    ((0, 256, 4, 7, 11, 1, 1), 1),    # vector width out of range
    ((0, 256, 4, 0, 8, 1, 1), 1),     # k_unroll 0
    ((0, 256, 4, 7, 8, -1, 1), 1),    # negative m tile
    ((0, 1024, 4, 7, 8, 1, 1), 3),    # well-formed but not built
    ((9, 256, 4, 7, 8, 1, 1), 3),     # unknown path
])
def test_config_checks(L, cfg, expect):
    c = _lib.SkinnyConfig(*cfg)
    assert L.skinny_addmm_bf16_with_config(A16, A16, A16, A16, 1, 8, 8, ctypes.byref(c), None) == expect


@pytest.mark.parametrize("ldr,ldy,M,flags,out_is_r,expect", [
    (7, 8, 2, 0, False, 1),          # R pitch below N
    (8, 7, 2, 0, False, 1),          # Y pitch below N
    (-8, 8, 1, 0, False, 1),         # negative pitch
    (8, 8, 2, 4, False, 1),          # unknown flag bit
    (8, 16, 2, 0, True, 1),          # Y is R with another pitch
    (8, 8, 0, 3, False, 0),          # M == 0: no-op, flags known
])
def test_shard_argument_checks(L, ldr, ldy, M, flags, out_is_r, expect):
    Y = A16 if out_is_r else A16 + 0x1000
    assert L.skinny_addmm_bf16_shard(A16, A16, A16, ldr, Y, ldy, M, 8, 8, flags, None, None) == expect
    if not out_is_r:  # the fp32 test output never aliases R
        assert L.skinny_addmm_bf16_shard_acc_f32(A16, A16, A16, ldr, A16 + 0x1000, ldy, M, 8, 8, flags,
                                                 None, None) == expect


@pytest.mark.parametrize("args,expect", [
    ((A16, A16, A16, A16, 1, A16, A16, 1, 8, 64), 1),      # kbits below 2
    ((A16, A16, A16, A16, 6, A16, A16, 1, 8, 64), 1),      # kbits above 5
    ((A16, A16, A16, A16, 4, A16, A16, -1, 8, 64), 1),     # negative M
    ((A16, A16, A16, A16, 4, A16, A16, 1, 8, 48), 3),      # K % 32 != 0
    ((A16, A16, A16, A16, 4, A16, A16, 1, 8, 32 * 513), 3),  # K beyond one lane per block
    ((A16, A16, A16, None, 4, A16, A16, 1, 8, 64), 1),     # NULL codebook
    ((None, A16, A16, A16, 4, A16, A16, 1, 8, 64), 1),     # NULL X with K > 0
    ((A16, None, A16, A16, 4, A16, A16, 1, 8, 64), 1),     # NULL planes with K > 0
    ((A16, A16, A16, A16, 4, None, A16, 1, 8, 64), 1),     # NULL residual
    ((A16 + 8, A16, A16, A16, 4, A16, A16, 1, 8, 64), 2),  # X not 16-byte aligned
    ((A16, A16 + 2, A16, A16, 4, A16, A16, 1, 8, 64), 2),  # plane words not 4-byte aligned
    ((A16, A16, A16, A16 + 2, 4, A16, A16, 1, 8, 64), 2),  # codebook not 4-byte aligned
    ((A16, A16, A16, A16, 4, A2 + 1, A16, 1, 8, 64), 2),   # R odd address
    ((None, None, None, A16, 4, None, None, 0, 8, 64), 0),  # M == 0: no-op
])
def test_kbit_argument_checks(L, args, expect):
    assert L.skinny_kbit_gemv_bf16(*args, None) == expect
    if args[6] is not None:
        assert L.skinny_kbit_gemv_bf16_acc_f32(*args, None) == expect


def _kda_args(**over):
    base = dict(mixed=A16, conv_w=A16, conv_b=A16, conv_pool=A16, cache_idx=A16, inter_idx=A16, a=A16, b=A16,
                A_log=A16, dt_bias=A16, ssm=A16, conv_win=A16, snap=A16, ring_v=None, ring_k=None, ring_g=None,
                ring_beta=None, out=A16, B=2, T=4, H=1, HV=1, K=128, V=16, lines=3, slots=3, ring_len=0,
                scale=0.088)
    base.update(over)
    return _lib.SkinnyKdaArgs(**base)


@pytest.mark.parametrize("over,expect", [
    (dict(K=64), 3),                                   # head dimension other than 128
    (dict(T=17), 3),                                   # more than 16 draft tokens
    (dict(V=8), 3),                                    # V not a multiple of 16
    (dict(T=0), 1),                                    # no tokens
    (dict(H=2, HV=3), 1),                              # value heads not a multiple of q/k heads
    (dict(ring_v=A16), 1),                             # ring buffers given in part
    (dict(ring_v=A16, ring_k=A16, ring_g=A16, ring_beta=A16, ring_len=2), 1),   # ring shorter than T
    (dict(mixed=None), 1),                             # missing input
    (dict(inter_idx=None), 1),                         # windows/snapshots without their index
    (dict(ssm=A16 + 4), 2),                            # state not 16-byte aligned
    (dict(snap=A16 + 8), 2),                           # snapshots not 16-byte aligned
    (dict(mixed=A2 + 1), 2),                           # bf16 input at an odd address
    (dict(B=0, mixed=None, ssm=None), 0),              # empty batch: no-op
])
def test_kda_argument_checks(L, over, expect):
    args = _kda_args(**over)
    assert L.skinny_kda_verify_bf16(ctypes.byref(args), None) == expect


def test_kda_null_args(L):
    assert L.skinny_kda_verify_bf16(None, None) == 1


def test_kda_sizes_beyond_int_range(L):
    args = _kda_args(lines=2 ** 31)
    assert L.skinny_kda_verify_bf16(ctypes.byref(args), None) == 3
