"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Inputs are the seeded synthetic tensors of decode_skinny_addmm_amd.synth; the oracle sees
the same bytes. Tolerances are those of tests/parity.py."""
import numpy as np
import pytest
import torch

import oracle
import parity as P
from decode_skinny_addmm_amd import synth

pytestmark = pytest.mark.gpu

N_FULL, K_FULL = 7168, 3584


@pytest.fixture(scope="module")
def sk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_skinny_addmm_amd as d
    d.ops.lib()  # raises if the library is missing: no fallback
    return d


def _dev(*ts):
    return [t.to("cuda") for t in ts]


def run_both(sk, X, W, R, config=None):
    Xd, Wd, Rd = _dev(X, W, R)
    Y = sk.addmm(Xd, Wd, Rd, config=config)
    A = sk.addmm_acc_f32(Xd, Wd, Rd, config=config)
    torch.cuda.synchronize()
    return P.bits_of(Y), A.cpu().numpy()


def full_oracle(X, W, R):
    return oracle.addmm_bf16(synth.bits(X), synth.bits(W), synth.bits(R))


SMALL_SHAPES = [(1, 64, 512), (3, 100, 1032), (5, 33, 3584), (8, 130, 776), (16, 257, 520),
                (17, 70, 264), (2, 1, 8), (4, 96, 4096 + 8), (1, 3, 24), (2, 20, 9000),
                (33, 70, 256), (65, 130, 1024), (130, 200, 384), (64, 64, 128)]


def refuses(cfg, K):
    """Instances that must refuse this K with SKINNY_ENOTSUP: GEMV and LDS-MFMA hold their K
    slice on chip; the direct-to-LDS GEMMs take whole K stages only (128 wide, or k_stage)."""
    return ((cfg["path"] == 0 and K > cfg["k_unroll"] * cfg["k_split"] * 512) or
            (cfg["path"] == 2 and K > cfg["k_split"] * 512) or
            (cfg["path"] == 5 and K % 128 != 0) or
            (cfg["path"] in (6, 7) and K % cfg["k_stage"] != 0))


def all_configs(sk, K=None):
    return [c for c in sk.configs() if K is None or not refuses(c, K)]


def test_small_shapes_every_config(sk):
    for (M, N, K) in SMALL_SHAPES:
        X, ws, rs = synth.make_inputs(M, N, K)
        Yo, Ao = full_oracle(X, ws[0], rs[0])
        for cfg in all_configs(sk):
            print("small shape", (M, N, K), "config", cfg, flush=True)
            if refuses(cfg, K):
                with pytest.raises(sk.ops.SkinnyError) as ei:
                    run_both(sk, X, ws[0], rs[0], cfg)
                assert ei.value.status == 3
                continue
            Yg, Ag = run_both(sk, X, ws[0], rs[0], cfg)
            P.check_y(Yg, Yo, Ao, "Y %s %s" % ((M, N, K), cfg))
            P.check_acc(Ag, Ao, "ACC %s %s" % ((M, N, K), cfg))
            assert np.array_equal(Yg.reshape(-1), P.rne_torch(Ag).reshape(-1)), "Y != RNE(ACC)"


@pytest.mark.parametrize("M", P.FULL_ORACLE_SMALL_M)
def test_full_size_full_oracle(sk, M):
    """Full N x K problem, every output against the oracle, at the selected configuration."""
    X, ws, rs = synth.make_inputs(M, N_FULL, K_FULL)
    print("full size M=%d config %s" % (M, sk.select_config(M)), flush=True)
    Yg, Ag = run_both(sk, X, ws[0], rs[0])
    Yo, Ao = full_oracle(X, ws[0], rs[0])
    st = P.check_y(Yg, Yo, Ao, "M=%d" % M)
    P.check_acc(Ag, Ao, "M=%d" % M)
    assert np.array_equal(Yg.reshape(-1), P.rne_torch(Ag).reshape(-1))
    print(st)


def sample_positions(M, N, count, seed):
    rng = np.random.default_rng(seed)
    ms = list(rng.integers(0, M, count))
    ns = list(rng.integers(0, N, count))
    # corners and tile edges
    for m in {0, M - 1, M // 2}:
        for n in (0, 1, 15, 16, 63, 64, N // 2, N - 2, N - 1):
            ms.append(m)
            ns.append(n)
    return np.array(ms, np.int64), np.array(ns, np.int64)


@pytest.mark.parametrize("M", P.FULL_ORACLE_LARGE_M)
def test_full_size_full_oracle_large_m(sk, M):
    """Every table row above M = 16 (and the M just past each boundary) at the full N x K
    problem: every output against the oracle, at the selected configuration."""
    X, ws, rs = synth.make_inputs(M, N_FULL, K_FULL)
    print("full size M=%d config %s" % (M, sk.select_config(M)), flush=True)
    Yg, Ag = run_both(sk, X, ws[0], rs[0])
    Yo, Ao = full_oracle(X, ws[0], rs[0])
    st = P.check_y(Yg, Yo, Ao, "M=%d" % M)
    P.check_acc(Ag, Ao, "M=%d" % M)
    assert np.array_equal(Yg.reshape(-1), P.rne_torch(Ag).reshape(-1))
    print(st)


@pytest.mark.parametrize("M", [4, 16])
def test_every_config_full_size_sampled(sk, M):
    X, ws, rs = synth.make_inputs(M, N_FULL, K_FULL)
    ms, ns = sample_positions(M, N_FULL, 2000, 100 + M)
    yo, ao = oracle.addmm_bf16_points(synth.bits(X), synth.bits(ws[0]), synth.bits(rs[0]), ms, ns)
    for cfg in all_configs(sk):
        print("full size M=%d config %s" % (M, cfg), flush=True)
        Yg, Ag = run_both(sk, X, ws[0], rs[0], cfg)
        P.check_y(Yg[ms, ns], yo, ao, "M=%d %s" % (M, cfg))
        P.check_acc(Ag[ms, ns], ao, "M=%d %s" % (M, cfg))


@pytest.mark.parametrize("M", [64, 256])
def test_matrix_core_configs_full_size_sampled(sk, M):
    """Every matrix-core K-loop instance (direct MFMA, GEMM, direct-to-LDS GEMM) at the full
    problem size and large M: sampled outputs against the oracle."""
    X, ws, rs = synth.make_inputs(M, N_FULL, K_FULL)
    ms, ns = sample_positions(M, N_FULL, 2000, 200 + M)
    yo, ao = oracle.addmm_bf16_points(synth.bits(X), synth.bits(ws[0]), synth.bits(rs[0]), ms, ns)
    for cfg in all_configs(sk, K_FULL):
        if cfg["path"] not in (1, 3, 5, 6, 7):
            continue
        print("full size M=%d config %s" % (M, cfg), flush=True)
        Yg, Ag = run_both(sk, X, ws[0], rs[0], cfg)
        P.check_y(Yg[ms, ns], yo, ao, "M=%d %s" % (M, cfg))
        P.check_acc(Ag[ms, ns], ao, "M=%d %s" % (M, cfg))
        assert np.array_equal(Yg.reshape(-1), P.rne_torch(Ag).reshape(-1))


@pytest.mark.parametrize("M,N,K", [(1, 300, 4104), (4, 256, 8), (16, 200, 9000), (64, 130, 24),
                                   (300, 1000, 1032), (257, 515, 3584), (33, 70, 512),
                                   (8, 300, 1032), (48, 300, 3712)])
def test_selected_config_any_shape(sk, M, N, K):
    """The library's own choice (tuned table, with its second choices and fallbacks for other K)
    at shapes off the tuned one: ragged N, K outside a kernel's on-chip slice or not a whole
    number of its stages, M above the table."""
    X, ws, rs = synth.make_inputs(M, N, K, seed=M + N + K)
    print("selected config", (M, N, K), sk.select_config(M, N, K), flush=True)
    Xd, Wd, Rd = _dev(X, ws[0], rs[0])
    Y = sk.addmm_default(Xd, Wd, Rd, torch.empty_like(Rd))
    A = sk.addmm_acc_f32(Xd, Wd, Rd)
    torch.cuda.synchronize()
    Yg, Ag = P.bits_of(Y), A.cpu().numpy()
    ms, ns = sample_positions(M, N, 1500, K)
    yo, ao = oracle.addmm_bf16_points(synth.bits(X), synth.bits(ws[0]), synth.bits(rs[0]), ms, ns)
    P.check_y(Yg[ms, ns], yo, ao, "selected %s" % ((M, N, K),))
    P.check_acc(Ag[ms, ns], ao, "selected %s" % ((M, N, K),))
    assert np.array_equal(Yg.reshape(-1), P.rne_torch(Ag).reshape(-1))


# ------------------------------------------------------------------ exact cases (bit-exact)

@pytest.mark.parametrize("M,N,K", [(4, N_FULL, K_FULL), (3, 77, 264), (70, 150, 640)])
def test_x_zero_gives_r(sk, M, N, K):
    _, ws, rs = synth.make_inputs(M, N, K)
    X = torch.zeros((M, K), dtype=torch.bfloat16)
    for cfg in [None] + all_configs(sk, K):
        Yg, _ = run_both(sk, X, ws[0], rs[0], cfg)
        Rb = synth.bits(rs[0])
        same = (Yg == Rb) | (((Yg & 0x7FFF) == 0) & ((Rb & 0x7FFF) == 0))
        assert same.all(), cfg


@pytest.mark.parametrize("M,N,K", [(4, N_FULL, K_FULL), (16, 130, 520), (70, 150, 640)])
def test_one_hot_rows(sk, M, N, K):
    X, _, rs = synth.make_inputs(M, N, K, seed=21)
    cols = (np.arange(N) * 131 + 7) % K
    W = synth.one_hot_rows(N, K, cols)
    Yo, Ao = full_oracle(X, W, rs[0])
    for cfg in [None] + all_configs(sk, K):
        Yg, Ag = run_both(sk, X, W, rs[0], cfg)
        assert np.array_equal(Yg, Yo), cfg
        assert np.array_equal(Ag.astype(np.float64), Ao), cfg


@pytest.mark.parametrize("M,N,K", [(4, N_FULL, K_FULL), (8, 100, 1032), (40, 100, 1024)])
def test_small_integers_exact(sk, M, N, K):
    X, W, R = synth.small_int_inputs(M, N, K)
    Yo, Ao = full_oracle(X, W, R)
    for cfg in [None] + all_configs(sk, K):
        Yg, Ag = run_both(sk, X, W, R, cfg)
        assert np.array_equal(Ag.astype(np.float64), Ao), cfg
        assert np.array_equal(Yg, Yo), cfg


# ------------------------------------------------------------------ edge cases

def test_k_zero_gives_r(sk):
    M, N = 3, 50
    R = synth.make_inputs(M, N, 8)[2][0]
    X = torch.empty((M, 0), dtype=torch.bfloat16)
    W = torch.empty((N, 0), dtype=torch.bfloat16)
    Yg, Ag = run_both(sk, X, W, R)
    assert np.array_equal(Yg, synth.bits(R))


def test_empty_m_and_n_are_noops(sk):
    X = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda")
    R = torch.zeros((0, 8), dtype=torch.bfloat16, device="cuda")
    Y = sk.addmm(X, W, R)
    assert Y.shape == (0, 8)
    X = torch.zeros((2, 64), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    R = torch.zeros((2, 0), dtype=torch.bfloat16, device="cuda")
    assert sk.addmm(X, W, R).shape == (2, 0)


@pytest.mark.parametrize("M", [1, 4, 16, 64, 256])
def test_in_place_residual(sk, M):
    X, ws, rs = synth.make_inputs(M, N_FULL, K_FULL)
    Xd, Wd, Rd = _dev(X, ws[0], rs[0])
    Y = sk.addmm(Xd, Wd, Rd)
    R2 = Rd.clone()
    sk.addmm(Xd, Wd, R2, out=R2)
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), R2.view(torch.int16))


def test_poisoned_output_fully_written(sk):
    for M in (1, 2, 5, 16, 33, 100, 257):
        X, ws, rs = synth.make_inputs(M, 1000, 1024)
        Xd, Wd, Rd = _dev(X, ws[0], rs[0])
        Y = torch.full_like(Rd, float("nan"))
        sk.addmm(Xd, Wd, Rd, out=Y)
        torch.cuda.synchronize()
        assert not torch.isnan(Y.float()).any(), M


def test_misaligned_and_bad_arguments_raise(sk):
    X, ws, rs = synth.make_inputs(2, 64, 72)
    Xd, Wd, Rd = _dev(X, ws[0], rs[0])
    big = torch.zeros(2 * 72 + 8, dtype=torch.bfloat16, device="cuda")
    Xmis = big[1:1 + 2 * 72].view(2, 72)  # 2-byte offset: not 16-byte aligned
    with pytest.raises(sk.ops.SkinnyError if hasattr(sk.ops, "SkinnyError") else RuntimeError):
        sk.addmm(Xmis, Wd, Rd)
    with pytest.raises(ValueError):
        sk.addmm(Xd.float(), Wd, Rd)
    with pytest.raises(ValueError):
        sk.addmm(Xd, Wd.t(), Rd)
    with pytest.raises(ValueError):
        sk.addmm(Xd.cpu(), Wd, Rd)
    # the output may be R itself, but never overlap X or W or only part of R
    buf = torch.zeros(2 * 72 + 2 * 64 + 16, dtype=torch.bfloat16, device="cuda")
    Xa = buf[:2 * 72].view(2, 72)
    Xa.copy_(Xd)
    with pytest.raises(ValueError):
        sk.addmm(Xa, Wd, Rd, out=buf[2 * 72 - 8:2 * 72 - 8 + 2 * 64].view(2, 64))
    Rb = buf[2 * 72:2 * 72 + 2 * 64].view(2, 64)
    Rb.copy_(Rd)
    with pytest.raises(ValueError):
        sk.addmm(Xd, Wd, Rb, out=buf[2 * 72 + 8:2 * 72 + 8 + 2 * 64].view(2, 64))
    with pytest.raises(ValueError):
        sk.addmm(Xd, Wd, Rd, out=Wd.view(-1)[:2 * 64].view(2, 64))
    Xk = torch.zeros((2, 12), dtype=torch.bfloat16, device="cuda")
    Wk = torch.zeros((64, 12), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError):
        sk.addmm(Xk, Wk, Rd)  # K % 8 != 0 -> SKINNY_ENOTSUP


# ------------------------------------------------------------------ determinism and graphs

@pytest.mark.parametrize("M", [4, 64, 256])
def test_deterministic_and_default_entry(sk, M):
    X, ws, rs = synth.make_inputs(M, N_FULL, K_FULL)
    Xd, Wd, Rd = _dev(X, ws[0], rs[0])
    a = sk.addmm(Xd, Wd, Rd)
    b = sk.addmm(Xd, Wd, Rd)
    c = sk.addmm_default(Xd, Wd, Rd, torch.empty_like(Rd))
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))


@pytest.mark.parametrize("M", [4, 64, 256])
def test_graph_replay_matches_eager(sk, M):
    print("graph replay M=%d config %s" % (M, sk.select_config(M)), flush=True)
    X, ws, rs = synth.make_inputs(M, N_FULL, K_FULL, copies=3)
    Xd = X.cuda()
    Wds = [w.cuda() for w in ws]
    Rds = [r.cuda() for r in rs]
    eager = [sk.addmm(Xd, w, r) for w, r in zip(Wds, Rds)]
    outs = [torch.empty_like(r) for r in Rds]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for w, r, o in zip(Wds, Rds, outs):
            sk.addmm(Xd, w, r, out=o)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for w, r, o in zip(Wds, Rds, outs):
            sk.addmm(Xd, w, r, out=o)
    for rep in range(4):
        for o in outs:
            o.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for e, o in zip(eager, outs):
            assert torch.equal(e.view(torch.int16), o.view(torch.int16)), rep
        _ = sk.addmm(Xd, Wds[0], Rds[0])  # eager work between replays
        torch.cuda.synchronize()
