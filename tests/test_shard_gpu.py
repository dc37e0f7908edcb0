"""GPU parity of the tensor-parallel shard form (skinny_addmm_bf16_shard): R and Y as column
blocks of wider row-major matrices, and the shard epilogue's two flags, against the CPU
oracle (its *_ex entry points with the same flags). Tolerances are those of tests/parity.py."""
import numpy as np
import pytest
import torch

import oracle
import parity as P
from decode_skinny_addmm_amd import synth
from test_parity_gpu import all_configs

pytestmark = pytest.mark.gpu

ROUND = oracle.ROUND_PRODUCT
NONEG = oracle.NO_NEG_ZERO
SENTINEL = 0x4D4D  # a finite bf16 pattern no output of these inputs produces in the padding


@pytest.fixture(scope="module")
def sk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_skinny_addmm_amd as d
    d.ops.lib()
    return d


def wide(block_cpu, ld, c0, fill_bits):
    """A [M, ld] bf16 GPU matrix filled with `fill_bits`, with `block_cpu` copied into columns
    c0 .. c0+N; returns (wide matrix, view of the block)."""
    M, N = block_cpu.shape
    full = torch.full((M, ld), fill_bits, dtype=torch.int16).view(torch.bfloat16).cuda()
    view = full[:, c0:c0 + N]
    view.copy_(block_cpu.cuda())
    return full, view


def shard_case(sk, M, N, K, ldr, c0r, ldy, c0y, flags, config, seed):
    X, ws, rs = synth.make_inputs(M, N, K, seed=seed)
    Xd, Wd = X.cuda(), ws[0].cuda()
    _, Rv = wide(rs[0], ldr, c0r, 0x3F80)
    Yfull, Yv = wide(torch.zeros((M, N), dtype=torch.bfloat16), ldy, c0y, SENTINEL)
    before = P.bits_of(Yfull).copy()
    sk.addmm_shard(Xd, Wd, Rv, out=Yv, round_product=bool(flags & ROUND), no_neg_zero=bool(flags & NONEG),
                   config=config)
    Afull = torch.full((M, ldy), float("nan"), dtype=torch.float32, device="cuda")
    Av = Afull[:, c0y:c0y + N]
    sk.addmm_shard_acc_f32(Xd, Wd, Rv, out=Av, round_product=bool(flags & ROUND), config=config)
    torch.cuda.synchronize()
    after = P.bits_of(Yfull)
    outside = np.ones(after.shape, dtype=bool)
    outside[:, c0y:c0y + N] = False
    assert np.array_equal(after[outside], before[outside]), "shard call wrote outside its block"
    assert torch.isnan(Afull[:, :c0y]).all() and torch.isnan(Afull[:, c0y + N:]).all()
    return X, ws[0], rs[0], after[:, c0y:c0y + N], Av.cpu().numpy()


@pytest.mark.parametrize("M,N,K,ldr,c0r,ldy,c0y", [
    (4, 896, 3584, 7168, 896 * 3, 7168, 896 * 5),     # one of eight shards of the 7168-wide output
    (3, 100, 1032, 333, 17, 250, 101),
    (33, 130, 512, 300, 5, 131, 1),
    (1, 7, 264, 7, 0, 64, 40),
])
def test_shard_block_single_rounding(sk, M, N, K, ldr, c0r, ldy, c0y):
    X, W, R, Yg, Ag = shard_case(sk, M, N, K, ldr, c0r, ldy, c0y, 0, None, M + N)
    Yo, Ao = oracle.addmm_bf16(synth.bits(X), synth.bits(W), synth.bits(R))
    P.check_y(Yg, Yo, Ao, "shard %s" % ((M, N, K),))
    P.check_acc(Ag, Ao, "shard %s" % ((M, N, K),))
    assert np.array_equal(Yg.reshape(-1), P.rne_torch(Ag).reshape(-1))


@pytest.mark.parametrize("M", [1, 2, 4, 5, 8, 16, 24, 32])
def test_shard_production_shape_selected(sk, M):
    """One rank of an 8-way split of the 7168 output columns (N = 896, rank 3, R and Y as column
    blocks of [M, 7168] matrices), K = 3584, at the configuration the library selects for that
    shape (the narrow-output table), every output against the oracle. Flags off: the dense
    rule. Flags on (two roundings, no -0): the fp32 sum meets the accumulator bar, Y is exactly
    the two-rounding epilogue of that sum, and Y equals the oracle's twice-rounded output bit for
    bit wherever the sum rounds to the same bf16 value as the exact sum."""
    N, K, ld, c0 = 896, 3584, 7168, 896 * 3
    print("shard production M=%d config %s" % (M, sk.select_config(M, N, K)), flush=True)
    # flags off
    X, W, R, Yg, Ag = shard_case(sk, M, N, K, ld, c0, ld, c0, 0, None, 1000 + M)
    Yo, Ao = oracle.addmm_bf16(synth.bits(X), synth.bits(W), synth.bits(R))
    P.check_y(Yg, Yo, Ao, "shard M=%d" % M)
    P.check_acc(Ag, Ao, "shard M=%d" % M)
    assert np.array_equal(Yg.reshape(-1), P.rne_torch(Ag).reshape(-1))
    # flags on, same inputs, same (selected) kernel
    flags = ROUND | NONEG
    _, _, _, Yf, Af = shard_case(sk, M, N, K, ld, c0, ld, c0, flags, None, 1000 + M)
    _, Rz = wide(torch.zeros((M, N), dtype=torch.bfloat16), ld, c0, 0)
    Sz = sk.addmm_shard_acc_f32(X.cuda(), W.cuda(), Rz).cpu().numpy().astype(np.float64)  # the fp32 sum
    _, So = oracle.addmm_bf16(synth.bits(X), synth.bits(W), np.zeros((M, N), dtype=np.uint16))
    P.check_acc(Sz, So, "shard sum M=%d" % M)
    r = oracle.bf16_bits_to_f64(synth.bits(R))
    gr = (oracle.bf16_bits_to_f64(oracle.round_bf16(Sz)).astype(np.float32) + r.astype(np.float32)).astype(np.float64)
    assert np.array_equal(Af.astype(np.float64), gr), "ACC is not fp32(bf16(sum) + r)"
    want = oracle.round_bf16(gr)
    want = np.where(want == 0x8000, 0, want).astype(np.uint16)
    assert np.array_equal(Yf, want), "Y is not the two-rounding epilogue of the fp32 sum"
    assert not np.any(Yf == 0x8000)
    Yof, _ = oracle.addmm_bf16(synth.bits(X), synth.bits(W), synth.bits(R), flags=flags)
    same_sum = oracle.round_bf16(Sz) == oracle.round_bf16(So)
    assert np.array_equal(Yf[same_sum], Yof[same_sum]), "differs from the oracle where the rounded sums agree"
    assert same_sum.mean() > 0.99


def test_shard_every_config(sk):
    """Every built configuration writes the strided block correctly (flags off and on)."""
    for (M, N, K) in [(5, 70, 512), (33, 130, 512)]:
        X, ws, rs = synth.make_inputs(M, N, K, seed=3)
        Yo, Ao = oracle.addmm_bf16(synth.bits(X), synth.bits(ws[0]), synth.bits(rs[0]))
        for cfg in all_configs(sk, K):
            print("shard config", (M, N, K), cfg, flush=True)
            _, _, _, Yg, Ag = shard_case(sk, M, N, K, N + 9, 3, N + 21, 11, 0, cfg, 3)
            P.check_y(Yg, Yo, Ao, "shard %s %s" % ((M, N, K), cfg))
            P.check_acc(Ag, Ao, "shard %s %s" % ((M, N, K), cfg))


@pytest.mark.parametrize("M,N,K", [(4, 896, 3584), (40, 300, 1024), (2, 50, 264)])
def test_round_product_is_exact_given_the_sum(sk, M, N, K):
    """Two roundings: the fp32 sum meets the accumulator bar against the oracle's exact sum,
    and Y is exactly RNE(RNE(sum) + r) of that fp32 sum (the oracle's rounding applied)."""
    X, ws, rs = synth.make_inputs(M, N, K, seed=M * N)
    Xd, Wd, Rd = X.cuda(), ws[0].cuda(), rs[0].cuda()
    zeros = torch.zeros_like(Rd)
    S = sk.addmm_acc_f32(Xd, Wd, zeros).cpu().numpy().astype(np.float64)   # fp32 sum, exactly
    _, So = oracle.addmm_bf16(synth.bits(X), synth.bits(ws[0]), np.zeros((M, N), dtype=np.uint16))
    P.check_acc(S, So, "sum %s" % ((M, N, K),))
    Y = sk.addmm_shard(Xd, Wd, Rd, round_product=True)
    A = sk.addmm_shard_acc_f32(Xd, Wd, Rd, round_product=True).cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    g = oracle.bf16_bits_to_f64(oracle.round_bf16(S))
    r = oracle.bf16_bits_to_f64(synth.bits(rs[0]))
    gr = (g.astype(np.float32) + r.astype(np.float32)).astype(np.float64)   # the fp32 addition
    assert np.array_equal(A, gr)                          # ACC is fp32(bf16(sum) + r)
    want = oracle.round_bf16(gr)
    assert np.array_equal(P.bits_of(Y), want)
    # the inputs exercise the difference between one and two roundings
    assert np.any(oracle.round_bf16(S + r) != want)


@pytest.mark.parametrize("M,N,K", [(4, 300, 3584), (8, 100, 1032), (40, 100, 1024)])
def test_round_product_small_integers_exact(sk, M, N, K):
    """Integer inputs: every sum is exact, so the two-rounding result equals the oracle's bit
    for bit, for every configuration that takes this K."""
    X, W, R = synth.small_int_inputs(M, N, K, seed=13)
    X, W = X.abs(), W + 2
    Yo, Ao = oracle.addmm_bf16(synth.bits(X), synth.bits(W), synth.bits(R), flags=ROUND)
    Xd, Wd, Rd = X.cuda(), W.cuda(), R.cuda()
    for cfg in [None] + all_configs(sk, K):
        Y = sk.addmm_shard(Xd, Wd, Rd, round_product=True, config=cfg)
        A = sk.addmm_shard_acc_f32(Xd, Wd, Rd, round_product=True, config=cfg)
        torch.cuda.synchronize()
        assert np.array_equal(P.bits_of(Y), Yo), cfg
        assert np.array_equal(A.cpu().numpy().astype(np.float64), Ao), cfg


def test_no_neg_zero(sk):
    """Results that round to -0: with the flag no 0x8000 is written; without it the output equals
    the oracle up to the sign of zero (the device may flush fp32 denormals, the oracle does not)."""
    M, N, K = 3, 40, 264
    X = torch.zeros((M, K), dtype=torch.bfloat16)
    W = torch.zeros((N, K), dtype=torch.bfloat16)
    X[:, 0] = 2.0 ** -70
    W[::2, 0] = -(2.0 ** -70)             # even rows: product -2^-140, rounds to -0
    W[1::2, 0] = 2.0 ** -70               # odd rows: +2^-140, rounds to +0
    R = torch.zeros((M, N), dtype=torch.bfloat16)
    R.view(torch.int16)[:, ::3] = -32768  # -0 in every third column
    Xd, Wd, Rd = X.cuda(), W.cuda(), R.cuda()
    for flags in (0, NONEG, ROUND, ROUND | NONEG):
        Yo, _ = oracle.addmm_bf16(synth.bits(X), synth.bits(W), synth.bits(R), flags=flags)
        for cfg in [None] + all_configs(sk, K):
            Y = P.bits_of(sk.addmm_shard(Xd, Wd, Rd, round_product=bool(flags & ROUND),
                                         no_neg_zero=bool(flags & NONEG), config=cfg))
            assert np.array_equal(Y & 0x7FFF, Yo & 0x7FFF), (flags, cfg)
            if flags & NONEG:
                assert not np.any(Y == 0x8000), (flags, cfg)
        if not flags & NONEG:
            assert np.any(Yo == 0x8000)   # the case does produce -0 by the definition


def test_shard_in_place_and_errors(sk):
    M, N, K = 4, 256, 512
    X, ws, rs = synth.make_inputs(M, N, K, seed=5)
    Xd, Wd = X.cuda(), ws[0].cuda()
    full, Rv = wide(rs[0], 600, 100, 0x3F80)
    want = P.bits_of(sk.addmm_shard(Xd, Wd, Rv.clone()))
    sk.addmm_shard(Xd, Wd, Rv, out=Rv)    # Y is R: same block, same pitch
    torch.cuda.synchronize()
    assert np.array_equal(P.bits_of(Rv), want)
    L = sk.ops.lib()
    Yd = torch.empty((M, 600), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    # pitch below N, unknown flag, Y == R with another pitch
    assert L.skinny_addmm_bf16_shard(Xd.data_ptr(), Wd.data_ptr(), Rv.data_ptr(), N - 1, Yd.data_ptr(), 600,
                                     M, N, K, 0, None, s) == 1
    assert L.skinny_addmm_bf16_shard(Xd.data_ptr(), Wd.data_ptr(), Rv.data_ptr(), 600, Yd.data_ptr(), 600,
                                     M, N, K, 4, None, s) == 1
    assert L.skinny_addmm_bf16_shard(Xd.data_ptr(), Wd.data_ptr(), Rv.data_ptr(), 600, Rv.data_ptr(), 601,
                                     M, N, K, 0, None, s) == 1
    with pytest.raises(ValueError):
        sk.addmm_shard(Xd, Wd, Rv.t())    # not row-major
