"""GPU parity of the k-bit quantized GEMV (skinny_kbit_gemv_bf16) against the CPU oracle
(oracle/kbit.c). Tolerances are those of tests/parity.py (fp32 accumulation, one rounding)."""
import numpy as np
import pytest
import torch

import oracle
import parity as P
from decode_skinny_addmm_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_skinny_addmm_amd as d
    d.ops.lib()
    return d


def _u32(planes):
    return planes.numpy().view(np.uint32)


def run_gpu(sk, X, planes, absmax, cb, kb, R):
    d = [t.cuda() for t in (X, planes, absmax, cb, R)]
    Y = sk.kbit_gemv(d[0], d[1], d[2], d[3], kb, d[4])
    A = sk.kbit_gemv_acc_f32(d[0], d[1], d[2], d[3], kb, d[4])
    torch.cuda.synchronize()
    return P.bits_of(Y), A.cpu().numpy()


@pytest.mark.parametrize("kb", [2, 3, 4, 5])
@pytest.mark.parametrize("M,N,K", [(1, 300, 512), (2, 77, 1024), (3, 130, 3584), (4, 64, 32), (5, 50, 288),
                                   (4, 1000, 2048)])
def test_kbit_matches_oracle(sk, kb, M, N, K):
    X, ps, As, rs, cb = synth.make_kbit_inputs(M, N, K, kbits=kb, seed=M * 100 + kb)
    print("kbit", kb, (M, N, K), flush=True)
    Yg, Ag = run_gpu(sk, X, ps[0], As[0], cb, kb, rs[0])
    Yo, Ao = oracle.kbit_gemv_bf16(synth.bits(X), _u32(ps[0]), As[0].numpy(), cb.numpy(), kb, synth.bits(rs[0]))
    P.check_y(Yg, Yo, Ao, "kbit %d %s" % (kb, (M, N, K)))
    P.check_acc(Ag, Ao, "kbit %d %s" % (kb, (M, N, K)))
    assert np.array_equal(Yg.reshape(-1), P.rne_torch(Ag).reshape(-1))


@pytest.mark.parametrize("kb", [2, 3, 4])
@pytest.mark.parametrize("M,N,K", [(5, 130, 512), (8, 64, 3584), (16, 300, 1024), (17, 40, 128), (40, 33, 384),
                                   (9, 1000, 2048)])
def test_kbit_matrix_core_form(sk, kb, M, N, K):
    """M >= 5 with k = 2, 3 and 4 and K a multiple of 128 (at most 3584) run on the matrix cores:
    one and several 16-row passes over X, ragged N, waves whose K slice is partly or wholly past K."""
    X, ps, As, rs, cb = synth.make_kbit_inputs(M, N, K, kbits=kb, seed=M * 100 + kb + 7)
    print("kbit mfma", kb, (M, N, K), flush=True)
    Yg, Ag = run_gpu(sk, X, ps[0], As[0], cb, kb, rs[0])
    Yo, Ao = oracle.kbit_gemv_bf16(synth.bits(X), _u32(ps[0]), As[0].numpy(), cb.numpy(), kb, synth.bits(rs[0]))
    P.check_y(Yg, Yo, Ao, "kbit mfma %d %s" % (kb, (M, N, K)))
    P.check_acc(Ag, Ao, "kbit mfma %d %s" % (kb, (M, N, K)))
    assert np.array_equal(Yg.reshape(-1), P.rne_torch(Ag).reshape(-1))


@pytest.mark.parametrize("M", [1, 4, 16])
def test_kbit_full_size(sk, M):
    """The decode shape, N = 7168, K = 3584, k = 4, against the whole oracle (M = 16: the matrix-
    core form)."""
    X, ps, As, rs, cb = synth.make_kbit_inputs(M, 7168, 3584, kbits=4)
    Yg, Ag = run_gpu(sk, X, ps[0], As[0], cb, 4, rs[0])
    Yo, Ao = oracle.kbit_gemv_bf16(synth.bits(X), _u32(ps[0]), As[0].numpy(), cb.numpy(), 4, synth.bits(rs[0]))
    P.check_y(Yg, Yo, Ao, "kbit full M=%d" % M)
    P.check_acc(Ag, Ao, "kbit full M=%d" % M)


@pytest.mark.parametrize("kb", [2, 4, 5])
def test_kbit_quantized_weights_end_to_end(sk, kb):
    """Weights quantized by the oracle with its normal-float codebook: the GPU GEMV equals the
    oracle's on them, and stays close to the dense product with the unquantized weights."""
    M, N, K = 2, 256, 1024
    X, ws, rs = synth.make_inputs(M, N, K, seed=kb)
    W = oracle.bf16_bits_to_f64(synth.bits(ws[0]))
    cb = oracle.nf_codebook(kb).astype(np.float32)
    planes, amax, _ = oracle.kbit_quantize(W, kb, cb)
    pt = torch.from_numpy(planes.view(np.int32).copy())
    at = torch.from_numpy(amax.copy())
    ct = torch.from_numpy(cb.copy())
    Yg, Ag = run_gpu(sk, X, pt, at, ct, kb, rs[0])
    Yo, Ao = oracle.kbit_gemv_bf16(synth.bits(X), planes, amax, cb, kb, synth.bits(rs[0]))
    P.check_y(Yg, Yo, Ao, "kbit e2e %d" % kb)
    P.check_acc(Ag, Ao, "kbit e2e %d" % kb)
    dense = oracle.bf16_bits_to_f64(synth.bits(X)) @ W.T
    quant = Ao - oracle.bf16_bits_to_f64(synth.bits(rs[0]))
    sqnr = 10 * np.log10((dense ** 2).sum() / ((dense - quant) ** 2).sum())
    assert sqnr > {2: 5.0, 4: 15.0, 5: 20.0}[kb], sqnr


def test_kbit_x_zero_and_errors(sk):
    M, N, K = 3, 100, 256
    X, ps, As, rs, cb = synth.make_kbit_inputs(M, N, K, kbits=3)
    Yg, _ = run_gpu(sk, torch.zeros_like(X), ps[0], As[0], cb, 3, rs[0])
    Rb = synth.bits(rs[0])
    assert np.all((Yg == Rb) | (((Yg & 0x7FFF) == 0) & ((Rb & 0x7FFF) == 0)))
    L = sk.ops.lib()
    d = [t.cuda() for t in (X, ps[0], As[0], cb, rs[0])]
    Y = torch.empty_like(d[4])
    s = torch.cuda.current_stream().cuda_stream
    args = [d[0].data_ptr(), d[1].data_ptr(), d[2].data_ptr(), d[3].data_ptr()]
    assert L.skinny_kbit_gemv_bf16(*args, 6, d[4].data_ptr(), Y.data_ptr(), M, N, K, s) == 1      # kbits
    assert L.skinny_kbit_gemv_bf16(*args, 3, d[4].data_ptr(), Y.data_ptr(), M, N, K - 8, s) == 3  # K % 32
    assert L.skinny_kbit_gemv_bf16(*args, 3, d[4].data_ptr(), Y.data_ptr(), M, N, 32 * 513, s) == 3  # K max
    assert L.skinny_kbit_gemv_bf16(d[0].data_ptr() + 2, *args[1:], 3, d[4].data_ptr(), Y.data_ptr(), M, N, K,
                                   s) == 2                                                        # X alignment
    with pytest.raises(ValueError):
        sk.kbit_gemv(d[0], d[1], d[2], d[3], 4, d[4])                                             # shape of planes


def test_kbit_k_zero_is_residual(sk):
    M, N = 3, 40
    R = torch.randn(M, N).to(torch.bfloat16).cuda()
    X = torch.empty((M, 0), dtype=torch.bfloat16, device="cuda")
    planes = torch.empty((N, 0, 4), dtype=torch.int32, device="cuda")
    amax = torch.empty((N, 0), dtype=torch.uint8, device="cuda")
    cb = torch.linspace(-1, 1, 16, dtype=torch.float32, device="cuda")
    Y = sk.kbit_gemv(X, planes, amax, cb, 4, R)
    torch.cuda.synchronize()
    assert torch.equal(Y.cpu().view(torch.int16), R.cpu().view(torch.int16))


@pytest.mark.parametrize("kb", [3, 4, 5])
@pytest.mark.parametrize("M,K", [(2, 16384), (1, 14336), (4, 8192), (8, 4096)])
def test_kbit_long_rows(sk, kb, M, K):
    """Long rows: one lane per block up to 512 blocks, a row group of one row per workgroup;
    k = 3 and 4 take the pair table (4-bit index fields, the top one clear at k = 3), k = 5 the
    one-index-per-lookup decode."""
    X, ps, As, rs, cb = synth.make_kbit_inputs(M, 48, K, kbits=kb, seed=K + kb)
    Yg, Ag = run_gpu(sk, X, ps[0], As[0], cb, kb, rs[0])
    Yo, Ao = oracle.kbit_gemv_bf16(synth.bits(X), _u32(ps[0]), As[0].numpy(), cb.numpy(), kb, synth.bits(rs[0]))
    P.check_y(Yg, Yo, Ao, "kbit %d long K=%d" % (kb, K))
    P.check_acc(Ag, Ao, "kbit %d long K=%d" % (kb, K))


@pytest.mark.parametrize("kb", [3, 4, 5])
def test_kbit_poisoned_output_fully_written(sk, kb):
    """Every output is written: Y starts as NaN (bf16 and fp32 entry) and must hold none after
    (k = 3: the pair table, k = 5: pairs 8 apart, k = 4 at M >= 5: the matrix-core form)."""
    for M, N, K in ((1, 300, 512), (4, 1000, 3584), (3, 77, 1024), (21, 70, 1024)):
        X, ps, As, rs, cb = synth.make_kbit_inputs(M, N, K, kbits=kb, seed=M)
        d = [t.cuda() for t in (X, ps[0], As[0], cb, rs[0])]
        Y = torch.full_like(d[4], float("nan"))
        sk.kbit_gemv(d[0], d[1], d[2], d[3], kb, d[4], out=Y)
        A = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        sk.kbit_gemv_acc_f32(d[0], d[1], d[2], d[3], kb, d[4], out=A)
        torch.cuda.synchronize()
        assert not torch.isnan(Y.float()).any() and not torch.isnan(A).any(), (M, N, K)
