"""GPU parity of the KDA chain-verify step (skinny_kda_verify_bf16) against the CPU oracle
(oracle/kda.c), in snapshot and ring mode.

Bars (the kernel computes in fp32 after the bf16 conv outputs, the oracle in fp64):
  * conv windows: bit-exact (data movement);
  * ring k and v (the bf16 conv outputs): at most 1 bf16 step, and equal wherever the exact
    conv value is more than 1e-6 from a rounding midpoint (fp32 and fp64 sums may round a
    value that close either way);
  * ring g and beta: relative 1e-5;
  * o: the dense path's rule, 2 bf16 ULP where |o| >= 2^-12, else 2^-18 absolute;
  * snapshots: |S - S_exact| <= 1e-5 |S_exact| + 5e-4 rms(S_exact) (fp32 state arithmetic is
    ~1e-6 relative). A state row
    whose value input v, at that token or an earlier one, lies within 1e-6 of a bf16 rounding
    midpoint (the oracle's fp64 conv value; the kernel's fp32 one may round the other way) may
    move by one bf16 step of v times beta times |k^|: that row gets 2^-8 max|v| max|k^| more.
    Likewise a key value k_c near a midpoint moves column c of the head's states by u dk^_c,
    |u| <= max|v| + sqrt(K) max|S|, dk^_c <= 2^-7 max|k^|: that column, from that token on,
    gets 2^-7 max|k^| (max|v| + sqrt(K) max|S|) more. A wrong decay, beta or head mapping moves
    every state by 1e-2 or more.
"""
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


def midpoint_distance(x):
    """Distance of each float64 value to the nearest bf16 rounding midpoint."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    m, e = np.frexp(x)
    scaled = m * 256.0                       # bf16 steps at 1.0 in these units
    frac = scaled - np.floor(scaled)
    return np.abs(frac - 0.5) * np.ldexp(1.0 / 256.0, e)


def run_case(sk, B, T, H, HV, K, V, ring, seed=0, permute=True):
    t_inp = synth.make_kda_inputs(B, T=T, H=H, HV=HV, K=K, V=V, seed=seed)
    if permute:
        lines = B + 1
        t_inp["cache_indices"] = torch.tensor([lines - 1 - i for i in range(B)], dtype=torch.int32)
        t_inp["inter_indices"] = torch.tensor([(i + 1) % lines for i in range(B)], dtype=torch.int32)
    n_inp = synth.kda_to_numpy(t_inp)
    scale = K ** -0.5
    print("kda", dict(B=B, T=T, H=H, HV=HV, K=K, V=V, ring=ring, seed=seed), flush=True)
    d = {k: v.cuda() for k, v in t_inp.items()}
    o = sk.kda_verify(d, T, H, HV, K, V, scale, snapshots=not ring, ring=ring)
    torch.cuda.synchronize()
    ref = oracle.kda_verify(n_inp, T, H, HV, K, V, scale, snapshots=not ring, ring_len=16 if ring else 0)
    what = "kda B=%d T=%d H=%d HV=%d V=%d ring=%s" % (B, T, H, HV, V, ring)
    assert np.array_equal(synth.bits(d["win_pool"].cpu()), ref["win_pool"]), what + ": windows"
    P.check_y(P.bits_of(o), ref["o"], ref["o_exact"], what + ": o")
    dim = 2 * H * K + HV * V
    conv_bits = oracle.round_bf16(ref["conv_exact"])
    near = midpoint_distance(ref["conv_exact"]) < 1e-6
    if ring:
        for name in ("rawv", "rawk"):
            g = synth.bits(d[name].cpu()).astype(np.int64)
            r = ref[name].astype(np.int64)
            diff = np.abs(P.ordered(g) - P.ordered(r))
            assert diff.max() <= 1, what + ": " + name
            assert (diff > 0).sum() <= int(near.sum()), what + ": %s differs away from a midpoint" % name
        assert np.allclose(d["g"].cpu().numpy(), ref["g"], rtol=1e-5, atol=1e-7), what + ": g"
        assert np.allclose(d["beta"].cpu().numpy(), ref["beta"], rtol=1e-5, atol=1e-7), what + ": beta"
    else:
        S = d["inter_ssm"].cpu().numpy().astype(np.float64)
        Se = ref["inter_ssm"]
        rms = float(np.sqrt(np.mean(Se ** 2)))
        err = np.abs(S - Se)
        lim = 1e-5 * np.abs(Se) + 5e-4 * rms
        # rows (line, t, hv, v) whose v input at a token <= t is near a midpoint
        vnear = near[:, 2 * H * K:].reshape(B, T, HV, V)
        vnear = np.cumsum(vnear, axis=1) > 0                       # at this token or before
        conv = oracle.bf16_bits_to_f64(conv_bits)
        vmax = float(np.abs(conv[:, 2 * H * K:]).max())
        khat_max = 0.0
        for row in range(B * T):
            for h in range(H):
                k = conv[row, H * K + h * K:H * K + (h + 1) * K]
                khat_max = max(khat_max, float(np.abs(k).max() / np.sqrt(k @ k + 1e-6)))
        extra = 2.0 ** -8 * vmax * khat_max
        lines = np.array([int(i) for i in n_inp["inter_indices"]])
        knear = near[:, H * K:2 * H * K].reshape(B, T, H, K)
        knear = np.cumsum(knear, axis=1) > 0
        extra_k = 2.0 ** -7 * khat_max * (vmax + np.sqrt(K) * float(np.abs(Se).max()))
        group = HV // H
        for bi in range(B):
            lim[lines[bi]] += np.where(vnear[bi][:, :, :, None], extra, 0.0)
            kcols = np.repeat(knear[bi], group, axis=1)            # [T, HV, K]
            lim[lines[bi]] += np.where(kcols[:, :, None, :], extra_k, 0.0)
        bad = err > lim
        msg = ": %d snapshot values off, max err %g (rms %g, %d rows and %d columns near a midpoint)" % (
            int(bad.sum()), err.max(), rms, int(vnear.sum()), int(knear.sum()))
        assert not bad.any(), what + msg
    assert conv_bits.shape == (B * T, dim)


@pytest.mark.parametrize("ring", [False, True])
@pytest.mark.parametrize("B,T,H,HV,V", [(1, 4, 1, 1, 16), (3, 4, 2, 4, 32), (2, 1, 1, 2, 16), (2, 16, 1, 1, 16),
                                        (5, 3, 2, 2, 48), (2, 6, 1, 2, 32), (3, 8, 2, 2, 16), (1, 11, 1, 1, 16)])
def test_kda_small(sk, B, T, H, HV, V, ring):
    run_case(sk, B, T, H, HV, 128, V, ring)


@pytest.mark.parametrize("ring", [False, True])
@pytest.mark.parametrize("B", [1, 4, 16, 32])
def test_kda_page_shape(sk, B, ring):
    """The page's layer: H = HV = 8, K = V = 128, 4 draft tokens. The launch takes 16 state rows
    per workgroup at B = 1 and 4, 32 at B = 16 and 64 at B = 32 (128 at B = 64, in the ring test
    below)."""
    run_case(sk, B, 4, 8, 8, 128, 128, ring, permute=B > 1)


def test_kda_gqa_page(sk):
    run_case(sk, 2, 4, 8, 16, 128, 128, False)


def test_kda_ring_bitwise_between_launch_shapes(sk):
    """The page's guard compares the ring bytes of two implementations; here the same inputs
    run through launches with different rows per workgroup (B = 1 uses 16 rows, the same batch
    row inside B = 64 uses 128) must fill identical ring bytes for that row."""
    T, H, HV, K, V = 4, 8, 8, 128, 128
    big = synth.make_kda_inputs(64, T=T, H=H, HV=HV, K=K, V=V, seed=3)
    db = {k: v.cuda() for k, v in big.items()}
    sk.kda_verify(db, T, H, HV, K, V, K ** -0.5, snapshots=False, ring=True)
    one = {}
    for k, v in big.items():
        if k in ("mixed", "a", "b"):
            one[k] = v[:T].clone()
        elif k in ("cache_indices", "inter_indices"):
            one[k] = v[:1].clone()
        elif k in ("w", "bias", "A_log", "dt_bias"):
            one[k] = v.clone()
        else:
            one[k] = v[:2].clone()      # lines/slots 0 and 1
    d1 = {k: v.cuda() for k, v in one.items()}
    d1["rawv"].zero_(); d1["rawk"].zero_(); d1["g"].zero_(); d1["beta"].zero_()
    sk.kda_verify(d1, T, H, HV, K, V, K ** -0.5, snapshots=False, ring=True)
    torch.cuda.synchronize()
    for name in ("rawv", "rawk", "g", "beta"):
        a = db[name][0, :, :T].cpu()
        b = d1[name][0, :, :T].cpu()
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)), name


def test_kda_argument_errors(sk):
    T, H, HV, K, V = 4, 1, 1, 128, 16
    d = {k: v.cuda() for k, v in synth.make_kda_inputs(2, T=T, H=H, HV=HV, K=K, V=V).items()}
    with pytest.raises(ValueError):
        sk.kda_verify(d, T, H, HV, K, 32, K ** -0.5)          # V does not match the tensors
    with pytest.raises(ValueError):
        sk.kda_verify(d, T + 1, H, HV, K, V, K ** -0.5)       # T does not match the tensors


@pytest.mark.parametrize("ring", [False, True])
def test_kda_poisoned_outputs_fully_written(sk, ring):
    """o, the windows of the batch rows' lines and their snapshots (or ring positions < T) start
    as NaN and must hold none after the call; lines and slots of no batch row stay NaN."""
    B, T, H, HV, K, V = 3, 4, 2, 4, 128, 32
    d = {k: v.cuda() for k, v in synth.make_kda_inputs(B, T=T, H=H, HV=HV, K=K, V=V).items()}
    d["cache_indices"] = torch.tensor([3, 0, 2], dtype=torch.int32, device="cuda")
    d["inter_indices"] = torch.tensor([1, 3, 0], dtype=torch.int32, device="cuda")
    nan = float("nan")
    d["win_pool"].fill_(nan)
    d["inter_ssm"].fill_(nan)
    for k in ("rawv", "rawk", "g", "beta"):
        d[k].fill_(nan)
    out = torch.full((B * T, HV, V), nan, dtype=torch.bfloat16, device="cuda")
    sk.kda_verify(d, T, H, HV, K, V, K ** -0.5, snapshots=not ring, ring=ring, out=out)
    torch.cuda.synchronize()
    assert not torch.isnan(out.float()).any()
    lines = [1, 3, 0]
    assert not torch.isnan(d["win_pool"][lines].float()).any()
    assert torch.isnan(d["win_pool"][2].float()).all()
    if ring:
        for k in ("rawv", "rawk", "g", "beta"):
            t = d[k][[3, 0, 2]][:, :, :T].float()
            assert not torch.isnan(t).any(), k
            assert torch.isnan(d[k][[3, 0, 2]][:, :, T:].float()).all(), k
            assert torch.isnan(d[k][1].float()).all(), k
    else:
        assert not torch.isnan(d["inter_ssm"][lines]).any()
        assert torch.isnan(d["inter_ssm"][2]).all()
