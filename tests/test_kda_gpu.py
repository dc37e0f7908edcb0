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


def near_midpoint(x, n_inp, B, T, dim):
    """Conv values an fp32 evaluation may round differently from the fp64 one: within
    2^-21 (sum of |terms| + |value|) of a bf16 rounding midpoint, eight times the unit
    roundoff of an fp32 sum and silu (conv_term_magnitude gives the terms)."""
    x = np.asarray(x, dtype=np.float64)
    return midpoint_distance(x) < 2.0 ** -21 * (conv_term_magnitude(n_inp, B, T, dim) + np.abs(x))


def midpoint_distance(x):
    """Distance of each float64 value to the nearest bf16 rounding midpoint."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    m, e = np.frexp(x)
    scaled = m * 256.0                       # bf16 steps at 1.0 in these units
    frac = scaled - np.floor(scaled)
    return np.abs(frac - 0.5) * np.ldexp(1.0 / 256.0, e)


def run_case(sk, B, T, H, HV, K, V, ring, seed=0, permute=True, clean=True, snapshots=None):
    """One verify call against the oracle. clean: inputs moved away from conv rounding
    midpoints first (clean_inputs), so every allowance below is empty and the bars are the
    tight ones; otherwise the allowances cover values that fp32 and fp64 may round apart.
    snapshots: defaults to `not ring`; False with ring False asks for o (and windows) only."""
    snap = (not ring) if snapshots is None else snapshots
    t_inp = synth.make_kda_inputs(B, T=T, H=H, HV=HV, K=K, V=V, seed=seed)
    if permute:
        lines = B + 1
        t_inp["cache_indices"] = torch.tensor([lines - 1 - i for i in range(B)], dtype=torch.int32)
        t_inp["inter_indices"] = torch.tensor([(i + 1) % lines for i in range(B)], dtype=torch.int32)
    if clean:
        t_inp = clean_inputs(t_inp, T, H, HV, K, V)
    n_inp = synth.kda_to_numpy(t_inp)
    scale = K ** -0.5
    print("kda", dict(B=B, T=T, H=H, HV=HV, K=K, V=V, ring=ring, snapshots=snap, seed=seed), flush=True)
    d = {k: v.cuda() for k, v in t_inp.items()}
    o = sk.kda_verify(d, T, H, HV, K, V, scale, snapshots=snap, ring=ring)
    torch.cuda.synchronize()
    ref = oracle.kda_verify(n_inp, T, H, HV, K, V, scale, snapshots=snap, ring_len=16 if ring else 0)
    what = "kda B=%d T=%d H=%d HV=%d V=%d ring=%s snapshots=%s" % (B, T, H, HV, V, ring, snap)
    assert np.array_equal(synth.bits(d["win_pool"].cpu()), ref["win_pool"]), what + ": windows"
    dim = 2 * H * K + HV * V
    conv_bits = oracle.round_bf16(ref["conv_exact"])
    near = near_midpoint(ref["conv_exact"], n_inp, B, T, dim)
    assert not (clean and near.any())
    # o: the dense rule, except on (token, value head) whose q input at that token, or k or v
    # input at that token or before, is near a midpoint: a one-step flip of q_c moves q^ by at
    # most 2^-6 max|q^| in 2-norm, and a flip of k or v moves the state (see the snapshot
    # allowances), so such o may move by up to 2^-5 scale sqrt(K) max|S| there
    rows = near.reshape(B, T, dim)
    qn = rows[:, :, :H * K].reshape(B, T, H, K).any(-1)
    kn = np.cumsum(rows[:, :, H * K:2 * H * K].reshape(B, T, H, K).any(-1), axis=1) > 0
    vn = np.cumsum(rows[:, :, 2 * H * K:].reshape(B, T, HV, V).any(-1), axis=1) > 0
    group = HV // H
    aff = np.repeat(qn | kn, group, axis=2) | vn                    # [B, T, HV]
    aff = np.broadcast_to(aff.reshape(B * T, HV, 1), (B * T, HV, V))
    og, oe = P.bits_of(o), ref["o_exact"]
    P.check_y(og[~aff], ref["o"][~aff], oe[~aff], what + ": o")
    if aff.any():
        s_max = float(np.abs(ref["inter_ssm"] if snap else n_inp["ssm"]).max()) * 4.0
        lim_o = 2.0 ** -5 * scale * np.sqrt(K) * s_max
        assert np.abs(oracle.bf16_bits_to_f64(og[aff]) - oe[aff]).max() <= lim_o, what + ": o near a flip"
    if ring:
        # ring entry (slot cache_idx[b], head, position t, channel) holds conv output
        # (row b*T + t, channel); only entries whose exact conv value is near a midpoint may differ
        cidx = np.array([int(i) for i in n_inp["cache_indices"]])
        near_rows = near.reshape(B, T, dim)
        near_ring = {"rawv": np.zeros(ref["rawv"].shape, dtype=bool), "rawk": np.zeros(ref["rawk"].shape, dtype=bool)}
        for bi in range(B):
            near_ring["rawv"][cidx[bi], :, :T, :] = near_rows[bi, :, 2 * H * K:].reshape(T, HV, V).transpose(1, 0, 2)
            near_ring["rawk"][cidx[bi], :, :T, :] = near_rows[bi, :, H * K:2 * H * K].reshape(T, H, K).transpose(1, 0, 2)
        for name in ("rawv", "rawk"):
            g = synth.bits(d[name].cpu()).astype(np.int64)
            r = ref[name].astype(np.int64)
            diff = np.abs(P.ordered(g) - P.ordered(r))
            assert diff.max() <= 1, what + ": " + name
            assert not (diff[~near_ring[name]] > 0).any(), what + ": %s differs away from a midpoint" % name
        assert np.allclose(d["g"].cpu().numpy(), ref["g"], rtol=1e-5, atol=1e-7), what + ": g"
        assert np.allclose(d["beta"].cpu().numpy(), ref["beta"], rtol=1e-5, atol=1e-7), what + ": beta"
    elif snap:
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
@pytest.mark.parametrize("B", [1, 4, 8, 16, 32, 64])
def test_kda_page_shape(sk, B, ring):
    """The page's layer: H = HV = 8, K = V = 128, 4 draft tokens. The launch takes 16 state rows
    per workgroup at B = 1 and 4, 32 at B = 8, 64 at B = 16 and 32 and 128 at B = 64."""
    run_case(sk, B, 4, 8, 8, 128, 128, ring, permute=B > 1)


@pytest.mark.parametrize("B,T,H,HV,V", [(64, 4, 8, 8, 128), (3, 1, 2, 4, 32), (3, 3, 2, 4, 32), (2, 5, 1, 2, 64),
                                        (4, 8, 2, 2, 128), (2, 9, 1, 1, 16), (2, 16, 1, 2, 32)])
def test_kda_outputs_only(sk, B, T, H, HV, V):
    """Neither snapshots nor ring: only o (and the conv windows) are written; the 4-, 8- and
    16-token instances of the kernel, against the oracle."""
    run_case(sk, B, T, H, HV, 128, V, False, snapshots=False)


@pytest.mark.parametrize("ring", [False, True])
def test_kda_unfiltered_inputs(sk, ring):
    """The page's layer on inputs as drawn (some conv outputs within an fp32 error of a bf16
    midpoint): ring, snapshots and o within the bars widened only where such a value feeds
    them."""
    run_case(sk, 16, 4, 8, 8, 128, 128, ring, clean=False)


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


def conv_term_magnitude(n_inp, B, T, dim):
    """|bias| + sum over the four taps of |weight * input| for every conv output [B*T, dim]:
    the scale of the fp32 rounding error of that output's sum."""
    f = lambda b: oracle.bf16_bits_to_f64(b)
    w, bias, pool, mixed = f(n_inp["w"]), f(n_inp["bias"]), f(n_inp["conv_pool"]), f(n_inp["mixed"])
    cidx = [int(i) for i in n_inp["cache_indices"]]
    mag = np.zeros((B * T, dim))
    for bi in range(B):
        seq = np.concatenate([pool[cidx[bi]], mixed[bi * T:(bi + 1) * T]], axis=0)   # [3 + T, dim]
        for t in range(T):
            mag[bi * T + t] = np.abs(bias) + sum(np.abs(w[:, j] * seq[t + j]) for j in range(4))
    return mag


def clean_inputs(t_inp, T, H, HV, K, V):
    """The same inputs with every conv output moved away from bf16 rounding midpoints (judged
    by the oracle's fp64 conv values with near_midpoint's margin): any token input feeding a
    near-midpoint value is moved by 1/16 (doubling every fourth round, so that outputs too
    small for any fp32 sum to round reliably leave that range) until none is left. The bf16 conv tensor
    is then the same for any correct fp32 evaluation, and the parity bars need no midpoint
    allowance."""
    t_inp = {k: v.clone() for k, v in t_inp.items()}
    B = int(t_inp["cache_indices"].shape[0])
    dim = 2 * H * K + HV * V
    for it in range(40):
        n_inp = synth.kda_to_numpy(t_inp)
        ref = oracle.kda_verify(n_inp, T, H, HV, K, V, K ** -0.5, snapshots=False)
        near = near_midpoint(ref["conv_exact"], n_inp, B, T, dim)
        if not near.any():
            return t_inp
        rows, cols = (torch.from_numpy(i) for i in np.nonzero(near))
        m = t_inp["mixed"].float()
        m[rows, cols] += 0.0625 * 2.0 ** (it // 4)
        t_inp["mixed"] = m.to(torch.bfloat16)
    raise AssertionError("could not move every conv output away from a midpoint")


@pytest.mark.parametrize("B,H,HV,V", [(4, 8, 8, 128), (16, 8, 8, 128), (3, 2, 4, 32)])
def test_kda_exact_conv_tight_bars(sk, B, H, HV, V):
    """Inputs with every conv output away from a rounding midpoint, both layouts of the same
    inputs: ring v and k equal to the oracle's bit for bit, g and beta within 1e-5, every
    snapshot within 1e-5 |S| + 5e-4 rms(S) with no midpoint allowance, o within the dense rule."""
    T, K = 4, 128
    t_inp = clean_inputs(synth.make_kda_inputs(B, T=T, H=H, HV=HV, K=K, V=V, seed=11), T, H, HV, K, V)
    n_inp = synth.kda_to_numpy(t_inp)
    scale = K ** -0.5
    what = "kda clean B=%d H=%d HV=%d V=%d" % (B, H, HV, V)
    print(what, flush=True)
    ref_s = oracle.kda_verify(n_inp, T, H, HV, K, V, scale, snapshots=True)
    ref_r = oracle.kda_verify(n_inp, T, H, HV, K, V, scale, snapshots=False, ring_len=16)
    ds = {k: v.cuda() for k, v in t_inp.items()}
    o_s = sk.kda_verify(ds, T, H, HV, K, V, scale, snapshots=True, ring=False)
    dr = {k: v.cuda() for k, v in t_inp.items()}
    o_r = sk.kda_verify(dr, T, H, HV, K, V, scale, snapshots=False, ring=True)
    torch.cuda.synchronize()
    for name in ("rawv", "rawk"):
        assert np.array_equal(synth.bits(dr[name].cpu()), ref_r[name]), what + ": " + name
    assert np.allclose(dr["g"].cpu().numpy(), ref_r["g"], rtol=1e-5, atol=1e-7), what + ": g"
    assert np.allclose(dr["beta"].cpu().numpy(), ref_r["beta"], rtol=1e-5, atol=1e-7), what + ": beta"
    S = ds["inter_ssm"].cpu().numpy().astype(np.float64)
    Se = ref_s["inter_ssm"]
    rms = float(np.sqrt(np.mean(Se ** 2)))
    err = np.abs(S - Se)
    bad = err > 1e-5 * np.abs(Se) + 5e-4 * rms
    assert not bad.any(), what + ": %d snapshot values off, max err %g (rms %g)" % (int(bad.sum()), err.max(), rms)
    for o, ref in ((o_s, ref_s), (o_r, ref_r)):
        P.check_y(P.bits_of(o), ref["o"], ref["o_exact"], what + ": o")
    assert np.array_equal(synth.bits(ds["win_pool"].cpu()), ref_s["win_pool"])
