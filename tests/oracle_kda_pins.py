"""Pins for the KDA chain-verify part of the CPU oracle (oracle/kda.c).

Each pin takes an ``oracle.Oracle`` handle and raises AssertionError on a mismatch; they run on
the real oracle (tests/test_oracle_kda.py) and on planted-mistake copies of kda.c
(tests/test_oracle_kda_mutants.py). What fixes the expected values, never the oracle's own
arithmetic:

  * special cases with closed forms: one-hot conv taps select a single input (the output is
    silu of it), zero taps leave silu(bias); x above the softplus threshold passes through,
    softplus(0) = ln 2, sigmoid(0) = 1/2;
  * invariants of the delta rule: with beta = 1 the updated state maps the normalised key
    onto the value (S k^ = v, up to the 1e-6 of the norm); with beta = 0 only the decay acts,
    S_t = S_0 * exp(sum of the gates); from a zero state one step gives the outer product
    beta v k^T; the output is the post-update state applied to the scaled normalised query;
  * the page's data movement, checked by numpy slicing: the window written after token t,
    the ring positions, the head of the query/key for each value head, untouched slots;
  * an independent round-to-nearest-even on float64 bits for the bf16 outputs.
"""
from __future__ import annotations

import math

import numpy as np

from decode_skinny_addmm_amd import synth


# ---------------------------------------------------------------- independent helpers

def rne_bf16_f64(x) -> np.ndarray:
    """float64 -> bf16 bits, round to nearest even on the float64 value (normal range)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m * 2^e, 0.5 <= |m| < 1
    r = np.round(m * 256.0)                 # 8 significant bits; numpy rounds half to even
    y = np.ldexp(r / 256.0, e).astype(np.float32)
    return (y.view(np.uint32) >> 16).astype(np.uint16)


def bf(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_bf16_bits(x) -> np.ndarray:
    """float values that are exactly bf16 -> bits."""
    x = np.asarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0), "value not exact in bf16"
    return (bits >> 16).astype(np.uint16)


def silu(x):
    return x / (1.0 + np.exp(-x))


def inputs(B, T, H, HV, K, V, seed=0, permute=True):
    inp = synth.kda_to_numpy(synth.make_kda_inputs(B, T=T, H=H, HV=HV, K=K, V=V, seed=seed))
    if permute:   # slots and lines other than 0..B-1, in another order
        lines = inp["conv_pool"].shape[0]
        inp["cache_indices"] = np.array([(lines - 1 - i) for i in range(B)], dtype=np.int32)
        inp["inter_indices"] = np.array([(i + 1) % lines for i in range(B)], dtype=np.int32)
    return inp


def seq_of(inp, T, b, d):
    """The conv sequence of channel d of batch row b: 3 cached inputs then T tokens."""
    line = inp["cache_indices"][b]
    state = bf(inp["conv_pool"][line, :, d])
    toks = bf(inp["mixed"][b * T:(b + 1) * T, d])
    return np.concatenate([state, toks])


def dims(H, HV, K, V):
    return 2 * H * K + HV * V


# ---------------------------------------------------------------- conv

def pin_conv_one_hot_taps(orc):
    B, T, H, HV, K, V = 2, 3, 1, 2, 8, 4
    dim = dims(H, HV, K, V)
    for j in range(4):
        inp = inputs(B, T, H, HV, K, V, seed=j)
        w = np.zeros((dim, 4), dtype=np.float32)
        w[:, j] = 1.0
        inp["w"] = to_bf16_bits(w)
        inp["bias"] = np.zeros(dim, dtype=np.uint16)
        r = orc.kda_verify(inp, T, H, HV, K, V, K ** -0.5)
        for b in range(B):
            for d in range(dim):
                s = seq_of(inp, T, b, d)
                want = silu(s[j:j + T])
                got = r["conv_exact"][b * T:(b + 1) * T, d]
                assert np.allclose(got, want, rtol=1e-13, atol=1e-300), (j, b, d, got, want)


def pin_conv_zero_taps_is_bias(orc):
    B, T, H, HV, K, V = 2, 2, 1, 1, 8, 8
    dim = dims(H, HV, K, V)
    inp = inputs(B, T, H, HV, K, V)
    inp["w"] = np.zeros((dim, 4), dtype=np.uint16)
    r = orc.kda_verify(inp, T, H, HV, K, V, 1.0)
    want = silu(bf(inp["bias"]))
    assert np.allclose(r["conv_exact"], np.broadcast_to(want, r["conv_exact"].shape), rtol=1e-13)


def pin_conv_window(orc):
    B, T, H, HV, K, V = 3, 4, 1, 1, 8, 8
    dim = dims(H, HV, K, V)
    inp = inputs(B, T, H, HV, K, V)
    start = np.random.default_rng(1).integers(0, 65535, (B + 1, T, 3, dim)).astype(np.uint16)
    inp["win_pool"] = start
    r = orc.kda_verify(inp, T, H, HV, K, V, 1.0)
    win = r["win_pool"]
    for b in range(B):
        line = inp["inter_indices"][b]
        cl = inp["cache_indices"][b]
        seq = np.concatenate([inp["conv_pool"][cl], inp["mixed"][b * T:(b + 1) * T]], axis=0)  # [3+T, dim] bits
        for t in range(T):
            assert np.array_equal(win[line, t], seq[t + 1:t + 4]), (b, t)
    untouched = sorted(set(range(B + 1)) - set(int(i) for i in inp["inter_indices"]))
    for line in untouched:
        assert np.array_equal(win[line], start[line])


# ---------------------------------------------------------------- gates

def pin_gate_closed_forms(orc):
    B, T, H, HV, K, V, R = 1, 4, 1, 2, 4, 4, 16
    inp = inputs(B, T, H, HV, K, V, permute=False)
    a = np.zeros((B * T, HV * K), dtype=np.float32)
    a[0, :] = 0.0          # softplus(0) = ln 2
    a[1, :] = 25.0         # above the threshold: passes through
    a[2, :] = -30.0        # softplus(-30) = log1p(e^-30)
    a[3, :] = 10.0         # below the threshold: log1p(e^10), not 10
    inp["a"] = to_bf16_bits(a)
    inp["dt_bias"] = np.zeros(HV * K, dtype=np.float32)
    bvals = np.array([[0.0, 2.0], [-1.0, 0.5], [3.0, -3.0], [1.0, -1.0]], dtype=np.float32)
    inp["b"] = to_bf16_bits(bvals)
    r = orc.kda_verify(inp, T, H, HV, K, V, 1.0, snapshots=False, ring_len=R)
    slot = inp["cache_indices"][0]
    for hv in range(HV):
        A = math.exp(float(np.float32(inp["A_log"][hv])))
        want = [-A * math.log(2.0), -A * 25.0, -A * math.log1p(math.exp(-30.0)), -A * math.log1p(math.exp(10.0))]
        for t in range(T):
            assert np.allclose(r["g"][slot, hv, t], want[t], rtol=1e-14), (hv, t)
            assert abs(r["beta"][slot, hv, t] - 1.0 / (1.0 + math.exp(-float(bvals[t, hv])))) < 1e-15


# ---------------------------------------------------------------- recurrence

def _qk_hat(r, inp, T, H, K, b, t, h, scale):
    row = b * T + t
    c = bf(rne_bf16_f64(r["conv_exact"][row]))
    q = c[h * K:(h + 1) * K]
    k = c[H * K + h * K:H * K + (h + 1) * K]
    qh = q / math.sqrt(float(q @ q) + 1e-6) * scale
    kh = k / math.sqrt(float(k @ k) + 1e-6)
    return qh, kh, c


def pin_beta_one_projects_key_to_value(orc):
    B, T, H, HV, K, V = 2, 4, 1, 2, 16, 8
    inp = inputs(B, T, H, HV, K, V)
    inp["b"] = to_bf16_bits(np.full((B * T, HV), 60.0, dtype=np.float32))   # sigmoid(60) = 1 in fp64
    r = orc.kda_verify(inp, T, H, HV, K, V, K ** -0.5)
    for b in range(B):
        line = inp["inter_indices"][b]
        for hv in range(HV):
            h = hv // (HV // H)
            for t in range(T):
                _, kh, c = _qk_hat(r, inp, T, H, K, b, t, h, K ** -0.5)
                v = c[2 * H * K + hv * V:2 * H * K + (hv + 1) * V]
                S = r["inter_ssm"][line, t, hv]
                # S k^ = v (k^ . k^ = 1 - 1e-6 / |k|^2 leaves a part of the decayed state)
                assert np.allclose(S @ kh, v, atol=1e-5), (b, hv, t)


def pin_beta_zero_is_decay_only(orc):
    B, T, H, HV, K, V, R = 1, 4, 1, 1, 8, 4, 16
    inp = inputs(B, T, H, HV, K, V)
    inp["b"] = to_bf16_bits(np.full((B * T, HV), -60.0, dtype=np.float32))
    r = orc.kda_verify(inp, T, H, HV, K, V, 1.0, snapshots=True, ring_len=0)
    r2 = orc.kda_verify(inp, T, H, HV, K, V, 1.0, snapshots=False, ring_len=R)
    slot, line = inp["cache_indices"][0], inp["inter_indices"][0]
    S0 = inp["ssm"][slot, 0].astype(np.float64)
    gsum = np.zeros(K)
    for t in range(T):
        gsum += r2["g"][slot, 0, t]
        assert np.allclose(r["inter_ssm"][line, t, 0], S0 * np.exp(gsum)[None, :], rtol=1e-12, atol=1e-20), t


def pin_single_step_from_zero_state(orc):
    B, T, H, HV, K, V = 1, 1, 1, 1, 16, 8
    inp = inputs(B, T, H, HV, K, V)
    inp["ssm"][:] = 0.0
    scale = 0.25
    r = orc.kda_verify(inp, T, H, HV, K, V, scale, ring_len=16)
    slot = inp["cache_indices"][0]
    beta = 1.0 / (1.0 + math.exp(-float(bf(inp["b"][0, 0]))))
    qh, kh, c = _qk_hat(r, inp, T, H, K, 0, 0, 0, scale)
    v = c[2 * H * K:2 * H * K + V]
    want = beta * v * float(kh @ qh)
    assert np.allclose(r["o_exact"][0, 0], want, rtol=1e-12, atol=1e-15)
    assert np.allclose(r["inter_ssm"][inp["inter_indices"][0], 0, 0], beta * np.outer(v, kh), rtol=1e-12, atol=1e-18)
    assert abs(r["beta"][slot, 0, 0] - beta) < 1e-15


def pin_output_is_post_update_state_times_query(orc):
    B, T, H, HV, K, V = 2, 3, 2, 4, 16, 8     # two value heads per query/key head
    inp = inputs(B, T, H, HV, K, V)
    scale = K ** -0.5
    r = orc.kda_verify(inp, T, H, HV, K, V, scale)
    for b in range(B):
        line = inp["inter_indices"][b]
        for hv in range(HV):
            h = hv // (HV // H)
            for t in range(T):
                qh, _, _ = _qk_hat(r, inp, T, H, K, b, t, h, scale)
                want = r["inter_ssm"][line, t, hv] @ qh
                assert np.allclose(r["o_exact"][b * T + t, hv], want, rtol=1e-12, atol=1e-15), (b, hv, t)


def pin_ring_contents(orc):
    B, T, H, HV, K, V, R = 2, 3, 1, 2, 8, 4, 16
    inp = inputs(B, T, H, HV, K, V)
    start = {k: inp[k].copy() for k in ("rawv", "rawk", "g", "beta")}
    r = orc.kda_verify(inp, T, H, HV, K, V, 1.0, snapshots=False, ring_len=R)
    touched = set()
    for b in range(B):
        slot = inp["cache_indices"][b]
        touched.add(int(slot))
        for t in range(T):
            c = rne_bf16_f64(r["conv_exact"][b * T + t])
            for hv in range(HV):
                assert np.array_equal(r["rawv"][slot, hv, t], c[2 * H * K + hv * V:2 * H * K + (hv + 1) * V])
            for h in range(H):
                assert np.array_equal(r["rawk"][slot, h, t], c[H * K + h * K:H * K + (h + 1) * K])
        for name in ("rawv", "rawk", "g", "beta"):   # positions past T keep their contents
            assert np.array_equal(r[name][slot][:, T:], start[name][slot][:, T:].astype(r[name].dtype))
    for slot in set(range(B + 1)) - touched:
        for name in ("rawv", "rawk", "g", "beta"):
            assert np.array_equal(r[name][slot], start[name][slot].astype(r[name].dtype))


def pin_output_rounding(orc):
    B, T, H, HV, K, V = 2, 2, 1, 1, 16, 16
    inp = inputs(B, T, H, HV, K, V)
    r = orc.kda_verify(inp, T, H, HV, K, V, K ** -0.5)
    assert np.array_equal(r["o"], rne_bf16_f64(r["o_exact"]))


ALL_KDA_PINS = [
    pin_conv_one_hot_taps,
    pin_conv_zero_taps_is_bias,
    pin_conv_window,
    pin_gate_closed_forms,
    pin_beta_one_projects_key_to_value,
    pin_beta_zero_is_decay_only,
    pin_single_step_from_zero_state,
    pin_output_is_post_update_state_times_query,
    pin_ring_contents,
    pin_output_rounding,
]
