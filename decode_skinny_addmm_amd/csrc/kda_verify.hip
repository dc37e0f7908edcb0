// kda_verify.hip -- one layer of the KDA chain-verify step (conv1d update, KDA gate, gated delta
// rule with per-token state snapshots or ring entries), fused into one kernel.
//
// Operation: the sglang page "benchmark/kernels/bench_kda_verify_sweep.py" (make_inputs and
// make_runner: causal_conv1d_update then fused_sigmoid_gating_delta_rule_update with is_kda,
// or fused_kda_conv_gating_verify), as defined in the C ABI header next to
// skinny_kda_verify_bf16.
//
// Where the bytes are: per (batch row, value head) the fp32 state [V, K] is read once (64 KB
// at V = K = 128) and, in snapshot mode, written T times; everything else (the conv inputs
// of 2K + V channels, the gates) is a few KB. So the kernel is an HBM stream of states, and
// the layout is chosen for it:
//   * a workgroup owns BV rows of one state; 16 lanes per row, 8 K channels per lane in two
//     runs of four (lch): the state slice lives in registers for all T tokens, every load and
//     snapshot store is a 16-byte vector, and a 16-lane group's access covers whole 128-byte
//     lines of the row's 512 contiguous bytes; the state loads are nontemporal;
//   * the state loads are issued right after the conv and gate inputs, so that their latency
//     hides behind the conv and gate work, which never waits for them; conv outputs (rounded
//     to bf16, the precision the unfused path materialises), the normalised q and k, exp(g)
//     and beta of all T tokens are staged in LDS once;
//   * per token: decay, S k^ and S q^ as 8-wide partial dots closed by a 16-lane DPP sum;
//   * the conv over q/k channels is recomputed by every workgroup of the head (256 channels
//     x T tokens, a few hundred FMAs per lane) instead of a second kernel and a round trip;
//     windows and ring entries shared by several workgroups are written by one of them.
#include "common.hpp"

namespace skinny {
namespace {

constexpr int KD = 128;        // head dimension of q and k (the page's shape)
constexpr int TLIM = 16;       // most draft tokens per verify
constexpr int CPL = KD / 16;   // K channels per lane

// K channel c (0..7) of lane j of a 16-lane group: two runs of four, at 4j and at 64 + 4j, so a
// group's 16-byte accesses to a 512-byte state row cover whole 128-byte lines (two per access)
__device__ __forceinline__ int lch(int j, int c) { return (c >> 2) * (KD / 2) + 4 * j + (c & 3); }

__device__ __forceinline__ float row16_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));  // ror 8
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));  // ror 4
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xF, 0xF, false));  // ror 2
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xF, 0xF, false));  // ror 1
    return v;
}

// 16-byte load marked nontemporal: the states are read once per call, and keeping them out of
// the caches' retained set leaves room for the snapshot writes (29 against 37 us at B = 64)
__device__ __forceinline__ float4 ldnt4(const float *p) {
    typedef float vf4 __attribute__((ext_vector_type(4)));
    const vf4 v = __builtin_nontemporal_load(reinterpret_cast<const vf4 *>(p));
    return make_float4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Fast exp / log (the hardware exp2 and log2 with one scaling multiply, ~2 ulp): gate math
// whose results are compared at 1e-5 relative, or that only feed fp32 state arithmetic.
__device__ __forceinline__ float fexp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
__device__ __forceinline__ float flog(float x) { return __builtin_amdgcn_logf(x) * 0.6931471805599453f; }

// softplus with beta 1 and threshold 20; below -15 log1p(e^x) = e^x to fp32 precision
__device__ __forceinline__ float softplus20(float x) {
    return x > 20.0f ? x : (x < -15.0f ? fexp(x) : flog(1.0f + fexp(x)));
}

// grid (V / BV, HV, B), block GR * 16 lanes: GR groups of 16 lanes, each group owning RPG
// consecutive state rows (BV = GR * RPG rows per workgroup).
// TMAX: token bound of this instance (4, 8 or 16 >= T): token loops unroll to it, token loads
// past T repeat token T - 1 (unconditional loads keep the memory waits exact).
template <int GR, int RPG, int TMAX>
__global__ __launch_bounds__(GR * 16) void kda_verify_kernel(skinny_kda_args a) {
    constexpr int NT = GR * 16, BV = GR * RPG;
    constexpr int GCH = (KD + NT - 1) / NT;   // gate channels per lane
    __shared__ float sq[TMAX][KD], sk[TMAX][KD], seg[TMAX][KD];
    __shared__ float sv[TMAX][BV];
    __shared__ float sbeta[TMAX], sqn[TMAX], skn[TMAX];

    const int tid = threadIdx.x;
    const int v0 = blockIdx.x * BV, hv = blockIdx.y, b = blockIdx.z;
    const int T = (int)a.T, H = (int)a.H, HV = (int)a.HV, V = (int)a.V, R = (int)a.ring_len;
    const int group = HV / H, h = hv / group;
    const size_t dim = (size_t)2 * H * KD + (size_t)HV * V;
    // the cache indices, issued first and both at once (the second reads cache_idx again when
    // no output needs inter_idx), through the vector memory path (an opaque zero offset), and
    // first used after the loads below that do not depend on them (the asm there): those go out
    // without waiting for the indices' round trip. (As scalar loads the compiler may wait for
    // them before the first vector load; measured 0.3-0.5 us slower at B = 1 and 4.)
    const bool need_iline = a.conv_win || a.snap;
    const int32_t *iptr = need_iline ? a.inter_idx : a.cache_idx;
    int zero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
    int cidx = a.cache_idx[b + zero], iraw = iptr[b + zero];
    const bool qk_writer = v0 == 0 && hv % group == 0;   // writes the q/k windows and ring k of head h
    const bool head_writer = v0 == 0;                    // writes ring g and beta of value head hv
    const bool ring = a.ring_v != nullptr;

    // Loads, in the order they are used (the memory counter is waited on in issue order): this
    // lane's conv weights and new inputs and its gate inputs (none depends on the cache
    // indices), the indices, the cached conv inputs, then the state rows (the largest part,
    // needed last: its transfer overlaps the conv, the gates and the first rows).
    constexpr int NCH = 2 * KD + BV;             // conv channels of this workgroup
    constexpr int CCH = (NCH + NT - 1) / NT;     // ... per lane
    const int gi = tid >> 4, j = tid & 15;
    const uint16_t *mixed = static_cast<const uint16_t *>(a.mixed);
    const uint16_t *cw = static_cast<const uint16_t *>(a.conv_w);
    const uint16_t *cb = static_cast<const uint16_t *>(a.conv_b);
    const uint16_t *pool = static_cast<const uint16_t *>(a.conv_pool);
    uint16_t *win = static_cast<uint16_t *>(a.conv_win);
    size_t chs[CCH];
    uint16_t wraw[CCH][4], braw_c[CCH], seq[CCH][TMAX + 3];   // fully unrolled: registers
#pragma unroll
    for (int u = 0; u < CCH; ++u) {
        const int i = min(tid + u * NT, NCH - 1);
        const size_t ch = i < KD ? (size_t)h * KD + i
                                 : i < 2 * KD ? (size_t)H * KD + (size_t)h * KD + (i - KD)
                                              : (size_t)2 * H * KD + (size_t)hv * V + v0 + (i - 2 * KD);
        chs[u] = ch;
#pragma unroll
        for (int q = 0; q < 4; ++q) wraw[u][q] = cw[ch * 4 + q];
        braw_c[u] = cb[ch];
#pragma unroll
        for (int t = 0; t < TMAX; ++t) seq[u][3 + t] = mixed[((size_t)b * T + min(t, T - 1)) * dim + ch];
    }
    const uint16_t *ag = static_cast<const uint16_t *>(a.a);
    const uint16_t *bg = static_cast<const uint16_t *>(a.b);
    uint16_t araw[GCH][TMAX];
    float dtb[GCH];
#pragma unroll
    for (int u = 0; u < GCH; ++u) {
        const int c = min(tid + u * NT, KD - 1);
#pragma unroll
        for (int t = 0; t < TMAX; ++t)
            araw[u][t] = ag[((size_t)b * T + min(t, T - 1)) * HV * KD + (size_t)hv * KD + c];
        dtb[u] = a.dt_bias[hv * KD + c];
    }
    const uint16_t braw = bg[((size_t)b * T + min(tid, T - 1)) * HV + hv];
    const float alog = a.A_log[hv];
    asm volatile("" : "+v"(cidx), "+v"(iraw) : : "memory");   // the indices are first used here
    const int slot = clampi(cidx, 0, (int)a.slots - 1);
    const int cline = clampi(cidx, 0, (int)a.lines - 1);
    const int iline = need_iline ? clampi(iraw, 0, (int)a.lines - 1) : 0;
#pragma unroll
    for (int u = 0; u < CCH; ++u)
#pragma unroll
        for (int s2 = 0; s2 < 3; ++s2) seq[u][s2] = pool[((size_t)cline * 3 + s2) * dim + chs[u]];
    float4 s4[RPG][2];
#pragma unroll
    for (int r = 0; r < RPG; ++r) {
        const float *srow = a.ssm + (((size_t)slot * HV + hv) * V + v0 + gi * RPG + r) * KD + 4 * j;
        s4[r][0] = ldnt4(srow);
        s4[r][1] = ldnt4(srow + KD / 2);
    }
    const float negA = -fexp(alog);

    // conv over the q, k (head h) and v (rows v0 .. v0+BV of head hv) channels: all T outputs
    // of a channel from its 3 cached and T new inputs. The arithmetic runs on every lane and
    // token (lanes past the last channel repeat it, tokens past T repeat token T - 1, as their
    // loads did) and only the writes are guarded; each result is also consumed outside the
    // guard (the empty asm), so the compiler cannot move the loads into the guarded code, behind
    // the state loads, where waiting for them would mean waiting for the whole state.
#pragma unroll
    for (int u = 0; u < CCH; ++u) {
        const int i = tid + u * NT;
        const bool live = i < NCH;
        const size_t ch = chs[u];
        float w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = bf16_bits_to_f32(wraw[u][q]);
        const float bias = bf16_bits_to_f32(braw_c[u]);
        const bool write_win = win && (i >= 2 * KD || qk_writer);
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
            float acc = bias;
#pragma unroll
            for (int q = 0; q < 4; ++q) acc = fmaf(w[q], bf16_bits_to_f32(seq[u][t + q]), acc);
            // silu with the accurate exp and an IEEE division: this value is rounded to bf16
            const uint16_t c = f32_to_bf16_rne(acc / (1.0f + expf(-acc)));
            const float cf = bf16_bits_to_f32(c);
            asm volatile("" : : "v"(cf));
            if (live && t < T) {
                if (i < KD) {
                    sq[t][i] = cf;
                } else if (i < 2 * KD) {
                    sk[t][i - KD] = cf;
                    if (ring && qk_writer)
                        static_cast<uint16_t *>(a.ring_k)[(((size_t)slot * H + h) * R + t) * KD + (i - KD)] = c;
                } else {
                    sv[t][i - 2 * KD] = cf;
                    if (ring)
                        static_cast<uint16_t *>(a.ring_v)[(((size_t)slot * HV + hv) * R + t) * V + v0 + (i - 2 * KD)] = c;
                }
                if (write_win)
#pragma unroll
                    for (int w2 = 0; w2 < 3; ++w2)
                        win[(((size_t)iline * T + t) * 3 + w2) * dim + ch] = seq[u][t + 1 + w2];
            }
        }
    }

    // gates from the registers loaded above: exp(g) per token and K channel, beta per token
    // (unconditional arithmetic, guarded writes, as for the conv)
#pragma unroll
    for (int u = 0; u < GCH; ++u) {
        const int c = tid + u * NT;
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
            const float g = negA * softplus20(bf16_bits_to_f32(araw[u][t]) + dtb[u]);
            const float e = fexp(g);
            asm volatile("" : : "v"(e));
            if (c < KD && t < T) {
                seg[t][c] = e;
                if (ring && head_writer) a.ring_g[(((size_t)slot * HV + hv) * R + t) * KD + c] = g;
            }
        }
    }
    {
        const float beta = 1.0f / (1.0f + fexp(-bf16_bits_to_f32(braw)));
        asm volatile("" : : "v"(beta));
        if (tid < T) {
            sbeta[tid] = beta;
            if (ring && head_writer) a.ring_beta[((size_t)slot * HV + hv) * R + tid] = beta;
        }
    }
    __syncthreads();

    // L2 norms of q and k per token: one 16-lane group per (token, q|k)
    for (int r = gi; r < 2 * T; r += GR) {
        const float *src = r < T ? sq[r] : sk[r - T];
        float p = 0.0f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) p = fmaf(src[lch(j, c)], src[lch(j, c)], p);
        p = row16_sum(p);
        if (j == 0) {
            const float n = 1.0f / sqrtf(p + 1e-6f);
            if (r < T) sqn[r] = n * a.scale;
            else skn[r - T] = n;
        }
    }
    __syncthreads();

    uint16_t *out = static_cast<uint16_t *>(a.out);
    // the recurrence, row by row (all T tokens of a row before the next): each row waits only
    // for its own 512 bytes of state, so the state stream overlaps the arithmetic
    if constexpr (TMAX == 4) {
        // up to 4 tokens: this lane's exp(g), k^ and q^ slices of every token, beta and the v
        // values of its rows move to registers once; the row pairs below then run on VALU and
        // DPP alone
        float e[4][CPL], kk[4][CPL], qq[4][CPL], bt[4], vv[4][RPG];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int tc = min(t, T - 1);
            const float kn = skn[tc], qn = sqn[tc];
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                e[t][c] = seg[tc][lch(j, c)];
                kk[t][c] = sk[tc][lch(j, c)] * kn;
                qq[t][c] = sq[tc][lch(j, c)] * qn;
            }
            bt[t] = sbeta[tc];
#pragma unroll
            for (int r = 0; r < RPG; ++r) vv[t][r] = sv[tc][gi * RPG + r];
        }
        constexpr int RP = RPG >= 4 ? 4 : RPG;   // rows per step of the loop (independent chains)
#pragma unroll
        for (int r0 = 0; r0 < RPG; r0 += RP) {
            float S[RP][CPL];
#pragma unroll
            for (int x = 0; x < RP; ++x) {
                S[x][0] = s4[r0 + x][0].x; S[x][1] = s4[r0 + x][0].y; S[x][2] = s4[r0 + x][0].z;
                S[x][3] = s4[r0 + x][0].w; S[x][4] = s4[r0 + x][1].x; S[x][5] = s4[r0 + x][1].y;
                S[x][6] = s4[r0 + x][1].z; S[x][7] = s4[r0 + x][1].w;
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if (t < T) {
                    float skp[RP], op[RP];
#pragma unroll
                    for (int x = 0; x < RP; ++x) {
                        skp[x] = 0.0f;
#pragma unroll
                        for (int c = 0; c < CPL; ++c) {
                            S[x][c] *= e[t][c];
                            skp[x] = fmaf(S[x][c], kk[t][c], skp[x]);
                        }
                    }
#pragma unroll
                    for (int x = 0; x < RP; ++x) skp[x] = row16_sum(skp[x]);
#pragma unroll
                    for (int x = 0; x < RP; ++x) {
                        const float u = bt[t] * (vv[t][r0 + x] - skp[x]);
                        op[x] = 0.0f;
#pragma unroll
                        for (int c = 0; c < CPL; ++c) {
                            S[x][c] = fmaf(u, kk[t][c], S[x][c]);
                            op[x] = fmaf(S[x][c], qq[t][c], op[x]);
                        }
                    }
#pragma unroll
                    for (int x = 0; x < RP; ++x) op[x] = row16_sum(op[x]);
#pragma unroll
                    for (int x = 0; x < RP; ++x) {
                        const int vl = gi * RPG + r0 + x;
                        if (j == 0) out[(((size_t)b * T + t) * HV + hv) * V + v0 + vl] = f32_to_bf16_rne(op[x]);
                        if (a.snap) {
                            float *dst = a.snap + ((((size_t)iline * T + t) * HV + hv) * V + v0 + vl) * KD + 4 * j;
                            *reinterpret_cast<float4 *>(dst) = make_float4(S[x][0], S[x][1], S[x][2], S[x][3]);
                            *reinterpret_cast<float4 *>(dst + KD / 2) = make_float4(S[x][4], S[x][5], S[x][6], S[x][7]);
                        }
                    }
                }
            }
        }
    } else {
#pragma unroll
        for (int r = 0; r < RPG; ++r) {
            const int vl = gi * RPG + r;            // row within the workgroup
            float S[CPL] = {s4[r][0].x, s4[r][0].y, s4[r][0].z, s4[r][0].w,
                            s4[r][1].x, s4[r][1].y, s4[r][1].z, s4[r][1].w};
            for (int t = 0; t < T; ++t) {
                const float kn = skn[t];
                float skp = 0.0f;
                float kk[CPL];
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    kk[c] = sk[t][lch(j, c)] * kn;
                    S[c] *= seg[t][lch(j, c)];
                    skp = fmaf(S[c], kk[c], skp);
                }
                skp = row16_sum(skp);
                const float u = sbeta[t] * (sv[t][vl] - skp);
                const float qn = sqn[t];
                float op = 0.0f;
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    S[c] = fmaf(u, kk[c], S[c]);
                    op = fmaf(S[c], sq[t][lch(j, c)] * qn, op);
                }
                op = row16_sum(op);
                if (j == 0) out[(((size_t)b * T + t) * HV + hv) * V + v0 + vl] = f32_to_bf16_rne(op);
                if (a.snap) {
                    float *dst = a.snap + ((((size_t)iline * T + t) * HV + hv) * V + v0 + vl) * KD + 4 * j;
                    *reinterpret_cast<float4 *>(dst) = make_float4(S[0], S[1], S[2], S[3]);
                    *reinterpret_cast<float4 *>(dst + KD / 2) = make_float4(S[4], S[5], S[6], S[7]);
                }
            }
        }
    }
}

template <int GR, int RPG>
hipError_t launch_shape(const skinny_kda_args &a, hipStream_t stream) {
    constexpr int BV = GR * RPG;
    dim3 grid((unsigned)(a.V / BV), (unsigned)a.HV, (unsigned)a.B);
    if (a.T <= 4)
        hipLaunchKernelGGL((kda_verify_kernel<GR, RPG, 4>), grid, dim3(GR * 16), 0, stream, a);
    else if (a.T <= 8)
        hipLaunchKernelGGL((kda_verify_kernel<GR, RPG, 8>), grid, dim3(GR * 16), 0, stream, a);
    else
        hipLaunchKernelGGL((kda_verify_kernel<GR, RPG, TLIM>), grid, dim3(GR * 16), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_kda_verify(const skinny_kda_args &a, hipStream_t stream) {
    // Rows per workgroup: the conv of the q/k channels and the gates are recomputed by every
    // workgroup of a (batch row, value head), so rows per workgroup are as many as still fill the
    // chip: 128 while that gives >= 512 workgroups (two per CU), else the most of 64, 32, 16 that
    // gives >= 256 (measured at B = 1 ... 64 in both layouts: within 1 % of the best forced shape
    // everywhere; one ">= 512" threshold for every size loses 5-10 % at B = 8 and 16), and
    // never fewer than 16 (at B = 1, 64 workgroups of 16 rows beat 256 of 4).
    const int64_t rows = a.B * a.HV * a.V;
    if (a.V % 128 == 0 && rows / 128 >= 512) return launch_shape<16, 8>(a, stream);
    if (a.V % 64 == 0 && rows / 64 >= 256) return launch_shape<16, 4>(a, stream);
    if (a.V % 32 == 0 && rows / 32 >= 256) return launch_shape<16, 2>(a, stream);
    return launch_shape<16, 1>(a, stream);
}

}  // namespace skinny
