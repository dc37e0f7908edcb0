/*
 * kda.c -- TEST INFRASTRUCTURE ONLY (built into the same liboracle.so as oracle.c).
 *
 * Plain CPU definition of one layer of the KDA chain-verify step benchmarked on the sglang
 * page "benchmark/kernels/bench_kda_verify_sweep.py" (its make_inputs and make_runner: the
 * unfused leg runs causal_conv1d_update, splits the result into q, k, v and runs
 * fused_sigmoid_gating_delta_rule_update with is_kda, the q/k L2 norm, the sigmoid gate and
 * disable_state_update; the fused legs compute the same in one kernel; "+ring" legs store
 * the step inputs in ring buffers instead of per-step state snapshots).
 *
 * The page gives the calls, argument names, shapes and dtypes, not the kernels' arithmetic.
 * The readings taken (each is the plain meaning of an argument name on the page, or the
 * standard definition of the named operation):
 *  - conv: per channel d, the sequence is the W-1 = 3 cached inputs (oldest first) followed
 *    by the T new tokens; output t = silu(bias[d] + sum_w weight[d, w] * seq[t + w]); the
 *    result is materialised in bf16 (the page's tensors are bf16) before the split into q,
 *    k (H heads of K channels each) and v (HV heads of V channels);
 *  - conv state: read only (a verify step commits nothing); after token t the window
 *    seq[t+1 .. t+3] is written to intermediate_conv_window[inter_idx[b], t];
 *  - gate (is_kda, no lower bound): g[t, hv, c] = -exp(A_log[hv]) * softplus(a + dt_bias)
 *    per K channel c, softplus with beta 1 and threshold 20 (x above 20 passes through);
 *    beta[t, hv] = sigmoid(b);
 *  - q and k are L2-normalised over K as x / sqrt(sum x^2 + 1e-6); q is multiplied by
 *    scale (the page passes K^-0.5); q/k head of v head hv is hv / (HV / H);
 *  - the state S[V, K] of (b, hv) starts as ssm[cache_idx[b], hv]; per token:
 *        S[v, c] *= exp(g[c]);  u[v] = beta * (v_t[v] - sum_c S[v, c] k[c]);
 *        S[v, c] += u[v] * k[c];  o_t[v] = sum_c S[v, c] q[c];
 *    ssm itself is not written (disable_state_update);
 *  - snapshot mode: S after token t goes to intermediate_states[inter_idx[b], t, hv];
 *  - ring mode: token t's conv outputs v (per hv) and k (per q/k head, before the norm),
 *    its gate g and beta go to position t of the ring of slot cache_idx[b] (the page sizes
 *    the ring at twice the draft tokens; where a verify starts in the ring is not on the
 *    page, position t is the plain reading);
 *  - o is written in bf16, [B*T, HV, V].
 * Everything after the bf16 conv outputs is fp64; o and the conv outputs are rounded to
 * bf16 directly from fp64 (oracle_round_bf16).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

uint16_t oracle_round_bf16(double v);      /* oracle.c */
double oracle_bf16_to_double(uint16_t b);  /* oracle.c */

#define KDA_W 4

static double silu(double x) { return x / (1.0 + exp(-x)); }

static double softplus_b1_t20(double x) { return x > 20.0 ? x : log1p(exp(x)); }

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* Conv output of channel d for token t of batch row bi (before the bf16 rounding). */
static double conv_value(const uint16_t *mixed, const uint16_t *conv_w, const uint16_t *conv_b,
                         const uint16_t *state_line, int64_t dim, int64_t T, int64_t bi, int64_t t,
                         int64_t d) {
    double acc = oracle_bf16_to_double(conv_b[d]);
    for (int w = 0; w < KDA_W; ++w) {
        const int64_t s = t + w;   /* index into [state(3), tokens(T)] */
        const uint16_t x = s < KDA_W - 1 ? state_line[s * dim + d] : mixed[(bi * T + (s - (KDA_W - 1))) * dim + d];
        acc += oracle_bf16_to_double(conv_w[d * KDA_W + w]) * oracle_bf16_to_double(x);
    }
    return silu(acc);
}

int oracle_kda_verify(int64_t B, int64_t T, int64_t H, int64_t HV, int64_t K, int64_t V, int64_t lines,
                      int64_t slots, int64_t ring_len, double scale, const uint16_t *mixed,
                      const uint16_t *conv_w, const uint16_t *conv_b, const uint16_t *conv_state,
                      const int32_t *conv_idx, const int32_t *inter_idx, const uint16_t *a,
                      const uint16_t *bgate, const float *A_log, const float *dt_bias, const float *ssm,
                      const int32_t *cache_idx, uint16_t *conv_win, double *snap, uint16_t *ring_v,
                      uint16_t *ring_k, double *ring_g, double *ring_beta, uint16_t *out,
                      double *out_exact, double *conv_exact) {
    if (B < 0 || T < 1 || H < 1 || HV < 1 || HV % H != 0 || K < 1 || V < 1 || lines < 1 || slots < 1)
        return -1;
    if ((ring_v || ring_k || ring_g || ring_beta) && ring_len < T) return -1;
    const int64_t dim = 2 * H * K + HV * V;
    const int64_t group = HV / H;

    /* conv outputs of every token and channel, rounded to bf16 (the materialised tensor) */
    uint16_t *cv = malloc(sizeof(uint16_t) * (size_t)(B * T * dim));
    double *S = malloc(sizeof(double) * (size_t)(V * K));
    double *q = malloc(sizeof(double) * (size_t)K), *k = malloc(sizeof(double) * (size_t)K);
    double *g = malloc(sizeof(double) * (size_t)K);
    if (!cv || !S || !q || !k || !g) {
        free(cv); free(S); free(q); free(k); free(g);
        return -2;
    }
    for (int64_t bi = 0; bi < B; ++bi) {
        const uint16_t *state_line = conv_state + (int64_t)conv_idx[bi] * (KDA_W - 1) * dim;
        for (int64_t t = 0; t < T; ++t)
            for (int64_t d = 0; d < dim; ++d) {
                const double c = conv_value(mixed, conv_w, conv_b, state_line, dim, T, bi, t, d);
                if (conv_exact) conv_exact[(bi * T + t) * dim + d] = c;
                cv[(bi * T + t) * dim + d] = oracle_round_bf16(c);
            }
        if (conv_win) {   /* window after token t: seq[t+1 .. t+3] */
            for (int64_t t = 0; t < T; ++t)
                for (int w = 0; w < KDA_W - 1; ++w) {
                    const int64_t s = t + 1 + w;
                    for (int64_t d = 0; d < dim; ++d) {
                        const uint16_t x = s < KDA_W - 1 ? state_line[s * dim + d]
                                                         : mixed[(bi * T + (s - (KDA_W - 1))) * dim + d];
                        conv_win[(((int64_t)inter_idx[bi] * T + t) * (KDA_W - 1) + w) * dim + d] = x;
                    }
                }
        }
    }

    for (int64_t bi = 0; bi < B; ++bi) {
        const int64_t slot = cache_idx[bi];
        for (int64_t hv = 0; hv < HV; ++hv) {
            const int64_t h = hv / group;
            const float *s0 = ssm + (slot * HV + hv) * V * K;
            for (int64_t i = 0; i < V * K; ++i) S[i] = (double)s0[i];
            const double decay_a = exp((double)A_log[hv]);
            for (int64_t t = 0; t < T; ++t) {
                const int64_t row = bi * T + t;
                const uint16_t *c_row = cv + row * dim;
                double qq = 0.0, kk = 0.0;
                for (int64_t c = 0; c < K; ++c) {
                    q[c] = oracle_bf16_to_double(c_row[h * K + c]);
                    k[c] = oracle_bf16_to_double(c_row[H * K + h * K + c]);
                    qq += q[c] * q[c];
                    kk += k[c] * k[c];
                }
                const double qn = 1.0 / sqrt(qq + 1e-6), kn = 1.0 / sqrt(kk + 1e-6);
                for (int64_t c = 0; c < K; ++c) {
                    const double x = oracle_bf16_to_double(a[row * HV * K + hv * K + c]) + (double)dt_bias[hv * K + c];
                    g[c] = -decay_a * softplus_b1_t20(x);
                }
                const double beta = sigmoid(oracle_bf16_to_double(bgate[row * HV + hv]));
                if (ring_v || ring_k || ring_g || ring_beta) {
                    const int64_t pos = t;
                    if (ring_v)
                        for (int64_t v = 0; v < V; ++v)
                            ring_v[((slot * HV + hv) * ring_len + pos) * V + v] = c_row[2 * H * K + hv * V + v];
                    if (ring_k && hv % group == 0)
                        for (int64_t c = 0; c < K; ++c)
                            ring_k[((slot * H + h) * ring_len + pos) * K + c] = c_row[H * K + h * K + c];
                    if (ring_g)
                        for (int64_t c = 0; c < K; ++c) ring_g[((slot * HV + hv) * ring_len + pos) * K + c] = g[c];
                    if (ring_beta) ring_beta[(slot * HV + hv) * ring_len + pos] = beta;
                }
                for (int64_t c = 0; c < K; ++c) {
                    q[c] *= qn * scale;
                    k[c] *= kn;
                }
                for (int64_t v = 0; v < V; ++v) {
                    double *Sv = S + v * K;
                    double sk = 0.0;
                    for (int64_t c = 0; c < K; ++c) {
                        Sv[c] *= exp(g[c]);
                        sk += Sv[c] * k[c];
                    }
                    const double u = beta * (oracle_bf16_to_double(c_row[2 * H * K + hv * V + v]) - sk);
                    double o = 0.0;
                    for (int64_t c = 0; c < K; ++c) {
                        Sv[c] += u * k[c];
                        o += Sv[c] * q[c];
                    }
                    if (out_exact) out_exact[(row * HV + hv) * V + v] = o;
                    if (out) out[(row * HV + hv) * V + v] = oracle_round_bf16(o);
                }
                if (snap) {
                    double *dst = snap + ((((int64_t)inter_idx[bi] * T + t) * HV + hv) * V) * K;
                    memcpy(dst, S, sizeof(double) * (size_t)(V * K));
                }
            }
        }
    }
    free(cv); free(S); free(q); free(k); free(g);
    return 0;
}
