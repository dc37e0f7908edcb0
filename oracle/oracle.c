/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU definition of the skinny residual
 * GEMM  Y = X * W^T + R  (X bf16[M,K], W bf16[N,K], R bf16[M,N], Y bf16[M,N]).
 *
 * Source of the definition: the vLLM benchmark page
 * "benchmarks/kernels/benchmark_k3_cutedsl_residual.py" -- its module docstring
 * states the operation (bf16 inputs, fp32 accumulation, bf16 output) and its
 * cuBLAS leg expresses it as torch.addmm(residual, a, b.t()) with alpha = beta = 1.
 *
 * What this file computes, per output element (m, n):
 *   exact   = sum_{k<K} x[m,k] * w[n,k]  +  r[m,n]      (real arithmetic)
 *   Y[m,n]  = round_to_nearest_even_bf16(exact)           (one rounding)
 * The sum is carried in fp64. Every bf16 x bf16 product has at most 16
 * significant bits, so it is exact in fp64; the K products and r are added
 * with Neumaier's compensated summation (A. Neumaier, 1974), which leaves an
 * error of about one fp64 rounding of the result plus O(K * 2^-106 * sum|terms|).
 * The fp64 value is rounded straight to bf16 (never through fp32, which would
 * round twice).
 *
 * Readings taken where the pages leave a step open:
 *  - one rounding of (accumulator + residual), not the page-2 kernel's
 *    "round the product to bf16, add the residual, round again";
 *  - round-to-nearest, ties-to-even; NaN stays NaN; overflow goes to +-Inf;
 *  - no sanitising of negative zero.
 *
 * The page-2 epilogue itself (the vLLM API page "fused_add_multicast_skinny_gemm",
 * FusedAddMulticastSkinnyGemm.kernel, tensor-parallel shard form) is available through
 * the *_ex entry points and two flags:
 *  - ORACLE_ROUND_PRODUCT: g = bf16(sum_k x*w) first, then Y = bf16(g + r). g and r are
 *    bf16 values, so g + r is exact in fp64 whenever their exponents differ by at most
 *    45; otherwise the smaller one is below 2^-45 of the larger and cannot move the
 *    bf16 rounding of the sum, so fp64 gives the exact rounded result either way;
 *  - ORACLE_NO_NEG_ZERO: a bf16 result of -0 is written as +0 (that page keeps -0 as
 *    its not-yet-written marker).
 * With no flag the *_ex functions compute exactly what the plain ones do.
 *
 * Who may use this: only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg. The GPU library never links or calls it, and
 * this file includes nothing from the GPU library.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* bf16 bits -> exact double (a bf16 is the upper half of an IEEE binary32). */
static double bf16_bits_to_double(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

double oracle_bf16_to_double(uint16_t b) { return bf16_bits_to_double(b); }

/*
 * Round a double to the nearest bf16 (8 significant bits, binary32 exponent
 * range), ties to even, written from the format's definition:
 *   - the representable magnitudes with exponent e (2^e <= |v| < 2^(e+1)) are
 *     multiples of q = 2^(e-7); below 2^-126 the spacing stays 2^-133
 *     (subnormals);
 *   - v/q is rounded to an integer, a tie goes to the even integer;
 *   - a result of 2^128 or more is infinity.
 */
uint16_t oracle_round_bf16(double v) {
    if (isnan(v)) return (uint16_t)0x7FC0;
    uint16_t sign = signbit(v) ? (uint16_t)0x8000 : (uint16_t)0;
    double a = fabs(v);
    if (isinf(a)) return (uint16_t)(sign | 0x7F80);
    if (a == 0.0) return sign;

    int e2;
    (void)frexp(a, &e2);          /* a = f * 2^e2, f in [0.5, 1): 2^(e2-1) <= a */
    int e = e2 - 1;               /* 2^e <= a < 2^(e+1) */
    if (e < -126) e = -126;       /* subnormal range keeps the 2^-133 spacing */
    double q = ldexp(1.0, e - 7);
    double t = a / q;             /* exact: division by a power of two */
    double fl = floor(t);
    double frac = t - fl;         /* exact */
    double n;
    if (frac > 0.5) n = fl + 1.0;
    else if (frac < 0.5) n = fl;
    else n = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;   /* tie: to even */
    double r = n * q;             /* exact */
    if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80);

    float rf = (float)r;          /* exact: r is a bf16 value */
    uint32_t u;
    memcpy(&u, &rf, sizeof u);
    return (uint16_t)(sign | ((u >> 16) & 0x7FFF));
}

#define ORACLE_ROUND_PRODUCT 1u
#define ORACLE_NO_NEG_ZERO 2u

/* One output element, by the definition above. With ORACLE_ROUND_PRODUCT the residual is
 * left out of the compensated sum and added after the sum has been rounded to bf16; acc_out
 * then receives bf16(sum) + r, the value the second rounding applies to. */
static void one_element(const uint16_t *X, const uint16_t *W, const uint16_t *R,
                        int64_t N, int64_t K, int64_t m, int64_t n, unsigned flags,
                        uint16_t *y_out, double *acc_out) {
    const int round_product = (flags & ORACLE_ROUND_PRODUCT) != 0;
    double s = 0.0, c = 0.0;      /* Neumaier: running sum and compensation */
    for (int64_t k = 0; k <= K; ++k) {
        if (k == K && round_product) break;
        double p = (k < K) ? bf16_bits_to_double(X[m * K + k]) * bf16_bits_to_double(W[n * K + k])
                           : bf16_bits_to_double(R[m * N + n]);
        double t = s + p;
        if (fabs(s) >= fabs(p)) c += (s - t) + p;
        else c += (p - t) + s;
        s = t;
    }
    double exact = s + c;
    if (round_product)
        exact = bf16_bits_to_double(oracle_round_bf16(exact)) + bf16_bits_to_double(R[m * N + n]);
    if (acc_out) *acc_out = exact;
    if (y_out) {
        uint16_t y = oracle_round_bf16(exact);
        if ((flags & ORACLE_NO_NEG_ZERO) && y == 0x8000) y = 0;
        *y_out = y;
    }
}

typedef struct {
    const uint16_t *X, *W, *R;
    uint16_t *Y;
    double *ACC;
    int64_t M, N, K;
    unsigned flags;
    int64_t begin, end;           /* flat element range [begin, end) over M*N */
} job_t;

static void *run_job(void *arg) {
    job_t *j = (job_t *)arg;
    for (int64_t i = j->begin; i < j->end; ++i) {
        int64_t m = i / j->N, n = i % j->N;
        one_element(j->X, j->W, j->R, j->N, j->K, m, n, j->flags,
                    j->Y ? &j->Y[i] : NULL, j->ACC ? &j->ACC[i] : NULL);
    }
    return NULL;
}

/*
 * Full product. X [M,K], W [N,K], R [M,N] are row-major bf16 bit patterns in
 * host memory; Y (bf16 bits, [M,N]) and ACC (fp64 exact sums, [M,N]) are
 * written when non-NULL. Work is split over `threads` POSIX threads by
 * contiguous element ranges; each element's summation order is fixed, so the
 * result does not depend on the thread count. Returns 0, or -1 on bad
 * arguments / thread failure.
 */
int oracle_addmm_bf16_ex(const uint16_t *X, const uint16_t *W, const uint16_t *R,
                         uint16_t *Y, double *ACC, int64_t M, int64_t N, int64_t K,
                         unsigned flags, int threads) {
    if (M < 0 || N < 0 || K < 0) return -1;
    if (flags & ~(ORACLE_ROUND_PRODUCT | ORACLE_NO_NEG_ZERO)) return -1;
    int64_t total = M * N;
    if (total == 0) return 0;
    if (threads < 1) threads = 1;
    if (threads > 256) threads = 256;
    if ((int64_t)threads > total) threads = (int)total;
    pthread_t tid[256];
    int joined[256];
    job_t jobs[256];
    for (int t = 0; t < threads; ++t) {
        jobs[t] = (job_t){X, W, R, Y, ACC, M, N, K, flags, total * t / threads, total * (t + 1) / threads};
        joined[t] = 0;
        if (t == threads - 1 || pthread_create(&tid[t], NULL, run_job, &jobs[t]) != 0)
            run_job(&jobs[t]);    /* last range (or a failed spawn) runs here */
        else
            joined[t] = 1;
    }
    for (int t = 0; t < threads; ++t)
        if (joined[t]) pthread_join(tid[t], NULL);
    return 0;
}

/* The plain definition (one rounding, no sanitising). */
int oracle_addmm_bf16(const uint16_t *X, const uint16_t *W, const uint16_t *R,
                      uint16_t *Y, double *ACC, int64_t M, int64_t N, int64_t K,
                      int threads) {
    return oracle_addmm_bf16_ex(X, W, R, Y, ACC, M, N, K, 0u, threads);
}

/*
 * Selected elements only: for i < count, element (ms[i], ns[i]) is written to
 * Y[i] / ACC[i]. Used to check large problems at sampled positions.
 * Returns 0, or -1 if an index is out of range or a flag is unknown.
 */
int oracle_addmm_bf16_points_ex(const uint16_t *X, const uint16_t *W, const uint16_t *R,
                                int64_t M, int64_t N, int64_t K,
                                const int64_t *ms, const int64_t *ns, int64_t count,
                                unsigned flags, uint16_t *Y, double *ACC) {
    if (flags & ~(ORACLE_ROUND_PRODUCT | ORACLE_NO_NEG_ZERO)) return -1;
    for (int64_t i = 0; i < count; ++i) {
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N) return -1;
        one_element(X, W, R, N, K, ms[i], ns[i], flags, Y ? &Y[i] : NULL, ACC ? &ACC[i] : NULL);
    }
    return 0;
}

int oracle_addmm_bf16_points(const uint16_t *X, const uint16_t *W, const uint16_t *R,
                             int64_t M, int64_t N, int64_t K,
                             const int64_t *ms, const int64_t *ns, int64_t count,
                             uint16_t *Y, double *ACC) {
    return oracle_addmm_bf16_points_ex(X, W, R, M, N, K, ms, ns, count, 0u, Y, ACC);
}

/* Elementwise rounding of a double array (for tests of the rounding step). */
void oracle_round_bf16_array(const double *v, uint16_t *out, int64_t count) {
    for (int64_t i = 0; i < count; ++i) out[i] = oracle_round_bf16(v[i]);
}
