/*
 * kbit.c -- TEST INFRASTRUCTURE ONLY (built into the same liboracle.so as oracle.c).
 *
 * Plain CPU definition of the k-bit quantized decode GEMV described on the bitsandbytes
 * page "compare/main...QLORA-2.diff" (agents/kbit_gemm_context.md: section 1.2 codebook,
 * 1.3 quantize, 1.4 dequantize, 1.5 E4M4 absmax, 1.6 bit-plane packing, 12 error budget;
 * the QLoRA guide's section 7, "Kernel 1: Scalar GEMV"):
 *
 *   - weights W[N, K] are quantized in blocks of 32 consecutive elements of a row;
 *   - a block keeps its absolute maximum as one E4M4 byte (4-bit exponent, bias 11, 4-bit
 *     mantissa) and, per element, a k-bit index (k = 2..5) into a 2^k-entry codebook;
 *   - the indices are stored as k bit-plane words per block: bit j of word b is bit b of
 *     element j's index; blocks follow each other in row-major element order;
 *   - dequantized weight = codebook[index] * decode(absmax byte);
 *   - the GEMV: Y[m, n] = bf16( sum_k X[m, k] * What[n, k] + R[m, n] ), one rounding,
 *     as the skinny residual GEMM of oracle.c with W replaced by its dequantized values.
 *
 * Everything is computed in fp64. A codebook entry (fp32) times a decoded E4M4 scale
 * (5 significant bits) is exact in fp64, and so is each product with a bf16 x; the sum is
 * compensated (Neumaier) and rounded straight to bf16 by oracle_round_bf16 (oracle.c).
 *
 * Readings taken where the page leaves a step open:
 *  - E4M4 encoding (the page gives only the decoder): the nearest representable value, a
 *    tie going to the even code; values above 31 saturate to 31 (0xFF);
 *  - the index of an element is the nearest codebook entry to w / max(absmax, 1e-8), with
 *    the unencoded absmax as on the page (computed here in fp64, the page's kernel uses
 *    fp32); a tie goes to the lower index (the page's search keeps the first best);
 *  - the GEMV keeps this library's operation: bf16 X, R and Y, fp32-or-better accumulation,
 *    residual added before the one rounding (the page benchmarks fp16 without a residual).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

uint16_t oracle_round_bf16(double v);      /* oracle.c */
double oracle_bf16_to_double(uint16_t b);  /* oracle.c */

/* E4M4 decode, from the page's definition: e = byte >> 4, m = byte & 15;
 * e > 0: 2^(e - 11) * (1 + m/16); e == 0: 2^(1 - 11) * (m/16) (zero for m == 0). */
double oracle_e4m4_decode(uint8_t byte) {
    const int e = byte >> 4, m = byte & 15;
    if (e == 0) return ldexp((double)m / 16.0, 1 - 11);
    return ldexp(1.0 + (double)m / 16.0, e - 11);
}

/* Nearest E4M4 code to v >= 0 (ties to the even code; above the largest value saturates;
 * NaN or negative gives 0). The codes are searched exhaustively. */
uint8_t oracle_e4m4_encode(double v) {
    if (!(v > 0.0)) return 0;
    int best = 0;
    double bestd = fabs(oracle_e4m4_decode(0) - v);
    for (int c = 1; c < 256; ++c) {
        const double d = fabs(oracle_e4m4_decode((uint8_t)c) - v);
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            bestd = d;
        }
    }
    return (uint8_t)best;
}

/* Standard normal CDF and density. */
static double phi_cdf(double z) { return 0.5 * erfc(-z / sqrt(2.0)); }
static double phi_pdf(double z) { return isinf(z) ? 0.0 : exp(-0.5 * z * z) / 2.5066282746310002; }  /* sqrt(2 pi) */

/* Inverse CDF by bisection (p in (0, 1)); plenty for the codebook edges. */
static double phi_inv(double p) {
    double lo = -40.0, hi = 40.0;
    for (int i = 0; i < 200; ++i) {
        const double mid = 0.5 * (lo + hi);
        if (phi_cdf(mid) < p) lo = mid; else hi = mid;
    }
    return 0.5 * (lo + hi);
}

/*
 * Normal-float codebook with 2^k levels: the expected value of N(0,1) inside each of 2^k
 * equiprobable bins, E[Z | a < Z < b] = (pdf(a) - pdf(b)) / (1 / 2^k), sorted ascending and
 * divided by the largest magnitude so that the outer levels are -1 and +1.
 * Returns 0, or -1 for k outside 1..8.
 */
int oracle_nf_codebook(int k, double *cb) {
    if (k < 1 || k > 8) return -1;
    const int L = 1 << k;
    double maxabs = 0.0;
    for (int i = 0; i < L; ++i) {
        const double a = (i == 0) ? -INFINITY : phi_inv((double)i / L);
        const double b = (i == L - 1) ? INFINITY : phi_inv((double)(i + 1) / L);
        cb[i] = (phi_pdf(a) - phi_pdf(b)) * L;
        if (fabs(cb[i]) > maxabs) maxabs = fabs(cb[i]);
    }
    for (int i = 0; i < L; ++i) cb[i] /= maxabs;
    return 0;
}

/*
 * Blockwise quantization of W (n values, n % 32 == 0, read as consecutive blocks of 32):
 * planes[blk*k + b] and absmax_e4m4[blk] as described above; absmax_raw[blk] (optional)
 * receives the unencoded block maximum. cb holds the 2^k codebook values (fp32, sorted).
 * Returns 0, or -1 on bad arguments.
 */
int oracle_kbit_quantize(const double *w, int64_t n, int k, const float *cb, uint32_t *planes,
                         uint8_t *absmax_e4m4, double *absmax_raw) {
    if (k < 2 || k > 5 || n < 0 || n % 32 != 0) return -1;
    const int L = 1 << k;
    for (int64_t blk = 0; blk < n / 32; ++blk) {
        const double *x = w + blk * 32;
        double amax = 0.0;
        for (int j = 0; j < 32; ++j)
            if (fabs(x[j]) > amax) amax = fabs(x[j]);
        const double s = amax > 1e-8 ? amax : 1e-8;
        uint32_t words[5] = {0, 0, 0, 0, 0};
        for (int j = 0; j < 32; ++j) {
            const double v = x[j] / s;
            int best = 0;
            double bestd = fabs(v - (double)cb[0]);
            for (int i = 1; i < L; ++i) {
                const double d = fabs(v - (double)cb[i]);
                if (d < bestd) { best = i; bestd = d; }
            }
            for (int b = 0; b < k; ++b)
                words[b] |= (uint32_t)((best >> b) & 1) << j;
        }
        for (int b = 0; b < k; ++b) planes[blk * k + b] = words[b];
        absmax_e4m4[blk] = oracle_e4m4_encode(amax);
        if (absmax_raw) absmax_raw[blk] = amax;
    }
    return 0;
}

/* Index of element j of block blk, read back from its k bit-plane words. */
static int kbit_index(const uint32_t *planes, int k, int64_t blk, int j) {
    int idx = 0;
    for (int b = 0; b < k; ++b) idx |= (int)((planes[blk * k + b] >> j) & 1u) << b;
    return idx;
}

/* Dequantized values of n elements (n % 32 == 0): out[i] = cb[index] * decode(absmax). */
int oracle_kbit_dequant(const uint32_t *planes, const uint8_t *absmax_e4m4, const float *cb, int k,
                        int64_t n, double *out) {
    if (k < 2 || k > 5 || n < 0 || n % 32 != 0) return -1;
    for (int64_t i = 0; i < n; ++i) {
        const int64_t blk = i / 32;
        out[i] = (double)cb[kbit_index(planes, k, blk, (int)(i % 32))] * oracle_e4m4_decode(absmax_e4m4[blk]);
    }
    return 0;
}

/*
 * The GEMV: X bf16 [M, K], R bf16 [M, N] (bit patterns), W as planes/absmax of N rows of K
 * (K % 32 == 0; row n is blocks n*K/32 .. (n+1)*K/32 - 1), codebook cb[2^k] (fp32).
 * Y (bf16 bits [M, N]) and ACC (the exact sum before rounding, [M, N]) written when non-NULL.
 */
int oracle_kbit_gemv_bf16(const uint16_t *X, const uint32_t *planes, const uint8_t *absmax_e4m4,
                          const float *cb, int k, const uint16_t *R, uint16_t *Y, double *ACC,
                          int64_t M, int64_t N, int64_t K) {
    if (k < 2 || k > 5 || M < 0 || N < 0 || K < 0 || K % 32 != 0) return -1;
    const int64_t bpr = K / 32;   /* blocks per row of W */
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            double s = 0.0, c = 0.0;
            for (int64_t kk = 0; kk <= K; ++kk) {
                double p;
                if (kk < K) {
                    const int64_t blk = n * bpr + kk / 32;
                    const double w = (double)cb[kbit_index(planes, k, blk, (int)(kk % 32))] *
                                     oracle_e4m4_decode(absmax_e4m4[blk]);
                    p = oracle_bf16_to_double(X[m * K + kk]) * w;
                } else {
                    p = oracle_bf16_to_double(R[m * N + n]);
                }
                const double t = s + p;
                if (fabs(s) >= fabs(p)) c += (s - t) + p;
                else c += (p - t) + s;
                s = t;
            }
            const double exact = s + c;
            if (ACC) ACC[m * N + n] = exact;
            if (Y) Y[m * N + n] = oracle_round_bf16(exact);
        }
    }
    return 0;
}
