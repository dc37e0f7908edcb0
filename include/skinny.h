/*
 * skinny.h -- C ABI of libskinny.so: the skinny residual GEMM on MI355X (gfx950).
 *
 * Operation (the vLLM benchmark page "benchmarks/kernels/benchmark_k3_cutedsl_residual.py",
 * module docstring and its torch.addmm leg; the vLLM API page
 * "fused_add_multicast_skinny_gemm", class FusedAddMulticastSkinnyGemm, for the kernel
 * family it comes from):
 *
 *     Y[m, n] = bf16( sum_{k<K} X[m, k] * W[n, k]  +  R[m, n] )
 *
 *   X  bf16 [M, K]  row-major, K contiguous (the activations)
 *   W  bf16 [N, K]  row-major, K contiguous (nn.Linear weight layout; the op uses W^T)
 *   R  bf16 [M, N]  row-major (the residual)
 *   Y  bf16 [M, N]  row-major (the output)
 * The products are summed in fp32, R is added in fp32, and the fp32 total is rounded once
 * to bf16, round-to-nearest-even (alpha = beta = 1). The order of the fp32 additions is
 * fixed per configuration, so a call is deterministic for a given configuration.
 *
 * Conventions shared by every entry point:
 *  - All array pointers are DEVICE pointers on the current HIP device. The caller owns every
 *    buffer; the library allocates no device memory and never synchronises.
 *  - `stream` is a hipStream_t (NULL = the null stream). Calls are asynchronous on it and
 *    may be captured into a HIP graph.
 *  - Sizes: M, N, K >= 0. M == 0 or N == 0 is a no-op returning SKINNY_OK. K == 0 gives
 *    Y = R. K must be a multiple of 8 (rows of X and W are read in 16-byte vectors).
 *  - Alignment: X and W must be 16-byte aligned; R and Y 2-byte aligned (ACC 4-byte).
 *    A pointer may be NULL only when its buffer is empty.
 *  - Aliasing: Y may be exactly R (in-place residual update). Any other overlap between
 *    an output and an input is undefined.
 *  - Errors: argument errors are reported before anything is launched; a HIP launch error
 *    is reported as SKINNY_EHIP (skinny_last_hip_error() gives the hipError_t value).
 *    No C++ exception crosses this interface.
 */
#ifndef SKINNY_H
#define SKINNY_H

#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define SKINNY_API __attribute__((visibility("default")))
#else
#define SKINNY_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum skinny_status {
    SKINNY_OK = 0,
    SKINNY_EINVAL = 1,  /* NULL pointer for a non-empty buffer, negative size, bad config field */
    SKINNY_EALIGN = 2,  /* X or W not 16-byte aligned, R/Y not 2-byte aligned, ACC not 4-byte */
    SKINNY_ENOTSUP = 3, /* K % 8 != 0, or configuration not built into this library / too large */
    SKINNY_EHIP = 4     /* the HIP runtime reported an error when launching */
} skinny_status;

/* Kernel families. */
enum {
    SKINNY_PATH_GEMV = 0, /* VALU path: bf16 dot products into fp32, cross-lane reduction */
    SKINNY_PATH_MFMA = 1, /* matrix-core path, fragments loaded straight from memory; any K */
    SKINNY_PATH_MFMA_LDS = 2, /* matrix-core path, W streamed in 1 KB row pieces and turned
                                 into fragments through LDS; K <= 512 * k_split */
    SKINNY_PATH_GEMM = 3,     /* matrix-core K-loop GEMM with LDS-staged operand tiles, for
                                 larger M; any K */
    SKINNY_PATH_SIMT = 4,     /* the vLLM API page's SIMT decomposition, knobs taken as named:
                                 thread t of a block_size workgroup takes vector t of every
                                 block_size * vector_width K-tile of outputs_per_block W rows,
                                 k_unroll tiles per step, X loaded through the cache; any K.
                                 Built for the page-1 sweep grid at m_tile 16 */
    SKINNY_PATH_GEMM_DMA = 5, /* matrix-core K-loop GEMM whose operand tiles are loaded from
                                 memory straight into a ring of LDS stages (k_unroll = stages;
                                 k_split 4: the 4 waves split each stage's K steps, 1: they
                                 split the output block); K must be a multiple of 128 (else
                                 SKINNY_ENOTSUP) */
    SKINNY_PATH_GEMM_RING = 6, /* the same operand pipeline with k_stage-wide stages (64 or 128)
                                 and 4 or 8 waves (block_size 256 or 512); k_split = waves
                                 taking alternate K steps of a stage, the others split the
                                 block; K must be a multiple of k_stage (else SKINNY_ENOTSUP) */
    SKINNY_PATH_GEMM_WS = 7   /* the ring of SKINNY_PATH_GEMM_RING with wave-specialised roles:
                                 4 waves only load the stages, 4 only run the matrix
                                 instructions (block_size 512); k_split = compute waves taking
                                 alternate K steps; vector_width 8 = each loading wave takes W
                                 and X rows, 9 = W rows and X rows on different waves;
                                 outputs_per_block 28 or 56 = blocks owning 7/8 of a 32- or
                                 64-row matrix tile (256 or 128 blocks at N = 7168); K must be
                                 a multiple of k_stage (else SKINNY_ENOTSUP) */
};

/*
 * One launch configuration (the knobs of the page-1 benchmark's Config record, re-read for
 * 64-wide wavefronts; see each field). A configuration is usable only if the library was
 * built with it: skinny_num_configs()/skinny_get_config() list them.
 */
typedef struct skinny_config {
    int32_t path;              /* one of the SKINNY_PATH_* values */
    int32_t block_size;        /* threads per workgroup, a multiple of 64 */
    int32_t outputs_per_block; /* output columns (rows of W) per workgroup */
    int32_t k_unroll;          /* GEMV: vectors of one W row in flight per lane per step;
                                  MFMA: 32-wide K steps in flight per wave */
    int32_t vector_width;      /* bf16 elements per W load per lane: 8 (16 B) or, SIMT only,
                                  4 (8 B). GEMV and MFMA_LDS encode their row order here:
                                  8 = rows strided over the grid, 9 = contiguous rows per
                                  workgroup, 10 (MFMA_LDS) = contiguous with X loaded first;
                                  all three load 16 B. GEMM_WS encodes its loader roles here
                                  (8 or 9, see SKINNY_PATH_GEMM_WS) */
    int32_t m_tile;            /* rows of X handled per pass (compile-time tile); M larger
                                  than m_tile runs ceil(M / m_tile) passes; 0 = let the
                                  library pick the smallest built tile >= M */
    int32_t k_split;           /* waves of a workgroup that share the same output columns
                                  and split K between them (their partial sums meet in LDS) */
    int32_t k_stage;           /* K per LDS stage of SKINNY_PATH_GEMM_RING (64 or 128) and
                                  SKINNY_PATH_GEMM_WS (64, 128 or 256); 0 for every other path */
} skinny_config;

/*
 * The name of the kernel (the instance whose epilogue writes a plain bf16 [M, N] output, for a
 * K that needs no ragged-tail handling: what skinny_addmm_bf16 launches with this
 * configuration at the tuned shape) as the HIP runtime reports it, copied with its
 * terminating NUL into buf (len bytes). Lets measurements made under a profiler be matched to
 * a configuration. SKINNY_ENOTSUP if the configuration is not built, SKINNY_EINVAL if buf is
 * too short, SKINNY_EHIP if the runtime has no name for it.
 */
SKINNY_API skinny_status skinny_config_kernel_name(const skinny_config *cfg, char *buf, int32_t len);

/* Register and scratch use of one built configuration (hipFuncGetAttributes). */
typedef struct skinny_resources {
    int32_t num_vgprs;         /* registers per lane reported by the runtime */
    int32_t spill_bytes;       /* private (scratch) bytes per lane; > 0 means spills */
    int32_t lds_bytes_static;  /* static LDS per workgroup */
    int32_t max_threads;       /* maximum threads per block for the kernel */
} skinny_resources;

/*
 * Y = bf16(X W^T + R) with the configuration skinny_select_config() picks for (M, N, K).
 */
SKINNY_API skinny_status skinny_addmm_bf16(const void *X, const void *W, const void *R, void *Y,
                                int64_t M, int64_t N, int64_t K, void *stream);

/*
 * The tuned configuration for a problem size (an M-indexed table measured on MI355X; the
 * page-1 benchmark's per-M "residual_config" lookup plays the same role). Host-only, no
 * HIP call. Returns SKINNY_EINVAL for a NULL `out` or negative sizes.
 *
 * Override for sweeps and experiments: if the environment variable SKINNY_CONFIG is set when
 * the library first needs a configuration, its value replaces the table for the whole process,
 * here and in every call that passes no configuration (skinny_addmm_bf16, and the calls below
 * with cfg == NULL). The value is 5 to 8 comma-separated decimal integers,
 * PATH,BLOCK,OUTPUTS,K_UNROLL,VECTOR_WIDTH[,M_TILE[,K_SPLIT[,K_STAGE]]] (the skinny_config
 * fields in order; missing trailing fields are 0, 1 and 0). A malformed value makes those calls
 * return SKINNY_EINVAL; a configuration that is not built, or does not take the shape, makes
 * the compute calls return SKINNY_ENOTSUP, as an explicit one would. It is read once.
 */
SKINNY_API skinny_status skinny_select_config(int64_t M, int64_t N, int64_t K, skinny_config *out);

/*
 * As skinny_addmm_bf16, with an explicit configuration (NULL = the selected one).
 * SKINNY_ENOTSUP if that configuration is not built into the library.
 */
SKINNY_API skinny_status skinny_addmm_bf16_with_config(const void *X, const void *W, const void *R, void *Y,
                                            int64_t M, int64_t N, int64_t K,
                                            const skinny_config *cfg, void *stream);

/*
 * Test entry: the same kernel and summation order as the bf16 call, but the epilogue
 * writes the fp32 value that would be rounded, ACC[m, n] = fp32(sum) + fp32(R[m, n]),
 * to ACC (float [M, N], row-major). cfg NULL = the selected configuration.
 */
SKINNY_API skinny_status skinny_addmm_bf16_acc_f32(const void *X, const void *W, const void *R, float *ACC,
                                        int64_t M, int64_t N, int64_t K,
                                        const skinny_config *cfg, void *stream);

/*
 * Tensor-parallel shard form (the vLLM API page "fused_add_multicast_skinny_gemm": each rank
 * multiplies its N/g rows of W and writes its columns of a wider output, with R taken from the
 * same wide layout):
 *
 *     Y[m*ldy + n] = bf16( sum_k X[m, k] * W[n, k]  +  R[m*ldr + n] ),  0 <= n < N
 *
 * R and Y are row-major with row pitches ldr and ldy (elements, each >= N when M > 1); Y and
 * R may point at a column offset inside a wider matrix, and elements outside the M x N block
 * are neither read nor written. `flags` is a bit set of SKINNY_FLAG_*:
 *   SKINNY_FLAG_ROUND_PRODUCT  round the fp32 sum of products to bf16 first, then add R in
 *                              fp32 and round again (that page's epilogue; two roundings);
 *   SKINNY_FLAG_NO_NEG_ZERO    write +0 wherever the bf16 result is -0 (that page reserves -0
 *                              as its not-yet-written marker).
 * Unknown flag bits give SKINNY_EINVAL. Y may be exactly R only with ldy == ldr (else
 * SKINNY_EINVAL). cfg NULL = the selected configuration. Everything else as
 * skinny_addmm_bf16_with_config.
 */
enum {
    SKINNY_FLAG_ROUND_PRODUCT = 1u,
    SKINNY_FLAG_NO_NEG_ZERO = 2u
};
SKINNY_API skinny_status skinny_addmm_bf16_shard(const void *X, const void *W, const void *R, int64_t ldr,
                                                 void *Y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                                                 uint32_t flags, const skinny_config *cfg, void *stream);

/*
 * Test entry of the shard form: the fp32 value each output would be rounded from (with
 * SKINNY_FLAG_ROUND_PRODUCT: bf16(sum) + R), written to ACC (float, row pitch ldacc).
 * SKINNY_FLAG_NO_NEG_ZERO acts on bf16 results only and is accepted and ignored here.
 */
SKINNY_API skinny_status skinny_addmm_bf16_shard_acc_f32(const void *X, const void *W, const void *R,
                                                         int64_t ldr, float *ACC, int64_t ldacc,
                                                         int64_t M, int64_t N, int64_t K, uint32_t flags,
                                                         const skinny_config *cfg, void *stream);

/*
 * Decode GEMV with k-bit quantized weights (the bitsandbytes page "compare/main...QLORA-2.diff":
 * agents/kbit_gemm_context.md sections 1.2-1.6 for the format, its QLoRA guide's section 7 for
 * the scalar decode GEMV):
 *
 *     Y[m, n] = bf16( sum_k X[m, k] * What[n, k]  +  R[m, n] ),
 *     What[n, k] = codebook[idx(n, k)] * e4m4(absmax[n, k / 32])
 *
 *   X        bf16 [M, K] row-major, 16-byte aligned
 *   planes   uint32 [N, K/32, kbits]: for the 32-element block (n, b), word i holds bit i of the
 *            indices of its elements (bit j of the word = element j); 4-byte aligned
 *   absmax   uint8 [N, K/32]: the block scale in E4M4 (4-bit exponent, bias 11, 4-bit
 *            mantissa: e > 0 gives 2^(e-11) * (1 + m/16), e == 0 gives m * 2^-14)
 *   codebook float [2^kbits] (e.g. the normal-float levels); 4-byte aligned
 *   R, Y     bf16 [M, N] row-major (Y may be exactly R)
 * kbits is 2..5 (else SKINNY_EINVAL); K must be a multiple of 32 and at most 16384 (one lane
 * per 32-element block of a row, 512 lanes per workgroup), else SKINNY_ENOTSUP. Sums are fp32,
 * one RNE rounding. M of any size runs in passes: of up to 4 rows on the VALU (the decode
 * form), or, for M >= 5 with kbits 2..4, K a multiple of 128 up to 3584, planes aligned to
 * 4 * kbits bytes (4 at kbits 3) and absmax to 4, of up to 16 rows on the matrix cores, with
 * each codebook value split into three bf16 parts whose sum is that fp32 value exactly. Same
 * conventions as above otherwise (device pointers, asynchronous, no allocation).
 */
SKINNY_API skinny_status skinny_kbit_gemv_bf16(const void *X, const uint32_t *planes, const uint8_t *absmax,
                                               const float *codebook, int32_t kbits, const void *R, void *Y,
                                               int64_t M, int64_t N, int64_t K, void *stream);

/* Test entry: the fp32 value each output is rounded from, fp32(sum) + fp32(R), to ACC [M, N]. */
SKINNY_API skinny_status skinny_kbit_gemv_bf16_acc_f32(const void *X, const uint32_t *planes,
                                                       const uint8_t *absmax, const float *codebook,
                                                       int32_t kbits, const void *R, float *ACC,
                                                       int64_t M, int64_t N, int64_t K, void *stream);

/*
 * One layer of the KDA chain-verify step of speculative decoding (the sglang page
 * "benchmark/kernels/bench_kda_verify_sweep.py": its make_inputs gives the tensors below, its
 * make_runner the calls; the unfused leg is causal_conv1d_update followed by
 * fused_sigmoid_gating_delta_rule_update with is_kda, the fused legs are
 * fused_kda_conv_gating_verify). For batch row b (T draft tokens), per channel d of the
 * mixed q|k|v projection and per value head hv:
 *
 *   conv:  c[t, d] = bf16( silu( bias[d] + sum_w conv_w[d, w] * seq_d[t + w] ) ),
 *          seq_d = conv_pool[cache_idx[b], 0..2, d] then mixed[b*T + 0..T-1, d];
 *          q = c[:, h*K ..], k = c[:, H*K + h*K ..], v = c[:, 2*H*K + hv*V ..], h = hv / (HV/H)
 *   gate:  g[t, c] = -exp(A_log[hv]) * softplus(a[b*T+t, hv*K + c] + dt_bias[hv*K + c])
 *          (softplus with beta 1, threshold 20); beta_t = sigmoid(b[b*T+t, hv])
 *   norm:  q^ = scale * q / sqrt(|q|^2 + 1e-6),  k^ = k / sqrt(|k|^2 + 1e-6)
 *   state: S = ssm[cache_idx[b], hv] ([V, K] fp32); per token t:
 *          S *= exp(g[t]) per K channel; u = beta_t (v_t - S k^); S += u k^T; o_t = S q^
 *   outputs: out[b*T + t, hv, :] = bf16(o_t);
 *          conv_win[inter_idx[b], t, w, d] = seq_d[t + 1 + w] (w = 0..2), when non-NULL;
 *          snapshot mode (snap non-NULL): snap[inter_idx[b], t, hv] = S after token t;
 *          ring mode (ring pointers non-NULL), position t of slot cache_idx[b]:
 *          ring_v[., hv, t, :] = v_t, ring_k[., h, t, :] = k_t (bf16 conv outputs, before the
 *          norm), ring_g[., hv, t, :] = g[t], ring_beta[., hv, t] = beta_t.
 *   ssm and conv_pool are read only (the verify step commits no state).
 * What comes from that page and what is a reading where it is silent: the page gives the
 * calls, argument names, tensor shapes and dtypes (and sizes the ring at 2T positions); it
 * does not print the kernels' arithmetic. Taken as the plain meaning of an argument name or
 * the standard definition of the named operation:
 *   - the conv window is the 3 cached inputs, oldest first, then the T tokens; its output is
 *     materialised in bf16 (the page's tensors are bf16) before the q | k | v split;
 *   - the gate is the standard KDA gate (is_kda, no lower bound): softplus with beta 1 and
 *     threshold 20, scaled by -exp(A_log); beta is the sigmoid of b;
 *   - the L2 norm adds its 1e-6 inside the square root; q is then multiplied by scale (the
 *     page passes K^-0.5); value head hv reads q/k head hv / (HV / H);
 *   - the delta rule decays S per K channel, then u = beta (v - S k^), S += u k^T, o = S q^
 *     (the output is read after the update);
 *   - a verify step writes no state: ssm and conv_pool are read only;
 *   - where in the ring a verify starts is not on the page; token t goes to position t;
 *   - not built: the page's lower-bound ("safe") gate and parent-token retrieval, whose
 *     arithmetic the page does not give.
 *
 * Layouts (row-major, device pointers, all bf16 unless noted):
 *   mixed [B*T, dim], dim = 2*H*K + HV*V;  conv_w [dim, 4];  conv_b [dim];
 *   conv_pool [lines, 3, dim];  conv_win [lines, T, 3, dim];
 *   a [B*T, HV*K];  b [B*T, HV];  A_log float [HV];  dt_bias float [HV*K];
 *   ssm float [slots, HV, V, K];  snap float [lines, T, HV, V, K];
 *   ring_v [slots, HV, ring_len, V];  ring_k [slots, H, ring_len, K];
 *   ring_g float [slots, HV, ring_len, K];  ring_beta float [slots, HV, ring_len];
 *   cache_idx, inter_idx int32 [B] (values outside 0..slots-1 / 0..lines-1 are clamped);
 *   out [B*T, HV, V].
 * Supported: K == 128, V a multiple of 16, 1 <= T <= 16, HV a multiple of H, ring_len >= T
 * when the ring is used (else SKINNY_ENOTSUP / SKINNY_EINVAL). ssm and snap must be 16-byte
 * aligned. B == 0 is a no-op. Asynchronous on `stream`, no allocation, capturable.
 */
typedef struct skinny_kda_args {
    const void *mixed, *conv_w, *conv_b, *conv_pool;
    const int32_t *cache_idx, *inter_idx;
    const void *a, *b;
    const float *A_log, *dt_bias, *ssm;
    void *conv_win;                 /* may be NULL */
    float *snap;                    /* may be NULL */
    void *ring_v, *ring_k;          /* ring mode: all four non-NULL, or all four NULL */
    float *ring_g, *ring_beta;
    void *out;
    int64_t B, T, H, HV, K, V, lines, slots, ring_len;
    float scale;
} skinny_kda_args;

SKINNY_API skinny_status skinny_kda_verify_bf16(const skinny_kda_args *args, void *stream);

/* Number of configurations built into the library, and the i-th of them (0-based). */
SKINNY_API int32_t skinny_num_configs(void);
SKINNY_API skinny_status skinny_get_config(int32_t index, skinny_config *out);

/* Register/LDS/spill figures of a built configuration (calls hipFuncGetAttributes). */
SKINNY_API skinny_status skinny_config_resources(const skinny_config *cfg, skinny_resources *out);

/* Static text for a status code; never NULL. */
SKINNY_API const char *skinny_status_string(skinny_status s);

/* The hipError_t of the most recent SKINNY_EHIP on the calling thread (0 if none). */
SKINNY_API int32_t skinny_last_hip_error(void);

/* Library version string, e.g. "0.1.0". */
SKINNY_API const char *skinny_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SKINNY_H */
