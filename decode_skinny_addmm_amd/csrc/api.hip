// api.hip -- the C ABI of libskinny.so (declared in include/skinny.h): argument checks,
// configuration lookup and dispatch to the compiled kernel instances.
#include <errno.h>
#include <stdlib.h>
#include <string.h>

#include <climits>
#include <vector>

#include "common.hpp"

namespace skinny {
namespace {

thread_local int32_t g_last_hip_error = 0;

#include "config_table.inc"

struct Registry {
    std::vector<const KernelEntry *> all;
    Registry() {
        int n = 0;
        const KernelEntry *g = gemv_entries(&n);
        for (int i = 0; i < n; ++i) all.push_back(&g[i]);
        const KernelEntry *f = mfma_entries(&n);
        for (int i = 0; i < n; ++i) all.push_back(&f[i]);
        const KernelEntry *l = mfma_lds_entries(&n);
        for (int i = 0; i < n; ++i) all.push_back(&l[i]);
        const KernelEntry *t = gemm_entries(&n);
        for (int i = 0; i < n; ++i) all.push_back(&t[i]);
        const KernelEntry *s = simt_entries(&n);
        for (int i = 0; i < n; ++i) all.push_back(&s[i]);
        const KernelEntry *d = dma_entries(&n);
        for (int i = 0; i < n; ++i) all.push_back(&d[i]);
        const KernelEntry *g2 = ring_entries(&n);
        for (int i = 0; i < n; ++i) all.push_back(&g2[i]);
    }
};

const Registry &registry() {
    static const Registry r;
    return r;
}

bool same_shape(const skinny_config &a, const skinny_config &b) {
    return a.path == b.path && a.block_size == b.block_size &&
           a.outputs_per_block == b.outputs_per_block && a.k_unroll == b.k_unroll &&
           a.vector_width == b.vector_width && a.k_split == b.k_split && a.k_stage == b.k_stage;
}

// Exact match; with m_tile == 0 the smallest built m_tile >= M (else the largest) is used.
const KernelEntry *find_entry(const skinny_config &c, int64_t M) {
    const KernelEntry *best = nullptr;
    for (const KernelEntry *e : registry().all) {
        if (!same_shape(e->cfg, c)) continue;
        if (c.m_tile != 0) {
            if (e->cfg.m_tile == c.m_tile) return e;
            continue;
        }
        if (!best) {
            best = e;
            continue;
        }
        const bool e_fits = e->cfg.m_tile >= M, b_fits = best->cfg.m_tile >= M;
        if (e_fits && (!b_fits || e->cfg.m_tile < best->cfg.m_tile)) best = e;
        else if (!e_fits && !b_fits && e->cfg.m_tile > best->cfg.m_tile) best = e;
    }
    return best;
}

skinny_config table_row(int64_t M, int64_t N) {
    const int nn = (int)(sizeof(kTableNarrow) / sizeof(kTableNarrow[0]));
    if (N <= kNarrowN && M <= kTableNarrow[nn - 1].max_m)
        for (int i = 0; i < nn; ++i)
            if (M <= kTableNarrow[i].max_m) return kTableNarrow[i].cfg;
    const int n = (int)(sizeof(kTable) / sizeof(kTable[0]));
    for (int i = 0; i < n; ++i)
        if (M <= kTable[i].max_m) return kTable[i].cfg;
    return kTable[n - 1].cfg;
}

// The table's choice for (M, N), unless that kernel cannot take this K (GEMV instances hold
// their K slice in registers; the direct-to-LDS GEMMs need whole K stages); then a second
// choice for the M range if it can (the LDS-MFMA kernel for M <= 16: any K up to its on-chip
// slice; 128-wide stages above), else the general configuration for that M range, which takes
// any K.
skinny_config select(int64_t M, int64_t N, int64_t K) {
    auto takes = [&](const skinny_config &c) {
        const KernelEntry *e = find_entry(c, M);
        return e && K <= e->max_k() && K % e->k_align == 0;
    };
    const skinny_config c = table_row(M, N);
    if (takes(c)) return c;
    if (M <= 16 && takes(kSecondSmall)) return kSecondSmall;
    if (M > 16 && takes(kSecondLarge)) return kSecondLarge;
    return M <= 16 ? kFallbackSmall : kFallbackLarge;
}

// SKINNY_CONFIG: "PATH,BLOCK,OUTPUTS,K_UNROLL,VECTOR_WIDTH[,M_TILE[,K_SPLIT[,K_STAGE]]]", decimal
// integers, the missing trailing fields 0, 1 and 0. Parsed once per process.
struct EnvConfig {
    bool set = false, valid = false;
    skinny_config cfg{};
};

EnvConfig parse_env_config() {
    EnvConfig r;
    const char *s = getenv("SKINNY_CONFIG");
    if (!s) return r;
    r.set = true;
    int64_t v[8];
    int n = 0;
    const char *p = s;
    for (;;) {
        char *end = nullptr;
        errno = 0;
        const long long x = strtoll(p, &end, 10);
        if (end == p || errno != 0 || x < INT32_MIN || x > INT32_MAX || n == 8) return r;
        v[n++] = x;
        while (*end == ' ') ++end;
        if (*end == '\0') break;
        if (*end != ',') return r;
        p = end + 1;
    }
    if (n < 5) return r;
    r.cfg = skinny_config{(int32_t)v[0], (int32_t)v[1], (int32_t)v[2], (int32_t)v[3], (int32_t)v[4],
                          n > 5 ? (int32_t)v[5] : 0, n > 6 ? (int32_t)v[6] : 1, n > 7 ? (int32_t)v[7] : 0};
    r.valid = true;
    return r;
}

const EnvConfig &env_config() {
    static const EnvConfig e = parse_env_config();
    return e;
}

// The configuration of a call that names none: SKINNY_CONFIG when set, else the table.
skinny_status default_config(int64_t M, int64_t N, int64_t K, skinny_config *out) {
    const EnvConfig &e = env_config();
    if (e.set) {
        if (!e.valid) return SKINNY_EINVAL;
        *out = e.cfg;
        return SKINNY_OK;
    }
    *out = select(M, N, K);
    return SKINNY_OK;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr uint32_t kKnownFlags = SKINNY_FLAG_ROUND_PRODUCT | SKINNY_FLAG_NO_NEG_ZERO;

skinny_status run(const void *X, const void *W, const void *R, int64_t ldr, void *out, int64_t ldo,
                  bool acc_out, int64_t M, int64_t N, int64_t K, uint32_t flags,
                  const skinny_config *cfg, void *stream) {
    if (M < 0 || N < 0 || K < 0) return SKINNY_EINVAL;
    if (flags & ~kKnownFlags) return SKINNY_EINVAL;
    if (M > 1 && (ldr < N || ldo < N)) return SKINNY_EINVAL;
    if (ldr < 0 || ldo < 0) return SKINNY_EINVAL;
    if (K % 8 != 0) return SKINNY_ENOTSUP;
    if (M == 0 || N == 0) return SKINNY_OK;
    if (!R || !out) return SKINNY_EINVAL;
    if (!acc_out && out == R && ldo != ldr) return SKINNY_EINVAL;
    if (K > 0 && (!X || !W)) return SKINNY_EINVAL;
    if ((X && !aligned(X, 16)) || (W && !aligned(W, 16)) || !aligned(R, 2) ||
        !aligned(out, acc_out ? 4 : 2))
        return SKINNY_EALIGN;
    // kernel index arithmetic is 32-bit for sizes, 64-bit for offsets
    if (M > INT_MAX || N > INT_MAX || K > INT_MAX || ldr > INT_MAX || ldo > INT_MAX) return SKINNY_ENOTSUP;
    skinny_config c;
    if (cfg) {
        c = *cfg;
    } else {
        const skinny_status st = default_config(M, N, K, &c);
        if (st != SKINNY_OK) return st;
    }
    if (c.block_size <= 0 || c.block_size % 64 != 0 || c.outputs_per_block <= 0 ||
        c.k_unroll <= 0 || c.vector_width < 4 || c.vector_width > 10 || c.m_tile < 0 ||
        c.k_split <= 0 || (c.block_size / 64) % c.k_split != 0 ||
        (c.path == SKINNY_PATH_GEMM_RING ? (c.k_stage != 64 && c.k_stage != 128)
         : c.path == SKINNY_PATH_GEMM_WS ? (c.k_stage != 64 && c.k_stage != 128 && c.k_stage != 256)
                                          : c.k_stage != 0))
        return SKINNY_EINVAL;
    const KernelEntry *e = find_entry(c, M);
    if (!e) return SKINNY_ENOTSUP;
    if (K > e->max_k() || K % e->k_align != 0) return SKINNY_ENOTSUP;
    // K == 0 (Y = R): all kernels but the direct MFMA one issue their first loads unconditionally, so the empty
    // sum goes to the general kernel, whose K loop simply does not run.
    if (K == 0 && e->cfg.path != SKINNY_PATH_MFMA)
        e = find_entry(kFallbackSmall, M);
    if (!e) return SKINNY_ENOTSUP;
    const int64_t mt = e->cfg.m_tile;
    if ((M + mt - 1) / mt > 65535) return SKINNY_ENOTSUP;
    LaunchArgs a{static_cast<const uint16_t *>(X), static_cast<const uint16_t *>(W),
                 static_cast<const uint16_t *>(R), out, M, N, K, acc_out,
                 static_cast<hipStream_t>(stream),
                 Epilogue{(int)ldr, (int)ldo, acc_out ? (flags & SKINNY_FLAG_ROUND_PRODUCT) : flags}};
    const hipError_t err = e->launch(a);
    if (err != hipSuccess) {
        g_last_hip_error = (int32_t)err;
        return SKINNY_EHIP;
    }
    return SKINNY_OK;
}

skinny_status run_kbit(const void *X, const uint32_t *planes, const uint8_t *absmax, const float *codebook,
                       int32_t kbits, const void *R, void *out, bool acc_out, int64_t M, int64_t N, int64_t K,
                       void *stream) {
    if (M < 0 || N < 0 || K < 0 || kbits < 2 || kbits > 5) return SKINNY_EINVAL;
    if (K % 32 != 0 || K > kbit_max_k()) return SKINNY_ENOTSUP;
    if (M == 0 || N == 0) return SKINNY_OK;
    if (!R || !out) return SKINNY_EINVAL;
    if (K > 0 && (!X || !planes || !absmax)) return SKINNY_EINVAL;
    if (!codebook) return SKINNY_EINVAL;
    if ((X && !aligned(X, 16)) || (planes && !aligned(planes, 4)) || !aligned(codebook, 4) ||
        !aligned(R, 2) || !aligned(out, acc_out ? 4 : 2))
        return SKINNY_EALIGN;
    if (M > INT_MAX || N > INT_MAX || (M + 3) / 4 > 65535) return SKINNY_ENOTSUP;
    // K == 0: no weights, Y = R; the dense kernels' empty-K path does exactly that
    if (K == 0) return run(X, nullptr, R, N, out, N, acc_out, M, N, 0, 0u, nullptr, stream);
    KbitArgs a{static_cast<const uint16_t *>(X), planes, absmax, codebook, kbits,
               static_cast<const uint16_t *>(R), out, M, N, K, acc_out, static_cast<hipStream_t>(stream)};
    const hipError_t err = launch_kbit_gemv(a);
    if (err != hipSuccess) {
        g_last_hip_error = (int32_t)err;
        return SKINNY_EHIP;
    }
    return SKINNY_OK;
}

skinny_status run_kda(const skinny_kda_args *a, void *stream) {
    if (!a) return SKINNY_EINVAL;
    if (a->B < 0 || a->T < 1 || a->H < 1 || a->HV < 1 || a->K < 1 || a->V < 1 || a->lines < 1 || a->slots < 1)
        return SKINNY_EINVAL;
    if (a->HV % a->H != 0) return SKINNY_EINVAL;
    const bool ring_any = a->ring_v || a->ring_k || a->ring_g || a->ring_beta;
    const bool ring_all = a->ring_v && a->ring_k && a->ring_g && a->ring_beta;
    if (ring_any && !ring_all) return SKINNY_EINVAL;
    if (ring_all && a->ring_len < a->T) return SKINNY_EINVAL;
    if (a->K != 128 || a->V % 16 != 0 || a->T > 16) return SKINNY_ENOTSUP;
    if (a->B > 65535 || a->HV > 65535 || a->V > 65535 * 16 || a->H * a->K + a->HV * a->V > INT_MAX / 2 ||
        a->lines > INT_MAX || a->slots > INT_MAX || a->ring_len > INT_MAX)
        return SKINNY_ENOTSUP;
    if (a->B == 0) return SKINNY_OK;
    if (!a->mixed || !a->conv_w || !a->conv_b || !a->conv_pool || !a->cache_idx || !a->a || !a->b || !a->A_log ||
        !a->dt_bias || !a->ssm || !a->out)
        return SKINNY_EINVAL;
    if ((a->conv_win || a->snap) && !a->inter_idx) return SKINNY_EINVAL;
    const void *two[] = {a->mixed, a->conv_w, a->conv_b, a->conv_pool, a->a, a->b, a->out, a->conv_win,
                         a->ring_v, a->ring_k};
    for (const void *p : two)
        if (p && !aligned(p, 2)) return SKINNY_EALIGN;
    const void *four[] = {a->cache_idx, a->inter_idx, a->A_log, a->dt_bias, a->ring_g, a->ring_beta};
    for (const void *p : four)
        if (p && !aligned(p, 4)) return SKINNY_EALIGN;
    if (!aligned(a->ssm, 16) || (a->snap && !aligned(a->snap, 16))) return SKINNY_EALIGN;
    const hipError_t err = launch_kda_verify(*a, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) {
        g_last_hip_error = (int32_t)err;
        return SKINNY_EHIP;
    }
    return SKINNY_OK;
}

}  // namespace
}  // namespace skinny

extern "C" {

skinny_status skinny_kda_verify_bf16(const skinny_kda_args *args, void *stream) {
    return skinny::run_kda(args, stream);
}

skinny_status skinny_kbit_gemv_bf16(const void *X, const uint32_t *planes, const uint8_t *absmax,
                                    const float *codebook, int32_t kbits, const void *R, void *Y,
                                    int64_t M, int64_t N, int64_t K, void *stream) {
    return skinny::run_kbit(X, planes, absmax, codebook, kbits, R, Y, false, M, N, K, stream);
}

skinny_status skinny_kbit_gemv_bf16_acc_f32(const void *X, const uint32_t *planes, const uint8_t *absmax,
                                            const float *codebook, int32_t kbits, const void *R, float *ACC,
                                            int64_t M, int64_t N, int64_t K, void *stream) {
    return skinny::run_kbit(X, planes, absmax, codebook, kbits, R, ACC, true, M, N, K, stream);
}

skinny_status skinny_addmm_bf16(const void *X, const void *W, const void *R, void *Y, int64_t M,
                                int64_t N, int64_t K, void *stream) {
    return skinny::run(X, W, R, N, Y, N, false, M, N, K, 0, nullptr, stream);
}

skinny_status skinny_addmm_bf16_with_config(const void *X, const void *W, const void *R, void *Y,
                                            int64_t M, int64_t N, int64_t K,
                                            const skinny_config *cfg, void *stream) {
    return skinny::run(X, W, R, N, Y, N, false, M, N, K, 0, cfg, stream);
}

skinny_status skinny_addmm_bf16_acc_f32(const void *X, const void *W, const void *R, float *ACC,
                                        int64_t M, int64_t N, int64_t K,
                                        const skinny_config *cfg, void *stream) {
    return skinny::run(X, W, R, N, ACC, N, true, M, N, K, 0, cfg, stream);
}

skinny_status skinny_addmm_bf16_shard(const void *X, const void *W, const void *R, int64_t ldr,
                                      void *Y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                                      uint32_t flags, const skinny_config *cfg, void *stream) {
    return skinny::run(X, W, R, ldr, Y, ldy, false, M, N, K, flags, cfg, stream);
}

skinny_status skinny_addmm_bf16_shard_acc_f32(const void *X, const void *W, const void *R,
                                              int64_t ldr, float *ACC, int64_t ldacc,
                                              int64_t M, int64_t N, int64_t K, uint32_t flags,
                                              const skinny_config *cfg, void *stream) {
    return skinny::run(X, W, R, ldr, ACC, ldacc, true, M, N, K, flags, cfg, stream);
}

skinny_status skinny_select_config(int64_t M, int64_t N, int64_t K, skinny_config *out) {
    if (!out || M < 0 || N < 0 || K < 0) return SKINNY_EINVAL;
    return skinny::default_config(M, N, K, out);
}

int32_t skinny_num_configs(void) { return (int32_t)skinny::registry().all.size(); }

skinny_status skinny_get_config(int32_t index, skinny_config *out) {
    if (!out || index < 0 || index >= skinny_num_configs()) return SKINNY_EINVAL;
    *out = skinny::registry().all[(size_t)index]->cfg;
    return SKINNY_OK;
}

skinny_status skinny_config_resources(const skinny_config *cfg, skinny_resources *out) {
    if (!cfg || !out) return SKINNY_EINVAL;
    const skinny::KernelEntry *e = skinny::find_entry(*cfg, cfg->m_tile > 0 ? cfg->m_tile : 1);
    if (!e) return SKINNY_ENOTSUP;
    hipFuncAttributes attr;
    const hipError_t err = hipFuncGetAttributes(&attr, e->fn_bf16);
    if (err != hipSuccess) {
        skinny::g_last_hip_error = (int32_t)err;
        return SKINNY_EHIP;
    }
    out->num_vgprs = attr.numRegs;
    out->spill_bytes = (int32_t)attr.localSizeBytes;
    out->lds_bytes_static = (int32_t)attr.sharedSizeBytes;
    out->max_threads = attr.maxThreadsPerBlock;
    return SKINNY_OK;
}

skinny_status skinny_config_kernel_name(const skinny_config *cfg, char *buf, int32_t len) {
    if (!cfg || !buf || len <= 0) return SKINNY_EINVAL;
    const skinny::KernelEntry *e = skinny::find_entry(*cfg, cfg->m_tile > 0 ? cfg->m_tile : 1);
    if (!e) return SKINNY_ENOTSUP;
    const char *name = hipKernelNameRefByPtr(e->fn_bf16, nullptr);
    if (!name) {
        skinny::g_last_hip_error = (int32_t)hipErrorInvalidDeviceFunction;
        return SKINNY_EHIP;
    }
    if ((int64_t)strlen(name) >= len) return SKINNY_EINVAL;
    memcpy(buf, name, strlen(name) + 1);
    return SKINNY_OK;
}

const char *skinny_status_string(skinny_status s) {
    switch (s) {
        case SKINNY_OK: return "ok";
        case SKINNY_EINVAL: return "invalid argument (NULL pointer for a non-empty buffer, negative size or bad config field)";
        case SKINNY_EALIGN: return "misaligned pointer (X and W need 16 bytes, R and Y 2, ACC 4)";
        case SKINNY_ENOTSUP: return "not supported (K % 8 != 0, size limit, or configuration not built into the library)";
        case SKINNY_EHIP: return "HIP runtime error at launch";
    }
    return "unknown status";
}

int32_t skinny_last_hip_error(void) { return skinny::g_last_hip_error; }

const char *skinny_version(void) { return "0.1.0"; }

}  // extern "C"
