// mfma_gemm.hip -- LDS-tiled matrix-core path for larger M (tens to hundreds of rows of X).
//
// Operation: vLLM benchmark page "benchmarks/kernels/benchmark_k3_cutedsl_residual.py"
// (module docstring; torch.addmm leg): Y = bf16(X W^T + R), fp32 accumulation. When M is in
// the tens or hundreds, every workgroup can no longer hold all of X on chip, so this kernel
// is a classic K-loop GEMM shaped for gfx950:
//   * a workgroup computes a BN x BM block of Y^T (BN rows of W = output columns n, BM rows
//     of X) with KG groups of 4 waves; the waves of a group are in a 2 x 2 layout, each a
//     (BN/2) x (BM/2) block of v_mfma_f32_16x16x32_bf16 tiles, and the KG groups take
//     alternate K stages (more waves per CU when the grid is small), adding their partial
//     blocks at the end;
//   * K advances in stages of 128: both operand tiles are fetched with 16-byte loads, D
//     stages ahead into registers so HBM latency is covered, then written to one of two LDS
//     buffers (rows padded to 272 bytes: fragment reads hit distinct banks) while the matrix
//     cores work on the other, one barrier per stage, and read back as A (W) and B (X^T)
//     fragments; larger wave blocks read less LDS per MFMA;
//   * block ids are laid out so that the M-tiles of one W row tile are consecutive on the
//     same XCD (blocks are dealt to the 8 XCDs round-robin): they run together and share
//     the W tile through that XCD's L2, so W leaves HBM once;
//   * R is fetched into registers at the start (its latency hides behind the K loop); the
//     epilogue stages the fp32 block in LDS and walks it row by row of Y, so residual loads
//     and output stores are contiguous; R is added in fp32, one RNE rounding to bf16.
#include "common.hpp"

namespace skinny {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kKC = 128;                 // K per stage (bf16 elements)
constexpr int kPitch = kKC * 2 + 16;     // bytes per staged row (256 + 16 padding)

__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// BN: rows of W per workgroup; BM: rows of X per workgroup; D: stages in flight per group;
// KG: groups of 4 waves splitting the K stages.
template <int BN, int BM, int D, int KG, bool ACC>
__global__ __launch_bounds__(256 * KG) void mfma_gemm_kernel(const uint16_t *__restrict__ X,
                                                        const uint16_t *__restrict__ W,
                                                        const uint16_t *R, void *out,
                                                        int M, int N, int K, int n_tiles, int m_tiles, Epilogue ep) {
    constexpr int WN = BN / 2, WM = BM / 2;          // wave block
    constexpr int TN = WN / 16, TM = WM / 16;        // MFMA tiles per wave
    constexpr int LW = BN * 16 / 256;                // 16-byte W loads per thread per stage
    constexpr int LX = BM * 16 / 256;                // 16-byte X loads per thread per stage
    static_assert(LW >= 1 && LX >= 1 && TN >= 1 && TM >= 1, "tile too small");
    constexpr int STAGE_BYTES = (BN + BM) * kPitch;
    constexpr int CBYTES = BN * (BM + 4) * 4;        // fp32 block for the epilogue (padded)
    constexpr int LDS_BYTES = 2 * KG * STAGE_BYTES > CBYTES ? 2 * KG * STAGE_BYTES : CBYTES;
    __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
    // group kg, stage buffer q: W tile at lds + (2*kg + q)*STAGE_BYTES, X tile right after it

    // XCD-aware block order: block b runs on XCD b % 8; consecutive blocks of one XCD take
    // the m-tiles of one n-tile
    const int b = blockIdx.x;
    const int xcd = b & 7, j = b >> 3;
    const int mt = j % m_tiles;
    const int nt = (j / m_tiles) * 8 + xcd;
    if (nt >= n_tiles) return;                       // padding block (uniform)
    const int n0 = nt * BN, m0 = mt * BM;

    const int tid = threadIdx.x & 255;               // thread within the group
    const int kg = threadIdx.x >> 8;                 // K group: stages kg, kg + KG, ...
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wn = (wave & 1) * WN, wm = (wave >> 1) * WM;
    const int KV = K >> 3;                           // 16-byte vectors per row
    const int stages = (K + kKC - 1) / kKC;
    const int gstages = (stages + KG - 1) / KG;      // stages of this group (some may be empty)
    uint8_t *const glds = lds + 2 * kg * STAGE_BYTES;
    const u32x4_t *Wv = reinterpret_cast<const u32x4_t *>(W);
    const u32x4_t *Xv = reinterpret_cast<const u32x4_t *>(X);

    // thread -> (row, 16-byte column) of the stage tiles: 16 threads cover one 256-byte row
    const int lrow = tid >> 4, lcol = tid & 15;
    // s below is the group-local stage; it covers the K stage s*KG + kg (stage numbers at or
    // past `stages` are empty and zero-filled)
    auto kstage = [&](int s) { return s * KG + kg; };
    auto fetch = [&](int s, u32x4_t (&wr)[LW], u32x4_t (&xr)[LX]) {
        const int v = min(kstage(s) * (kKC / 8) + lcol, KV - 1);  // clamped; zeroed if past K
#pragma unroll
        for (int i = 0; i < LW; ++i) {
            const int n = min(n0 + lrow + 16 * i, N - 1);
            wr[i] = Wv[(size_t)n * KV + v];  // cached: the other m-tiles read it from L2
        }
#pragma unroll
        for (int i = 0; i < LX; ++i) {
            const int m = min(m0 + lrow + 16 * i, M - 1);
            xr[i] = Xv[(size_t)m * KV + v];
        }
    };
    auto stash = [&](int s, u32x4_t (&wr)[LW], u32x4_t (&xr)[LX]) {
        uint8_t *Ws = glds + (s & 1) * STAGE_BYTES;
        uint8_t *Xs = Ws + BN * kPitch;
        const bool kok = kstage(s) * (kKC / 8) + lcol < KV;
#pragma unroll
        for (int i = 0; i < LW; ++i)
            *reinterpret_cast<u32x4_t *>(Ws + (lrow + 16 * i) * kPitch + 16 * lcol) = kok ? wr[i] : u32x4_t{};
#pragma unroll
        for (int i = 0; i < LX; ++i)
            *reinterpret_cast<u32x4_t *>(Xs + (lrow + 16 * i) * kPitch + 16 * lcol) = kok ? xr[i] : u32x4_t{};
    };

    // residual prefetch: thread t finishes elements e = t + 256*KG*i of the block, taken row by
    // row of Y (ml = e / BN, nl = e % BN); clamped addresses keep the loads unconditional, and
    // their latency hides behind the K loop
    constexpr int EPT = BN * BM / (256 * KG);
    static_assert(EPT * 256 * KG == BN * BM, "epilogue split");
    uint16_t rv[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int e = threadIdx.x + 256 * KG * i;
        rv[i] = R[(size_t)min(m0 + e / BN, M - 1) * ep.ldr + min(n0 + e % BN, N - 1)];
    }

    f32x4_t acc[TN][TM];
#pragma unroll
    for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int c = 0; c < TM; ++c) acc[a][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // The loop body is branch-free so the compiler keeps D stages of loads in flight (a
    // branch around a load makes it wait for every outstanding load): prefetches past the
    // last stage re-read the last stage (never used), stages past K are zero-filled.
    // Stage s lives in LDS buffer s&1: during stage s the next stage is written to the other
    // buffer while the matrix cores read this one, with one barrier per stage.
    u32x4_t wr[D][LW], xr[D][LX];
#pragma unroll
    for (int d = 0; d < D; ++d) fetch(min(d, gstages - 1), wr[d], xr[d]);
    stash(0, wr[0], xr[0]);
    fetch(min(D, gstages - 1), wr[0], xr[0]);

    const int frow = lane & 15, fk = 16 * (lane >> 4);  // fragment row / byte offset in a k-step
    const int groups = (gstages + D - 1) / D;
    for (int g0 = 0; g0 < groups; ++g0) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int s = g0 * D + d;
            const int dn = (d + 1) % D;              // register slot of stage s + 1
            __syncthreads();                         // stage s is in LDS; stage s-1 reads are done
            stash(s + 1, wr[dn], xr[dn]);            // zero-filled when s + 1 is past K
            fetch(min(s + 1 + D, gstages - 1), wr[dn], xr[dn]);
            const uint8_t *Ws = glds + (s & 1) * STAGE_BYTES;
            const uint8_t *Xs = Ws + BN * kPitch;
            // each stage sums into a fresh tile that is then added to the total: the longest
            // fp32 rounding chain is 4 + K/128 steps instead of K/32
            f32x4_t st[TN][TM];
#pragma unroll
            for (int a = 0; a < TN; ++a)
#pragma unroll
                for (int c = 0; c < TM; ++c) st[a][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < kKC / 32; ++kk) {
                u32x4_t af[TN], bfr[TM];
#pragma unroll
                for (int a = 0; a < TN; ++a)
                    af[a] = *reinterpret_cast<const u32x4_t *>(Ws + (wn + 16 * a + frow) * kPitch + 64 * kk + fk);
#pragma unroll
                for (int c = 0; c < TM; ++c)
                    bfr[c] = *reinterpret_cast<const u32x4_t *>(Xs + (wm + 16 * c + frow) * kPitch + 64 * kk + fk);
#pragma unroll
                for (int a = 0; a < TN; ++a)
#pragma unroll
                    for (int c = 0; c < TM; ++c) st[a][c] = mfma16(af[a], bfr[c], st[a][c]);
            }
#pragma unroll
            for (int a = 0; a < TN; ++a)
#pragma unroll
                for (int c = 0; c < TM; ++c) acc[a][c] += st[a][c];
        }
    }

    // epilogue: acc[a][c][r] = Y^T[n0 + wn + 16a + 4*(lane/16) + r][m0 + wm + 16c + lane%16]
    // (partial over this group's stages); the groups add into C in group order
    __syncthreads();
    float *C = reinterpret_cast<float *>(lds);       // C[n][m], row pitch BM + 4 floats
#pragma unroll
    for (int q = 0; q < KG; ++q) {
        if (kg == q) {
#pragma unroll
            for (int a = 0; a < TN; ++a)
#pragma unroll
                for (int c = 0; c < TM; ++c)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float &slot = C[(wn + 16 * a + 4 * (lane >> 4) + r) * (BM + 4) + wm + 16 * c + (lane & 15)];
                        slot = (q == 0) ? acc[a][c][r] : slot + acc[a][c][r];
                    }
        }
        __syncthreads();
    }
    // walk the block row by row of Y: neighbouring threads take neighbouring n
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int e = threadIdx.x + 256 * KG * i;
        const int ml = e / BN, nl = e % BN;
        const int m = m0 + ml, n = n0 + nl;
        if (m < M && n < N) {
            store_output<ACC>(out, ep, m, n, C[nl * (BM + 4) + ml], bf16_bits_to_f32(rv[i]));
        }
    }
}

template <int BN, int BM, int D, int KG>
hipError_t launch_gemm(const LaunchArgs &a) {
    const int n_tiles = (int)((a.N + BN - 1) / BN);
    const int m_tiles = (int)((a.M + BM - 1) / BM);
    const int groups = (n_tiles + 7) / 8;            // n-tiles per XCD, rounded up
    dim3 grid((unsigned)(groups * 8 * m_tiles));
    dim3 block(256 * KG);
    if (a.acc_out)
        hipLaunchKernelGGL((mfma_gemm_kernel<BN, BM, D, KG, true>), grid, block, 0, a.stream, a.X, a.W, a.R, a.out,
                           (int)a.M, (int)a.N, (int)a.K, n_tiles, m_tiles, a.ep);
    else
        hipLaunchKernelGGL((mfma_gemm_kernel<BN, BM, D, KG, false>), grid, block, 0, a.stream, a.X, a.W, a.R, a.out,
                           (int)a.M, (int)a.N, (int)a.K, n_tiles, m_tiles, a.ep);
    return hipGetLastError();
}

int64_t gemm_max_k() { return INT64_MAX; }

// Public knobs: path SKINNY_PATH_GEMM, block_size = 256*KG, outputs_per_block = BN,
// k_unroll = D (stages in flight per group), vector_width = 8, m_tile = BM, k_split = KG
// (groups of 4 waves; a wave's block is fixed by BN, BM).
#define GEMM_ENTRY(BN, BM, D, KG)                                                                  \
    KernelEntry {                                                                                  \
        skinny_config{SKINNY_PATH_GEMM, 256 * KG, BN, D, 8, BM, KG}, &launch_gemm<BN, BM, D, KG>,  \
            (const void *)&mfma_gemm_kernel<BN, BM, D, KG, false>,                                 \
            (const void *)&mfma_gemm_kernel<BN, BM, D, KG, true>, &gemm_max_k                      \
    }

const KernelEntry kGemmEntries[] = {
    GEMM_ENTRY(32, 32, 4, 1),
    GEMM_ENTRY(32, 64, 4, 1),
    GEMM_ENTRY(64, 64, 4, 1),
    GEMM_ENTRY(64, 64, 2, 1),
    GEMM_ENTRY(64, 128, 2, 1),
    GEMM_ENTRY(32, 32, 2, 2),
    GEMM_ENTRY(32, 64, 2, 2),
    GEMM_ENTRY(32, 64, 4, 2),
    GEMM_ENTRY(64, 64, 2, 2),
    GEMM_ENTRY(64, 64, 4, 2),
};

}  // namespace

const KernelEntry *gemm_entries(int *count) {
    *count = (int)(sizeof(kGemmEntries) / sizeof(kGemmEntries[0]));
    return kGemmEntries;
}

}  // namespace skinny
