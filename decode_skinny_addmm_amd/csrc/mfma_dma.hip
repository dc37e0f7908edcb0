// mfma_dma.hip -- matrix-core K-loop GEMM whose operand tiles go from memory straight into
// LDS (gfx950 global_load_lds_dwordx4), for tens to hundreds of rows of X.
//
// Operation: vLLM benchmark page "benchmarks/kernels/benchmark_k3_cutedsl_residual.py"
// (module docstring; torch.addmm leg): Y = bf16(X W^T + R), fp32 accumulation.
// Design for gfx950:
//   * a workgroup of 4 waves computes a BN x BM block of Y^T (BN rows of W, BM rows of X)
//     with v_mfma_f32_16x16x32_bf16 tiles, split over the waves in one of two ways:
//     KW = false: a 2 x 2 layout, each wave a (BN/2) x (BM/2) block over the whole stage
//     (every fragment is read from LDS by the two waves that share it);
//     KW = true: each wave takes one of the stage's four 32-wide K steps for the whole block
//     (every fragment is read once; the waves' partial blocks are added in the epilogue,
//     in wave order);
//   * K advances in stages of 128. A stage is (BN + BM) rows of 256 bytes in LDS, held in a
//     ring of NS stages. Each wave moves its share of a stage with direct-to-LDS loads
//     (16 bytes per lane, 1 KB of LDS per instruction, four 256-byte rows), so operand
//     bytes never pass through registers and no LDS store instructions are issued; load i of
//     every wave covers rows 16i .. 16i + 15, so the W rows (read once) take the non-temporal
//     cache policy and the X rows (read by every W tile) the default one;
//   * the 16-byte chunks of a row are stored XOR-swizzled by the row index (chunk c of row r
//     sits at position c ^ (r & 15)): a lane's load still covers a 64-byte aligned piece of
//     one row, and the MFMA fragment reads (16 rows, one logical chunk) hit 16 distinct
//     bank groups;
//   * NS - 1 stages are in flight while the matrix cores work on one; each wave waits for
//     its own loads of the stage with an explicit vmcnt count, then one barrier publishes
//     the stage to the workgroup and frees the slot read in the previous iteration, which
//     is refilled right after the barrier;
//   * KW = false: each stage sums into a fresh tile that is then added to the total, so the
//     longest fp32 rounding chain is 4 + K/128 additions; KW = true: K/128 accumulations per
//     wave, then the three additions of the wave partials;
//   * block ids are laid out so that the M-tiles of one W row tile are consecutive on one XCD
//     (blocks are dealt to the 8 XCDs round-robin): they share the W tile through that
//     XCD's L2, so W leaves HBM once;
//   * R is fetched into registers at the start (its latency hides behind the K loop); the
//     epilogue stages the fp32 block in LDS and walks it row by row of Y, so R and Y are
//     accessed contiguously; R added in fp32, one RNE rounding to bf16.
// K must be a multiple of 128 (whole stages: direct-to-LDS loads cannot zero a ragged tail).
#include "common.hpp"

namespace skinny {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kKC = 128;          // K per stage (bf16 elements)
constexpr int kRowBytes = 256;    // one staged row: 128 bf16, no padding (swizzled instead)

__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// s_waitcnt immediate that waits until at most n vector-memory operations are outstanding
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at their maxima).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Barrier that orders the workgroup's LDS accesses without waiting for outstanding
// direct-to-LDS loads (each wave has already waited for the loads it needs).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

typedef __attribute__((address_space(3))) void lds_void;

// BN: rows of W per workgroup; BM: rows of X per workgroup; NS: LDS stages in the ring;
// KW: the waves split each stage's K steps (true) or the block (false).
template <int BN, int BM, int NS, bool KW, bool ACC, bool GEN>
__global__ __launch_bounds__(256) void mfma_dma_kernel(const uint16_t *__restrict__ X,
                                                       const uint16_t *__restrict__ W,
                                                       const uint16_t *R, void *out,
                                                       int M, int N, int K, int n_tiles, int m_tiles, Epilogue ep) {
    const Epilogue epi = GEN ? ep : Epilogue{N, N, 0u};  // see plain_epilogue
    constexpr int WN = KW ? BN : BN / 2, WM = KW ? BM : BM / 2;  // wave block
    constexpr int TN = WN / 16, TM = WM / 16;        // MFMA tiles per wave
    static_assert(TN >= 1 && TM >= 1, "tile too small");
    constexpr int ROWS = BN + BM;                    // staged rows: W rows, then X rows
    constexpr int STAGE_BYTES = ROWS * kRowBytes;
    constexpr int BLOCKS = ROWS / 4;                 // 1 KB load blocks per stage
    static_assert(BLOCKS % 4 == 0, "stage blocks must split evenly over 4 waves");
    constexpr int PW = BLOCKS / 4;                   // load instructions per wave per stage
    static_assert(PW * (NS - 2) < 64 && NS >= 2, "vmcnt budget");
    constexpr int CBYTES = (KW ? 4 : 1) * BN * (BM + 4) * 4;  // fp32 block(s) for the epilogue (padded)
    constexpr int LDS_BYTES = NS * STAGE_BYTES > CBYTES ? NS * STAGE_BYTES : CBYTES;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];

    // XCD-aware block order: block b runs on XCD b % 8; consecutive blocks of one XCD take
    // the m-tiles of one n-tile
    const int b = blockIdx.x;
    const int xcd = b & 7, j = b >> 3;
    const int mt = j % m_tiles;
    const int nt = (j / m_tiles) * 8 + xcd;
    if (nt >= n_tiles) return;                       // padding block (uniform)
    const int n0 = nt * BN, m0 = mt * BM;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wn = KW ? 0 : (wave & 1) * WN, wm = KW ? 0 : (wave >> 1) * WM;
    const int S = K / kKC;                           // stages (K % 128 == 0)

    // This lane's source row and chunk for each of the wave's load blocks. Block q = 4i + wave
    // covers staged rows 4q..4q+3; lane l fills position l: row 4q + l/16, stored chunk l%16,
    // which holds logical chunk (l%16) ^ (row & 15). Rows past M or N re-read the last valid
    // row (their outputs are never written).
    const uint16_t *src[PW];
#pragma unroll
    for (int i = 0; i < PW; ++i) {
        const int q = 4 * i + wave;                  // load i of every wave covers rows 16i..16i+15
        const int sr = 4 * q + (lane >> 4);
        const int c = (lane & 15) ^ (sr & 15);
        const uint16_t *row = sr < BN ? W + (size_t)min(n0 + sr, N - 1) * K
                                      : X + (size_t)min(m0 + sr - BN, M - 1) * K;
        src[i] = row + 8 * c;
    }
    static_assert(BN % 16 == 0, "W loads are whole 16-row groups");
    auto issue = [&](int s) {                        // stage s -> ring slot s % NS
        uint8_t *st = lds + (s % NS) * STAGE_BYTES + wave * 1024;
#pragma unroll
        for (int i = 0; i < BN / 16; ++i)            // W rows: read once, non-temporal
            __builtin_amdgcn_global_load_lds((const void *)(src[i] + (size_t)s * kKC),
                                             (lds_void *)((__attribute__((address_space(3))) uint8_t *)st + i * 4096),
                                             16, 0, 2);
#pragma unroll
        for (int i = BN / 16; i < PW; ++i)           // X rows: shared by every W tile, cached
            __builtin_amdgcn_global_load_lds((const void *)(src[i] + (size_t)s * kKC),
                                             (lds_void *)((__attribute__((address_space(3))) uint8_t *)st + i * 4096),
                                             16, 0, 0);
    };

    // residual prefetch: thread t finishes elements e = t + 256 i of the block, taken row by
    // row of Y (ml = e / BN, nl = e % BN); clamped addresses, so the loads are unconditional
    // and their latency hides behind the K loop (they are the oldest loads, so every wait
    // below also covers them)
    constexpr int EPT = BN * BM / 256;
    static_assert(EPT * 256 == BN * BM, "epilogue split");
    uint16_t rv[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int e = tid + 256 * i;
        rv[i] = R[(size_t)min(m0 + e / BN, M - 1) * epi.ldr + min(n0 + e % BN, N - 1)];
    }

    f32x4_t acc[TN][TM];
#pragma unroll
    for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int c = 0; c < TM; ++c) acc[a][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int p = 0; p < NS - 1; ++p)
        if (p < S) issue(p);

    // fragment reads: row r (a multiple of 16 plus lane%16) and logical chunk 4*kk + lane/16
    // sit at r*256 + ((4*kk + lane/16) ^ (lane%16))*16
    const int frow = lane & 15, fq = lane >> 4;
    for (int s = 0; s < S; ++s) {
        const int later = min(NS - 2, S - 1 - s);    // stages issued after s, still in flight
        if (later >= 2) wait_vmcnt<PW * 2 < 64 ? PW * 2 : 63>();
        else if (later == 1) wait_vmcnt<PW>();
        else wait_vmcnt<0>();
        lds_barrier();                               // stage s visible; slot (s-1)%NS free
        if (s + NS - 1 < S) issue(s + NS - 1);
        const uint8_t *Ws = lds + (s % NS) * STAGE_BYTES;
        const uint8_t *Xs = Ws + BN * kRowBytes;
        if constexpr (KW) {
            // this wave's K step of the stage, every tile of the block, straight into acc
            const int off = (((4 * wave + fq) ^ frow) << 4) + frow * kRowBytes;
            u32x4_t af[TN], bfr[TM];
#pragma unroll
            for (int a = 0; a < TN; ++a) af[a] = *reinterpret_cast<const u32x4_t *>(Ws + 16 * a * kRowBytes + off);
#pragma unroll
            for (int c = 0; c < TM; ++c) bfr[c] = *reinterpret_cast<const u32x4_t *>(Xs + 16 * c * kRowBytes + off);
#pragma unroll
            for (int a = 0; a < TN; ++a)
#pragma unroll
                for (int c = 0; c < TM; ++c) acc[a][c] = mfma16(af[a], bfr[c], acc[a][c]);
            continue;
        }
        f32x4_t st[TN][TM];
#pragma unroll
        for (int a = 0; a < TN; ++a)
#pragma unroll
            for (int c = 0; c < TM; ++c) st[a][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < kKC / 32; ++kk) {
            const int off = (((4 * kk + fq) ^ frow) << 4) + frow * kRowBytes;
            u32x4_t af[TN], bfr[TM];
#pragma unroll
            for (int a = 0; a < TN; ++a)
                af[a] = *reinterpret_cast<const u32x4_t *>(Ws + (wn + 16 * a) * kRowBytes + off);
#pragma unroll
            for (int c = 0; c < TM; ++c)
                bfr[c] = *reinterpret_cast<const u32x4_t *>(Xs + (wm + 16 * c) * kRowBytes + off);
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

    // epilogue: acc[a][c][r] = Y^T[n0 + wn + 16a + 4*(lane/16) + r][m0 + wm + 16c + lane%16]
    __syncthreads();                                 // every wave is done with the ring
    float *C = reinterpret_cast<float *>(lds);       // C[n][m], row pitch BM + 4 floats
    constexpr int CB = BN * (BM + 4);                // floats per block copy
    float *Cw = C + (KW ? wave * CB : 0);            // KW: one partial block per wave
#pragma unroll
    for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int c = 0; c < TM; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Cw[(wn + 16 * a + 4 * (lane >> 4) + r) * (BM + 4) + wm + 16 * c + (lane & 15)] = acc[a][c][r];
    __syncthreads();
    // walk the block row by row of Y: neighbouring threads take neighbouring n
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int e = tid + 256 * i;
        const int ml = e / BN, nl = e % BN;
        const int m = m0 + ml, n = n0 + nl;
        if (m < M && n < N) {
            float t = C[nl * (BM + 4) + ml];
            if constexpr (KW) t = ((t + C[CB + nl * (BM + 4) + ml]) + C[2 * CB + nl * (BM + 4) + ml]) +
                                  C[3 * CB + nl * (BM + 4) + ml];
            store_output<ACC>(out, epi, m, n, t, bf16_bits_to_f32(rv[i]));
        }
    }
}

template <int BN, int BM, int NS, bool KW>
hipError_t launch_dma(const LaunchArgs &a) {
    const int n_tiles = (int)((a.N + BN - 1) / BN);
    const int m_tiles = (int)((a.M + BM - 1) / BM);
    const int groups = (n_tiles + 7) / 8;            // n-tiles per XCD, rounded up
    dim3 grid((unsigned)(groups * 8 * m_tiles));
    dim3 block(256);
    if (a.acc_out)
        hipLaunchKernelGGL((mfma_dma_kernel<BN, BM, NS, KW, true, true>), grid, block, 0, a.stream, a.X, a.W, a.R,
                           a.out, (int)a.M, (int)a.N, (int)a.K, n_tiles, m_tiles, a.ep);
    else if (plain_epilogue(a))
        hipLaunchKernelGGL((mfma_dma_kernel<BN, BM, NS, KW, false, false>), grid, block, 0, a.stream, a.X, a.W, a.R,
                           a.out, (int)a.M, (int)a.N, (int)a.K, n_tiles, m_tiles, a.ep);
    else
        hipLaunchKernelGGL((mfma_dma_kernel<BN, BM, NS, KW, false, true>), grid, block, 0, a.stream, a.X, a.W, a.R,
                           a.out, (int)a.M, (int)a.N, (int)a.K, n_tiles, m_tiles, a.ep);
    return hipGetLastError();
}

int64_t dma_max_k() { return INT64_MAX; }

// Public knobs: path SKINNY_PATH_GEMM_DMA, block_size = 256, outputs_per_block = BN,
// k_unroll = NS (LDS stages in the ring), vector_width = 8, m_tile = BM, k_split = 1 for the
// 2 x 2 wave layout or 4 for the four waves splitting each stage's K steps.
#define DMA_ENTRY_K(BN, BM, NS, KW)                                                                \
    KernelEntry {                                                                                  \
        skinny_config{SKINNY_PATH_GEMM_DMA, 256, BN, NS, 8, BM, (KW) ? 4 : 1},                     \
            &launch_dma<BN, BM, NS, KW>, (const void *)&mfma_dma_kernel<BN, BM, NS, KW, false, false>, \
            (const void *)&mfma_dma_kernel<BN, BM, NS, KW, true, true>, &dma_max_k, kKC            \
    }
#define DMA_ENTRY(BN, BM, NS) DMA_ENTRY_K(BN, BM, NS, false)

const KernelEntry kDmaEntries[] = {
    DMA_ENTRY(32, 32, 4),
    DMA_ENTRY(32, 64, 4),
    DMA_ENTRY(64, 32, 4),
    DMA_ENTRY(64, 64, 2),
    DMA_ENTRY(64, 64, 3),
    DMA_ENTRY(64, 64, 4),
    DMA_ENTRY(128, 64, 2),
    DMA_ENTRY(128, 64, 3),
    DMA_ENTRY(64, 128, 3),
    DMA_ENTRY_K(32, 32, 4, true),
    DMA_ENTRY_K(32, 64, 4, true),
    DMA_ENTRY_K(64, 32, 4, true),
    DMA_ENTRY_K(64, 64, 3, true),
    DMA_ENTRY_K(64, 64, 4, true),
    DMA_ENTRY_K(128, 64, 3, true),
    DMA_ENTRY_K(64, 128, 3, true),
    // 32 W rows by as many X rows as M needs: 224 workgroups for N = 7168, W read once
    DMA_ENTRY_K(32, 48, 4, true),
    DMA_ENTRY_K(32, 80, 4, true),
};

}  // namespace

const KernelEntry *dma_entries(int *count) {
    *count = (int)(sizeof(kDmaEntries) / sizeof(kDmaEntries[0]));
    return kDmaEntries;
}

}  // namespace skinny
