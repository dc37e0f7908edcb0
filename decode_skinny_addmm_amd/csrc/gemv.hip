// gemv.hip -- VALU path of the skinny residual GEMM  Y = bf16(X W^T + R)  for small M.
//
// Operation: vLLM benchmark page "benchmarks/kernels/benchmark_k3_cutedsl_residual.py"
// (module docstring; torch.addmm leg). The SIMT decomposition it starts from is the kernel
// of the vLLM API page "fused_add_multicast_skinny_gemm" (FusedAddMulticastSkinnyGemm:
// threads of a block stride over K in vectors, fp32 FMAs, warp then cross-warp reduction,
// residual added in the epilogue). Re-designed for gfx950:
//   * a workgroup is KS 64-lane waves that split K; lane l of wave w reads the 16-byte
//     vectors (j*KS + w)*64 + l of a row, so each load instruction of a wave is one
//     contiguous 1 KB piece of a W row (non-temporal: W is read once per call);
//   * workgroup g owns RB*NB rows, either g + i*G (G = number of workgroups: the chip
//     streams a compact window of W in address order) or g*RB*NB + i (contiguous rows:
//     outputs and residuals of a workgroup are contiguous), taken in NB batches of RB rows;
//     batch b+1's loads are in flight while batch b is multiplied and reduced;
//   * the lane's slice of X (KV 16-byte vectors per row of X) is loaded once into
//     registers and reused for every row of the workgroup;
//   * products: v_dot2c_f32_bf16 (two bf16 products into an fp32 accumulator per lane);
//   * the 64-lane reduction transposes (v_permlane32/16_swap, DPP), so RB*MT sums cost
//     about RB*MT exchange steps; the KS partial sums of every batch meet in LDS once;
//   * the epilogue adds R (prefetched at kernel start) in fp32 and rounds once to bf16.
// TAIL = false is the fast path for K a multiple of KV*KS*512 (no clamping, no selects);
// TAIL = true clamps vector indices past K and zeroes them in both operands.
#include "common.hpp"

namespace skinny {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// MT: rows of X per pass; KS: waves (K split); RB: rows per batch; NB: batches per
// workgroup; KV: 16-byte vectors per lane per row (K <= KV * KS * 512).
template <int MT, int KS, int RB, int NB, int KV, bool CONTIG, bool TAIL, bool ACC, bool GEN>
__global__ __launch_bounds__(KS * 64) void gemv_kernel(const uint16_t *__restrict__ X,
                                                       const uint16_t *__restrict__ W,
                                                       const uint16_t *R, void *out,
                                                       int M, int N, int K, Epilogue ep) {
    const Epilogue epi = GEN ? ep : Epilogue{N, N, 0u};  // see plain_epilogue
    constexpr int V = RB * MT;                  // sums per lane per batch, index = m * RB + r
    constexpr int S = ilog2(V) < 6 ? ilog2(V) : 6;
    constexpr int CF = V > 64 ? V / 64 : 1;     // sums per lane after the reduction
    constexpr int NBW = (NB + KS - 1) / KS;     // batches whose epilogue one wave runs
    static_assert((V & (V - 1)) == 0, "RB*MT must be a power of two");

    const int lane = threadIdx.x & 63;
    const int ks = threadIdx.x >> 6;
    const int G = gridDim.x;
    const int g = xcd_run(blockIdx.x, gridDim.x);  // contiguous row groups per XCD
    const int m0 = blockIdx.y * MT;
    const int NV = K >> 3;                      // 16-byte vectors per row
    const u32x4_t *Wv = reinterpret_cast<const u32x4_t *>(W);
    const u32x4_t *Xv = reinterpret_cast<const u32x4_t *>(X);

    auto vec_index = [&](int j) {
        const int v = (j * KS + ks) * 64 + lane;
        return TAIL ? min(v, NV - 1) : v;
    };
    // rows of this workgroup: contiguous (CONTIG) or strided over the grid
    auto row_of = [&](int i) { return CONTIG ? g * (RB * NB) + i : g + i * G; };
    auto load_batch = [&](int b, u32x4_t (&w)[RB][KV]) {
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const int n = min(row_of(b * RB + r), N - 1);  // rows past N: never stored
            const u32x4_t *row = Wv + (size_t)n * NV;
#pragma unroll
            for (int j = 0; j < KV; ++j) w[r][j] = __builtin_nontemporal_load(row + vec_index(j));
        }
    };

    // 1. this lane's slice of X, then the first two batches of W, then residuals (the wait
    // counter retires loads in issue order, so X and batch 0 must not sit behind batch 1)
    u32x4_t x[KV][MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const u32x4_t *row = Xv + (size_t)min(m0 + m, M - 1) * NV;  // rows past M: never stored
#pragma unroll
        for (int j = 0; j < KV; ++j) x[j][m] = row[vec_index(j)];
    }
    u32x4_t wbuf[2][RB][KV];
    __builtin_amdgcn_sched_barrier(0);  // keep the issue order: X, batch 0, batch 1
    load_batch(0, wbuf[0]);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NB > 1) load_batch(1, wbuf[1]);
    __builtin_amdgcn_sched_barrier(0);
    const bool writer_lane = (lane & ((64 >> S) - 1)) == 0;
    const int base = CF * (lane >> (6 - S));
    float rres[NBW][CF];
#pragma unroll
    for (int q = 0; q < NBW; ++q) {
        const int b = min(ks + q * KS, NB - 1);
#pragma unroll
        for (int c = 0; c < CF; ++c) {
            const int idx = base + c;
            const int n = min(row_of(b * RB + idx % RB), N - 1);
            const int m = min(m0 + idx / RB, M - 1);
            rres[q][c] = bf16_bits_to_f32(R[(size_t)m * epi.ldr + n]);
        }
    }
    if constexpr (TAIL) {
#pragma unroll
        for (int j = 0; j < KV; ++j)
            if ((j * KS + ks) * 64 + lane >= NV) {
#pragma unroll
                for (int m = 0; m < MT; ++m) x[j][m] = u32x4_t{};
            }
    }

    __shared__ float red[NB][KS][V];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        u32x4_t (&w)[RB][KV] = wbuf[b & 1];
        if constexpr (TAIL) {
#pragma unroll
            for (int j = 0; j < KV; ++j)
                if ((j * KS + ks) * 64 + lane >= NV) {
#pragma unroll
                    for (int r = 0; r < RB; ++r) w[r][j] = u32x4_t{};
                }
        }
        float acc[V];
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] = 0.0f;
#pragma unroll
        for (int j = 0; j < KV; ++j)
#pragma unroll
            for (int r = 0; r < RB; ++r)
#pragma unroll
                for (int m = 0; m < MT; ++m)
#pragma unroll
                    for (int d = 0; d < 4; ++d)
                        acc[m * RB + r] = dot2_bf16(x[j][m][d], w[r][j][d], acc[m * RB + r]);
        if (b + 2 < NB) load_batch(b + 2, w);  // refill this buffer while the next batch lands
        wave_transpose_reduce<V, 32>(acc, lane);
        if (writer_lane) {
#pragma unroll
            for (int c = 0; c < CF; ++c) red[b][ks][base + c] = acc[c];
        }
    }
    __syncthreads();

    if (!writer_lane) return;
#pragma unroll
    for (int q = 0; q < NBW; ++q) {
        const int b = ks + q * KS;
        if (b >= NB) break;
#pragma unroll
        for (int c = 0; c < CF; ++c) {
            const int idx = base + c;
            const int n = row_of(b * RB + idx % RB);
            const int m = m0 + idx / RB;
            if (m < M && n < N) {
                float t = red[b][0][idx];
#pragma unroll
                for (int p = 1; p < KS; ++p) t += red[b][p][idx];
                store_output<ACC>(out, epi, m, n, t, rres[q][c]);
            }
        }
    }
}

template <int MT, int KS, int RB, int NB, int KV, bool CONTIG, bool TAIL>
void launch_one(const LaunchArgs &a, dim3 grid, dim3 block) {
    if (a.acc_out)
        hipLaunchKernelGGL((gemv_kernel<MT, KS, RB, NB, KV, CONTIG, TAIL, true, true>), grid, block, 0, a.stream,
                           a.X, a.W, a.R, a.out, (int)a.M, (int)a.N, (int)a.K, a.ep);
    else if (plain_epilogue(a))
        hipLaunchKernelGGL((gemv_kernel<MT, KS, RB, NB, KV, CONTIG, TAIL, false, false>), grid, block, 0, a.stream,
                           a.X, a.W, a.R, a.out, (int)a.M, (int)a.N, (int)a.K, a.ep);
    else
        hipLaunchKernelGGL((gemv_kernel<MT, KS, RB, NB, KV, CONTIG, TAIL, false, true>), grid, block, 0, a.stream,
                           a.X, a.W, a.R, a.out, (int)a.M, (int)a.N, (int)a.K, a.ep);
}

template <int MT, int KS, int RB, int NB, int KV, bool CONTIG>
hipError_t launch_gemv(const LaunchArgs &a) {
    constexpr int64_t rows = (int64_t)RB * NB;
    dim3 grid((unsigned)((a.N + rows - 1) / rows), (unsigned)((a.M + MT - 1) / MT));
    dim3 block(KS * 64);
    if (a.K % ((int64_t)KV * KS * 512) == 0)
        launch_one<MT, KS, RB, NB, KV, CONTIG, false>(a, grid, block);
    else
        launch_one<MT, KS, RB, NB, KV, CONTIG, true>(a, grid, block);
    return hipGetLastError();
}

template <int KS, int KV>
int64_t gemv_max_k() { return (int64_t)KV * KS * 64 * 8; }

// Public knobs: block_size = 64*KS, outputs_per_block = RB*NB, k_unroll = KV,
// vector_width = 8 (rows strided over the grid) or 9 (contiguous rows), m_tile = MT,
// k_split = KS; rows per batch RB = outputs_per_block / NB.
#define GEMV_ENTRY(MT, KS, RB, NB, KV, CONTIG)                                                     \
    KernelEntry {                                                                                  \
        skinny_config{SKINNY_PATH_GEMV, 64 * KS, RB * NB, KV, CONTIG ? 9 : 8, MT, KS},             \
            &launch_gemv<MT, KS, RB, NB, KV, CONTIG>,                                              \
            (const void *)&gemv_kernel<MT, KS, RB, NB, KV, CONTIG, false, false, false>,           \
            (const void *)&gemv_kernel<MT, KS, RB, NB, KV, CONTIG, false, true, true>, &gemv_max_k<KS, KV> \
    }

#include "gemv_instances.inc"

}  // namespace

const KernelEntry *gemv_entries(int *count) {
    *count = (int)(sizeof(kGemvEntries) / sizeof(kGemvEntries[0]));
    return kGemvEntries;
}

}  // namespace skinny
