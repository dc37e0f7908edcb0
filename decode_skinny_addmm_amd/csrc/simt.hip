// simt.hip -- the block-strided SIMT family, for tuning sweeps over the launch knobs.
//
// Operation: vLLM benchmark page "benchmarks/kernels/benchmark_k3_cutedsl_residual.py"
// (module docstring; torch.addmm leg). Decomposition: the kernel of the vLLM API page
// "fused_add_multicast_skinny_gemm" (FusedAddMulticastSkinnyGemm) -- one workgroup per
// `outputs_per_block` output columns; its `block_size` threads stride over K in vectors of
// `vector_width` bf16 (thread t takes vectors t, t + block, ...), `k_unroll` vectors of every
// row in flight per step; fp32 accumulation, a warp (here: 64-lane wave) reduction, then a
// cross-wave reduction, residual added in the epilogue. The benchmark page sweeps exactly
// these four knobs; this family exposes them unchanged so the same grid can be timed on
// gfx950. Written for 64-lane waves: products with v_dot2c_f32_bf16, the in-wave reduction
// with permlane swaps and DPP (transposing, so M*opb sums cost about M*opb steps), the waves'
// partial sums meet in LDS; loads are unconditional (clamped indices, K tail zeroed).
#include "common.hpp"

namespace skinny {
namespace {

template <int VW> struct Vec;
template <> struct Vec<8> { typedef uint32_t type __attribute__((ext_vector_type(4))); };
template <> struct Vec<4> { typedef uint32_t type __attribute__((ext_vector_type(2))); };

// MT: rows of X per pass; BS: threads per workgroup; OPB: output columns per workgroup;
// KU: vectors per row in flight per step; VW: bf16 per vector.
template <int MT, int BS, int OPB, int KU, int VW, bool ACC>
__global__ __launch_bounds__(BS) void simt_kernel(const uint16_t *__restrict__ X, const uint16_t *__restrict__ W,
                                                  const uint16_t *R, void *out, int M, int N, int K,
                                                  Epilogue ep) {
    using vec = typename Vec<VW>::type;
    constexpr int DW = VW / 2;                   // dwords per vector
    constexpr int WAVES = BS / 64;
    constexpr int V = MT * OPB;                  // sums per lane, index = m * OPB + o
    constexpr int S = ilog2(V) < 6 ? ilog2(V) : 6;
    constexpr int CF = V > 64 ? V / 64 : 1;
    static_assert((V & (V - 1)) == 0, "MT * OPB must be a power of two");

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = blockIdx.x * OPB;
    const int m0 = blockIdx.y * MT;
    const int NV = K / VW;                       // vectors per row
    const vec *Wv = reinterpret_cast<const vec *>(W);
    const vec *Xv = reinterpret_cast<const vec *>(X);

    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.0f;

    const int steps = (NV + BS - 1) / BS;        // vectors per thread per row (last one ragged)
    for (int j0 = 0; j0 < steps; j0 += KU) {
        vec w[KU][OPB];
        vec x[KU][MT];
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int v = min((j0 + u) * BS + tid, NV - 1);
#pragma unroll
            for (int o = 0; o < OPB; ++o) w[u][o] = __builtin_nontemporal_load(&Wv[(size_t)min(n0 + o, N - 1) * NV + v]);
        }
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int v = min((j0 + u) * BS + tid, NV - 1);
#pragma unroll
            for (int m = 0; m < MT; ++m) x[u][m] = Xv[(size_t)min(m0 + m, M - 1) * NV + v];
        }
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            if ((j0 + u) * BS + tid >= NV) {     // past the end of the row (or of the step range)
#pragma unroll
                for (int m = 0; m < MT; ++m) x[u][m] = vec{};
            }
        }
#pragma unroll
        for (int u = 0; u < KU; ++u)
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int o = 0; o < OPB; ++o)
#pragma unroll
                    for (int d = 0; d < DW; ++d) acc[m * OPB + o] = dot2_bf16(x[u][m][d], w[u][o][d], acc[m * OPB + o]);
    }

    wave_transpose_reduce<V, 32>(acc, lane);
    const bool writer = (lane & ((64 >> S) - 1)) == 0;
    const int base = CF * (lane >> (6 - S));
    __shared__ float red[WAVES][V];
    if (writer) {
#pragma unroll
        for (int c = 0; c < CF; ++c) red[wave][base + c] = acc[c];
    }
    __syncthreads();
    // the first V threads finish one output each: neighbouring threads, neighbouring columns
    for (int idx = tid; idx < V; idx += BS) {
        const int m = m0 + idx / OPB, n = n0 + idx % OPB;
        if (m < M && n < N) {
            float t = red[0][idx];
#pragma unroll
            for (int q = 1; q < WAVES; ++q) t += red[q][idx];
            store_output<ACC>(out, ep, m, n, t, bf16_bits_to_f32(R[(size_t)m * ep.ldr + n]));
        }
    }
}

template <int MT, int BS, int OPB, int KU, int VW>
hipError_t launch_simt(const LaunchArgs &a) {
    dim3 grid((unsigned)((a.N + OPB - 1) / OPB), (unsigned)((a.M + MT - 1) / MT));
    dim3 block(BS);
    if (a.acc_out)
        hipLaunchKernelGGL((simt_kernel<MT, BS, OPB, KU, VW, true>), grid, block, 0, a.stream, a.X, a.W, a.R,
                           a.out, (int)a.M, (int)a.N, (int)a.K, a.ep);
    else
        hipLaunchKernelGGL((simt_kernel<MT, BS, OPB, KU, VW, false>), grid, block, 0, a.stream, a.X, a.W, a.R,
                           a.out, (int)a.M, (int)a.N, (int)a.K, a.ep);
    return hipGetLastError();
}

int64_t simt_max_k() { return INT64_MAX; }

// Public knobs: path SKINNY_PATH_SIMT, block_size, outputs_per_block, k_unroll, vector_width
// exactly as named; m_tile = MT; k_split = block_size / 64 (every wave shares every column).
#define SIMT_ENTRY(MT, BS, OPB, KU, VW)                                                            \
    KernelEntry {                                                                                  \
        skinny_config{SKINNY_PATH_SIMT, BS, OPB, KU, VW, MT, BS / 64},                             \
            &launch_simt<MT, BS, OPB, KU, VW>, (const void *)&simt_kernel<MT, BS, OPB, KU, VW, false>, \
            (const void *)&simt_kernel<MT, BS, OPB, KU, VW, true>, &simt_max_k                     \
    }
#define SIMT_KU(MT, BS, OPB, VW) SIMT_ENTRY(MT, BS, OPB, 1, VW), SIMT_ENTRY(MT, BS, OPB, 2, VW), SIMT_ENTRY(MT, BS, OPB, 4, VW)
#define SIMT_OPB(MT, BS, VW) SIMT_KU(MT, BS, 1, VW), SIMT_KU(MT, BS, 2, VW), SIMT_KU(MT, BS, 4, VW), SIMT_KU(MT, BS, 8, VW)
#define SIMT_GRID(MT, VW) SIMT_OPB(MT, 64, VW), SIMT_OPB(MT, 128, VW), SIMT_OPB(MT, 256, VW)

// The 72-point grid (block {64,128,256} x outputs {1,2,4,8} x k_unroll {1,2,4} x vector
// width {4,8}) at a 16-row X tile.
const KernelEntry kSimtEntries[] = {SIMT_GRID(16, 4), SIMT_GRID(16, 8)};

}  // namespace

const KernelEntry *simt_entries(int *count) {
    *count = (int)(sizeof(kSimtEntries) / sizeof(kSimtEntries[0]));
    return kSimtEntries;
}

}  // namespace skinny
