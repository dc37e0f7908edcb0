// mfma.hip -- matrix-core path of the skinny residual GEMM  Y = bf16(X W^T + R).
//
// Operation: vLLM benchmark page "benchmarks/kernels/benchmark_k3_cutedsl_residual.py"
// (module docstring; torch.addmm leg). The pages' kernel is SIMT; on gfx950 the same
// data flow maps onto v_mfma_f32_16x16x32_bf16 with:
//   * A operand = a 16-row tile of W (rows = output columns n), B operand = X^T
//     (columns = rows m of X, zero-padded to 16), D = a 16 x 16 fp32 block of Y^T;
//   * each lane loads its A fragment straight from HBM: 16 bytes = 8 consecutive k of one
//     W row (lane & 15 selects the row, lane >> 4 the 8-wide k group), non-temporal;
//     four k-steps of one row cover a 128-byte line;
//   * the B fragment comes the same way from X (L2-resident, lanes of padding rows skip
//     the load) and is reused across the T row tiles of the workgroup;
//   * a workgroup is KS waves that split K into KS contiguous slices; the matrix cores do
//     the reduction over k inside each slice, and the KS partial blocks meet in LDS;
//   * workgroup g owns the row tiles g, g + G, g + 2G, ... (G = number of workgroups), so
//     the chip streams a compact window of W in address order;
//   * the epilogue adds R in fp32 and rounds once to bf16 (RNE); residuals are fetched
//     before the K loop so their latency hides under the W stream.
#include "common.hpp"

namespace skinny {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// KS: waves per workgroup (K slices); T: 16-row W tiles per workgroup; KU: k-steps (32 wide)
// per batch; CT: 16-column X tiles per pass (m_tile = 16*CT); ACC: write fp32 instead of bf16.
template <int KS, int T, int KU, int CT, bool ACC>
__global__ __launch_bounds__(KS * 64) void mfma_kernel(const uint16_t *__restrict__ X,
                                                       const uint16_t *__restrict__ W,
                                                       const uint16_t *R, void *out,
                                                       int M, int N, int K, Epilogue ep) {
    constexpr int NT = KS * 64;                 // threads
    constexpr int OUTS = T * CT * 256;          // D elements per workgroup (incl. padding)
    constexpr int PER_THREAD = (OUTS + NT - 1) / NT;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int ks = tid >> 6;
    const int row = lane & 15;
    const int kg = lane >> 4;
    const int G = gridDim.x;
    const int m0 = blockIdx.y * 16 * CT;
    // first row of tile t: (blockIdx.x + t * G) * 16

    // residual prefetch for the outputs this thread finishes in the epilogue (indices are
    // clamped so the loads need no branch; out-of-range outputs are never stored)
    float rres[PER_THREAD];
#pragma unroll
    for (int p = 0; p < PER_THREAD; ++p) {
        const int e = min(tid + p * NT, OUTS - 1);
        const int tc = e >> 8, l = (e >> 2) & 63, r = e & 3;
        const int t = tc / CT, c = tc % CT;
        const int m = min(m0 + 16 * c + (l & 15), M - 1);
        const int n = min((blockIdx.x + t * G) * 16 + 4 * (l >> 4) + r, N - 1);
        rres[p] = bf16_bits_to_f32(R[(size_t)m * ep.ldr + n]);
    }

    // this wave's K slice, in 32-wide steps
    const int nsteps = (K + 31) / 32;
    const int per = (nsteps + KS - 1) / KS;
    const int s_begin = ks * per;
    const int s_end = min(nsteps, s_begin + per);

    const u32x4_t *Wv = reinterpret_cast<const u32x4_t *>(W);
    const u32x4_t *Xv = reinterpret_cast<const u32x4_t *>(X);
    const int kv = K / 8;  // 16-byte vectors per row

    f32x4_t acc[T][CT];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int c = 0; c < CT; ++c) acc[t][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Loads are unconditional: W rows past N and X rows past M are clamped to a valid row
    // (their results are never stored); k-steps past the slice or past K are clamped and
    // zeroed in both operands.
    for (int s0 = s_begin; s0 < s_end; s0 += KU) {
        u32x4_t a[KU][T];
        u32x4_t b[KU][CT];
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int v = min((s0 + u) * 4 + kg, kv - 1);  // 16-byte vector index along K
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const int n = min((int)(blockIdx.x + t * G) * 16 + row, N - 1);
                a[u][t] = __builtin_nontemporal_load(&Wv[(size_t)n * kv + v]);
            }
        }
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int v = min((s0 + u) * 4 + kg, kv - 1);
#pragma unroll
            for (int c = 0; c < CT; ++c) b[u][c] = Xv[(size_t)min(m0 + 16 * c + row, M - 1) * kv + v];
        }
        // keep every load of the batch in flight before the first use
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            if ((s0 + u) >= s_end || (s0 + u) * 4 + kg >= kv) {
#pragma unroll
                for (int t = 0; t < T; ++t) a[u][t] = u32x4_t{};
#pragma unroll
                for (int c = 0; c < CT; ++c) b[u][c] = u32x4_t{};
            }
        }
#pragma unroll
        for (int u = 0; u < KU; ++u)
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int c = 0; c < CT; ++c) acc[t][c] = mfma16(a[u][t], b[u][c], acc[t][c]);
    }

    // acc[t][c][i] = partial D[n = (blockIdx.x + t*G)*16 + 4*kg + i][m = m0 + 16c + row]
    __shared__ f32x4_t red[KS][T * CT][64];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int c = 0; c < CT; ++c) red[ks][t * CT + c][lane] = acc[t][c];
    __syncthreads();

    const float *redf = reinterpret_cast<const float *>(&red[0][0][0]);
#pragma unroll
    for (int p = 0; p < PER_THREAD; ++p) {
        const int e = tid + p * NT;
        if (e >= OUTS) break;
        const int tc = e >> 8, l = (e >> 2) & 63, r = e & 3;
        const int t = tc / CT, c = tc % CT;
        const int m = m0 + 16 * c + (l & 15);
        const int n = (blockIdx.x + t * G) * 16 + 4 * (l >> 4) + r;
        if (m >= M || n >= N) continue;
        float sum = redf[e];
#pragma unroll
        for (int g = 1; g < KS; ++g) sum += redf[g * OUTS + e];
        store_output<ACC>(out, ep, m, n, sum, rres[p]);
    }
}

template <int KS, int T, int KU, int CT>
hipError_t launch_mfma(const LaunchArgs &a) {
    dim3 grid((unsigned)((a.N + 16 * T - 1) / (16 * T)), (unsigned)((a.M + 16 * CT - 1) / (16 * CT)));
    dim3 block(KS * 64);
    if (a.acc_out)
        hipLaunchKernelGGL((mfma_kernel<KS, T, KU, CT, true>), grid, block, 0, a.stream, a.X, a.W, a.R,
                           a.out, (int)a.M, (int)a.N, (int)a.K, a.ep);
    else
        hipLaunchKernelGGL((mfma_kernel<KS, T, KU, CT, false>), grid, block, 0, a.stream, a.X, a.W, a.R,
                           a.out, (int)a.M, (int)a.N, (int)a.K, a.ep);
    return hipGetLastError();
}

int64_t no_k_limit() { return INT64_MAX; }

// Public knobs: block_size = 64*KS, outputs_per_block = 16*T, k_unroll = KU,
// vector_width = 8, m_tile = 16*CT, k_split = KS.
#define MFMA_ENTRY(KS, T, KU, CT)                                                                  \
    KernelEntry {                                                                                  \
        skinny_config{SKINNY_PATH_MFMA, 64 * KS, 16 * T, KU, 8, 16 * CT, KS},                      \
            &launch_mfma<KS, T, KU, CT>, (const void *)&mfma_kernel<KS, T, KU, CT, false>,         \
            (const void *)&mfma_kernel<KS, T, KU, CT, true>, &no_k_limit                           \
    }

#include "mfma_instances.inc"

}  // namespace

const KernelEntry *mfma_entries(int *count) {
    *count = (int)(sizeof(kMfmaEntries) / sizeof(kMfmaEntries[0]));
    return kMfmaEntries;
}

}  // namespace skinny
