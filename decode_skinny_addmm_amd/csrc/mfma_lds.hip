// mfma_lds.hip -- matrix-core path for small M with W streamed like the GEMV path.
//
// Operation: vLLM benchmark page "benchmarks/kernels/benchmark_k3_cutedsl_residual.py"
// (module docstring; torch.addmm leg). Data flow on gfx950:
//   * a workgroup is KS waves; wave w owns the K slice [512w, 512w + 512) (one 16-byte
//     vector per lane per row), so every W load instruction reads one contiguous 1 KB piece
//     of a row (non-temporal), exactly like the GEMV path;
//   * workgroup g owns rows g + i*G (G = number of workgroups), in NB batches of RB rows,
//     double-buffered in registers so batch b+1 is in flight while batch b is multiplied;
//   * each batch goes through a wave-private LDS slice (rows padded to 1040 bytes, so the
//     16 rows of a fragment read hit distinct banks) and comes back as A fragments of
//     v_mfma_f32_16x16x32_bf16: lane l takes row l%16 (rows repeat when RB < 16), k group
//     l/16; the matrix cores then do the whole 512-long dot product of the slice;
//   * the B fragments (X^T, rows of X padded to 16*CT) are loaded once per workgroup and
//     stay in registers for every batch;
//   * the KS partial tiles of every batch meet in LDS once at the end; the epilogue adds R
//     (prefetched at kernel start) in fp32 and rounds once to bf16 (RNE).
// K must be a multiple of 8 and at most 512*KS; a K that is not a multiple of 512*KS takes
// the TAIL variant, which clamps vector indices past K and zeroes them in both operands.
#include "common.hpp"

namespace skinny {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kRowPitch = 1040;  // bytes per staged row: 1 KB of W + 16 B of padding

__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// CONTIG: workgroup g owns the contiguous rows g*RB*NB + i instead of g + i*G.
// XL: the rows of X (those < M) are loaded first, in contiguous 1 KB pieces, and turned into
// fragments through the staging slice; otherwise the fragments are loaded in fragment order
// (16 rows x 64 B per instruction) after the W batches.
template <int KS, int RB, int NB, int CT, bool CONTIG, bool XL, bool TAIL, bool ACC, bool GEN>
__global__ __launch_bounds__(KS * 64) void mfma_lds_kernel(const uint16_t *__restrict__ X,
                                                           const uint16_t *__restrict__ W,
                                                           const uint16_t *R, void *out,
                                                           int M, int N, int K, Epilogue ep) {
    const Epilogue epi = GEN ? ep : Epilogue{N, N, 0u};  // see plain_epilogue
    static_assert(RB == 1 || RB == 2 || RB == 4 || RB == 8 || RB == 16, "RB must divide 16");
    constexpr int NT = KS * 64;
    constexpr int OUTS = NB * RB * 16 * CT;       // outputs per workgroup (incl. padded m)
    constexpr int PER = (OUTS + NT - 1) / NT;
    constexpr int LV = RB < 4 ? 16 : 4 * RB;      // lanes of a D tile that hold rows < RB

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int ks = tid >> 6;
    const int G = gridDim.x;
    const int g = xcd_run(blockIdx.x, gridDim.x);  // contiguous row groups per XCD
    const int m0 = blockIdx.y * 16 * CT;
    const int NV = K >> 3;
    const u32x4_t *Wv = reinterpret_cast<const u32x4_t *>(W);
    const u32x4_t *Xv = reinterpret_cast<const u32x4_t *>(X);

    constexpr int SROWS = (XL && RB < 16) ? 16 : RB;  // staged rows per wave (X needs 16)
    __shared__ __attribute__((aligned(16))) uint8_t stage[KS][SROWS * kRowPitch];
    __shared__ f32x4_t red[NB][KS][CT][LV];

    const int vlane = ks * 64 + lane;                       // this lane's W vector in a row
    const int vload = TAIL ? min(vlane, NV - 1) : vlane;
    auto row_of = [&](int br) { return CONTIG ? g * (RB * NB) + br : g + br * G; };
    auto load_batch = [&](int b, u32x4_t (&w)[RB]) {
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const int n = min(row_of(b * RB + r), N - 1);  // rows past N: never stored
            w[r] = __builtin_nontemporal_load(Wv + (size_t)n * NV + vload);
        }
    };

    u32x4_t wbuf[2][RB];
    u32x4_t xrow[XL ? 16 * CT : 1];
    if constexpr (XL && !TAIL) {
        // X first (only the rows < M; the first four of each column tile unconditionally):
        // waiting for X then does not wait for W, whose loads follow
#pragma unroll
        for (int i = 0; i < 16 * CT; ++i)
            if ((i & 15) < 4 || m0 + i < M) xrow[i] = Xv[(size_t)min(m0 + i, M - 1) * NV + vlane];
    }
    load_batch(0, wbuf[0]);
    if constexpr (NB > 1) load_batch(1, wbuf[1]);

    // B fragments: lane l holds X[m0 + 16c + l%16][512*ks + 32s + 8*(l/16) + 0..7]
    uint8_t *my = stage[ks];
    u32x4_t xf[16][CT];
    if constexpr (XL && !TAIL) {
#pragma unroll
        for (int c = 0; c < CT; ++c) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (i < 4 || m0 + 16 * c + i < M)
                    *reinterpret_cast<u32x4_t *>(my + i * kRowPitch + 16 * lane) = xrow[16 * c + i];
            const int valid = max(min(M - m0 - 16 * c, 16), 1);  // rows of this column tile < M
#pragma unroll
            for (int s = 0; s < 16; ++s)
                xf[s][c] = *reinterpret_cast<const u32x4_t *>(my + min(lane & 15, valid - 1) * kRowPitch +
                                                              64 * s + 16 * (lane >> 4));
        }
    } else {
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            const u32x4_t *row = Xv + (size_t)min(m0 + 16 * c + (lane & 15), M - 1) * NV;
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const int v = ks * 64 + 4 * s + (lane >> 4);
                xf[s][c] = row[TAIL ? min(v, NV - 1) : v];
            }
        }
    }
    // residuals of the outputs this thread writes; output e is (row br = e % (RB*NB),
    // column mc = e / (RB*NB)), so neighbouring threads touch neighbouring rows n of one m
    float rres[PER];
#pragma unroll
    for (int p = 0; p < PER; ++p) {
        const int e = min(tid + p * NT, OUTS - 1);
        const int br = e % (RB * NB);  // batch * RB + row
        const int m = min(m0 + e / (RB * NB), M - 1);
        const int n = min(row_of(br), N - 1);
        rres[p] = bf16_bits_to_f32(R[(size_t)m * epi.ldr + n]);
    }
    if constexpr (TAIL) {
#pragma unroll
        for (int s = 0; s < 16; ++s)
            if (ks * 64 + 4 * s + (lane >> 4) >= NV) {
#pragma unroll
                for (int c = 0; c < CT; ++c) xf[s][c] = u32x4_t{};
            }
    }

    const int rd_row = (lane & 15) % RB;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        u32x4_t (&w)[RB] = wbuf[b & 1];
        if constexpr (TAIL) {
            if (vlane >= NV) {
#pragma unroll
                for (int r = 0; r < RB; ++r) w[r] = u32x4_t{};
            }
        }
#pragma unroll
        for (int r = 0; r < RB; ++r)
            *reinterpret_cast<u32x4_t *>(my + r * kRowPitch + 16 * lane) = w[r];
        if (b + 2 < NB) load_batch(b + 2, w);
        f32x4_t acc[CT];
#pragma unroll
        for (int c = 0; c < CT; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const u32x4_t a =
                *reinterpret_cast<const u32x4_t *>(my + rd_row * kRowPitch + 64 * s + 16 * (lane >> 4));
#pragma unroll
            for (int c = 0; c < CT; ++c) acc[c] = mfma16(a, xf[s][c], acc[c]);
        }
        // acc[c][i] = partial D[row 4*(l/16) + i][m 16c + l%16] over this wave's K slice
        if (lane < LV) {
#pragma unroll
            for (int c = 0; c < CT; ++c) red[b][ks][c][lane] = acc[c];
        }
    }
    __syncthreads();

    const float *redf = reinterpret_cast<const float *>(&red[0][0][0][0]);
#pragma unroll
    for (int p = 0; p < PER; ++p) {
        const int e = tid + p * NT;
        if (e >= OUTS) break;
        const int br = e % (RB * NB);
        const int mc = e / (RB * NB);       // column within the padded m range
        const int b = br / RB, r = br % RB;
        const int m = m0 + mc;
        const int n = row_of(br);
        if (m >= M || n >= N) continue;
        // D[row r][col mc%16] of column tile mc/16 lives in lane 16*(r/4) + mc%16, element r%4
        const int idx = ((mc >> 4) * LV + 16 * (r >> 2) + (mc & 15)) * 4 + (r & 3);
        float t = 0.0f;
#pragma unroll
        for (int q = 0; q < KS; ++q) t += redf[(b * KS + q) * CT * LV * 4 + idx];
        store_output<ACC>(out, epi, m, n, t, rres[p]);
    }
}

template <int KS, int RB, int NB, int CT, bool CONTIG, bool XL, bool TAIL>
void launch_one(const LaunchArgs &a, dim3 grid, dim3 block) {
    if (a.acc_out)
        hipLaunchKernelGGL((mfma_lds_kernel<KS, RB, NB, CT, CONTIG, XL, TAIL, true, true>), grid, block, 0,
                           a.stream, a.X, a.W, a.R, a.out, (int)a.M, (int)a.N, (int)a.K, a.ep);
    else if (plain_epilogue(a))
        hipLaunchKernelGGL((mfma_lds_kernel<KS, RB, NB, CT, CONTIG, XL, TAIL, false, false>), grid, block, 0,
                           a.stream, a.X, a.W, a.R, a.out, (int)a.M, (int)a.N, (int)a.K, a.ep);
    else
        hipLaunchKernelGGL((mfma_lds_kernel<KS, RB, NB, CT, CONTIG, XL, TAIL, false, true>), grid, block, 0,
                           a.stream, a.X, a.W, a.R, a.out, (int)a.M, (int)a.N, (int)a.K, a.ep);
}

template <int KS, int RB, int NB, int CT, bool CONTIG, bool XL>
hipError_t launch_mfma_lds(const LaunchArgs &a) {
    static_assert(!XL || CONTIG, "X-first variants use contiguous rows");
    constexpr int64_t rows = (int64_t)RB * NB;
    dim3 grid((unsigned)((a.N + rows - 1) / rows), (unsigned)((a.M + 16 * CT - 1) / (16 * CT)));
    dim3 block(KS * 64);
    if (a.K % (512 * KS) == 0)
        launch_one<KS, RB, NB, CT, CONTIG, XL, false>(a, grid, block);
    else
        launch_one<KS, RB, NB, CT, CONTIG, XL, true>(a, grid, block);
    return hipGetLastError();
}

template <int KS>
int64_t lds_max_k() { return (int64_t)KS * 512; }

// Public knobs: path SKINNY_PATH_MFMA_LDS, block_size = 64*KS, outputs_per_block = RB*NB,
// k_unroll = RB (rows per batch), m_tile = 16*CT, k_split = KS; vector_width tells the
// variants of one shape apart: 8 = rows strided over the grid, 9 = contiguous rows,
// 10 = contiguous rows with X loaded first through LDS.
#define MFMA_LDS_ENTRY(KS, RB, NB, CT, CONTIG, XL)                                                 \
    KernelEntry {                                                                                  \
        skinny_config{SKINNY_PATH_MFMA_LDS, 64 * KS, RB * NB, RB, XL ? 10 : (CONTIG ? 9 : 8),     \
                      16 * CT, KS},                                                                \
            &launch_mfma_lds<KS, RB, NB, CT, CONTIG, XL>,                                          \
            (const void *)&mfma_lds_kernel<KS, RB, NB, CT, CONTIG, XL, false, false, false>,       \
            (const void *)&mfma_lds_kernel<KS, RB, NB, CT, CONTIG, XL, false, true, true>, &lds_max_k<KS> \
    }

const KernelEntry kMfmaLdsEntries[] = {
    MFMA_LDS_ENTRY(7, 16, 2, 1, true, false),
    MFMA_LDS_ENTRY(7, 16, 2, 1, true, true),
    MFMA_LDS_ENTRY(7, 8, 4, 1, true, true),
    MFMA_LDS_ENTRY(7, 8, 4, 1, true, false),
    MFMA_LDS_ENTRY(7, 16, 2, 1, false, false),
    MFMA_LDS_ENTRY(7, 16, 1, 1, true, false),
    MFMA_LDS_ENTRY(7, 16, 4, 1, true, false),
    MFMA_LDS_ENTRY(7, 16, 4, 1, true, true),
    MFMA_LDS_ENTRY(7, 4, 7, 1, true, true),
    MFMA_LDS_ENTRY(7, 16, 2, 2, true, false),
    MFMA_LDS_ENTRY(7, 16, 2, 2, true, true),
    MFMA_LDS_ENTRY(7, 8, 4, 2, true, true),
    // few rows per workgroup: enough workgroups for one rank's narrow share of N
    MFMA_LDS_ENTRY(7, 4, 1, 1, true, true),
    MFMA_LDS_ENTRY(7, 8, 1, 1, true, true),
};

}  // namespace

const KernelEntry *mfma_lds_entries(int *count) {
    *count = (int)(sizeof(kMfmaLdsEntries) / sizeof(kMfmaLdsEntries[0]));
    return kMfmaLdsEntries;
}

}  // namespace skinny
