// kbit_gemv.hip -- decode GEMV with k-bit quantized weights (k = 2..5), Y = bf16(X What^T + R).
//
// Format (the bitsandbytes page "compare/main...QLORA-2.diff", agents/kbit_gemm_context.md,
// sections 1.3-1.6): W is stored in blocks of 32 consecutive elements of a row; a block has
// k bit-plane words (bit j of word b = bit b of element j's codebook index) and one E4M4
// absmax byte (4-bit exponent with bias 11, 4-bit mantissa); the dequantized weight is
// codebook[index] * decode(absmax). The GEMV is that page's decode kernel ("Kernel 1: Scalar
// GEMV" of its QLoRA guide, section 7), here with this library's bf16 X, R and Y.
//
// Design for gfx950:
//   * a workgroup is 4 waves; a wave takes 4 rows of W at a time, 16 lanes per row, and
//     lane s of a row group walks the row's blocks s, s + 16, ...; so each lane stays on one
//     row, the 16 lanes of a group read 16 neighbouring blocks (contiguous plane words), and
//     the row's partial sums meet in a 16-lane DPP reduction;
//   * X (M <= MT rows) is copied to LDS once per workgroup with a 16-byte pad after every
//     32-element block, so the 16 lanes of a group (64-byte stride) read distinct banks;
//   * the codebook (2^k fp32 entries) sits in LDS: one ds_read_b32 per element, conflict-free
//     because the whole table spans fewer than 64 banks;
//   * per block: the k plane words and the scale byte are loaded together for U blocks
//     ahead; an element's index is assembled from bit j of each plane; the 32 products of a
//     block are summed in fp32 and scaled once by the decoded absmax;
//   * R is prefetched by the lanes that write; one RNE rounding to bf16 at the end.
#include "common.hpp"

namespace skinny {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kPadBlockBytes = 80;   // 64 bytes of a 32-element bf16 block + 16 bytes of padding
constexpr int kUnroll = 4;           // blocks in flight per lane

// E4M4 byte -> fp32 (the page's decoder): e > 0: 2^(e - 11) * (1 + m/16) built as IEEE bits;
// e == 0: m * 2^-14 (zero for m == 0).
__device__ __forceinline__ float e4m4_decode(uint32_t byte) {
    const uint32_t e = byte >> 4, m = byte & 15u;
    const float normal = __uint_as_float(((e + 116u) << 23) | (m << 19));
    const float sub = (float)m * 6.103515625e-05f;   // 2^-14
    return e ? normal : sub;
}

// MT: rows of X per pass; KB: bits per index.
template <int KB, int MT, bool ACC>
__global__ __launch_bounds__(256) void kbit_gemv_kernel(const uint16_t *__restrict__ X,
                                                        const uint32_t *__restrict__ planes,
                                                        const uint8_t *__restrict__ absmax,
                                                        const float *__restrict__ codebook,
                                                        const uint16_t *R, void *out, int M, int N, int K,
                                                        Epilogue ep) {
    constexpr int L = 1 << KB;
    extern __shared__ __attribute__((aligned(16))) uint8_t xs[];   // [MT][BPR] padded blocks
    __shared__ float cbs[L];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int BPR = K >> 5;                                  // blocks per row
    const int m0 = blockIdx.y * MT;
    const int n = blockIdx.x * 16 + wave * 4 + (lane >> 4);  // this lane's row of W
    const int s = lane & 15;                                 // position in the row group
    const int nc = min(n, N - 1);                            // rows past N: computed, not stored

    // residual of the output this lane writes (lanes s = (16/MT)*m of a group write row m)
    constexpr int WSTEP = 16 / MT;
    const int my_m = s / WSTEP;
    const bool writer = (s % WSTEP) == 0;
    const float rres = bf16_bits_to_f32(R[(size_t)min(m0 + my_m, M - 1) * ep.ldr + nc]);

    if (tid < L) cbs[tid] = codebook[tid];
    // X rows m0 .. m0+MT-1 (clamped) into LDS, 16 bytes per thread per step
    const int chunks = MT * BPR * 4;
    for (int c = tid; c < chunks; c += 256) {
        const int m = c / (BPR * 4), r = c % (BPR * 4);
        const u32x4_t v = *reinterpret_cast<const u32x4_t *>(X + (size_t)min(m0 + m, M - 1) * K + r * 8);
        *reinterpret_cast<u32x4_t *>(xs + (m * BPR + (r >> 2)) * kPadBlockBytes + (r & 3) * 16) = v;
    }
    __syncthreads();

    const uint32_t *prow = planes + (size_t)nc * BPR * KB;
    const uint8_t *arow = absmax + (size_t)nc * BPR;
    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.0f;

    // every lane runs the same trip count (blocks past the row are clamped and weighted 0)
    for (int base = 0; base < BPR; base += 16 * kUnroll) {
        const int b0 = base + s;
        uint32_t w[kUnroll][KB];
        uint32_t a[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int b = min(b0 + 16 * u, BPR - 1);         // clamped; masked below
#pragma unroll
            for (int i = 0; i < KB; ++i) w[u][i] = __builtin_nontemporal_load(prow + (size_t)b * KB + i);
            a[u] = arow[b];
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int b = b0 + 16 * u;
            const float scale = b < BPR ? e4m4_decode(a[u]) : 0.0f;   // past the row: adds 0
            const int bx = min(b, BPR - 1);
            float part[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m) part[m] = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {                   // 8 elements per 16-byte chunk of X
                u32x4_t xv[MT];
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    xv[m] = *reinterpret_cast<const u32x4_t *>(xs + (m * BPR + bx) * kPadBlockBytes + q * 16);
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const int j = q * 8 + t;
                    uint32_t idx = 0;
#pragma unroll
                    for (int i = 0; i < KB; ++i) idx |= ((w[u][i] >> j) & 1u) << i;
                    const float c = cbs[idx];
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
                        const uint32_t pair = xv[m][t >> 1];
                        const float x = __uint_as_float((t & 1) ? (pair & 0xFFFF0000u) : (pair << 16));
                        part[m] = fmaf(x, c, part[m]);
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[m] = fmaf(part[m], scale, acc[m]);
        }
    }

    // sum over the 16 lanes of the row group; afterwards lane s holds row m = s / WSTEP in acc[0]
    wave_transpose_reduce<MT, 8>(acc, lane);
    if (writer && n < N && m0 + my_m < M) store_output<ACC>(out, ep, m0 + my_m, n, acc[0], rres);
}

template <int KB, int MT>
hipError_t launch_kbit(const KbitArgs &a) {
    dim3 grid((unsigned)((a.N + 15) / 16), (unsigned)((a.M + MT - 1) / MT));
    const size_t shmem = (size_t)MT * (a.K / 32) * kPadBlockBytes;
    const Epilogue ep{(int)a.N, (int)a.N, 0u};
    if (a.acc_out)
        hipLaunchKernelGGL((kbit_gemv_kernel<KB, MT, true>), grid, dim3(256), shmem, a.stream, a.X, a.planes,
                           a.absmax, a.codebook, a.R, a.out, (int)a.M, (int)a.N, (int)a.K, ep);
    else
        hipLaunchKernelGGL((kbit_gemv_kernel<KB, MT, false>), grid, dim3(256), shmem, a.stream, a.X, a.planes,
                           a.absmax, a.codebook, a.R, a.out, (int)a.M, (int)a.N, (int)a.K, ep);
    return hipGetLastError();
}

template <int KB>
hipError_t launch_kbit_mt(const KbitArgs &a) {
    if (a.M <= 1) return launch_kbit<KB, 1>(a);
    if (a.M <= 2) return launch_kbit<KB, 2>(a);
    return launch_kbit<KB, 4>(a);
}

}  // namespace

int64_t kbit_max_k() {
    // X of 4 rows in padded LDS blocks: 4 * (K / 32) * 80 bytes, kept within 96 KB
    return (int64_t)(96 * 1024 / (4 * kPadBlockBytes)) * 32;
}

hipError_t launch_kbit_gemv(const KbitArgs &a) {
    switch (a.kbits) {
        case 2: return launch_kbit_mt<2>(a);
        case 3: return launch_kbit_mt<3>(a);
        case 4: return launch_kbit_mt<4>(a);
        case 5: return launch_kbit_mt<5>(a);
    }
    return hipErrorInvalidValue;
}

}  // namespace skinny
