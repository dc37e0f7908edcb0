// mfma_ring.hip -- matrix-core K-loop GEMM with operand tiles loaded from memory straight
// into a ring of narrow LDS stages, for tens to hundreds of rows of X.
//
// Operation: vLLM benchmark page "benchmarks/kernels/benchmark_k3_cutedsl_residual.py"
// (module docstring; torch.addmm leg): Y = bf16(X W^T + R), fp32 accumulation.
//
// Same operand pipeline as the direct-to-LDS GEMM (mfma_dma.hip), generalised where that one
// is fixed, so that more bytes can be in flight per compute unit for the same LDS:
//   * stages are KC = 64 or 128 bf16 of K (128- or 256-byte rows): with 64-wide stages the
//     ring holds twice as many stages, so the loads of more stages overlap the long HBM
//     latency of W;
//   * a workgroup is NW = 4 or 8 waves laid out WK x WN x WM: WK waves take alternate 32-wide
//     K steps of each stage (their blocks are added in wave order at the end), WN x WM split
//     the BN x BM block of Y^T; with 8 waves two waves share each SIMD, so one wave's LDS
//     reads overlap the other's matrix instructions;
//   * each stage is (BN + BM) rows in LDS, filled by direct-to-LDS loads (16 bytes per lane,
//     1 KB per instruction), W rows non-temporal, X rows with the default policy;
//   * 16-byte chunks are XOR-swizzled so the 16-row fragment reads of v_mfma_f32_16x16x32_bf16
//     hit 16 distinct bank groups: chunk c of row r at c ^ (r & 15) for 256-byte rows (and the
//     512-byte rows of the wave-specialised form), c ^ ((r >> 1) & 7) for 128-byte rows (rows r
//     and r + 1 share a 256-byte bank window);
//   * each wave waits for its own loads of a stage with an explicit vmcnt, then one barrier
//     publishes the stage and frees the slot read one iteration earlier, which is refilled;
//   * R is fetched into registers before the K loop; the epilogue stages the block in LDS,
//     adds the K-step groups in wave order and R in fp32, rounds once to bf16 and writes Y
//     row-contiguously;
//   * blocks are ordered so that each XCD takes a contiguous run of n-tiles and the m-tiles
//     sharing one W tile run consecutively on it.
// A second kernel below runs the same ring with the waves split into loaders and compute waves.
// K must be a multiple of KC.
#include "common.hpp"

namespace skinny {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// s_waitcnt immediate: at most n vector-memory operations outstanding (gfx9 encoding: vmcnt
// bits 3:0 and 15:14; expcnt and lgkmcnt at their maxima, i.e. not waited for).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until at most `later` stages of PW loads each are outstanding (later is uniform).
template <int PW, int MAXL>
__device__ __forceinline__ void wait_stages(int later) {
    if constexpr (MAXL >= 1) {
        if (later >= MAXL) {
            wait_vmcnt<PW * MAXL>();
            return;
        }
        wait_stages<PW, MAXL - 1>(later);
    } else {
        wait_vmcnt<0>();
    }
}

// Barrier ordering the workgroup's LDS accesses without waiting for outstanding
// direct-to-LDS loads (each wave has already waited for the loads it needs).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int RB>
__device__ __forceinline__ int swizzle(int r) {
    return RB >= 256 ? (r & 15) : ((r >> 1) & 7);
}

// BN, BM: rows of W and of X per block; KC: K per stage; NS: ring stages; NW waves laid out
// WK x WN x WM.
template <int BN, int BM, int KC, int NS, int NW, int WK, int WN, int WM, bool ACC, bool GEN>
__global__ __launch_bounds__(NW * 64) void mfma_ring_kernel(const uint16_t *__restrict__ X,
                                                            const uint16_t *__restrict__ W,
                                                            const uint16_t *R, void *out, int M, int N, int K,
                                                            int n_tiles, int m_tiles, Epilogue ep) {
    static_assert(WK * WN * WM == NW && (NW == 4 || NW == 8), "wave layout");
    static_assert(KC == 64 || KC == 128, "stage width");
    static_assert((KC / 32) % WK == 0, "K steps per stage must split evenly over the K waves");
    const Epilogue epi = GEN ? ep : Epilogue{N, N, 0u};  // see plain_epilogue
    constexpr int NT = NW * 64;
    constexpr int RB = KC * 2;                       // bytes per staged row
    constexpr int CPR = RB / 16;                     // 16-byte chunks per row
    constexpr int RPL = 1024 / RB;                   // rows per 1 KB load block
    constexpr int STAGE_BYTES = (BN + BM) * RB;
    constexpr int BLOCKS = STAGE_BYTES / 1024;
    static_assert(BLOCKS % NW == 0, "stage blocks must split evenly over the waves");
    constexpr int PW = BLOCKS / NW;                  // load instructions per wave per stage
    static_assert(BN % (NW * RPL) == 0, "each load instruction is all W rows or all X rows");
    constexpr int WLOADS = BN / (NW * RPL);          // loads per wave per stage that carry W rows
    constexpr int WNB = BN / WN, WMB = BM / WM;      // wave block
    constexpr int TN = WNB / 16, TM = WMB / 16;
    static_assert(TN >= 1 && TM >= 1 && WNB % 16 == 0 && WMB % 16 == 0, "wave block of whole tiles");
    constexpr int KSTEPS = KC / 32 / WK;             // 32-wide K steps per wave per stage
    constexpr int CP = BM + 4;                       // row pitch (floats) of the fp32 block in LDS
    constexpr int CB = BN * CP;                      // floats per block copy
    constexpr int CBYTES = WK * CB * 4;
    constexpr int LDS_BYTES = NS * STAGE_BYTES > CBYTES ? NS * STAGE_BYTES : CBYTES;
    constexpr int EPT = BN * BM / NT;                // outputs finished per thread
    static_assert(EPT * NT == BN * BM, "epilogue split");
    static_assert(PW * (NS - 2) < 64 && NS >= 2, "vmcnt budget");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];

    // block order: block b runs on XCD b % 8; each XCD takes a contiguous run of n-tiles, and
    // its consecutive blocks take the m-tiles of one n-tile. Neighbouring n-tiles then share
    // their XCD's L2, so the 128-byte lines of R and Y that two blocks split (blocks of 32 or 28
    // columns) are fetched once and written back whole (M = 16 9.73 -> 9.49 us, 64 14.13 ->
    // 13.81 against n-tiles dealt round-robin over the XCDs)
    const int b = blockIdx.x;
    const int xcd = b & 7, j = b >> 3;
    const int mt = j % m_tiles;
    const int nt = xcd * ((n_tiles + 7) / 8) + j / m_tiles;
    if (nt >= n_tiles) return;                       // padding block (uniform)
    const int n0 = nt * BN, m0 = mt * BM;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wk = wave % WK, wn = ((wave / WK) % WN) * WNB, wm = (wave / (WK * WN)) * WMB;
    const int S = K / KC;                            // stages

    // load i of every wave covers load blocks NW*i + wave; lane l fills position l of its block:
    // row RPL*q + l/CPR, stored chunk l%CPR, holding logical chunk (l%CPR) ^ swizzle(row).
    // Rows past N or M re-read the last valid row (their outputs are never written).
    const uint16_t *src[PW];
#pragma unroll
    for (int i = 0; i < PW; ++i) {
        const int q = NW * i + wave;
        const int sr = RPL * q + lane / CPR;
        const int c = (lane % CPR) ^ swizzle<RB>(sr);
        const uint16_t *row = sr < BN ? W + (size_t)min(n0 + sr, N - 1) * K
                                      : X + (size_t)min(m0 + sr - BN, M - 1) * K;
        src[i] = row + 8 * c;
    }
    auto issue = [&](int s) {                        // stage s -> ring slot s % NS
        lds_u8 *st = (lds_u8 *)(lds + (s % NS) * STAGE_BYTES + wave * 1024);
#pragma unroll
        for (int i = 0; i < WLOADS; ++i)
            __builtin_amdgcn_global_load_lds((const void *)(src[i] + (size_t)s * KC),
                                             (lds_void *)(st + i * NW * 1024), 16, 0, 2);
#pragma unroll
        for (int i = WLOADS; i < PW; ++i)
            __builtin_amdgcn_global_load_lds((const void *)(src[i] + (size_t)s * KC),
                                             (lds_void *)(st + i * NW * 1024), 16, 0, 0);
    };

    // residual prefetch: thread t finishes elements e = t + NT i of the block, walked row by row
    // of Y (ml = e / BN, nl = e % BN); clamped addresses, so the loads are unconditional and
    // their latency hides behind the K loop (they are the oldest loads, so every wait below
    // also covers them)
    uint16_t rv[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int e = tid + NT * i;
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

    // fragment reads: row r (16-row group + lane%16), logical chunk 4*kk + lane/16
    const int frow = lane & 15, fq = lane >> 4;
    for (int s = 0; s < S; ++s) {
        wait_stages<PW, NS - 2>(min(NS - 2, S - 1 - s));
        lds_barrier();                               // stage s visible; slot (s-1)%NS free
        if (s + NS - 1 < S) issue(s + NS - 1);
        const uint8_t *Ws = lds + (s % NS) * STAGE_BYTES;
        const uint8_t *Xs = Ws + BN * RB;
#pragma unroll
        for (int u = 0; u < KSTEPS; ++u) {
            const int kk = u * WK + wk;              // this wave's K step of the stage
            u32x4_t af[TN], bfr[TM];
#pragma unroll
            for (int a = 0; a < TN; ++a) {
                const int r = wn + 16 * a + frow;
                af[a] = *reinterpret_cast<const u32x4_t *>(Ws + r * RB + (((4 * kk + fq) ^ swizzle<RB>(r)) << 4));
            }
#pragma unroll
            for (int c = 0; c < TM; ++c) {
                const int r = wm + 16 * c + frow;
                bfr[c] = *reinterpret_cast<const u32x4_t *>(Xs + r * RB + (((4 * kk + fq) ^ swizzle<RB>(r)) << 4));
            }
#pragma unroll
            for (int a = 0; a < TN; ++a)
#pragma unroll
                for (int c = 0; c < TM; ++c) acc[a][c] = mfma16(af[a], bfr[c], acc[a][c]);
        }
    }

    // acc[a][c][r] = partial Y^T[n0 + wn + 16a + 4*(lane/16) + r][m0 + wm + 16c + lane%16]
    __syncthreads();                                 // every wave is done with the ring
    float *C = reinterpret_cast<float *>(lds);       // C[wk][n][m], row pitch CP
    float *Cw = C + wk * CB;
#pragma unroll
    for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int c = 0; c < TM; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Cw[(wn + 16 * a + 4 * (lane >> 4) + r) * CP + wm + 16 * c + (lane & 15)] = acc[a][c][r];
    __syncthreads();
    // neighbouring threads take neighbouring n of one row of Y; K-step groups in wave order
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int e = tid + NT * i;
        const int ml = e / BN, nl = e % BN;
        const int m = m0 + ml, n = n0 + nl;
        if (m < M && n < N) {
            float t = C[nl * CP + ml];
#pragma unroll
            for (int q = 1; q < WK; ++q) t += C[q * CB + nl * CP + ml];
            store_output<ACC>(out, epi, m, n, t, bf16_bits_to_f32(rv[i]));
        }
    }
}

template <int BN, int BM, int KC, int NS, int NW, int WK, int WN, int WM>
hipError_t launch_ring(const LaunchArgs &a) {
    const int n_tiles = (int)((a.N + BN - 1) / BN);
    const int m_tiles = (int)((a.M + BM - 1) / BM);
    const int groups = (n_tiles + 7) / 8;            // n-tiles per XCD, rounded up
    dim3 grid((unsigned)(groups * 8 * m_tiles));
    dim3 block(NW * 64);
#define RING_ARGS a.X, a.W, a.R, a.out, (int)a.M, (int)a.N, (int)a.K, n_tiles, m_tiles, a.ep
    if (a.acc_out)
        hipLaunchKernelGGL((mfma_ring_kernel<BN, BM, KC, NS, NW, WK, WN, WM, true, true>), grid, block, 0, a.stream,
                           RING_ARGS);
    else if (plain_epilogue(a))
        hipLaunchKernelGGL((mfma_ring_kernel<BN, BM, KC, NS, NW, WK, WN, WM, false, false>), grid, block, 0,
                           a.stream, RING_ARGS);
    else
        hipLaunchKernelGGL((mfma_ring_kernel<BN, BM, KC, NS, NW, WK, WN, WM, false, true>), grid, block, 0, a.stream,
                           RING_ARGS);
#undef RING_ARGS
    return hipGetLastError();
}

// Wave-specialised form (path SKINNY_PATH_GEMM_WS): the same ring, blocks, swizzle and
// epilogue, but each wave of a workgroup has one role. NL loader waves only issue the
// direct-to-LDS loads: each waits for its own loads of a stage, meets the stage barrier and
// refills the slot that barrier freed. NC = WK x WN x WM compute waves only read fragments and
// run the matrix instructions. In the form above every wave issues its share of the next stage
// and then stalls until the memory pipeline takes it (a third of a stage's time at M = 256),
// with its matrix work queued behind the stall; here the stalls fall on waves that have nothing
// else to do, while the compute waves on the same SIMDs keep the matrix cores busy.
// SPLIT: the first NL / 2 loaders take a stage's W rows and the others its X rows, so no
// wave's in-order load completions mix HBM and L2 latencies; otherwise loader lw takes the
// stage's load blocks NL*i + lw.
//
// One loader's part of the ring: PW load blocks (1 KB) per stage, block q = first + step*i
// holding rows RPL*q ... of the stage (its BNV W rows first, then its BM X rows); the first NWI
// of them are W rows and carry the non-temporal policy. Lane l fills position l of a block, as
// in the kernel above.
template <int BNV, int BM, int KC, int NS, int PW, int NWI>
__device__ __forceinline__ void ring_loader(const uint16_t *X, const uint16_t *W, int M, int N, int K, int n0,
                                            int m0, int lane, int first, int step, uint8_t *lds, int S) {
    constexpr int RB = KC * 2, CPR = RB / 16, RPL = 1024 / RB;
    constexpr int STAGE_BYTES = (BNV + BM) * RB;
    const uint16_t *src[PW];
    int dst[PW];
#pragma unroll
    for (int i = 0; i < PW; ++i) {
        const int q = first + step * i;
        const int sr = RPL * q + lane / CPR;         // row of the stage
        const int orow = sr < BNV ? sr : sr - BNV;   // row of its operand (the swizzle's row)
        const int c = (lane % CPR) ^ swizzle<RB>(orow);
        const uint16_t *row = sr < BNV ? W + (size_t)min(n0 + sr, N - 1) * K
                                       : X + (size_t)min(m0 + orow, M - 1) * K;
        src[i] = row + 8 * c;
        dst[i] = q * 1024;
    }
    auto issue = [&](int s) {                        // stage s -> ring slot s % NS
        lds_u8 *st = (lds_u8 *)(lds + (s % NS) * STAGE_BYTES);
#pragma unroll
        for (int i = 0; i < PW; ++i) {
            if (i < NWI)
                __builtin_amdgcn_global_load_lds((const void *)(src[i] + (size_t)s * KC), (lds_void *)(st + dst[i]),
                                                 16, 0, 2);
            else
                __builtin_amdgcn_global_load_lds((const void *)(src[i] + (size_t)s * KC), (lds_void *)(st + dst[i]),
                                                 16, 0, 0);
        }
    };
#pragma unroll
    for (int p = 0; p < NS - 1; ++p)
        if (p < S) issue(p);
    for (int s = 0; s < S; ++s) {
        wait_stages<PW, NS - 2>(min(NS - 2, S - 1 - s));
        lds_barrier();                               // stage s visible; slot (s-1)%NS free
        if (s + NS - 1 < S) issue(s + NS - 1);
    }
}

// The loaders of one role (W rows or X rows of a stage, SPLIT form): `blocks` load blocks from
// block `base` on, dealt round-robin over `count` loaders; when they do not split evenly the
// first blocks % count loaders take one more. Each loader's count is a compile-time constant,
// so its vmcnt waits count exactly its own loads.
template <int BNV, int BM, int KC, int NS, int BLOCKS, int COUNT, bool WROWS>
__device__ __forceinline__ void ring_loader_role(const uint16_t *X, const uint16_t *W, int M, int N, int K, int n0,
                                                 int m0, int lane, int idx, int base, uint8_t *lds, int S) {
    constexpr int PH = (BLOCKS + COUNT - 1) / COUNT, REM = BLOCKS % COUNT;
    static_assert(BLOCKS >= COUNT, "every loader of the role has a block");
    if (REM == 0 || idx < REM)
        ring_loader<BNV, BM, KC, NS, PH, WROWS ? PH : 0>(X, W, M, N, K, n0, m0, lane, base + idx, COUNT, lds, S);
    else
        ring_loader<BNV, BM, KC, NS, PH - 1, WROWS ? PH - 1 : 0>(X, W, M, N, K, n0, m0, lane, base + idx, COUNT,
                                                                 lds, S);
}

// Mixed form with load blocks that do not split evenly: loader w takes blocks w, w + NL, ...
// of the stage (W blocks first), so its load count and how many of them are W rows are
// compile-time constants of w; one instance per loader.
template <int BNV, int BM, int KC, int NS, int NL, int WBLK, int BLOCKS, int LW>
__device__ __forceinline__ void ring_loader_mixed(const uint16_t *X, const uint16_t *W, int M, int N, int K, int n0,
                                                  int m0, int lane, int wave, uint8_t *lds, int S) {
    if constexpr (LW < NL) {
        if (wave == LW) {
            constexpr int PW = (BLOCKS - LW + NL - 1) / NL;
            constexpr int NWI = WBLK > LW ? (WBLK - LW + NL - 1) / NL : 0;
            static_assert(PW >= 1, "every loader has a block");
            ring_loader<BNV, BM, KC, NS, PW, NWI>(X, W, M, N, K, n0, m0, lane, LW, NL, lds, S);
        } else {
            ring_loader_mixed<BNV, BM, KC, NS, NL, WBLK, BLOCKS, LW + 1>(X, W, M, N, K, n0, m0, lane, wave, lds, S);
        }
    }
}

// BN: W rows of the matrix-instruction block; BNV <= BN of them are a block's own (loaded,
// finished and stored): with BNV = 7/8 BN, N = 7168 splits into 256 blocks of 28 or 128 of 56
// W rows, one or two per compute unit, instead of 224 or 112. Fragment reads of the rows past
// BNV land on X rows of the same stage; their results are never stored.
template <int BN, int BNV, int BM, int KC, int NS, int NL, int WK, int WN, int WM, bool SPLIT, bool ACC, bool GEN>
__global__ __launch_bounds__((NL + WK * WN * WM) * 64) void mfma_ring_ws_kernel(
    const uint16_t *__restrict__ X, const uint16_t *__restrict__ W, const uint16_t *R, void *out, int M, int N, int K,
    int n_tiles, int m_tiles, Epilogue ep) {
    constexpr int NC = WK * WN * WM;
    constexpr int NW = NL + NC;
    static_assert(NW <= 16 && NL >= 1 && (!SPLIT || NL % 2 == 0), "wave layout");
    static_assert(BNV <= BN && BN - BNV <= BM, "fragment reads stay inside the stage");
    static_assert(KC == 64 || KC == 128 || KC == 256, "stage width");
    static_assert((KC / 32) % WK == 0, "K steps per stage must split evenly over the K waves");
    const Epilogue epi = GEN ? ep : Epilogue{N, N, 0u};  // see plain_epilogue
    constexpr int NT = NW * 64;
    constexpr int RB = KC * 2;
    constexpr int RPL = 1024 / RB;
    constexpr int STAGE_BYTES = (BNV + BM) * RB;
    constexpr int WBLK = BNV / RPL, XBLK = BM / RPL, BLOCKS = WBLK + XBLK;
    static_assert(BNV % RPL == 0 && BM % RPL == 0, "whole load blocks");
    constexpr int NLW = SPLIT ? NL / 2 : NL;         // loaders that carry W rows
    constexpr bool EVEN = WBLK % NL == 0 && XBLK % NL == 0;  // mixed form: every loader alike
    // most loads per stage of a W (or any) loader and of an X loader (one fewer for the last
    // loaders of a role, or of the mixed form, when the blocks do not split evenly)
    constexpr int PWW = SPLIT ? (WBLK + NLW - 1) / NLW : (BLOCKS + NL - 1) / NL;
    constexpr int PWX = SPLIT ? (XBLK + NL - NLW - 1) / (NL - NLW) : PWW;
    static_assert(PWW * (NS - 2) < 64 && PWX * (NS - 2) < 64 && NS >= 2, "vmcnt budget");
    constexpr int WNB = BN / WN, WMB = BM / WM;      // compute wave block
    constexpr int TN = WNB / 16, TM = WMB / 16;
    static_assert(TN >= 1 && TM >= 1 && WNB % 16 == 0 && WMB % 16 == 0, "wave block of whole tiles");
    constexpr int KSTEPS = KC / 32 / WK;
    constexpr int CP = BM + 4;
    constexpr int CB = BN * CP;
    constexpr int CBYTES = WK * CB * 4;
    // where the ring and the partial blocks fit side by side, the blocks get LDS of their own, and
    // no barrier has to separate the last fragment reads from their writes (0.1 us at M >= 32)
    constexpr bool CSEP = NS * STAGE_BYTES + CBYTES <= 160 * 1024;
    constexpr int LDS_BYTES = CSEP ? NS * STAGE_BYTES + CBYTES : (NS * STAGE_BYTES > CBYTES ? NS * STAGE_BYTES : CBYTES);
    constexpr int OUTS = BNV * BM;                  // outputs of a block
    constexpr int EPT = (OUTS + NT - 1) / NT;        // finished per thread (the last round ragged)
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];

    // block order as in the kernel above
    const int b = blockIdx.x;
    const int xcd = b & 7, j = b >> 3;
    const int mt = j % m_tiles;
    const int nt = xcd * ((n_tiles + 7) / 8) + j / m_tiles;
    if (nt >= n_tiles) return;                       // padding block (uniform)
    const int n0 = nt * BNV, m0 = mt * BM;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // a scalar role branch
    const int S = K / KC;

    uint16_t rv[EPT];                                // residual prefetch, as above
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int e = tid + NT * i;
        rv[i] = R[(size_t)min(m0 + e / BNV, M - 1) * epi.ldr + min(n0 + e % BNV, N - 1)];
    }

    // Every wave meets the same barriers: one per stage, one when the ring is done (unless the
    // partial blocks have LDS of their own), one when the partial blocks are in LDS.
    float *C = reinterpret_cast<float *>(lds + (CSEP ? NS * STAGE_BYTES : 0));  // C[wk][n][m], row pitch CP
    if (wave < NL) {
        if constexpr (SPLIT) {
            if (wave < NLW)
                ring_loader_role<BNV, BM, KC, NS, WBLK, NLW, true>(X, W, M, N, K, n0, m0, lane, wave, 0, lds, S);
            else
                ring_loader_role<BNV, BM, KC, NS, XBLK, NL - NLW, false>(X, W, M, N, K, n0, m0, lane, wave - NLW,
                                                                         WBLK, lds, S);
        } else if constexpr (EVEN) {
            ring_loader<BNV, BM, KC, NS, PWW, WBLK / NL>(X, W, M, N, K, n0, m0, lane, wave, NL, lds, S);
        } else {
            ring_loader_mixed<BNV, BM, KC, NS, NL, WBLK, BLOCKS, 0>(X, W, M, N, K, n0, m0, lane, wave, lds, S);
        }
        if (!CSEP) __syncthreads();                  // (its waits cover every load of the ring)
    } else {
        const int cw = wave - NL;
        const int wk = cw % WK, wn = ((cw / WK) % WN) * WNB, wm = (cw / (WK * WN)) * WMB;
        f32x4_t acc[TN][TM];
#pragma unroll
        for (int a = 0; a < TN; ++a)
#pragma unroll
            for (int c = 0; c < TM; ++c) acc[a][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        const int frow = lane & 15, fq = lane >> 4;
        for (int s = 0; s < S; ++s) {
            // the fragment reads of the previous stage have returned (lgkmcnt 0) before the
            // barrier that lets the loaders refill their slot
            __builtin_amdgcn_s_waitcnt(0xC07F);
            lds_barrier();
            const uint8_t *Ws = lds + (s % NS) * STAGE_BYTES;
            const uint8_t *Xs = Ws + BNV * RB;
#pragma unroll
            for (int u = 0; u < KSTEPS; ++u) {
                const int kk = u * WK + wk;
                u32x4_t af[TN], bfr[TM];
#pragma unroll
                for (int a = 0; a < TN; ++a) {
                    const int r = wn + 16 * a + frow;
                    af[a] = *reinterpret_cast<const u32x4_t *>(Ws + r * RB + (((4 * kk + fq) ^ swizzle<RB>(r)) << 4));
                }
#pragma unroll
                for (int c = 0; c < TM; ++c) {
                    const int r = wm + 16 * c + frow;
                    bfr[c] = *reinterpret_cast<const u32x4_t *>(Xs + r * RB + (((4 * kk + fq) ^ swizzle<RB>(r)) << 4));
                }
#pragma unroll
                for (int a = 0; a < TN; ++a)
#pragma unroll
                    for (int c = 0; c < TM; ++c) acc[a][c] = mfma16(af[a], bfr[c], acc[a][c]);
            }
        }
        if (!CSEP) __syncthreads();                  // every wave is done with the ring
        float *Cw = C + wk * CB;
#pragma unroll
        for (int a = 0; a < TN; ++a)
#pragma unroll
            for (int c = 0; c < TM; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Cw[(wn + 16 * a + 4 * (lane >> 4) + r) * CP + wm + 16 * c + (lane & 15)] = acc[a][c][r];
    }
    __syncthreads();
    // all waves finish the block: neighbouring threads take neighbouring n of one row of Y
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int e = tid + NT * i;
        const int ml = e / BNV, nl = e % BNV;
        const int m = m0 + ml, n = n0 + nl;
        if ((OUTS % NT == 0 || e < OUTS) && m < M && n < N) {
            float t = C[nl * CP + ml];
#pragma unroll
            for (int q = 1; q < WK; ++q) t += C[q * CB + nl * CP + ml];
            store_output<ACC>(out, epi, m, n, t, bf16_bits_to_f32(rv[i]));
        }
    }
}

template <int BN, int BNV, int BM, int KC, int NS, int NL, int WK, int WN, int WM, bool SPLIT>
hipError_t launch_ring_ws(const LaunchArgs &a) {
    const int n_tiles = (int)((a.N + BNV - 1) / BNV);
    const int m_tiles = (int)((a.M + BM - 1) / BM);
    const int groups = (n_tiles + 7) / 8;            // n-tiles per XCD, rounded up
    dim3 grid((unsigned)(groups * 8 * m_tiles));
    dim3 block((NL + WK * WN * WM) * 64);
#define RING_ARGS a.X, a.W, a.R, a.out, (int)a.M, (int)a.N, (int)a.K, n_tiles, m_tiles, a.ep
    if (a.acc_out)
        hipLaunchKernelGGL((mfma_ring_ws_kernel<BN, BNV, BM, KC, NS, NL, WK, WN, WM, SPLIT, true, true>), grid, block, 0,
                           a.stream, RING_ARGS);
    else if (plain_epilogue(a))
        hipLaunchKernelGGL((mfma_ring_ws_kernel<BN, BNV, BM, KC, NS, NL, WK, WN, WM, SPLIT, false, false>), grid, block, 0,
                           a.stream, RING_ARGS);
    else
        hipLaunchKernelGGL((mfma_ring_ws_kernel<BN, BNV, BM, KC, NS, NL, WK, WN, WM, SPLIT, false, true>), grid, block, 0,
                           a.stream, RING_ARGS);
#undef RING_ARGS
    return hipGetLastError();
}

int64_t ring_max_k() { return INT64_MAX; }

// Public knobs: path SKINNY_PATH_GEMM_RING, block_size = 64 * NW, outputs_per_block = BN,
// k_unroll = NS (ring stages), vector_width = 8, m_tile = BM, k_split = WK (waves taking
// alternate K steps of a stage; the other waves split the block, along W rows first:
// WN = 2 whenever NW / WK >= 2), k_stage = KC. K must be a multiple of KC.
#define RING_ENTRY(BN, BM, KC, NS, NW, WK, WN, WM)                                                    \
    KernelEntry {                                                                                     \
        skinny_config{SKINNY_PATH_GEMM_RING, 64 * NW, BN, NS, 8, BM, WK, KC},                         \
            &launch_ring<BN, BM, KC, NS, NW, WK, WN, WM>,                                             \
            (const void *)&mfma_ring_kernel<BN, BM, KC, NS, NW, WK, WN, WM, false, false>,            \
            (const void *)&mfma_ring_kernel<BN, BM, KC, NS, NW, WK, WN, WM, true, true>, &ring_max_k, KC \
    }

// Public knobs of the wave-specialised form: path SKINNY_PATH_GEMM_WS, block_size = 512 (4
// loader and 4 compute waves), outputs_per_block = BNV (the W rows a block owns: BN, or 7/8 of
// it, 28 of a 32-row or 56 of a 64-row matrix tile), k_unroll = NS, vector_width = 8 (every
// loader takes W and X rows) or 9 (W rows and X rows on different loaders), m_tile = BM,
// k_split = WK (compute waves taking alternate K steps of a stage; the others split the block,
// two along W rows), k_stage = KC (64, 128 or 256: 128-, 256- or 512-byte row pieces).
#define WS_ENTRY_V(BN, BNV, BM, KC, NS, WK, SPLIT)                                                    \
    KernelEntry {                                                                                     \
        skinny_config{SKINNY_PATH_GEMM_WS, 512, BNV, NS, (SPLIT) ? 9 : 8, BM, WK, KC},                \
            &launch_ring_ws<BN, BNV, BM, KC, NS, 4, WK, 2, 2 / (WK), SPLIT>,                          \
            (const void *)&mfma_ring_ws_kernel<BN, BNV, BM, KC, NS, 4, WK, 2, 2 / (WK), SPLIT, false, false>, \
            (const void *)&mfma_ring_ws_kernel<BN, BNV, BM, KC, NS, 4, WK, 2, 2 / (WK), SPLIT, true, true>,   \
            &ring_max_k, KC                                                                           \
    }
#define WS_ENTRY(BN, BM, KC, NS, WK, SPLIT) WS_ENTRY_V(BN, BN, BM, KC, NS, WK, SPLIT)

const KernelEntry kRingEntries[] = {
    // 32 W rows per block (224 workgroups at N = 7168)
    RING_ENTRY(32, 32, 64, 8, 4, 2, 1, 2),
    RING_ENTRY(32, 64, 64, 6, 4, 2, 1, 2),
    RING_ENTRY(32, 64, 64, 8, 4, 2, 1, 2),
    RING_ENTRY(32, 64, 128, 4, 4, 4, 1, 1),
    RING_ENTRY(32, 64, 128, 5, 4, 4, 1, 1),
    RING_ENTRY(32, 128, 64, 6, 4, 1, 2, 2),
    // 64 W rows per block
    RING_ENTRY(64, 64, 64, 6, 4, 2, 2, 1),
    RING_ENTRY(64, 64, 64, 8, 8, 2, 2, 2),
    RING_ENTRY(64, 64, 64, 6, 8, 2, 2, 2),
    RING_ENTRY(64, 128, 64, 4, 4, 1, 2, 2),
    RING_ENTRY(64, 128, 64, 6, 4, 1, 2, 2),
    RING_ENTRY(64, 128, 64, 4, 8, 2, 2, 2),
    RING_ENTRY(64, 128, 64, 6, 8, 2, 2, 2),
    RING_ENTRY(64, 256, 64, 3, 8, 2, 2, 2),
    // 128 W rows per block (112 workgroups)
    RING_ENTRY(128, 128, 64, 4, 8, 2, 2, 2),
    // eight waves on 32- and 64-row W tiles
    RING_ENTRY(32, 32, 128, 4, 8, 4, 1, 2),
    RING_ENTRY(32, 64, 128, 4, 8, 4, 1, 2),
    RING_ENTRY(32, 96, 128, 4, 8, 4, 1, 2),
    RING_ENTRY(64, 64, 128, 4, 8, 4, 2, 1),
    RING_ENTRY(64, 96, 128, 3, 8, 4, 2, 1),
    RING_ENTRY(64, 128, 128, 3, 8, 4, 2, 1),
    RING_ENTRY(64, 128, 64, 5, 8, 1, 2, 4),
    RING_ENTRY(64, 192, 64, 4, 8, 2, 2, 2),
    // wave-specialised form
    WS_ENTRY(32, 16, 128, 6, 2, false),
    WS_ENTRY(32, 32, 128, 4, 1, false),
    WS_ENTRY(32, 32, 128, 5, 2, false),
    WS_ENTRY(32, 48, 128, 4, 2, false),
    WS_ENTRY(32, 48, 256, 3, 2, false),
    WS_ENTRY(32, 64, 128, 4, 1, false),
    WS_ENTRY(32, 64, 128, 4, 1, true),
    WS_ENTRY(32, 64, 128, 5, 1, false),
    WS_ENTRY(32, 64, 256, 3, 1, false),
    WS_ENTRY(32, 80, 128, 4, 2, false),
    WS_ENTRY(32, 80, 128, 4, 2, true),
    WS_ENTRY(32, 96, 128, 4, 1, true),
    WS_ENTRY(64, 64, 128, 4, 1, false),
    WS_ENTRY(64, 64, 128, 4, 1, true),
    WS_ENTRY(64, 64, 128, 5, 1, true),
    WS_ENTRY(64, 64, 128, 4, 2, true),
    WS_ENTRY(64, 96, 128, 3, 1, false),
    WS_ENTRY(64, 96, 128, 3, 1, true),
    WS_ENTRY(64, 128, 128, 3, 1, false),
    WS_ENTRY(64, 128, 128, 3, 1, true),
    WS_ENTRY(64, 128, 128, 3, 2, false),
    // 7/8 of the matrix block's W rows per block: 256 (28 rows) or 128 (56 rows) blocks at N = 7168
    WS_ENTRY_V(32, 28, 16, 128, 6, 2, true),
    WS_ENTRY_V(32, 28, 16, 256, 4, 2, true),
    WS_ENTRY_V(32, 28, 32, 128, 5, 2, true),
    WS_ENTRY_V(32, 28, 32, 256, 4, 2, true),
    WS_ENTRY_V(32, 28, 48, 128, 4, 2, true),
    WS_ENTRY_V(32, 28, 64, 256, 3, 1, true),
    WS_ENTRY_V(32, 28, 80, 128, 4, 2, true),
    WS_ENTRY_V(64, 56, 64, 128, 4, 1, true),
    WS_ENTRY_V(64, 56, 96, 128, 3, 1, true),
    WS_ENTRY_V(64, 56, 128, 128, 3, 1, true),
    WS_ENTRY_V(32, 28, 16, 128, 6, 2, false),
    WS_ENTRY_V(32, 28, 32, 128, 5, 2, false),
    WS_ENTRY_V(32, 28, 48, 128, 4, 2, false),
    WS_ENTRY_V(32, 28, 80, 128, 4, 2, false),
    WS_ENTRY_V(64, 56, 64, 128, 4, 1, false),
    WS_ENTRY_V(64, 56, 128, 128, 3, 1, false),
    WS_ENTRY_V(32, 28, 64, 128, 4, 1, false),
    WS_ENTRY_V(32, 28, 64, 128, 4, 2, false),
    WS_ENTRY_V(32, 28, 64, 256, 3, 1, false),
    WS_ENTRY_V(64, 56, 80, 128, 4, 2, true),
    WS_ENTRY_V(64, 56, 80, 128, 4, 2, false),
    WS_ENTRY_V(32, 28, 96, 128, 4, 2, false),
};

}  // namespace

const KernelEntry *ring_entries(int *count) {
    *count = (int)(sizeof(kRingEntries) / sizeof(kRingEntries[0]));
    return kRingEntries;
}

}  // namespace skinny
