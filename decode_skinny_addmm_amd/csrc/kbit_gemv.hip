// kbit_gemv.hip -- decode GEMV with k-bit quantized weights (k = 2..5), Y = bf16(X What^T + R).
//
// Format (the bitsandbytes page "compare/main...QLORA-2.diff", agents/kbit_gemm_context.md,
// sections 1.3-1.6): W is stored in blocks of 32 consecutive elements of a row; a block has
// k bit-plane words (bit j of word i = bit i of element j's codebook index) and one E4M4
// absmax byte (4-bit exponent with bias 11, 4-bit mantissa); the dequantized weight is
// codebook[index] * decode(absmax). The GEMV is that page's decode kernel ("Kernel 1: Scalar
// GEMV" of its QLoRA guide, section 7), here with this library's bf16 X, R and Y.
//
// At M <= 4 the work per weight, not the bytes, sets the time (about 0.5 byte per weight at
// k = 4 against one codebook lookup and one FMA per weight and output row), so the design
// minimises VALU instructions per weight on gfx950:
//   * a lane owns one block position b of the K axis for the whole launch: the 32 X values
//     of that block (per output row) are converted to fp32 once and stay in VGPRs; the
//     workgroup's lanes cover r rows x K/32 blocks, and walk G such row groups;
//   * index decode without per-bit work: each plane word is rotated once so plane i lands on
//     bit i + 2 of a byte; for each c = 0..7 one AND-OR per plane collects elements
//     c, c+8, c+16, c+24 into one word whose bytes are the four indices times 4, i.e. the
//     LDS byte addresses of their codebook entries; one rotation re-aligns the word; one
//     bit-field extract per element feeds a ds_read_b32 (the 2^k-entry fp32 table spans at
//     most 32 banks, so every lookup is conflict-free). For k = 2, 3 and 4 the words instead
//     hold two indices per field, and one ds_read_b64 fetches both codebook values from a
//     table of pairs (block_dot_pair); k = 5 pairs the elements 8 apart, whose indices sit
//     in adjacent bytes of the collected word, in a sparse table (block_dot_pair8);
//   * one fp32 FMA per weight and row; the block's sum is scaled once by its decoded absmax;
//   * per-block partial sums meet in LDS; 16 lanes per output row add them and write
//     bf16(sum + R) with one rounding (R is loaded by the writing lane at kernel start).
#include <algorithm>

#include "common.hpp"

namespace skinny {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxThreads = 512;    // 2 waves per SIMD: up to 256 VGPRs (X of 4 rows takes 128)
constexpr int kMaxRowGroups = 8;        // G: row groups a workgroup walks (plane words kept in flight)
constexpr int kPartialBytes = 64 * 1024;  // LDS budget of the per-block partial sums

// E4M4 byte -> fp32 (the page's decoder): e > 0: 2^(e - 11) * (1 + m/16) built as IEEE bits;
// e == 0: m * 2^-14 (zero for m == 0).
__device__ __forceinline__ float e4m4_decode(uint32_t byte) {
    const uint32_t e = byte >> 4, m = byte & 15u;
    const float normal = __uint_as_float(((e + 116u) << 23) | (m << 19));
    const float sub = (float)m * 6.103515625e-05f;   // 2^-14
    return e ? normal : sub;
}

__device__ __forceinline__ uint32_t rotr(uint32_t v, int s) { return __builtin_amdgcn_alignbit(v, v, s); }

// (a & m) | acc as one VOP3 instruction (left to itself the compiler splits a chain of these
// into ANDs and a three-input OR, one instruction more per word)
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t acc) {
    uint32_t d;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(m), "v"(acc));
    return d;
}

constexpr uint32_t rotl_c(uint32_t v, int s) { return s == 0 ? v : (v << s) | (v >> (32 - s)); }

// Sum over the 16 lanes of a row of the wavefront (DPP row rotations stay within the row).
__device__ __forceinline__ float row16_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));  // ror 8
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));  // ror 4
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xF, 0xF, false));  // ror 2
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xF, 0xF, false));  // ror 1
    return v;
}

// Partial sum of one block for MT rows: decode the 32 indices of the block from its plane
// words and accumulate x * codebook[index] (scaled by the block's absmax at the end).
template <int KB, int MT>
__device__ __forceinline__ void block_dot(const uint32_t (&P)[KB], uint32_t a, const float (&x)[MT][32],
                                          const uint32_t (&msk)[8], const char *cbb, float (&out)[MT]) {
    uint32_t Q[KB];
#pragma unroll
    for (int i = 0; i < KB; ++i) Q[i] = rotr(P[i], 30 - i);   // element j, plane i -> bit j + 2 + i
    float s[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) s[m] = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        // elements c + 8t (t = 0..3): their plane-i bits sit at 8t + 2 + i + c (mod 32)
        // mask of plane i for this c: bit 2 + i of every byte rotated by c, i.e. msk[(c + i) % 8]
        uint32_t w = Q[0] & msk[c];
#pragma unroll
        for (int i = 1; i < KB; ++i) w = and_or(Q[i], msk[(c + i) & 7], w);
        if (c) w = rotr(w, c);                                   // byte t = 4 * index(c + 8t)
        // hide w's known-zero bits so each byte is taken with one bit-field extract
        // instead of a shift and a mask
        asm("" : "+v"(w));
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float cv = *reinterpret_cast<const float *>(cbb + ((w >> (8 * t)) & 0xFFu));
#pragma unroll
            for (int m = 0; m < MT; ++m) s[m] = fmaf(x[m][c + 8 * t], cv, s[m]);
        }
    }
    const float scale = e4m4_decode(a);
#pragma unroll
    for (int m = 0; m < MT; ++m) out[m] = s[m] * scale;
}

// k = 2, 3 and 4: the same partial sum with two indices per lookup. Each index takes an F-bit
// field (F = 2 for k = 2, 4 for k = 3 and 4; at k = 3 the top bit is always clear). Word c'
// (c' in [0, 8) with c' mod 2F < F) of each half of the block collects the elements e, e + F,
// e + 16, e + 16 + F (e = c' in the low half, c' + 8 in the high half; the words cover all 32
// elements): plane i is rotated once per half so that element j's bit lands at j + 3 + i (low)
// or j - 5 + i (high), and one AND-OR per plane with the mask of positions c' + 3 + i + {0, F,
// 16, 16 + F} leaves index(e) + index(e + F) << F at bits c' + 3 ... and index(e + 16) +
// index(e + 16 + F) << F at bits c' + 19 ..., each field 3 + 2F bits long with its low 3 bits
// clear: one bit-field extract gives the byte address of a float2 (codebook[a], codebook[b])
// in a 2^(2F)-entry LDS table. Per 4 weights: k + 2 VALU instructions and two 8-byte lookups
// (the byte form: k + 5 and four). k = 5 takes block_dot_pair8: 5-bit fields at distance 5 do
// not tile a 16-element half.
template <int KB, int MT>
__device__ __forceinline__ void block_dot_pair(const uint32_t (&P)[KB], uint32_t a, const float (&x)[MT][32],
                                               const uint32_t (&pm)[7], const char *pairb, float (&out)[MT]) {
    constexpr int KF = KB == 2 ? 2 : 4;                // field stride: element distance in a pair
    constexpr int FW = 3 + 2 * KF;                     // field width in bits
    uint32_t Qlo[KB], Qhi[KB];
#pragma unroll
    for (int i = 0; i < KB; ++i) {
        Qlo[i] = rotr(P[i], 29 - i);                   // element j -> bit j + 3 + i
        Qhi[i] = rotr(P[i], 5 - i);                    // element j -> bit j - 5 + i (mod 32)
    }
    float s[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) s[m] = 0.0f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int cp = 0; cp < 8; ++cp) {
            if (cp % (2 * KF) >= KF) continue;
            const uint32_t(&Q)[KB] = h ? Qhi : Qlo;
            uint32_t w = Q[0] & pm[cp];
#pragma unroll
            for (int i = 1; i < KB; ++i) w = and_or(Q[i], pm[cp + i], w);
            const uint32_t f0 = __builtin_amdgcn_ubfe(w, cp, FW);
            const uint32_t f1 = __builtin_amdgcn_ubfe(w, cp + 16, FW);
            const float2 v0 = *reinterpret_cast<const float2 *>(pairb + f0);
            const float2 v1 = *reinterpret_cast<const float2 *>(pairb + f1);
            const int e = cp + 8 * h;
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                s[m] = fmaf(x[m][e], v0.x, s[m]);
                s[m] = fmaf(x[m][e + KF], v0.y, s[m]);
                s[m] = fmaf(x[m][e + 16], v1.x, s[m]);
                s[m] = fmaf(x[m][e + 16 + KF], v1.y, s[m]);
            }
        }
    }
    const float scale = e4m4_decode(a);
#pragma unroll
    for (int m = 0; m < MT; ++m) out[m] = s[m] * scale;
}

// k = 3 and 4: the same pairs (e, e + 4) from a transposed block. A 4 x 4 bit-block transpose
// of the plane words (two passes of bit-field swaps between word pairs) leaves in word c, nibble
// g, the index of element 4g + c (bit i from plane i; at k = 3 the fourth plane is zero), so
// byte b of word c is index(8b + c) + 16 index(8b + c + 4): the pair table's entry number as it
// stands. Its byte address is that byte times 8, one instruction (a byte-select shift) per
// lookup. Per 32 weights: 16 instructions for the transpose and 16 for the addresses, against
// 56 in block_dot_pair.
// (zero: a register holding 0 that the compiler cannot see through, the fourth plane at k = 3; a
// literal zero lets it fold the transpose into a longer sequence without byte-select shifts)
template <int KB, int MT>
__device__ __forceinline__ void block_dot_tr(const uint32_t (&P)[KB], uint32_t a, const float (&x)[MT][32],
                                             const char *pairb, uint32_t zero, float (&out)[MT]) {
    static_assert(KB == 3 || KB == 4, "four planes at most");
    auto bfi = [](uint32_t m, uint32_t v, uint32_t w) { return (m & v) | (~m & w); };
    uint32_t w0 = P[0], w1 = P[1], w2 = P[2], w3 = KB == 4 ? P[KB - 1] : zero;
    // first swap: bits 4g + 2, 4g + 3 of words 0, 1 <-> bits 4g, 4g + 1 of words 2, 3
    uint32_t n0 = bfi(0xCCCCCCCCu, w2 << 2, w0), n2 = bfi(0x33333333u, w0 >> 2, w2);
    uint32_t n1 = bfi(0xCCCCCCCCu, w3 << 2, w1), n3 = bfi(0x33333333u, w1 >> 2, w3);
    // second swap: bits 4g + 1, 4g + 3 of words 0, 2 <-> bits 4g, 4g + 2 of words 1, 3
    const uint32_t W[4] = {bfi(0xAAAAAAAAu, n1 << 1, n0), bfi(0x55555555u, n0 >> 1, n1),
                           bfi(0xAAAAAAAAu, n3 << 1, n2), bfi(0x55555555u, n2 >> 1, n3)};
    float s[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) s[m] = 0.0f;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int e = 8 * b + c;
            const float2 v = *reinterpret_cast<const float2 *>(pairb + (__builtin_amdgcn_ubfe(W[c], 8 * b, 8) << 3));
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                s[m] = fmaf(x[m][e], v.x, s[m]);
                s[m] = fmaf(x[m][e + 4], v.y, s[m]);
            }
        }
    const float scale = e4m4_decode(a);
#pragma unroll
    for (int m = 0; m < MT; ++m) out[m] = s[m] * scale;
}

// k = 5: the word of the byte form (byte t of rotr(w, c) holds index(c + 8t) times 8, with
// planes rotated one place further than there) read as two half-words: the low half-word is
// 8 * (index(c) + 256 * index(c + 8)) and the high one the same for c + 16 and c + 24, the
// byte addresses of float2 entries (codebook[a], codebook[b]) at a + 256 b of a sparse LDS
// table (32 x 32 used entries of 7968). Per 4 weights: 8 VALU instructions (7 at c = 0) and
// two 8-byte lookups, against 10 and four lookups in the byte form.
template <int MT>
__device__ __forceinline__ void block_dot_pair8(const uint32_t (&P)[5], uint32_t a, const float (&x)[MT][32],
                                                const uint32_t (&m8)[8], const char *pairb, float (&out)[MT]) {
    uint32_t Q[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) Q[i] = rotr(P[i], 29 - i);   // element j, plane i -> bit j + 3 + i
    float s[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) s[m] = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        // plane i of elements c + 8t sits at bits 8t + 3 + i + c (mod 32): mask m8[(c + i) % 8]
        uint32_t w = Q[0] & m8[c];
#pragma unroll
        for (int i = 1; i < 5; ++i) w = and_or(Q[i], m8[(c + i) & 7], w);
        if (c) w = rotr(w, c);
        asm("" : "+v"(w));                                       // one instruction per half-word
        const uint32_t f0 = w & 0xFFFFu, f1 = w >> 16;
        const float2 v0 = *reinterpret_cast<const float2 *>(pairb + f0);
        const float2 v1 = *reinterpret_cast<const float2 *>(pairb + f1);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            s[m] = fmaf(x[m][c], v0.x, s[m]);
            s[m] = fmaf(x[m][c + 8], v0.y, s[m]);
            s[m] = fmaf(x[m][c + 16], v1.x, s[m]);
            s[m] = fmaf(x[m][c + 24], v1.y, s[m]);
        }
    }
    const float scale = e4m4_decode(a);
#pragma unroll
    for (int m = 0; m < MT; ++m) out[m] = s[m] * scale;
}

// One launch: grid.x = ceil(N / (r * G)), grid.y = ceil(M / MT); blockDim.x = T (a multiple of
// 64 with r * BPR <= T and r * G <= T / 16); K >= 32. Lane t < r * BPR owns row offset t / BPR and
// block t % BPR; the other lanes compute a clamped copy that is not stored, and help with the
// final sums.
template <int KB, int MT, bool ACC>
__global__ __launch_bounds__(kMaxThreads) void kbit_gemv_kernel(const uint16_t *__restrict__ X,
                                                                const uint32_t *__restrict__ planes,
                                                                const uint8_t *__restrict__ absmax,
                                                                const float *__restrict__ codebook,
                                                                const uint16_t *R, void *out, int M, int N, int K,
                                                                int r, int G) {
    constexpr int L = 1 << KB;
    constexpr bool PAIR = KB <= 4;               // two indices per lookup (block_dot_pair)
    constexpr bool PAIR8 = KB == 5;              // the same with pairs 8 apart (block_dot_pair8)
    // pairs from a transposed block (block_dot_tr): at k = 4, and at k = 3 for one or two rows
    // (measured at K = 3584: k = 3 with four rows was 0.2 us faster with block_dot_pair)
    constexpr bool TR = KB == 4 || (KB == 3 && MT <= 2);
    constexpr int KF = KB == 2 ? 2 : 4;          // block_dot_pair's field stride
    constexpr int LP = PAIR ? 1 << (2 * KF) : PAIR8 ? 31 + 256 * 31 + 1 : 1;  // pair-table entries
    __shared__ float cbs[L];
    __shared__ float2 pairs[LP];
    extern __shared__ float part[];        // [r * G][MT][BPR]

    const int tid = threadIdx.x;
    const int BPR = K >> 5;
    const int rows = r * G;                  // rows of W this workgroup covers
    const int n0 = blockIdx.x * rows;
    const int m0 = blockIdx.y * MT;
    const bool active = tid < r * BPR;
    const int roff = active ? tid / BPR : 0;
    const int blk = active ? tid - roff * BPR : 0;

    // every load is unconditional (clamped addresses) and issued before the first wait, in
    // about the order the data is needed (the memory counter is waited on in issue order): X
    // of this lane's block, the writer lanes' residuals, then the plane words and scale bytes
    // of all kMaxRowGroups row groups (groups past G repeat group G - 1 and are not used). The
    // codebook load is issued first. Where the words and the scale bytes go is the compiler's
    // choice (the empty asm statements do not bind loads of memory the kernel never writes);
    // the two source forms below lead it to different schedules, chosen per k by measurement
    // at K = 3584 (0.1 - 0.5 us apart). The schedule to avoid: the first group's scale byte
    // issued behind every word and widened before the pair-table writes, which makes the
    // first wait one for all loads (k = 5 took it when its words and bytes were loaded in one
    // loop).
    const int lane = tid & 63;
    float cbv = codebook[lane & (L - 1)];
    asm volatile("" ::: "memory");             // the codebook load stays first
    u32x4 xv[MT][4];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const uint16_t *xr = X + (size_t)min(m0 + m, M - 1) * K + blk * 32;
#pragma unroll
        for (int q = 0; q < 4; ++q) xv[m][q] = *reinterpret_cast<const u32x4 *>(xr + q * 8);
    }
    const int grp = tid >> 4, s16 = tid & 15;   // writer lanes: 16 per local row
    const int wn = n0 + grp;
    uint16_t rbits[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) rbits[m] = R[(size_t)min(m0 + m, M - 1) * N + min(wn, N - 1)];

    uint32_t P[kMaxRowGroups][KB];
    uint32_t A[kMaxRowGroups];
    if constexpr (KB == 3 || KB == 5) {
        size_t bi[kMaxRowGroups];
#pragma unroll
        for (int g = 0; g < kMaxRowGroups; ++g) {
            const int n = min(n0 + min(g, G - 1) * r + roff, N - 1);
            bi[g] = (size_t)n * BPR + blk;
            A[g] = absmax[bi[g]];
        }
        asm volatile("" ::: "memory");
#pragma unroll
        for (int g = 0; g < kMaxRowGroups; ++g)
#pragma unroll
            for (int i = 0; i < KB; ++i) P[g][i] = __builtin_nontemporal_load(planes + bi[g] * KB + i);
    } else {
#pragma unroll
        for (int g = 0; g < kMaxRowGroups; ++g) {
            const int n = min(n0 + min(g, G - 1) * r + roff, N - 1);
            const size_t b = (size_t)n * BPR + blk;
#pragma unroll
            for (int i = 0; i < KB; ++i) P[g][i] = __builtin_nontemporal_load(planes + b * KB + i);
            A[g] = absmax[b];
            asm volatile("" ::: "memory");
        }
    }

    // every wave writes the whole codebook itself (all waves write identical values), so
    // its lookups need no workgroup barrier; the asm (with a memory clobber) keeps this after
    // the loads above, so that its wait counts only the codebook load
    asm volatile("" : "+v"(cbv) :: "memory");
    if (lane < L) cbs[lane] = cbv;
    if constexpr (PAIR) {
        // the pair table, also per wave: entry a + (b << F) = (codebook[a], codebook[b]), read
        // from this wave's own codebook writes above (a wave's LDS operations run in order);
        // at k = 3 the entries with a or b >= 8 are never read (clamped here)
#pragma unroll
        for (int e0 = 0; e0 < LP; e0 += 64)
            if (e0 + lane < LP) {
                const int ea = (e0 + lane) & ((1 << KF) - 1), eb = (e0 + lane) >> KF;
                pairs[e0 + lane] = make_float2(cbs[min(ea, L - 1)], cbs[min(eb, L - 1)]);
            }
    }
    if constexpr (PAIR8) {
        // the 32 x 32 used entries a + 256 b, per wave as above: lane l writes a = l % 32 (its
        // own codebook value) for b = 2 i + l / 32, i = 0..15
        float2 *prow = pairs + (lane & 31) + 256 * (lane >> 5);
#pragma unroll
        for (int i = 0; i < 16; ++i) prow[512 * i] = make_float2(cbv, cbs[2 * i + (lane >> 5)]);
    }
    uint32_t pm[7];                              // pair masks: positions s + 3 + {0, F, 16, 16 + F}
#pragma unroll
    for (int j = 0; j < 7; ++j) {
        pm[j] = rotl_c((1u | (1u << KF) | (1u << 16) | (1u << (16 + KF))) << 3, j);
        asm("" : "+v"(pm[j]));
    }
    uint32_t msk[8], m8[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        msk[j] = rotl_c(0x04040404u, j);
        m8[j] = rotl_c(0x08080808u, j);
        asm("" : "+v"(msk[j]), "+v"(m8[j]));     // keep in VGPRs: a VOP3 AND-OR takes no literal
    }
    // X to fp32: pinning xv here keeps its wait (and the conversion) from being scheduled
    // between the loads above, where it would hold back their issue
    float x[MT][32];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            asm volatile("" : "+v"(xv[m][q]));
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                x[m][q * 8 + 2 * h] = __uint_as_float(xv[m][q][h] << 16);
                x[m][q * 8 + 2 * h + 1] = __uint_as_float(xv[m][q][h] & 0xFFFF0000u);
            }
        }

    const char *cbb = reinterpret_cast<const char *>(cbs);
    const char *pairb = reinterpret_cast<const char *>(pairs);
    uint32_t zero = 0u;
    asm("" : "+v"(zero));
    // two row groups per step, so that their lookups and FMAs interleave; the empty asm
    // pins each group's words to its step, so that the compiler cannot hoist their decode
    // (and the wait for their loads) above the barrier and the groups before
#pragma unroll
    for (int g = 0; g < kMaxRowGroups; g += 2) {
#pragma unroll
        for (int i = 0; i < KB; ++i) asm volatile("" : "+v"(P[g][i]), "+v"(P[g + 1][i]));
        asm volatile("" : "+v"(A[g]), "+v"(A[g + 1]));
        if (g + 1 < G) {
            float o0[MT], o1[MT];
            if constexpr (TR) {
                block_dot_tr<KB, MT>(P[g], A[g], x, pairb, zero, o0);
                block_dot_tr<KB, MT>(P[g + 1], A[g + 1], x, pairb, zero, o1);
            } else if constexpr (PAIR) {
                block_dot_pair<KB, MT>(P[g], A[g], x, pm, pairb, o0);
                block_dot_pair<KB, MT>(P[g + 1], A[g + 1], x, pm, pairb, o1);
            } else if constexpr (PAIR8) {
                block_dot_pair8<MT>(P[g], A[g], x, m8, pairb, o0);
                block_dot_pair8<MT>(P[g + 1], A[g + 1], x, m8, pairb, o1);
            } else {
                block_dot<KB, MT>(P[g], A[g], x, msk, cbb, o0);
                block_dot<KB, MT>(P[g + 1], A[g + 1], x, msk, cbb, o1);
            }
            if (active) {
                float *p0 = part + (size_t)(g * r + roff) * MT * BPR + blk;
                float *p1 = p0 + (size_t)r * MT * BPR;
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    p0[m * BPR] = o0[m];
                    p1[m * BPR] = o1[m];
                }
            }
        } else if (g < G) {
            float o0[MT];
            if constexpr (TR) block_dot_tr<KB, MT>(P[g], A[g], x, pairb, zero, o0);
            else if constexpr (PAIR) block_dot_pair<KB, MT>(P[g], A[g], x, pm, pairb, o0);
            else if constexpr (PAIR8) block_dot_pair8<MT>(P[g], A[g], x, m8, pairb, o0);
            else block_dot<KB, MT>(P[g], A[g], x, msk, cbb, o0);
            if (active) {
                float *p0 = part + (size_t)(g * r + roff) * MT * BPR + blk;
#pragma unroll
                for (int m = 0; m < MT; ++m) p0[m * BPR] = o0[m];
            }
        }
    }
    __syncthreads();

    // 16 lanes per local row: add the row's BPR partial sums, one rounding with R
    if (grp < rows) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const float *pr = part + (size_t)grp * MT * BPR + m * BPR;
            // up to 8 partials per lane in one batch of independent LDS reads (BPR <= 128),
            // then a loop for longer rows
            float part8[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) part8[u] = pr[min(s16 + 16 * u, BPR - 1)];
            float v = 0.0f;
#pragma unroll
            for (int u = 0; u < 8; ++u) v += s16 + 16 * u < BPR ? part8[u] : 0.0f;
            for (int b = s16 + 128; b < BPR; b += 16) v += pr[b];
            v = row16_sum(v);
            if (s16 == 0 && wn < N && m0 + m < M) store_output<ACC>(out, Epilogue{N, N, 0u}, m0 + m, wn, v, bf16_bits_to_f32(rbits[m]));
        }
    }
}

// ---------------------------------------------------------------------------------------------
// Matrix-core form for 5 <= M (k = 2, 3 and 4; K a multiple of 128, at most 3584; the plane
// words of a block read as one 8-, 12- or 16-byte vector, the scale bytes of four blocks as one dword): the
// products go to v_mfma_f32_16x16x32_bf16 with X as the A operand (16 rows of X) and the decoded
// weights as the B operand (16 W rows), so one MFMA covers one 32-element block of 16 W rows
// for up to 16 rows of X. A W row's block is split over four lanes (lane l: W row l % 16, part
// g = l / 16), each decoding two of the pair words of block_dot_pair (planes rotated one bit
// further, so a field is the entry index times 16): 8 elements per lane, in the order e, e + F,
// e + 16, e + 16 + F for its two word positions; X's fragments take the same order. A pair-table
// entry holds the two codebook values as three bf16 pairs (hi, mid, lo: each fp32 value is
// exactly the sum of its three bf16 parts, so the three MFMAs reproduce the fp32 products; two
// parts, 2^-18 relative, miss the parity floor of outputs near zero); the block's
// D = X . (hi + mid + lo) is then scaled by the lane's W-row absmax (each D lane holds one W row)
// and added to the accumulator. The time barely depends on M (up to 16): about 60 VALU
// instructions per block and lane (the decode's rotations now serve 8 elements instead of 32,
// and 12 moves assemble the B fragments from the 16-byte entries) and conflicting 16-byte LDS
// lookups, which is why M <= 4 stays with the VALU form.
constexpr int kMfmaWaves = 7;          // K slices of 16 blocks (512 elements) per workgroup
constexpr int kMfmaBlocks = 16;        // blocks per wave
constexpr int kMfmaTiles = 2;          // 16-row W tiles per workgroup
constexpr int kXPitchB = 1040;         // bytes per staged X row (512 bf16 + 16)

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4_t mfma_bf16(u32x4 a, u32x4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}

// fp32 -> three bf16 parts whose sum is the value exactly (each part truncated from what the
// previous ones leave: 8 + 8 + 8 significant bits)
__device__ __forceinline__ void split3(float v, uint32_t &hi, uint32_t &mid, uint32_t &lo) {
    const uint32_t b0 = __float_as_uint(v) & 0xFFFF0000u;
    const float r1 = v - __uint_as_float(b0);
    const uint32_t b1 = __float_as_uint(r1) & 0xFFFF0000u;
    const float r2 = r1 - __uint_as_float(b1);
    hi = b0 >> 16;
    mid = b1 >> 16;
    lo = __float_as_uint(r2) >> 16;
}

template <int KB, bool ACC>
__global__ __launch_bounds__(kMfmaWaves * 64) void kbit_mfma_kernel(const uint16_t *__restrict__ X,
                                                                    const uint32_t *__restrict__ planes,
                                                                    const uint8_t *__restrict__ absmax,
                                                                    const float *__restrict__ codebook,
                                                                    const uint16_t *R, void *out, int M, int N,
                                                                    int K) {
    static_assert(KB >= 2 && KB <= 4, "plane words read as one 8-, 12- or 16-byte vector");
    constexpr int L = 1 << KB;
    constexpr int F = KB == 2 ? 2 : 4;           // pair distance (field stride)
    constexpr int FW = 4 + 2 * F;                // field width: entry index times 16
    constexpr int LP = 1 << (2 * F);             // pair-table entries
    constexpr int NT = kMfmaWaves * 64;
    constexpr int ROWS = 16 * kMfmaTiles;
    constexpr int OUTS = ROWS * 16;
    constexpr int PER = (OUTS + NT - 1) / NT;
    __shared__ float cbs[L];
    __shared__ u32x4 pairs[LP];
    __shared__ __attribute__((aligned(16))) uint8_t xst[kMfmaWaves][16 * kXPitchB];
    __shared__ f32x4_t red[kMfmaTiles][kMfmaWaves][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int BPR = K >> 5;
    const int NV = K >> 3;                       // 16-byte vectors of an X row
    const int n0 = blockIdx.x * ROWS;
    const int m0 = blockIdx.y * 16;
    const int b0 = w * kMfmaBlocks;              // this wave's first block
    const int nb = max(0, min(kMfmaBlocks, BPR - b0));
    const int rn = lane & 15, g = lane >> 4, h = g >> 1;

    // loads, in the order they are used, all before the first wait: the codebook, this wave's X
    // slice (16 rows x 512 elements, 1 KB per instruction), the residuals of the outputs this
    // thread writes, then per tile the scale dwords (16 blocks of the lane's W row) and the plane
    // words of the lane's W row for each of the wave's blocks (addresses clamped; blocks past the
    // wave's nb are loaded but never used)
    float cbv = codebook[lane & (L - 1)];
    asm volatile("" ::: "memory");
    u32x4 xr[16];
    {
        const int v = min(4 * b0 + lane, NV - 1);
#pragma unroll
        for (int r = 0; r < 16; ++r)
            xr[r] = *reinterpret_cast<const u32x4 *>(X + (size_t)min(m0 + r, M - 1) * K + 8 * v);
    }
    uint16_t rbits[PER];
#pragma unroll
    for (int p = 0; p < PER; ++p) {
        const int e = min(tid + p * NT, OUTS - 1);
        rbits[p] = R[(size_t)min(m0 + e / ROWS, M - 1) * N + min(n0 + e % ROWS, N - 1)];
    }
    uint32_t sc[kMfmaTiles][4];
    uint32_t P[kMfmaTiles][kMfmaBlocks][KB];
#pragma unroll
    for (int t = 0; t < kMfmaTiles; ++t) {
        const size_t row = (size_t)min(n0 + 16 * t + rn, N - 1);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            sc[t][q] = *reinterpret_cast<const uint32_t *>(absmax + row * BPR + min(b0 + 4 * q, BPR - 4));
#pragma unroll
        for (int j = 0; j < kMfmaBlocks; ++j) {
            const uint32_t *pw = planes + (row * BPR + min(b0 + j, BPR - 1)) * KB;
            if constexpr (KB == 4) {
                const u32x4 v = *reinterpret_cast<const u32x4 *>(pw);
#pragma unroll
                for (int i = 0; i < 4; ++i) P[t][j][i] = v[i];
            } else if constexpr (KB == 3) {
                const uint3 v = *reinterpret_cast<const uint3 *>(pw);   // one 12-byte load
                P[t][j][0] = v.x;
                P[t][j][1] = v.y;
                P[t][j][2] = v.z;
            } else {
                const u32x2 v = *reinterpret_cast<const u32x2 *>(pw);
                P[t][j][0] = v[0];
                P[t][j][1] = v[1];
            }
        }
    }

    // the codebook and the pair table of three-part entries, per wave (identical writes in every
    // wave, read back only by the writing wave: no workgroup barrier); entry a + (b << F)
    asm volatile("" : "+v"(cbv) :: "memory");
    if (lane < L) cbs[lane] = cbv;
#pragma unroll
    for (int e0 = 0; e0 < LP; e0 += 64)
        if (e0 + lane < LP) {
            const int ea = (e0 + lane) & ((1 << F) - 1), eb = (e0 + lane) >> F;
            uint32_t ha, ma, la, hb, mb, lb;
            split3(cbs[min(ea, L - 1)], ha, ma, la);
            split3(cbs[min(eb, L - 1)], hb, mb, lb);
            pairs[e0 + lane] = u32x4{ha | (hb << 16), ma | (mb << 16), la | (lb << 16), 0u};
        }

    // X fragments through this wave's LDS slice: lane (row rn, part g) takes, of block j, the
    // pairs (e, e + F) and (e + 16, e + 16 + F) for its two word positions e = cp + 8h, i.e. from
    // the 16-byte chunks 4j + h and 4j + 2 + h the dwords p and q (F = 4: p = g % 2, q = p + 2;
    // F = 2: p = 2 (g % 2), q = p + 1), low halves then high halves
    uint8_t *xs = xst[w];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        asm volatile("" : "+v"(xr[r]));
        *reinterpret_cast<u32x4 *>(xs + r * kXPitchB + 16 * lane) = xr[r];
    }
    const int pp = F == 4 ? (g & 1) : 2 * (g & 1);
    const int qq = F == 4 ? pp + 2 : pp + 1;
    u32x4 xf[kMfmaBlocks];
#pragma unroll
    for (int j = 0; j < kMfmaBlocks; ++j) {
        const uint32_t *ca = reinterpret_cast<const uint32_t *>(xs + rn * kXPitchB + 16 * (4 * j + h));
        const uint32_t *cb2 = reinterpret_cast<const uint32_t *>(xs + rn * kXPitchB + 16 * (4 * j + 2 + h));
        const uint32_t ap = ca[pp], aq = ca[qq], bp = cb2[pp], bq = cb2[qq];
        xf[j] = u32x4{(ap & 0xFFFFu) | (aq << 16), (bp & 0xFFFFu) | (bq << 16), (ap >> 16) | (aq & 0xFFFF0000u),
                      (bp >> 16) | (bq & 0xFFFF0000u)};
        if (j >= nb) xf[j] = u32x4{0u, 0u, 0u, 0u};  // past the wave's blocks: products exactly 0
    }

    // per lane: its two word positions and their masks (plane i of element j at bit j + 4 + i,
    // 8 lower for the high half)
    const int cpa = F == 4 ? 2 * (g & 1) : 4 * (g & 1);
    const int rot = h ? 4 : 28;
    uint32_t mk[2][KB];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < KB; ++i) {
            const uint32_t base = (1u | (1u << F) | (1u << 16) | (1u << (16 + F))) << 4;
            mk[u][i] = rotr(base, (32 - (cpa + u + i)) & 31);   // base rotated left by cp + i
        }
    const char *pairb = reinterpret_cast<const char *>(pairs);

    f32x4_t acc[kMfmaTiles];
#pragma unroll
    for (int t = 0; t < kMfmaTiles; ++t) {
        acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kMfmaBlocks; ++j) {   // blocks past nb add 0 (zero X fragment)
            uint32_t Q[KB];
#pragma unroll
            for (int i = 0; i < KB; ++i) Q[i] = rotr(P[t][j][i], rot - i);
            u32x4 bh, bm, bl;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                uint32_t wd = Q[0] & mk[u][0];
#pragma unroll
                for (int i = 1; i < KB; ++i) wd = and_or(Q[i], mk[u][i], wd);
                const int cp = cpa + u;
                const u32x4 e0 = *reinterpret_cast<const u32x4 *>(pairb + __builtin_amdgcn_ubfe(wd, cp, FW));
                const u32x4 e1 = *reinterpret_cast<const u32x4 *>(pairb + __builtin_amdgcn_ubfe(wd, cp + 16, FW));
                bh[2 * u] = e0[0]; bm[2 * u] = e0[1]; bl[2 * u] = e0[2];
                bh[2 * u + 1] = e1[0]; bm[2 * u + 1] = e1[1]; bl[2 * u + 1] = e1[2];
            }
            f32x4_t d = mfma_bf16(xf[j], bh, f32x4_t{0.f, 0.f, 0.f, 0.f});
            d = mfma_bf16(xf[j], bm, d);
            d = mfma_bf16(xf[j], bl, d);
            const float sv = e4m4_decode(__builtin_amdgcn_ubfe(sc[t][j >> 2], 8 * (j & 3), 8));
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[t][i] = fmaf(d[i], sv, acc[t][i]);
        }
        // acc[t][i] = partial Y[m0 + 4g + i][n0 + 16t + rn] over this wave's blocks
        red[t][w][lane] = acc[t];
    }
    __syncthreads();

    const float *redf = reinterpret_cast<const float *>(&red[0][0][0]);
#pragma unroll
    for (int p = 0; p < PER; ++p) {
        const int e = tid + p * NT;
        if (e >= OUTS) break;
        const int nl = e % ROWS, mc = e / ROWS;
        const int m = m0 + mc, n = n0 + nl;
        if (m >= M || n >= N) continue;
        const int t = nl >> 4, j = nl & 15;
        const int idx = (16 * (mc >> 2) + j) * 4 + (mc & 3);
        float v = 0.0f;
#pragma unroll
        for (int q = 0; q < kMfmaWaves; ++q) v += redf[(t * kMfmaWaves + q) * 64 * 4 + idx];
        store_output<ACC>(out, Epilogue{N, N, 0u}, m, n, v, bf16_bits_to_f32(rbits[p]));
    }
}

struct KbitShape {
    int r, T, G;
    size_t shmem;
};

// Rows per row group r and workgroup size T (a multiple of 64 holding r * BPR owner lanes and
// 16 writer lanes per row): the fewest idle lanes in the launched waves first, then a size of
// 256..512 lanes, then the smaller size (at K = 3584, BPR = 112: r = 4 and 448 threads, no idle
// lane; 2 rows in 256 threads leave 32 idle and measured 2-3 % slower). G row groups per
// workgroup so that every local row has a writer group, the partial sums fit their LDS budget
// and the grid still covers the chip.
KbitShape kbit_shape(int64_t N, int64_t K, int MT) {
    const int BPR = (int)(K / 32);
    KbitShape s{16, 256, 1, 0};
    if (BPR > 0) {
        double best_eff = -1.0;
        int best_pen = 2;
        for (int r = 1; r * BPR <= kMaxThreads && 16 * r <= kMaxThreads; ++r) {
            const int T = ((std::max(r * BPR, 16 * r) + 63) / 64) * 64;
            const double eff = (double)(r * BPR) / T;
            const int pen = (T >= 256 && T <= 512) ? 0 : 1;
            const bool better = eff > best_eff + 1e-9 ||
                                (eff > best_eff - 1e-9 && (pen < best_pen || (pen == best_pen && T < s.T)));
            if (better) {
                best_eff = eff;
                best_pen = pen;
                s.r = r;
                s.T = T;
            }
        }
    }
    // G: the row groups a workgroup walks. Each of the 256 CUs takes ceil(WGs / 256) workgroups
    // of G groups; pick the G with the least such work per CU, the largest on a tie (fewer,
    // longer workgroups pay the load latency at their start fewer times).
    const int64_t groups = (N + s.r - 1) / s.r;
    int Gmax = std::min(kMaxRowGroups, std::max(1, (s.T / 16) / s.r));
    if (BPR > 0) Gmax = std::min(Gmax, std::max(1, kPartialBytes / (s.r * MT * BPR * 4)));
    int64_t best = -1;
    for (int G = 1; G <= Gmax; ++G) {
        const int64_t wgs = (groups + G - 1) / G;
        const int64_t cost = ((wgs + 255) / 256) * G;
        if (best < 0 || cost <= best) {
            best = cost;
            s.G = G;
        }
    }
    s.shmem = (size_t)s.r * s.G * MT * std::max(BPR, 1) * sizeof(float);
    return s;
}

template <int KB, int MT>
hipError_t launch_kbit(const KbitArgs &a) {
    const KbitShape s = kbit_shape(a.N, a.K, MT);
    const int rows = s.r * s.G;
    dim3 grid((unsigned)((a.N + rows - 1) / rows), (unsigned)((a.M + MT - 1) / MT));
    if (a.acc_out)
        hipLaunchKernelGGL((kbit_gemv_kernel<KB, MT, true>), grid, dim3(s.T), s.shmem, a.stream, a.X, a.planes,
                           a.absmax, a.codebook, a.R, a.out, (int)a.M, (int)a.N, (int)a.K, s.r, s.G);
    else
        hipLaunchKernelGGL((kbit_gemv_kernel<KB, MT, false>), grid, dim3(s.T), s.shmem, a.stream, a.X, a.planes,
                           a.absmax, a.codebook, a.R, a.out, (int)a.M, (int)a.N, (int)a.K, s.r, s.G);
    return hipGetLastError();
}

template <int KB>
hipError_t launch_kbit_mt(const KbitArgs &a) {
    if (a.M <= 1) return launch_kbit<KB, 1>(a);
    if (a.M <= 2) return launch_kbit<KB, 2>(a);
    return launch_kbit<KB, 4>(a);
}

// The matrix-core form takes k = 2, 3 and 4 from M = 5 (where the VALU form needs a second 4-row
// pass; at K = 3584: M = 5 .. 8 15.9 against 17.2 - 17.5 us at k = 4, M = 16 16.2 against 33.2)
// when K fits its 7 x 16 blocks in whole dwords of scale bytes and the plane and scale pointers
// allow its vector loads; at M <= 4 the VALU form is faster (k = 4, M = 4: 9.4 against 15.9).
constexpr int64_t kKbitMfmaMinM = 5;
bool kbit_mfma_eligible(const KbitArgs &a) {
    const uintptr_t pl = reinterpret_cast<uintptr_t>(a.planes), am = reinterpret_cast<uintptr_t>(a.absmax);
    const uintptr_t pal = a.kbits == 3 ? 4 : 4 * a.kbits;   // 12-byte words: dword alignment
    return a.kbits <= 4 && a.M >= kKbitMfmaMinM && a.K % 128 == 0 && a.K <= 32 * kMfmaWaves * kMfmaBlocks &&
           pl % pal == 0 && am % 4 == 0;
}

}  // namespace

int64_t kbit_max_k() {
    // one lane per 32-element block of a row, at most kMaxThreads lanes per workgroup
    return (int64_t)kMaxThreads * 32;
}

hipError_t launch_kbit_gemv(const KbitArgs &a) {
    if (kbit_mfma_eligible(a)) {
        const dim3 grid((unsigned)((a.N + 16 * kMfmaTiles - 1) / (16 * kMfmaTiles)), (unsigned)((a.M + 15) / 16));
        const dim3 block(kMfmaWaves * 64);
#define KBIT_MFMA(KB, ACC)                                                                                      \
    hipLaunchKernelGGL((kbit_mfma_kernel<KB, ACC>), grid, block, 0, a.stream, a.X, a.planes, a.absmax, a.codebook, \
                       a.R, a.out, (int)a.M, (int)a.N, (int)a.K)
        if (a.kbits == 4) {
            if (a.acc_out) KBIT_MFMA(4, true);
            else KBIT_MFMA(4, false);
        } else if (a.kbits == 3) {
            if (a.acc_out) KBIT_MFMA(3, true);
            else KBIT_MFMA(3, false);
        } else {
            if (a.acc_out) KBIT_MFMA(2, true);
            else KBIT_MFMA(2, false);
        }
#undef KBIT_MFMA
        return hipGetLastError();
    }
    switch (a.kbits) {
        case 2: return launch_kbit_mt<2>(a);
        case 3: return launch_kbit_mt<3>(a);
        case 4: return launch_kbit_mt<4>(a);
        case 5: return launch_kbit_mt<5>(a);
    }
    return hipErrorInvalidValue;
}

}  // namespace skinny
