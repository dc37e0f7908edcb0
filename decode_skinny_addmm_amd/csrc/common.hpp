// common.hpp -- shared device helpers and the kernel registry of libskinny.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/skinny.h"

namespace skinny {

// ----------------------------------------------------------------------------- launch plumbing

// Epilogue layout and options, passed to every kernel by value: R[m, n] is R[m*ldr + n],
// the output element (m, n) is out[m*ldy + n]; flags are SKINNY_FLAG_* bits.
struct Epilogue {
    int ldr, ldy;
    uint32_t flags;
};

// Arguments of one call, already validated by the C ABI layer.
struct LaunchArgs {
    const uint16_t *X;  // bf16 [M, K]
    const uint16_t *W;  // bf16 [N, K]
    const uint16_t *R;  // bf16 [M, N], row pitch ep.ldr
    void *out;          // bf16 Y or float ACC [M, N], row pitch ep.ldy
    int64_t M, N, K;
    bool acc_out;       // true: write fp32 ACC instead of bf16 Y
    hipStream_t stream;
    Epilogue ep;
};

// True for the plain [M, N] output with no shard flags. The kernels on the tuned path have an
// instantiation for that case (GEN = false) whose epilogue takes the pitches from N and has
// no flag tests; the general instantiation (GEN = true) serves the shard form and the fp32
// test output. The sum of products is the same code in both.
inline bool plain_epilogue(const LaunchArgs &a) {
    return a.ep.flags == 0 && a.ep.ldr == a.N && a.ep.ldy == a.N;
}

// One compiled kernel instance: its public configuration, how to launch it, and the
// address of its device function (for attribute queries).
struct KernelEntry {
    skinny_config cfg;
    hipError_t (*launch)(const LaunchArgs &);
    const void *fn_bf16;            // kernel writing bf16 Y
    const void *fn_acc;             // kernel writing fp32 ACC
    int64_t (*max_k)();             // largest K the instance accepts (LDS limits), or INT64_MAX
    int32_t k_align = 8;            // K must be a multiple of this
};

// Arguments of one k-bit quantized GEMV call (kbit_gemv.hip), validated by the C ABI layer.
struct KbitArgs {
    const uint16_t *X;        // bf16 [M, K]
    const uint32_t *planes;   // [N, K/32, kbits] bit-plane words
    const uint8_t *absmax;    // [N, K/32] E4M4 bytes
    const float *codebook;    // [2^kbits]
    int kbits;                // 2 .. 5
    const uint16_t *R;        // bf16 [M, N]
    void *out;                // bf16 Y or float ACC [M, N]
    int64_t M, N, K;
    bool acc_out;
    hipStream_t stream;
};
hipError_t launch_kbit_gemv(const KbitArgs &a);
int64_t kbit_max_k();

// One KDA chain-verify call (kda_verify.hip), validated by the C ABI layer.
hipError_t launch_kda_verify(const skinny_kda_args &a, hipStream_t stream);

// Registries filled by each kernel family's translation unit.
const KernelEntry *gemv_entries(int *count);
const KernelEntry *mfma_entries(int *count);
const KernelEntry *mfma_lds_entries(int *count);
const KernelEntry *gemm_entries(int *count);
const KernelEntry *simt_entries(int *count);
const KernelEntry *dma_entries(int *count);
const KernelEntry *ring_entries(int *count);

// ----------------------------------------------------------------------------- device helpers

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even (gfx950 converts in hardware: v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// acc + a.lo*b.lo + a.hi*b.hi on two packed bf16 pairs (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// The one epilogue of every kernel: t is the fp32 sum of the K products for output (m, n),
// r the residual already widened to fp32. Y = bf16(t + r), rounded once (RNE); with
// SKINNY_FLAG_ROUND_PRODUCT the sum is first rounded to bf16 (the tensor-parallel shard
// epilogue of the vLLM API page "fused_add_multicast_skinny_gemm": GEMM result in bf16, then
// the residual added in fp32 and rounded again); with SKINNY_FLAG_NO_NEG_ZERO a -0 result is
// written as +0 (that page keeps -0 free as its not-yet-written marker). The fp32 test output
// (ACC) is the value that gets rounded.
template <bool ACC>
__device__ __forceinline__ void store_output(void *out, const Epilogue &ep, int m, int n, float t, float r) {
    const float g = (ep.flags & SKINNY_FLAG_ROUND_PRODUCT) ? bf16_bits_to_f32(f32_to_bf16_rne(t)) : t;
    const float y = g + r;
    const size_t o = (size_t)m * ep.ldy + n;
    if constexpr (ACC) {
        static_cast<float *>(out)[o] = y;
    } else {
        uint16_t b = f32_to_bf16_rne(y);
        if ((ep.flags & SKINNY_FLAG_NO_NEG_ZERO) && b == 0x8000u) b = 0;
        static_cast<uint16_t *>(out)[o] = b;
    }
}

// Block b of a 1-D grid of G blocks runs on XCD b % 8. xcd_run maps it to a contiguous run of
// indices per XCD (a bijection of 0 .. G-1: XCD x takes G / 8 indices, one more when x < G % 8),
// so blocks of neighbouring rows of W share an L2 and the 128-byte lines of R and Y that they
// split are fetched once and written back whole.
__device__ __forceinline__ int xcd_run(int b, int G) {
    const int x = b & 7, q = G >> 3, r = G & 7;
    return x * q + min(x, r) + (b >> 3);
}

// ---- cross-lane exchange steps (gfx950) ------------------------------------------------
// pair_step<D>(x, y): lanes whose lane-id bit D is clear return x + (x of their partner),
// lanes with the bit set return y + (y of their partner); partners differ exactly in bit D
// (distances 32, 16: v_permlane32_swap / v_permlane16_swap; 8: DPP row_ror:8) or pair the two
// halves of an 8- or 4-lane group (4: DPP row_half_mirror; 2, 1: DPP quad_perm).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int D>
__device__ __forceinline__ float pair_step(float x, float y, int lane) {
    if constexpr (D == 32) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    } else if constexpr (D == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    } else {
        constexpr int CTRL = D == 8 ? 0x128 : D == 4 ? 0x141 : D == 2 ? 0x4E : 0xB1;
        const float xs = x + dpp_f32<CTRL>(x);
        const float ys = y + dpp_f32<CTRL>(y);
        return (lane & D) ? ys : xs;
    }
}

// Transposing reduction of CNT per-lane values over the 64 lanes of a wavefront.
// At each lane distance D (32, 16, ..., 1) a lane keeps one half of its values (the upper
// half if its bit D is set) and adds its partner's copy of that half, so the value count
// halves per step instead of every value paying for all six steps. After
// s = min(log2 CNT, 6) halving steps (plain butterfly steps follow while D > 0), lane L
// holds in a[j] the wave-wide sum of original index  j + (CNT >> s) * (L >> (6 - s));
// lanes that differ only in their low (6 - s) bits hold the same sums.
template <int CNT, int D, int NV>
__device__ __forceinline__ void wave_transpose_reduce(float (&a)[NV], int lane) {
    if constexpr (D > 0) {
        if constexpr (CNT > 1) {
            constexpr int H = CNT / 2;
#pragma unroll
            for (int i = 0; i < H; ++i) a[i] = pair_step<D>(a[i], a[i + H], lane);
            wave_transpose_reduce<H, D / 2>(a, lane);
        } else {
            a[0] = pair_step<D>(a[0], a[0], lane);
            wave_transpose_reduce<1, D / 2>(a, lane);
        }
    }
}

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

}  // namespace skinny
