// probe.hip -- measurement reference kernels (include/skinny_probe.h): empty launch,
// streaming read, plain copy. Not part of the operation.
#include "../../include/skinny_probe.h"
#include "common.hpp"

#include <climits>

namespace skinny {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void null_kernel() {}

template <int U>
__global__ __launch_bounds__(256) void read_kernel(const u32x4 *__restrict__ p, int64_t n, float *sink) {
    float s = 0.0f;
    const int64_t stride = (int64_t)gridDim.x * 256 * U;
    for (int64_t base = (int64_t)blockIdx.x * 256 * U + threadIdx.x; base < n; base += stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + (int64_t)u * 256;
            v[u] = i < n ? __builtin_nontemporal_load(&p[i]) : u32x4{};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) s += __uint_as_float(v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3]);
    }
    if (s == 1.25e-37f) sink[0] = s;  // never true for real data; keeps the loads alive
}

// Read shaped like the small-M kernels: a workgroup of 7 waves owns RPB contiguous rows of
// 7168 bytes; lane t of the workgroup reads 16-byte vector t of every row (each wave
// instruction is one contiguous 1 KB piece of a row), and every load of the workgroup is
// issued before the first one is used.
template <int RPB>
__global__ __launch_bounds__(448) void read_rows_kernel(const u32x4 *__restrict__ p, int rows, float *sink) {
    const int t = threadIdx.x;
    const int r0 = blockIdx.x * RPB;
    u32x4 v[RPB];
#pragma unroll
    for (int r = 0; r < RPB; ++r) v[r] = __builtin_nontemporal_load(&p[(size_t)min(r0 + r, rows - 1) * 448 + t]);
    uint32_t x = 0;
#pragma unroll
    for (int r = 0; r < RPB; ++r) x ^= v[r][0] ^ v[r][1] ^ v[r][2] ^ v[r][3];
    if (x == 0x9E3779B9u && t == 0) sink[0] = 1.0f;  // data-dependent, so the loads stay
}

// Busy for `ticks` of the 100 MHz real-time counter from the workgroup's start.
__global__ void spin_kernel(uint64_t ticks) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (__builtin_amdgcn_s_memrealtime() - t0 < ticks) __builtin_amdgcn_s_sleep(1);
}

__global__ __launch_bounds__(256) void copy_kernel(u32x4 *__restrict__ d, const u32x4 *__restrict__ s,
                                                   int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) d[i] = s[i];
}

int cu_count() {
    static int cus = 0;
    if (!cus) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
    }
    return cus;
}

skinny_status finish(hipError_t e) { return e == hipSuccess ? SKINNY_OK : SKINNY_EHIP; }

}  // namespace
}  // namespace skinny

using namespace skinny;

extern "C" {

skinny_status skinny_probe_null(void *stream) {
    hipLaunchKernelGGL(null_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream);
    return finish(hipGetLastError());
}

skinny_status skinny_probe_read(const void *buf, int64_t bytes, float *sink, int32_t blocks, int32_t unroll,
                                void *stream) {
    if (bytes < 0 || !sink || (bytes > 0 && !buf)) return SKINNY_EINVAL;
    if (bytes % 16 || ((uintptr_t)buf % 16)) return SKINNY_EALIGN;
    if (unroll < 1 || unroll > 16 || blocks < 0) return SKINNY_EINVAL;
    if (bytes == 0) return SKINNY_OK;
    const int64_t n = bytes / 16;
    const int g = blocks ? blocks : 8 * cu_count();
    const u32x4 *p = (const u32x4 *)buf;
    hipStream_t s = (hipStream_t)stream;
    switch (unroll) {
        case 1: hipLaunchKernelGGL(read_kernel<1>, dim3(g), dim3(256), 0, s, p, n, sink); break;
        case 2: hipLaunchKernelGGL(read_kernel<2>, dim3(g), dim3(256), 0, s, p, n, sink); break;
        case 4: hipLaunchKernelGGL(read_kernel<4>, dim3(g), dim3(256), 0, s, p, n, sink); break;
        case 8: hipLaunchKernelGGL(read_kernel<8>, dim3(g), dim3(256), 0, s, p, n, sink); break;
        case 16: hipLaunchKernelGGL(read_kernel<16>, dim3(g), dim3(256), 0, s, p, n, sink); break;
        default: return SKINNY_EINVAL;
    }
    return finish(hipGetLastError());
}

skinny_status skinny_probe_read_rows(const void *buf, int64_t rows, int32_t rows_per_block, float *sink,
                                     void *stream) {
    if (rows < 0 || !sink || (rows > 0 && !buf) || rows > INT_MAX) return SKINNY_EINVAL;
    if ((uintptr_t)buf % 16) return SKINNY_EALIGN;
    if (rows == 0) return SKINNY_OK;
    const int rpb = rows_per_block;
    const dim3 grid((unsigned)((rows + rpb - 1) / rpb)), block(448);
    const u32x4 *p = (const u32x4 *)buf;
    hipStream_t s = (hipStream_t)stream;
    switch (rpb) {
        case 4: hipLaunchKernelGGL(read_rows_kernel<4>, grid, block, 0, s, p, (int)rows, sink); break;
        case 8: hipLaunchKernelGGL(read_rows_kernel<8>, grid, block, 0, s, p, (int)rows, sink); break;
        case 16: hipLaunchKernelGGL(read_rows_kernel<16>, grid, block, 0, s, p, (int)rows, sink); break;
        case 28: hipLaunchKernelGGL(read_rows_kernel<28>, grid, block, 0, s, p, (int)rows, sink); break;
        case 32: hipLaunchKernelGGL(read_rows_kernel<32>, grid, block, 0, s, p, (int)rows, sink); break;
        default: return SKINNY_EINVAL;
    }
    return finish(hipGetLastError());
}

skinny_status skinny_probe_spin(int64_t nanoseconds, int32_t blocks, int32_t threads, void *stream) {
    if (nanoseconds < 0 || blocks < 1 || threads < 1 || threads > 1024) return SKINNY_EINVAL;
    hipLaunchKernelGGL(spin_kernel, dim3(blocks), dim3(threads), 0, (hipStream_t)stream,
                       (uint64_t)(nanoseconds / 10));
    return finish(hipGetLastError());
}

skinny_status skinny_probe_copy(void *dst, const void *src, int64_t bytes, void *stream) {
    if (bytes < 0 || (bytes > 0 && (!dst || !src))) return SKINNY_EINVAL;
    if (bytes % 16 || ((uintptr_t)dst % 16) || ((uintptr_t)src % 16)) return SKINNY_EALIGN;
    if (bytes == 0) return SKINNY_OK;
    const int64_t n = bytes / 16;
    const int64_t want = (n + 255) / 256;
    const int g = (int)(want < 8 * cu_count() ? want : 8 * cu_count());
    hipLaunchKernelGGL(copy_kernel, dim3(g), dim3(256), 0, (hipStream_t)stream, (u32x4 *)dst,
                       (const u32x4 *)src, n);
    return finish(hipGetLastError());
}

}  // extern "C"
