// probe.hip -- measurement reference kernels (include/skinny_probe.h): empty launch,
// streaming read, plain copy. Not part of the operation.
#include "../../include/skinny_probe.h"
#include "common.hpp"

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
