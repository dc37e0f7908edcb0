/*
 * skinny_probe.h -- measurement reference kernels of libskinny.so (not part of the operation).
 *
 * The benchmark of the vLLM page "benchmarks/kernels/benchmark_k3_cutedsl_residual.py"
 * times the operation by batched graph replay; these kernels give the same harness its
 * reference rows on MI355X: the per-launch floor (an empty kernel), the HBM read rate a
 * plain streaming kernel reaches on the same buffers, and a plain copy of known size that
 * calibrates hardware byte counters. Device pointers, asynchronous on `stream`
 * (a hipStream_t, NULL = null stream); status codes as in skinny.h.
 */
#ifndef SKINNY_PROBE_H
#define SKINNY_PROBE_H

#include <stdint.h>

#include "skinny.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Launch one empty workgroup (the per-launch floor). */
SKINNY_API skinny_status skinny_probe_null(void *stream);

/*
 * Read `bytes` bytes at `buf` (16-byte aligned, bytes % 16 == 0) with 16-byte non-temporal
 * loads: `blocks` workgroups of 256 threads (0 = 8 per compute unit), each thread keeping
 * `unroll` (1, 2, 4, 8 or 16) loads in flight. `sink` (>= 4 bytes, device) is written only if the data
 * sums to a value that random data never produces, so the loads cannot be removed.
 */
SKINNY_API skinny_status skinny_probe_read(const void *buf, int64_t bytes, float *sink,
                                           int32_t blocks, int32_t unroll, void *stream);

/*
 * Read `rows` rows of 7168 bytes at `buf` (16-byte aligned) the way the small-M kernels
 * stream W at K = 3584: workgroups of 448 threads (7 waves) own `rows_per_block` (4, 8, 16,
 * 28 or 32) contiguous rows, thread t loads 16-byte vector t of each row non-temporally, and
 * every load of a workgroup is issued before any is used. The single-launch ceiling of that
 * access pattern. `sink` as for skinny_probe_read.
 */
SKINNY_API skinny_status skinny_probe_read_rows(const void *buf, int64_t rows, int32_t rows_per_block,
                                                float *sink, void *stream);

/*
 * Launch `blocks` workgroups of `threads` threads that each stay busy for `nanoseconds`
 * (the 100 MHz real-time counter, so 10 ns steps) and touch no memory: call time minus
 * that duration is what one launch costs around a kernel that is busy, not empty.
 */
SKINNY_API skinny_status skinny_probe_spin(int64_t nanoseconds, int32_t blocks, int32_t threads, void *stream);

/* dst[0:bytes) = src[0:bytes) with 16-byte loads and stores (bytes % 16 == 0, both 16-B aligned). */
SKINNY_API skinny_status skinny_probe_copy(void *dst, const void *src, int64_t bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SKINNY_PROBE_H */
