/* gsa_probe.h -- a measurement aid, not part of the operator.
 *
 * libgsa_probe.so holds two small kernels for the benchmark.  A plain
 * streaming-read kernel, run over >= 1 GiB of device memory, reports the HBM
 * read bandwidth a simple kernel achieves on the same GPU, beside the 8 TB/s
 * datasheet peak that the operator's roofline figure is taken against.  A
 * bounded spin kernel keeps the GPU busy while the host enqueues a timed
 * region, so that host-side launch work never shows in the measured time.
 * Neither computes anything the operator needs.
 */
#ifndef GSA_PROBE_H
#define GSA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes at device pointer `src` (16-byte aligned, bytes a
 * multiple of 16, bytes / 16 < 2^31) with non-temporal 128-bit loads, `grid`
 * workgroups of 256 threads, each over one contiguous segment of about
 * bytes / grid bytes, eight loads in flight per thread, and fold them into one word per
 * workgroup that is written to sink[blockIdx] only if it equals a value no
 * input is expected to produce (so the loads cannot be optimised away).
 * sink must hold `grid` uint32 words.  Enqueued on `stream` (a hipStream_t,
 * NULL = default stream).  Returns 0, -1 (bad argument) or -3 (launch
 * failed). */
int gsa_probe_read(const void *src, size_t bytes, uint32_t *sink, int grid, void *stream);

/* Enqueue one single-wave kernel on `stream` that spins for `us`
 * microseconds of device wall-clock time (1 <= us <= 1000000) and returns.
 * Returns 0, -1 (bad argument) or -3 (HIP query or launch failed). */
int gsa_probe_spin(uint32_t us, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GSA_PROBE_H */
