/* Measurement reference of libqoq: a plain streaming read.
 *
 * Not part of the quantized GEMM. It gives the bandwidth one kernel launch
 * achieves on this GPU for a buffer of a given size, the reference against
 * which the weight-streaming GEMM kernels of small batches (a few MB read in
 * a few microseconds, where the launch ramp dominates) are compared. */
#ifndef QOQ_MEASURE_H
#define QOQ_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#include "qoq.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes of device memory at `buf` once, in 16-byte loads
 * spread over `workgroups` workgroups of 256 threads (0 selects 1024), four
 * independent loads in flight per thread. The loaded words are XOR-reduced
 * and the result is stored to *sink only when it equals a fixed unlikely
 * value, so the loads cannot be elided while nothing else is written.
 *   buf        device, 16-byte aligned, read only.
 *   bytes      > 0, a multiple of 16, at most 2^40.
 *   workgroups 0..65536.
 *   sink       device, 4 bytes, written at most once (normally never).
 * Enqueued on `stream`; no allocation or synchronization.
 * Errors: QOQ_ERR_NULL, QOQ_ERR_SHAPE, QOQ_ERR_ALIGN, QOQ_ERR_HIP. */
qoq_status qoq_stream_read(const void* buf, size_t bytes, int32_t workgroups, uint32_t* sink,
                           void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QOQ_MEASURE_H */
