/*
 * swiglu_probe.h -- diagnostic kernels of libswiglu that measure what this
 * device actually sustains, for reading the fused kernel's roofline fraction
 * against more than the datasheet (the datasheet peaks assume the top clock
 * and ideal memory).  Not part of the fused product.
 *
 * Same conventions as swiglu.h: device pointers, `stream` is a hipStream_t
 * (NULL = default), calls enqueue and return, errors are swiglu_status codes.
 */
#ifndef SWIGLU_PROBE_H_
#define SWIGLU_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#include "swiglu.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Matrix-core ceiling: `blocks` workgroups of 256 threads each run `iters`
 * iterations of 8 independent v_mfma_f32_32x32x16_bf16 per wave on register
 * operands (no memory traffic).  Flops = blocks * 4 waves * iters * 8 * 32768.
 * `sink` (device, >= blocks * 256 floats) receives the accumulators so the
 * work cannot be elided.  blocks >= 1, iters >= 1. */
swiglu_status swiglu_probe_mfma(float *sink, int blocks, int iters, void *stream);

/* HBM read ceiling: streams `bytes` (multiple of 16, >= 16) from `src` with
 * 16-byte loads, grid-stride, and writes one 32-bit checksum per thread to
 * `sink` (device, >= blocks * 256 uint32).  blocks >= 1. */
swiglu_status swiglu_probe_read(const void *src, size_t bytes, uint32_t *sink, int blocks,
                                void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SWIGLU_PROBE_H_ */
