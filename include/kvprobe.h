/*
 * kvint2 measurement aid (not part of the quantisation or attention path):
 * the achievable matrix-core rate of the current GPU, which benchmarks
 * report as the measured denominator of an MFMA roofline beside the
 * vendor's dense fp16 figure.
 */
#ifndef KVPROBE_H
#define KVPROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Launches `blocks` blocks of 256 threads (four waves) on `stream`; every
 * wave issues iters x 8 independent v_mfma_f32_16x16x32_f16 (16 x 16 x 32
 * fp16 products, fp32 accumulation: 16384 flops each) on register operands
 * and touches no memory in its loop, so one launch performs
 * blocks * 4 * iters * 8 * 16384 flops; time it with events on `stream`.
 * out_dev: device f32 [blocks * 256], written (a checksum that keeps the
 * work live; its value is meaningless).  Errors: KVQ_EINVAL (null out_dev,
 * blocks outside 1..2^20, iters outside 1..2^24), KVQ_EHIP (launch error). */
int kvq_mfma_peak_probe(float* out_dev, int32_t blocks, int32_t iters, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* KVPROBE_H */
