/*
 * ssd_measure.h -- a measurement probe shipped with the library: an
 * achievable bf16 matrix-core rate on the current device, the denominator a
 * roofline needs next to the published peak. It computes nothing of the SSD
 * layer. Same conventions as ssd_api.h (device pointer, asynchronous on
 * `stream`, checks before the launch).
 */
#ifndef SSD_MEASURE_H
#define SSD_MEASURE_H

#include "ssd_api.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Launches `workgroups` work-groups of 4 waves; every wave runs `iters`
 * rounds of 8 independent v_mfma_f32_32x32x16_bf16 (32 x 32 x 16 products,
 * 32768 flops each) on register operands, then writes one float per lane to
 * out[workgroups * 256] so that nothing is optimised away. Flops per launch:
 * workgroups * 4 * iters * 8 * 32768. Time it with events on `stream`.
 * Errors: SSD_ERR_SHAPE (workgroups or iters < 1, or the flop count beyond
 * 2^62), SSD_ERR_NULL (out NULL), SSD_ERR_ALIGN, SSD_ERR_HIP.
 */
SSD_API ssd_status ssd_mfma_bf16_probe(int workgroups, int iters, float *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SSD_MEASURE_H */
