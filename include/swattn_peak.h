/*
 * swattn_peak.h — achievable-peak probes of libswattn.so (measurement utilities, not part of
 * the attention operations).
 *
 * Results of the attention kernels are priced against the published MI355X peaks (dense
 * bf16 MFMA 2.5 PFLOP/s, HBM3E 8 TB/s) and, beside them, against what these probes
 * measure on the same device: a loop of nothing but bf16 matrix instructions, and
 * streaming copies / reads of a large buffer. The caller times the enqueued launch (e.g.
 * with events on `stream`).
 *
 * Conventions as in swattn.h: asynchronous on `stream` (a hipStream_t), nothing allocated,
 * SWA_OK or a negative swa_status (SWA_ERR_NULL, SWA_ERR_ARG, SWA_ERR_LAYOUT,
 * SWA_ERR_LAUNCH) with nothing enqueued on a host-detected error.
 */
#ifndef SWATTN_PEAK_H_
#define SWATTN_PEAK_H_

#include <stdint.h>

#include "swattn.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * swa_peak_mfma_bf16 — one workgroup of 8 waves per compute unit of the current device; every
 * wave issues iters x 8 v_mfma_f32_32x32x16_bf16 on register operands (4 independent
 * accumulators, no memory traffic in the loop).
 *   sink   device f32 [1]; written only in the impossible case that the accumulators sum to a
 *          sentinel (keeps the loop from being optimised away)
 *   iters  >= 1
 * swa_peak_mfma_bf16_flops(iters) returns the floating-point operations one such launch
 * performs on the current device (0 on a bad argument or when the device cannot be queried).
 */
int32_t swa_peak_mfma_bf16(float* sink, int32_t iters, void* stream);
double swa_peak_mfma_bf16_flops(int32_t iters);

/*
 * swa_peak_copy — dst[0:bytes) = src[0:bytes), 16 bytes per lane per access, grid-stride over
 * 4 workgroups of 256 lanes per compute unit. bytes > 0 and a multiple of 16; src and dst
 * 16-byte aligned and not overlapping. Moves 2 * bytes through HBM.
 */
int32_t swa_peak_copy(const void* src, void* dst, int64_t bytes, void* stream);

/*
 * swa_peak_read — reads src[0:bytes) once (16 bytes per lane per access) and folds it into a
 * value that reaches sink (device f32 [1]) only when it equals a sentinel. Same size and
 * alignment rules as swa_peak_copy.
 */
int32_t swa_peak_read(const void* src, int64_t bytes, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SWATTN_PEAK_H_ */
