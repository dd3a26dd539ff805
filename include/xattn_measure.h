/*
 * xattn_measure.h -- measurement helpers of libxattn.so, kept apart from the
 * attention ABI (include/xattn.h): what the chip delivers, against which the
 * attention kernels' rates are read beside the published peaks.  Same
 * conventions as xattn.h: device pointers, asynchronous calls on `stream`,
 * status codes, nothing allocated.
 */
#ifndef XATTN_MEASURE_H
#define XATTN_MEASURE_H

#include "xattn.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * A matrix-core throughput probe.  Launches `blocks` workgroups of 256
 * threads, each wave running `iters` rounds of four independent
 * v_mfma_f32_32x32x16_bf16 chains on register operands, and writes one float per thread to `out` (device, at least
 * blocks * 256 floats; caller-owned).  *flops (if not NULL) receives the
 * floating-point operations the launch performs.  With both events given
 * (hipEvent_t, created and recorded by the caller) they are bound to the
 * dispatch, as in xattn_decode_timed; give both or neither.  The rate it
 * measures is what this chip's matrix cores deliver under a full load, at
 * the clock such a load holds: the reference against which the attention
 * kernels' MFMA fractions can be read beside the published peak.
 * Returns XATTN_EINVAL for iters or blocks < 1, a NULL or misaligned out,
 * or a single event.
 */
xattn_status xattn_peak_mfma_bf16(int32_t iters, int32_t blocks, float *out, void *stream,
                                  void *start_event, void *stop_event, double *flops);

/*
 * An HBM read probe.  `blocks` workgroups of 256 threads read the `bytes` (a positive multiple of 16) of
 * `src` (device, 16-byte aligned) once, with 16-byte non-temporal loads, and
 * write one word per thread to `out` (device, at least blocks * 256 words).
 * Events as for xattn_peak_mfma_bf16.  Its rate is the read bandwidth this
 * chip's HBM delivers to a plain stream: the reference for the attention
 * kernels' HBM fractions beside the published 8 TB/s.  Returns XATTN_EINVAL
 * for bad sizes, NULL or misaligned buffers, or a single event.
 */
xattn_status xattn_peak_read(const void *src, int64_t bytes, int32_t blocks, uint32_t *out,
                             void *stream, void *start_event, void *stop_event);

#ifdef __cplusplus
}
#endif

#endif /* XATTN_MEASURE_H */
