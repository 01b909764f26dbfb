/*
 * libmoe355 measurement probes: what one MI355X sustains, measured on the
 * same chip as the layer, so that the layer's kernels can be reported as a
 * fraction of a measured ceiling as well as of the published peaks
 * (HBM3E 8 TB/s, dense fp16 MFMA 2.5 PFLOP/s).  Not part of the layer.
 *
 * Conventions as in moe355.h: device pointers, asynchronous on `stream`,
 * MOE_OK or a negative MOE_ERR_* status; nothing is allocated.
 */
#ifndef MOE355_PROBE_H
#define MOE355_PROBE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* One launch that reads every byte of buf_dev[0 .. bytes) once in 16-byte
 * loads (bytes a multiple of 16, buf_dev 16-byte aligned) with `blocks`
 * workgroups of 256 threads; each block writes one word to sink_dev[block]
 * (sink_dev: `blocks` uint32 words).  Achieved HBM read bandwidth =
 * bytes / launch time when buf is not cached. */
int moe_probe_stream_read(const void* buf_dev, size_t bytes, uint32_t* sink_dev,
                          int32_t blocks, hipStream_t stream);

/* `blocks` workgroups of 4 waves, each wave running `iters` rounds of four
 * independent v_mfma_f32_32x32x16_f16 chains with register operands; every
 * thread writes one float to sink_dev[blocks * 256].  Flops of one launch:
 * moe_probe_mfma_f16_flops(iters, blocks). */
int moe_probe_mfma_f16(int32_t iters, float* sink_dev, int32_t blocks,
                       hipStream_t stream);
double moe_probe_mfma_f16_flops(int32_t iters, int32_t blocks);

#ifdef __cplusplus
}
#endif
#endif /* MOE355_PROBE_H */
