/* moe_probe.h -- C ABI of libmoe_probe: two measurement kernels that give the
 * rates this MI355X actually reaches, against which the layer's kernels are
 * reported next to the published peaks (HBM 8 TB/s, dense bf16 MFMA
 * 2.5 PFLOP/s).  No page defines them; they are part of the measurement, not
 * of the method, and the layer library does not use them.
 *
 * Both are asynchronous on `stream`, allocate nothing, and return 0 or a
 * hipError_t value (nonzero) from the launch.
 */
#ifndef MOE_PROBE_H
#define MOE_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read: every 4 KiB piece of buf (device, `bytes` long, a multiple
 * of 4096, 16-byte aligned) is read once, grid-stride, by `blocks` blocks of
 * 4 waves, through direct global -> LDS loads (the load the layer's
 * weight-streaming kernels use) into an LDS slot nothing reads.  sink
 * (device) is written only when bytes == 0, which the checks reject: it is
 * there so the call has an output.  Bytes read = `bytes`. */
int moe_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, int blocks,
                          hipStream_t stream);

/* MFMA loop: `blocks` blocks of 4 waves, each wave issuing `iters` rounds of 8
 * independent v_mfma_f32_16x16x32_bf16 on register operands (16,384 FLOP
 * each, accumulators in AGPRs, nothing else in the loop); one float per thread is written to out (device, blocks * 256
 * floats).  FLOP = blocks * 4 * iters * 8 * 16384. */
int moe_probe_mfma_bf16(float* out, int blocks, int iters, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif
