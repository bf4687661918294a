/*
 * gqa_peaks.h -- C ABI of the measurement microkernels (libgqa_peaks.so),
 * separate from the layer library.  They give what one MI355X delivers to
 * a bf16 matrix-core loop and to a streaming read, so that the layer's
 * kernels can be reported against measured peaks beside the published ones
 * (the layer's prefill is bounded by the bf16 MFMA rate, its decode by HBM
 * bandwidth: "num_heads Is Not a Capacity Knob", "Why the cost does not
 * move" -- projections and score work are matrix products, and a
 * flash-style kernel changes only their memory traffic).
 *
 * Both calls only enqueue work on `stream` (a hipStream_t, NULL = default
 * stream) and never synchronize; the caller times them (HIP events on the
 * same stream).  Device pointers are owned by the caller.  Arguments are
 * checked on the host first: on error nothing is launched and the return
 * value is nonzero (1 = bad argument, 2 = launch failure).
 */
#ifndef GQA_PEAKS_H_
#define GQA_PEAKS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* bf16 MFMA-only loop: `workgroups` workgroups of 4 waves; each wave runs
 * `iters` rounds of 8 independent v_mfma_f32_32x32x16_bf16 on register
 * operands (no memory traffic inside the loop) and writes one float per
 * lane to sink[workgroups * 256] at the end.
 * Algorithmic work: workgroups * 4 * iters * 8 * 32768 FLOP.
 * workgroups in [1, 1 << 20], iters in [1, 1 << 24]. */
int gqa_peak_mfma_bf16(int32_t workgroups, int32_t iters, float* sink, void* stream);

/* Streaming read of `bytes` bytes from `buf` (16-byte aligned, bytes a
 * multiple of 16 * 256 * 8 = 32768) by `workgroups` workgroups of 256
 * lanes, 16-byte loads, each byte read once; every lane writes the XOR of
 * what it read to sink[workgroups * 256] (uint32).
 * Algorithmic work: `bytes` bytes read.  workgroups in [1, 1 << 20]. */
int gqa_peak_stream_read(const void* buf, size_t bytes, int32_t workgroups, uint32_t* sink,
                         void* stream);

#ifdef __cplusplus
}
#endif
#endif /* GQA_PEAKS_H_ */
