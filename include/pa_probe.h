/*
 * pa_probe.h -- measurement kernels for the MI355X (gfx950) rooflines the attention library is
 * judged against.  They compute nothing of the method: they read memory and run the matrix
 * cores as fast as plain code can, so that a benchmark can report each attention kernel's rate
 * against a measured ceiling beside the published one.  Built as libpa_probe.so, separate
 * from libpa.so.
 *
 * Conventions: device pointers are HIP device addresses of caller-owned buffers; `stream` is a
 * hipStream_t (NULL = the default stream); every call only enqueues kernels (no allocation, no
 * synchronisation) and returns 0, or -1 for an argument out of range, or -13 if the launch
 * failed.  Timing is the caller's (events on the same stream).
 */
#ifndef PA_PROBE_H_
#define PA_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes of device memory at `src` once, with 16-byte loads from a grid of
 * `blocks` workgroups of 256 threads striding over the buffer (four loads in flight per
 * thread).  bytes must be a positive multiple of 16 and src 16-byte aligned; blocks in
 * [1, 65536].  The loaded values feed a checksum that is written to sink[blockIdx] only when it
 * equals a constant no real input produces, so the loads cannot be removed and nothing else is
 * written; sink must hold `blocks` uint32 values. */
int32_t pa_probe_read(const void* src, size_t bytes, int32_t blocks, void* sink, void* stream);

/* Run the matrix cores: `blocks` workgroups of 256 threads, each wavefront issuing `iters`
 * rounds of 8 independent bf16 MFMAs (shape 16: v_mfma_f32_16x16x32_bf16, 16,384 flops each;
 * shape 32: v_mfma_f32_32x32x16_bf16, 32,768 flops each) on register operands.  Flops of one
 * call = blocks * 4 * iters * 8 * (16,384 or 32,768).  blocks in [1, 65536], iters in
 * [1, 2^20], shape 16 or 32.  sink: `blocks` floats, written only under the same never-true
 * test. */
int32_t pa_probe_mfma(int32_t blocks, int32_t iters, int32_t shape, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H_ */
