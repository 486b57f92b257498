/* Peak microbenchmarks for MI355X (gfx950): what the chip reaches on this machine, so that the
 * roofline fractions reported by bench.py can be read against measured as well as
 * published peaks.  A measurement aid beside the attention library, built as its own
 * library (libssa_probe.so); no attention call uses it.
 *
 * Both calls only enqueue work on `stream` (a hipStream_t, NULL = the default stream) and
 * return the launch status as an int (0 = hipSuccess); the caller times them, e.g. with
 * events on the same stream.  Buffers are device memory the caller owns.
 */
#ifndef SSA_PROBE_H
#define SSA_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* blocks workgroups of four waves; every wave issues iters x 8 independent
 * v_mfma_f32_16x16x32_bf16 (16384 FLOP each) from registers, so the FLOP count is
 * blocks * 4 * iters * 8 * 16384.  out: blocks * 256 floats (the accumulators' sums, so
 * the products are not removed); blocks >= 1, iters >= 1. */
int ssa_probe_mfma_bf16(int blocks, int iters, float* out, void* stream);

/* Reads `bytes` (a multiple of 16, 16-byte aligned) of src once with 16-byte loads,
 * each of blocks workgroups of 256 threads reading one contiguous slice.  out: blocks * 256 * 16 bytes
 * (XOR of what each thread read, so the loads are not removed). */
int ssa_probe_hbm_read(const void* src, size_t bytes, int blocks, void* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif
