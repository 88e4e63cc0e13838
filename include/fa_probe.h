/*
 * fa_probe.h -- measurement aid of the MI355X attention library (not part of
 * the backward): the sustained rate of the matrix instruction the tile
 * kernels are built on, to put their roofline in context.
 */
#ifndef FA_PROBE_H
#define FA_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Enqueues `blocks` workgroups of four waves (one wave per SIMD with one
 * workgroup per CU), each issuing 16 * iters back-to-back
 * v_mfma_f32_32x32x16_bf16 products (32768 FLOPs each) on random operand
 * bits drawn from `seed`, into four independent accumulators:
 *   mode 0: both operands from registers;
 *   mode 1: the A operand of every product a fresh 16-byte-per-lane read of a
 *           random 64 KB LDS tile (the operand supply of the tile kernels).
 * `out` is a DEVICE float buffer of blocks * 256 elements, caller-owned; it
 * only keeps the products live and is in practice never written.  Time the
 * call with events on `stream` (a hipStream_t; NULL: the default stream).
 * Returns 0, 1 for invalid arguments (nothing enqueued), 4 if the launch
 * failed. */
int fa_probe_mfma_rate(int mode, int blocks, int iters, uint32_t seed, float *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_PROBE_H */
