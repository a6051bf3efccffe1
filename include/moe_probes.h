/* Measured ceilings of this GPU, kept outside the MoE layer library
 * (libmoe_probes.so): the rates the layer's kernels are set against beside
 * the datasheet peaks.  Used only by the benchmark and its tests.
 */
#ifndef MOE_PROBES_H
#define MOE_PROBES_H

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read: sums buf[0..n) (fp32), every element read once with
 * 16-byte loads, blocks grid-striding over the buffer.
 *
 * buf: device, n floats, 16-byte aligned, n % 4 == 0.
 * block_sums: device, `blocks` floats, written (block b's partial sum; the
 *   caller adds them).  blocks in [1, 65536].
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (n < 0, n % 4, blocks out of range,
 *   misaligned buf); nothing is written on error.  Asynchronous on `stream`;
 *   allocates nothing.
 */
int32_t moe_probe_stream_read(const float* buf, int64_t n, float* block_sums, int blocks,
                              moe_stream stream);

/* MFMA loop: `blocks` blocks of 8 waves, each wave issuing `iters` rounds of
 * 16 independent v_mfma_f32_16x16x32_bf16 on all-ones operands, with no
 * memory traffic: 2*16*16*32 * 16 * 8 * iters * blocks FLOP.  Every
 * accumulator element ends at 32 * iters.
 *
 * out: device, `blocks` floats, written (one accumulator element of each
 *   block).  blocks in [1, 65536], iters in [1, 2^19] (so 32 * iters stays
 *   exact in fp32).
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE; nothing is written on error.
 *   Asynchronous on `stream`; allocates nothing.
 */
int32_t moe_probe_mfma_loop(int64_t iters, float* out, int blocks, moe_stream stream);

#ifdef __cplusplus
}
#endif

#endif
