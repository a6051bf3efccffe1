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

/* Block-contiguous streaming read: block b sums floats
 * [b n/blocks, (b+1) n/blocks) with 16-byte loads, 32 KB per step (512
 * threads, four loads each).  Concurrent reads fall in `blocks` separate
 * regions instead of one window moving over the buffer.  nontemporal != 0:
 * the loads carry the non-temporal hint (data read once, not kept in the
 * caches).
 *
 * buf: device, n floats, 16-byte aligned; n a multiple of 8192 * blocks.
 * block_sums: device, `blocks` floats, written.  blocks in [1, 65536].
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE; nothing is written on error.
 *   Asynchronous on `stream`; allocates nothing.
 */
int32_t moe_probe_stream_read_blocks(const float* buf, int64_t n, float* block_sums, int blocks,
                                     int nontemporal, moe_stream stream);

/* The same read through direct-to-LDS loads (global_load_lds, the expert
 * GEMM's load kind): block b streams floats [b n/blocks, (b+1) n/blocks),
 * 4 KB per step, and sums what landed in LDS; the counter calibration of
 * the traffic records runs it beside a plain copy.
 *
 * buf: device, n floats, 16-byte aligned; n a multiple of 4096 * blocks.
 * block_sums: device, `blocks` floats, written.  blocks in [1, 65536].
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE; nothing is written on error.
 *   Asynchronous on `stream`; allocates nothing.
 */
int32_t moe_probe_stream_read_lds(const float* buf, int64_t n, float* block_sums, int blocks,
                                  moe_stream stream);

/* Row gather: n_idx / per_wave waves; wave w reads the table rows
 * idx[w*per_wave .. (w+1)*per_wave) whole (row_bytes each, 16-byte loads,
 * 8 rows in flight) and sums them as fp32: the access pattern of a token
 * gathering its k atomic experts' rows, with no other work.  n_idx *
 * row_bytes bytes are requested.
 *
 * table: device, n_rows * row_bytes bytes, 16-byte aligned; row_bytes in
 *   {1024, 2048, 4096, 8192}.  idx: device int32 [n_idx]; entries outside
 *   [0, n_rows) are clamped.  per_wave in [1, 64], n_idx % per_wave == 0.
 * wave_sums: device, n_idx / per_wave floats, written.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE; nothing is written on error.
 *   Asynchronous on `stream`; allocates nothing.
 */
int32_t moe_probe_row_gather(const void* table, int64_t n_rows, int row_bytes,
                             const int32_t* idx, int64_t n_idx, int per_wave,
                             float* wave_sums, moe_stream stream);

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

/* The expert GEMM's K-slice work alone, at its shape: `blocks` blocks of 8
 * waves, each wave a 128 x 64 tile of v_mfma_f32_16x16x32_bf16 (64 per wave
 * per 64-wide K tile), `iters` K tiles, one barrier per K tile.
 *   mode 0: the MFMAs only (fragments read from LDS once);
 *   mode 1: + every fragment read from LDS at every 32-wide K step;
 *   mode 2: + the next K tile's 64 KB copied into LDS with direct-to-LDS
 *           loads from src (src_rows rows of 128 bytes, re-read by every
 *           block: keep it a few MB, so that it stays in L2), all issued at
 *           the K tile's start;
 *   mode 3: the same copies issued one after each row of MFMAs of the K
 *           tile's first 32-wide step, the expert GEMM's own order.
 * 2*16*16*32 * 64 * 8 * iters * blocks FLOP.
 *
 * src: device, src_rows * 128 bytes, 16-byte aligned, src_rows >= 512 (modes
 *   2 and 3 only; ignored otherwise).  out: device, `blocks` floats, written.
 *   iters in [1, 2^20], blocks in [1, 65536].
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE; nothing is written on error.
 *   Asynchronous on `stream`; allocates nothing.
 */
int32_t moe_probe_gemm_slice(int mode, const void* src, int src_rows, int iters, float* out,
                             int blocks, moe_stream stream);

#ifdef __cplusplus
}
#endif

#endif
