// Ceiling probes (libmoe_probes.so): streaming reads (grid-stride,
// block-contiguous, direct-to-LDS), a row gather, a memory-free MFMA loop
// and the expert GEMM's K-slice mix, the measured rates the layer's kernels are set
// against beside the datasheet peaks.  Only the benchmark and its tests
// call them.
#include "../../include/moe_probes.h"
#include "../csrc/common.h"

namespace moe_probes {

using moe::f32x4;
using moe::u32x4;
using moe::wave_sum;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Grid-stride sum over n4 16-byte elements; each thread keeps four loads in
// flight; one partial sum per block.
__global__ __launch_bounds__(256) void k_stream_read(const f32x4* __restrict__ buf, int64_t n4,
                                                     float* __restrict__ block_sums) {
  __shared__ float ws[4];
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
  for (; i + 3 * stride < n4; i += 4 * stride) {
    const f32x4 a = buf[i], b = buf[i + stride], c = buf[i + 2 * stride], d = buf[i + 3 * stride];
    s0 += (a[0] + a[1]) + (a[2] + a[3]);
    s1 += (b[0] + b[1]) + (b[2] + b[3]);
    s2 += (c[0] + c[1]) + (c[2] + c[3]);
    s3 += (d[0] + d[1]) + (d[2] + d[3]);
  }
  for (; i < n4; i += stride) {
    const f32x4 a = buf[i];
    s0 += (a[0] + a[1]) + (a[2] + a[3]);
  }
  const float s = wave_sum((s0 + s1) + (s2 + s3));
  if ((threadIdx.x & 63) == 0) ws[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) block_sums[blockIdx.x] = (ws[0] + ws[1]) + (ws[2] + ws[3]);
}

// Block-contiguous streaming read: block b reads its own contiguous share
// [b n/blocks, (b+1) n/blocks) in 32 KB steps (512 threads, four 16-byte
// loads each, issued together), so that concurrent reads fall in `blocks`
// separate regions rather than in one window moving over the buffer.  NT:
// the loads carry the non-temporal hint.
template <bool NT>
__global__ __launch_bounds__(512) void k_stream_read_blocks(const f32x4* __restrict__ buf,
                                                            int64_t per_block,
                                                            float* __restrict__ block_sums) {
  __shared__ float ws[8];
  const f32x4* base = buf + (int64_t)blockIdx.x * per_block;
  const int tid = threadIdx.x;
  auto ld = [](const f32x4* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
  };
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
  for (int64_t off = 0; off < per_block; off += 2048) {
    const f32x4 a = ld(base + off + tid), b = ld(base + off + 512 + tid),
                c = ld(base + off + 1024 + tid), d = ld(base + off + 1536 + tid);
    s0 += (a[0] + a[1]) + (a[2] + a[3]);
    s1 += (b[0] + b[1]) + (b[2] + b[3]);
    s2 += (c[0] + c[1]) + (c[2] + c[3]);
    s3 += (d[0] + d[1]) + (d[2] + d[3]);
  }
  const float s = wave_sum((s0 + s1) + (s2 + s3));
  if ((tid & 63) == 0) ws[tid >> 6] = s;
  __syncthreads();
  if (tid == 0)
    block_sums[blockIdx.x] = ((ws[0] + ws[1]) + (ws[2] + ws[3])) + ((ws[4] + ws[5]) + (ws[6] + ws[7]));
}

// The same streaming read through direct-to-LDS loads (global_load_lds,
// the expert GEMM's load kind): each block streams its contiguous share,
// 4 KB per step (lane l's 16 bytes land at LDS offset 16 l of its wave's
// 1 KB), 4 steps in flight; every thread then reads its own 16 bytes back
// from LDS and sums them, so the sums show every element was read.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

__global__ __launch_bounds__(256) void k_stream_read_lds(const f32x4* __restrict__ buf,
                                                         int64_t per_block,
                                                         float* __restrict__ block_sums) {
  __shared__ __attribute__((aligned(16))) f32x4 lds[4 * 256];
  __shared__ float ws[4];
  const f32x4* base = buf + (int64_t)blockIdx.x * per_block;
  const int tid = threadIdx.x, wave = tid >> 6;
  float s = 0.f;
  for (int64_t off = 0; off < per_block; off += 4 * 256) {
#pragma unroll
    for (int st = 0; st < 4; st++)
      __builtin_amdgcn_global_load_lds((gbl_void_t*)(base + off + st * 256 + tid),
                                       (lds_void_t*)(lds + st * 256 + wave * 64), 16, 0, 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies landed
#pragma unroll
    for (int st = 0; st < 4; st++) {
      const f32x4 a = lds[st * 256 + tid];
      s += (a[0] + a[1]) + (a[2] + a[3]);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): reads done before the next copies
  }
  s = wave_sum(s);
  if ((tid & 63) == 0) ws[wave] = s;
  __syncthreads();
  if (tid == 0) block_sums[blockIdx.x] = (ws[0] + ws[1]) + (ws[2] + ws[3]);
}

// Row gather: wave w reads the rows idx[w*per .. w*per + per) of a table
// of 16-byte units (U units per lane and row: lane l takes units l, l+64,
// ...), 8 rows in flight at a time, and sums them; one partial per wave.
// Indexes outside [0, n_rows) are clamped.
template <int U>
__global__ __launch_bounds__(256) void k_row_gather(const f32x4* __restrict__ table,
                                                    int64_t n_rows, const int32_t* __restrict__ idx,
                                                    int64_t n_waves, int per,
                                                    float* __restrict__ wave_sums) {
  constexpr int CH = 8;
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= n_waves) return;
  int myrow = 0;
  if (lane < per) {
    const int64_t r = idx[w * per + lane];
    myrow = (int)(r < 0 ? 0 : (r >= n_rows ? n_rows - 1 : r));
  }
  float s = 0.f;
  for (int j0 = 0; j0 < per; j0 += CH) {
    f32x4 v[CH][U];
#pragma unroll
    for (int c = 0; c < CH; c++)
      if (j0 + c < per) {
        const f32x4* row = table + (int64_t)__builtin_amdgcn_readlane(myrow, j0 + c) * (64 * U);
#pragma unroll
        for (int i = 0; i < U; i++) v[c][i] = row[lane + 64 * i];
      }
#pragma unroll
    for (int c = 0; c < CH; c++)
      if (j0 + c < per)
#pragma unroll
        for (int i = 0; i < U; i++) s += (v[c][i][0] + v[c][i][1]) + (v[c][i][2] + v[c][i][3]);
  }
  s = wave_sum(s);
  if (lane == 0) wave_sums[w] = s;
}

// The expert GEMM's K-slice work alone, at its shape: a 512-thread block of
// 8 waves (two per SIMD), each wave a 128 x 64 tile of 16x16x32 bf16 MFMAs
// (128 fp32 accumulators), 64-wide K tiles of A (256 rows) and B (256 rows)
// in LDS, 128 bytes per row, 16-byte chunks swizzled as in the GEMM, one
// barrier per K tile.  MODE 0: the MFMAs only, on fragments read once;
// MODE 1: + every fragment read from LDS at every 32-wide K step (12
// ds_read_b128 per wave per step); MODE 2: + the next K tile's 64 KB copied
// into the other of two LDS buffers with direct-to-LDS loads (8 per thread
// per K tile) from `src`, src_rows rows of 128 bytes that every block
// re-reads (a few MB: they stay in L2), all issued at the K tile's start;
// MODE 3: the same copies issued one after each MFMA row of the K tile's
// first 32-wide step, the order of the GEMM's own loop (which issues its
// copies over the rows of the step that follows its barrier).  64 MFMAs per
// wave per K tile.
template <int MODE>
__global__ __launch_bounds__(512, 1) void k_gemm_slice(const uint16_t* __restrict__ src,
                                                       int src_rows, int iters,
                                                       float* __restrict__ out) {
  constexpr int ROWS = 512, BK = 64;  // A rows 0..255, B rows 256..511
  __shared__ __attribute__((aligned(1024))) uint16_t lds[2][ROWS * BK];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3, frow = lane & 15;
  for (int i = tid; i < 2 * ROWS * BK / 8; i += 512)
    reinterpret_cast<u32x4*>(&lds[0][0])[i] = u32x4{0x3f803f80u, 0x3f803f80u, 0u, 0u};
  __syncthreads();
  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = f32x4{};
  bf16x8 afr[8], bfr[4];
  auto frag = [&](int buf, int row, int ks) {
    const int ch = ((ks * 4 + (lane >> 4)) ^ ((row >> 1) & 7)) * 8;
    return *reinterpret_cast<const bf16x8*>(&lds[buf][row * BK + ch]);
  };
  auto read_frags = [&](int buf, int ks) {
#pragma unroll
    for (int fm = 0; fm < 8; fm++) afr[fm] = frag(buf, wm * 128 + fm * 16 + frow, ks);
#pragma unroll
    for (int fn = 0; fn < 4; fn++) bfr[fn] = frag(buf, 256 + wn * 64 + fn * 16 + frow, ks);
  };
  // copy i (0..7) of the next K tile: wave w fills rows 64w + 8i .. + 7 of
  // the other buffer
  auto copy = [&](int it, int cur, int i) {
    const int r = wave * 64 + 8 * i;
    const int64_t sr = ((int64_t)(it + 1) * ROWS + r + (lane >> 3)) % src_rows;
    __builtin_amdgcn_global_load_lds((gbl_void_t*)(src + sr * BK + (lane & 7) * 8),
                                     (lds_void_t*)&lds[cur ^ 1][r * BK], 16, 0, 0);
  };
  if (MODE == 0) read_frags(0, 0);
  for (int it = 0; it < iters; it++) {
    const int cur = it & 1;
    if (MODE == 2)
#pragma unroll
      for (int i = 0; i < 8; i++) copy(it, cur, i);
#pragma unroll
    for (int ks = 0; ks < 2; ks++) {
      if (MODE >= 1) read_frags(cur, ks);
#pragma unroll
      for (int fm = 0; fm < 8; fm++) {
#pragma unroll
        for (int fn = 0; fn < 4; fn++)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[fn], afr[fm], acc[fm][fn],
                                                                0, 0, 0);
        if (MODE == 3 && ks == 0) copy(it, cur, fm);
      }
    }
    if (MODE >= 2) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies landed
    __syncthreads();
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) s += (acc[i][j][0] + acc[i][j][1]) + (acc[i][j][2] + acc[i][j][3]);
  if (s == -1.f) out[blockIdx.x] = s;  // never: keeps every chain live
  else if (tid == 0) out[blockIdx.x] = acc[0][0][0];
}

// 16 independent accumulator chains per wave (started at different values
// so that none can be merged), all-ones operands: each MFMA adds 32 to
// every element.
__global__ __launch_bounds__(512) void k_mfma_loop(int64_t iters, float* __restrict__ out) {
  bf16x8 one;
#pragma unroll
  for (int q = 0; q < 8; q++) one[q] = (__bf16)1.0f;
  f32x4 acc[16];
#pragma unroll
  for (int j = 0; j < 16; j++) acc[j] = f32x4{(float)j, 0.f, 0.f, 0.f};
  for (int64_t it = 0; it < iters; it++) {
#pragma unroll
    for (int j = 0; j < 16; j++)
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(one, one, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; j++) s += (acc[j][0] + acc[j][1]) + (acc[j][2] + acc[j][3]);
  if (s == -1.f) out[blockIdx.x] = s;  // never: keeps every chain live
  else if (threadIdx.x == 0) out[blockIdx.x] = acc[0][0];
}

}  // namespace moe_probes

extern "C" int32_t moe_probe_stream_read(const float* buf, int64_t n, float* block_sums,
                                         int blocks, moe_stream stream) {
  using namespace moe_probes;
  if (!buf || !block_sums) return MOE_ERR_NULL;
  if (n < 0 || n % 4 != 0 || blocks < 1 || blocks > 65536 || (uintptr_t)buf % 16 != 0)
    return MOE_ERR_SHAPE;
  hipLaunchKernelGGL(k_stream_read, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     reinterpret_cast<const f32x4*>(buf), n / 4, block_sums);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

extern "C" int32_t moe_probe_stream_read_blocks(const float* buf, int64_t n, float* block_sums,
                                                int blocks, int nontemporal, moe_stream stream) {
  using namespace moe_probes;
  if (!buf || !block_sums) return MOE_ERR_NULL;
  if (n < 0 || blocks < 1 || blocks > 65536 || (uintptr_t)buf % 16 != 0 ||
      n % ((int64_t)blocks * 8192) != 0)
    return MOE_ERR_SHAPE;
  const f32x4* b4 = reinterpret_cast<const f32x4*>(buf);
  if (nontemporal)
    hipLaunchKernelGGL(k_stream_read_blocks<true>, dim3((unsigned)blocks), dim3(512), 0,
                       (hipStream_t)stream, b4, n / 4 / blocks, block_sums);
  else
    hipLaunchKernelGGL(k_stream_read_blocks<false>, dim3((unsigned)blocks), dim3(512), 0,
                       (hipStream_t)stream, b4, n / 4 / blocks, block_sums);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

extern "C" int32_t moe_probe_stream_read_lds(const float* buf, int64_t n, float* block_sums,
                                             int blocks, moe_stream stream) {
  using namespace moe_probes;
  if (!buf || !block_sums) return MOE_ERR_NULL;
  if (n < 0 || blocks < 1 || blocks > 65536 || (uintptr_t)buf % 16 != 0 ||
      n % ((int64_t)blocks * 4096) != 0)
    return MOE_ERR_SHAPE;
  hipLaunchKernelGGL(k_stream_read_lds, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     reinterpret_cast<const f32x4*>(buf), n / 4 / blocks, block_sums);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

extern "C" int32_t moe_probe_mfma_loop(int64_t iters, float* out, int blocks,
                                       moe_stream stream) {
  using namespace moe_probes;
  if (!out) return MOE_ERR_NULL;
  if (iters < 1 || iters > (1 << 19) || blocks < 1 || blocks > 65536) return MOE_ERR_SHAPE;
  hipLaunchKernelGGL(k_mfma_loop, dim3((unsigned)blocks), dim3(512), 0, (hipStream_t)stream,
                     iters, out);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

extern "C" int32_t moe_probe_gemm_slice(int mode, const void* src, int src_rows, int iters,
                                        float* out, int blocks, moe_stream stream) {
  using namespace moe_probes;
  if (!out || (mode >= 2 && !src)) return MOE_ERR_NULL;
  if (mode < 0 || mode > 3 || iters < 1 || iters > (1 << 20) || blocks < 1 || blocks > 65536 ||
      (mode >= 2 && (src_rows < 512 || (uintptr_t)src % 16 != 0)))
    return MOE_ERR_SHAPE;
  const uint16_t* s16 = reinterpret_cast<const uint16_t*>(src);
  hipStream_t st = (hipStream_t)stream;
  if (mode == 0)
    hipLaunchKernelGGL(k_gemm_slice<0>, dim3((unsigned)blocks), dim3(512), 0, st, s16, src_rows, iters, out);
  else if (mode == 1)
    hipLaunchKernelGGL(k_gemm_slice<1>, dim3((unsigned)blocks), dim3(512), 0, st, s16, src_rows, iters, out);
  else if (mode == 2)
    hipLaunchKernelGGL(k_gemm_slice<2>, dim3((unsigned)blocks), dim3(512), 0, st, s16, src_rows, iters, out);
  else
    hipLaunchKernelGGL(k_gemm_slice<3>, dim3((unsigned)blocks), dim3(512), 0, st, s16, src_rows, iters, out);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

extern "C" int32_t moe_probe_row_gather(const void* table, int64_t n_rows, int row_bytes,
                                        const int32_t* idx, int64_t n_idx, int per_wave,
                                        float* wave_sums, moe_stream stream) {
  using namespace moe_probes;
  if (!table || !idx || !wave_sums) return MOE_ERR_NULL;
  if (n_rows < 1 || n_idx < 1 || per_wave < 1 || per_wave > 64 || n_idx % per_wave != 0 ||
      (row_bytes != 1024 && row_bytes != 2048 && row_bytes != 4096 && row_bytes != 8192) ||
      (uintptr_t)table % 16 != 0)
    return MOE_ERR_SHAPE;
  const int64_t n_waves = n_idx / per_wave;
  if ((n_waves + 3) / 4 > 0x7fffffff) return MOE_ERR_SHAPE;
  const dim3 grid((unsigned)((n_waves + 3) / 4)), block(256);
  const f32x4* t = reinterpret_cast<const f32x4*>(table);
  hipStream_t st = (hipStream_t)stream;
  switch (row_bytes) {
    case 1024: hipLaunchKernelGGL(k_row_gather<1>, grid, block, 0, st, t, n_rows, idx, n_waves, per_wave, wave_sums); break;
    case 2048: hipLaunchKernelGGL(k_row_gather<2>, grid, block, 0, st, t, n_rows, idx, n_waves, per_wave, wave_sums); break;
    case 4096: hipLaunchKernelGGL(k_row_gather<4>, grid, block, 0, st, t, n_rows, idx, n_waves, per_wave, wave_sums); break;
    default: hipLaunchKernelGGL(k_row_gather<8>, grid, block, 0, st, t, n_rows, idx, n_waves, per_wave, wave_sums); break;
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
