// Ceiling probes (libmoe_probes.so): a streaming read and a memory-free
// MFMA loop, the measured rates the layer's kernels are set against beside
// the datasheet peaks.  Only the benchmark and its tests call them.
#include "../../include/moe_probes.h"
#include "../csrc/common.h"

namespace moe_probes {

using moe::f32x4;
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

extern "C" int32_t moe_probe_mfma_loop(int64_t iters, float* out, int blocks,
                                       moe_stream stream) {
  using namespace moe_probes;
  if (!out) return MOE_ERR_NULL;
  if (iters < 1 || iters > (1 << 19) || blocks < 1 || blocks > 65536) return MOE_ERR_SHAPE;
  hipLaunchKernelGGL(k_mfma_loop, dim3((unsigned)blocks), dim3(512), 0, (hipStream_t)stream,
                     iters, out);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
