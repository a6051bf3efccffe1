// Expert-centric dispatch: the batch's routing decisions flattened to tasks
// tau = t*k + j, grouped by expert id and sorted by token inside each group
// ("OmniMoE: An Efficient MoE by Orchestrating Atomic Experts at Scale",
// Technical Summary sec. 2.2, Expert-Centric Scheduling, steps Task
// Collection and Grouping & Sorting).
//
// The grouping is a stable LSD radix sort of the task ids keyed by expert
// id, 8 key bits per pass (one pass for up to 256 experts, two for 65,536).
// Each pass is a per-tile digit histogram, one exclusive scan over
// (digit, tile) in digit-major order, and a stable scatter whose in-tile
// ranks come from wave ballots.  Stability of every pass keeps tasks of one
// expert in task order, i.e. by token.  Only integer atomics on LDS or
// per-expert counters are used, and their results do not depend on order,
// so the output is bit-exact and deterministic.
#include "kernels.h"

namespace moe {

constexpr int kRadixThreads = 256;
constexpr int kRadixItems = 4;
constexpr int kRadixTile = kRadixThreads * kRadixItems;

__global__ void k_fill_i32(int32_t* p, int32_t v, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// ids outside [0, E) are not counted (they are a caller error; skipping
// them keeps every access in bounds)
__global__ void k_count_experts(const int32_t* __restrict__ idx, int64_t n, int E,
                                int32_t* counts) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    const int32_t e = idx[i];
    if ((uint32_t)e < (uint32_t)E) atomicAdd(&counts[e], 1);
  }
}

// Exclusive scan of n ints by one block of 1024 threads: out[0] = 0,
// out[i] = in[0] + ... + in[i-1]; also writes out[n] (the total) when
// write_total.  in and out may alias.
__global__ __launch_bounds__(1024) void k_scan_single_block(const int32_t* in, int32_t* out,
                                                            int64_t n, int write_total) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  const int64_t per = (n + 1023) / 1024;
  const int64_t lo = tid * per;
  const int64_t hi = lo + per < n ? lo + per : n;
  int32_t s = 0;
  for (int64_t i = lo; i < hi; i++) s += in[i];
  part[tid] = s;
  __syncthreads();
  // Hillis-Steele inclusive scan over the 1024 partial sums
  for (int o = 1; o < 1024; o <<= 1) {
    int32_t v = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int32_t run = tid ? part[tid - 1] : 0;
  for (int64_t i = lo; i < hi; i++) {
    int32_t v = in[i];
    out[i] = run;
    run += v;
  }
  if (write_total && tid == 1023) out[n] = part[1023];
}

// Multi-block exclusive scan for long arrays: each block of 256 threads
// covers 4096 consecutive ints (16 per thread, loaded as four 16-byte
// vectors); pass 1 writes block totals, the totals are scanned by one
// block, pass 2 rescans each block locally and adds its offset.
constexpr int kScanThreads = 256;
constexpr int kScanPer = 16;
constexpr int kScanTile = kScanThreads * kScanPer;

__device__ __forceinline__ int32_t block_exclusive_sum(int32_t v, int32_t* lds_w, int32_t& total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int32_t inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int32_t t = __shfl_up(inc, o, 64);
    if (lane >= o) inc += t;
  }
  if (lane == 63) lds_w[w] = inc;
  __syncthreads();
  int32_t wbase = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < kScanThreads / 64; i++) {
    const int32_t t = lds_w[i];
    if (i < w) wbase += t;
    total += t;
  }
  return wbase + inc - v;
}

__device__ __forceinline__ void load16(const int32_t* in, int64_t n, int64_t base, int32_t v[16]) {
  if (base + 16 <= n && ((uintptr_t)(in + base) & 15) == 0) {
#pragma unroll
    for (int q = 0; q < 4; q++) {
      int4 t = reinterpret_cast<const int4*>(in + base)[q];
      v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; i++) v[i] = base + i < n ? in[base + i] : 0;
  }
}

__global__ __launch_bounds__(kScanThreads) void k_scan_totals(const int32_t* __restrict__ in,
                                                              int64_t n,
                                                              int32_t* __restrict__ totals) {
  __shared__ int32_t lds_w[kScanThreads / 64];
  const int64_t base = (int64_t)blockIdx.x * kScanTile + threadIdx.x * kScanPer;
  int32_t v[16];
  load16(in, n, base, v);
  int32_t s = 0;
#pragma unroll
  for (int i = 0; i < 16; i++) s += v[i];
  int32_t total;
  block_exclusive_sum(s, lds_w, total);
  if (threadIdx.x == 0) totals[blockIdx.x] = total;
}

// out may alias in.  offsets: scanned block totals (nullptr: one block).
__global__ __launch_bounds__(kScanThreads) void k_scan_finish(const int32_t* in, int32_t* out,
                                                              int64_t n,
                                                              const int32_t* __restrict__ offsets,
                                                              int32_t* total_out) {
  __shared__ int32_t lds_w[kScanThreads / 64];
  const int64_t base = (int64_t)blockIdx.x * kScanTile + threadIdx.x * kScanPer;
  int32_t v[16];
  load16(in, n, base, v);
  int32_t s = 0;
#pragma unroll
  for (int i = 0; i < 16; i++) s += v[i];
  int32_t total;
  int32_t run = block_exclusive_sum(s, lds_w, total) + (offsets ? offsets[blockIdx.x] : 0);
#pragma unroll
  for (int i = 0; i < 16; i++) {
    if (base + i < n) out[base + i] = run;
    run += v[i];
  }
  if (total_out && blockIdx.x == gridDim.x - 1 && threadIdx.x == 0)
    *total_out = (offsets ? offsets[blockIdx.x] : 0) + total;
}

// exclusive scan of n ints (in may equal out); writes *total_out when given.
// scratch: cdiv(n, 4096) + 1 ints.
static void exclusive_scan(const int32_t* in, int32_t* out, int64_t n, int32_t* total_out,
                           int32_t* scratch, hipStream_t st) {
  const int64_t nblk = cdiv(n, kScanTile);
  if (nblk <= 1) {
    hipLaunchKernelGGL(k_scan_finish, dim3(1), dim3(kScanThreads), 0, st, in, out, n,
                       (const int32_t*)nullptr, total_out);
    return;
  }
  hipLaunchKernelGGL(k_scan_totals, dim3((unsigned)nblk), dim3(kScanThreads), 0, st, in, n,
                     scratch);
  hipLaunchKernelGGL(k_scan_single_block, dim3(1), dim3(1024), 0, st, scratch, scratch, nblk, 0);
  hipLaunchKernelGGL(k_scan_finish, dim3((unsigned)nblk), dim3(kScanThreads), 0, st, in, out, n,
                     (const int32_t*)scratch, total_out);
}

// Single-pass dispatch (E <= 256): exclusive scan of the digit-major tile
// histogram in place, and from it the expert offsets (the scanned value at
// (e, tile 0)) and counts.
__global__ __launch_bounds__(1024) void k_dispatch_scan(int32_t* hist, int64_t len, int nb, int E,
                                                        int64_t n, int32_t* __restrict__ counts,
                                                        int32_t* __restrict__ offsets) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  const int64_t per = (len + 1023) / 1024;
  const int64_t lo = tid * per;
  const int64_t hi = lo + per < len ? lo + per : len;
  int32_t s = 0;
  for (int64_t i = lo; i < hi; i++) s += hist[i];
  part[tid] = s;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    int32_t v = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int32_t run = tid ? part[tid - 1] : 0;
  for (int64_t i = lo; i < hi; i++) {
    int32_t v = hist[i];
    hist[i] = run;
    if (i % nb == 0 && i / nb < E) offsets[i / nb] = run;
    run += v;
  }
  if (tid == 0) offsets[E] = (int32_t)n;
  __syncthreads();
  for (int e = tid; e < E; e += 1024) counts[e] = offsets[e + 1] - offsets[e];
}

__device__ __forceinline__ int radix_digit(const int32_t* idx, int32_t task, int shift, int mask) {
  return (idx[task] >> shift) & mask;
}

// Per-tile digit histogram: hist[digit * nb + tile].
__global__ __launch_bounds__(kRadixThreads) void k_radix_hist(const int32_t* __restrict__ idx,
                                                              const int32_t* __restrict__ src,
                                                              int64_t n, int shift, int bits,
                                                              int32_t* __restrict__ hist, int nb) {
  __shared__ int32_t cnt[256];
  const int tid = threadIdx.x;
  const int mask = (1 << bits) - 1;
  cnt[tid] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * kRadixTile;
#pragma unroll
  for (int r = 0; r < kRadixItems; r++) {
    int64_t i = base + r * kRadixThreads + tid;
    if (i < n) {
      int32_t task = src ? src[i] : (int32_t)i;
      atomicAdd(&cnt[radix_digit(idx, task, shift, mask)], 1);
    }
  }
  __syncthreads();
  if (tid <= mask) hist[(int64_t)tid * nb + blockIdx.x] = cnt[tid];
}

// Stable scatter.  Items of a tile are taken in task order r*256 + w*64 + l;
// an item's destination is base[digit, tile] + (same-digit items earlier in
// the tile).  Same-digit lanes of a wave are found with one ballot per key
// bit.  The last pass also writes the inverse permutation.
__global__ __launch_bounds__(kRadixThreads) void k_radix_scatter(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ src, int64_t n, int shift,
    int bits, const int32_t* __restrict__ hist_scanned, int nb, int32_t* __restrict__ dst,
    int32_t* __restrict__ inv) {
  __shared__ int32_t run[256];
  __shared__ int32_t wcnt[kRadixThreads / 64][256];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int mask = (1 << bits) - 1;
  run[tid] = tid <= mask ? hist_scanned[(int64_t)tid * nb + blockIdx.x] : 0;
#pragma unroll
  for (int ww = 0; ww < kRadixThreads / 64; ww++) wcnt[ww][tid] = 0;
  __syncthreads();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t base = (int64_t)blockIdx.x * kRadixTile;
  for (int r = 0; r < kRadixItems; r++) {
    const int64_t i = base + r * kRadixThreads + tid;
    const bool valid = i < n;
    int32_t task = 0;
    int dg = 0;
    if (valid) {
      task = src ? src[i] : (int32_t)i;
      dg = radix_digit(idx, task, shift, mask);
    }
    uint64_t same = __ballot(valid);
    for (int b = 0; b < bits; b++) {
      uint64_t bb = __ballot(valid && ((dg >> b) & 1));
      same &= ((dg >> b) & 1) ? bb : ~bb;
    }
    const int rank = __popcll(same & lt_mask);
    if (valid && rank == 0) wcnt[w][dg] = __popcll(same);
    __syncthreads();
    if (valid) {
      int32_t pos = run[dg] + rank;
      for (int ww = 0; ww < w; ww++) pos += wcnt[ww][dg];
      dst[pos] = task;
      if (inv) inv[task] = pos;
    }
    __syncthreads();
    int32_t add = 0;
#pragma unroll
    for (int ww = 0; ww < kRadixThreads / 64; ww++) {
      add += wcnt[ww][tid];
      wcnt[ww][tid] = 0;
    }
    run[tid] += add;
    __syncthreads();
  }
}

// ------------------------------------------------------------------------

int64_t dispatch_scratch_ints(int64_t n, int E) {
  int bits = 0;
  while ((1ll << bits) < E) bits++;
  int passes = bits ? (bits + 7) / 8 : 1;
  int64_t nb = cdiv(n, kRadixTile);
  // hist (256 * nb) + for multi-pass sorts one temp array of n and the
  // scan's block totals
  const int64_t scan = cdiv((256 * nb > E ? 256 * nb : E), kScanTile) + 1;
  return 256 * nb + (passes > 1 ? n + scan : 0);
}

hipError_t launch_dispatch(const int32_t* idx, int64_t n, int E, int32_t* counts,
                           int32_t* offsets, int32_t* perm, int32_t* inv_perm, int32_t* scratch,
                           hipStream_t st) {
  int bits = 0;
  while ((1ll << bits) < E) bits++;
  if (bits == 0) bits = 1;  // one expert: a pass on a constant digit keeps task order
  const int nb = (int)cdiv(n, kRadixTile);
  int32_t* hist = scratch;
  int32_t* tmp = scratch + 256 * (int64_t)nb;
  if (n == 0) {
    hipLaunchKernelGGL(k_fill_i32, dim3((unsigned)cdiv(E, 256)), dim3(256), 0, st, counts, 0,
                       (int64_t)E);
    hipLaunchKernelGGL(k_fill_i32, dim3((unsigned)cdiv(E + 1, 256)), dim3(256), 0, st, offsets,
                       0, (int64_t)E + 1);
    return hipGetLastError();
  }
  if (bits <= 8) {
    // one pass: histogram, scan (+ counts and offsets), stable scatter
    hipLaunchKernelGGL(k_radix_hist, dim3(nb), dim3(kRadixThreads), 0, st, idx,
                       (const int32_t*)nullptr, n, 0, bits, hist, nb);
    hipLaunchKernelGGL(k_dispatch_scan, dim3(1), dim3(1024), 0, st, hist,
                       (int64_t)(1 << bits) * nb, nb, E, n, counts, offsets);
    hipLaunchKernelGGL(k_radix_scatter, dim3(nb), dim3(kRadixThreads), 0, st, idx,
                       (const int32_t*)nullptr, n, 0, bits, hist, nb, perm, inv_perm);
    return hipGetLastError();
  }
  // many experts: per-expert counts by atomics on global counters (spread
  // over many bins), then 8-bit LSD passes
  hipLaunchKernelGGL(k_fill_i32, dim3((unsigned)cdiv(E, 256)), dim3(256), 0, st, counts, 0,
                     (int64_t)E);
  hipLaunchKernelGGL(k_count_experts, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, st, idx, n, E,
                     counts);
  int32_t* scan_scratch = tmp + n;
  exclusive_scan(counts, offsets, (int64_t)E, offsets + E, scan_scratch, st);
  const int passes = (bits + 7) / 8;
  const int32_t* src = nullptr;
  for (int p = 0; p < passes; p++) {
    const int shift = 8 * p;
    const int pb = bits - shift < 8 ? bits - shift : 8;
    const bool last = p == passes - 1;
    // ping-pong so that the last pass lands in perm
    int32_t* dst = ((passes - 1 - p) % 2) ? tmp : perm;
    hipLaunchKernelGGL(k_radix_hist, dim3(nb), dim3(kRadixThreads), 0, st, idx, src, n, shift,
                       pb, hist, nb);
    exclusive_scan(hist, hist, (int64_t)(1 << pb) * nb, (int32_t*)nullptr, scan_scratch, st);
    hipLaunchKernelGGL(k_radix_scatter, dim3(nb), dim3(kRadixThreads), 0, st, idx, src, n, shift,
                       pb, hist, nb, dst, last ? inv_perm : (int32_t*)nullptr);
    src = dst;
  }
  return hipGetLastError();
}

}  // namespace moe
