// Expert-centric dispatch: the batch's routing decisions flattened to tasks
// tau = t*k + j, grouped by expert id and sorted by token inside each group
// ("OmniMoE: An Efficient MoE by Orchestrating Atomic Experts at Scale",
// Technical Summary sec. 2.2, Expert-Centric Scheduling, steps Task
// Collection and Grouping & Sorting).
//
// A group is a contiguous range of `width` expert ids (one expert for
// routed FFN experts; one row of the expert grid for atomic experts), so
// the key of a task is its expert id / width.  The grouping is a stable LSD
// radix sort of the task ids by that key, 8 key bits per pass (one pass for
// up to 256 groups).
// Each pass is a per-tile digit histogram, one exclusive scan over
// (digit, tile) in digit-major order, and a stable scatter whose in-tile
// ranks come from wave ballots.  Stability of every pass keeps tasks of one
// expert in task order, i.e. by token.  Group offsets come from the scan
// (one pass) or from the segment boundaries of the sorted order (several
// passes).  The only atomics are integer adds on LDS counters, whose results
// do not depend on order, so the output is bit-exact and deterministic.
#include "kernels.h"
#include "tiles.h"

namespace moe {

constexpr int kRadixThreads = 256;
constexpr int kRadixItems = 4;
constexpr int kRadixTile = kRadixThreads * kRadixItems;
// single pass with at most this many tiles: the scatter scans the histogram
// itself (each block reads all of it), no separate scan launch
constexpr int kSelfScanTiles = 64;

__global__ void k_fill_i32(int32_t* p, int32_t v, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// Exclusive scan over the 256 threads of a block (4 waves): returns the
// sum of v over lower threads and sets total.  wsum: 4 ints of LDS.  Ends
// with a barrier, so wsum can be reused at once.
__device__ __forceinline__ int32_t block256_exclusive(int32_t v, int32_t* wsum, int32_t& total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int32_t pre = 0;
#pragma unroll
  for (int ww = 0; ww < 4; ww++) pre += ww < w ? wsum[ww] : 0;
  total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  __syncthreads();
  return pre + x - v;
}

// Multi-pass sorts: block `digit` scans its row hist[digit, 0..nb) of the
// tile histogram in place (exclusive, tiles in order) and writes the row
// total; the scatter adds the exclusive scan of the totals over digits.
__global__ __launch_bounds__(256) void k_digit_scan(int32_t* __restrict__ hist, int nb,
                                                    int32_t* __restrict__ totals) {
  __shared__ int32_t wsum[4];
  int32_t* row = hist + (int64_t)blockIdx.x * nb;
  int32_t carry = 0;
  for (int base = 0; base < nb; base += 256) {
    const int i = base + threadIdx.x;
    const int32_t v = i < nb ? row[i] : 0;
    int32_t tot;
    const int32_t ex = block256_exclusive(v, wsum, tot);
    if (i < nb) row[i] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) totals[blockIdx.x] = carry;
}

// Group key of an expert id: id / width (a shift when width is a power of
// two: wshift >= 0).
struct GroupKey {
  int width, wshift;
};
__device__ __forceinline__ int32_t group_of(int32_t e, GroupKey g) {
  return g.wshift >= 0 ? (e >> g.wshift) : (int32_t)((uint32_t)e / (uint32_t)g.width);
}

__device__ __forceinline__ int radix_digit(const int32_t* idx, int32_t task, int shift, int mask,
                                           GroupKey g) {
  return (group_of(idx[task], g) >> shift) & mask;
}

// Per-tile digit histogram: hist[digit * nb + tile].  Also sets zero[0..nz)
// to 0 (the counts that a later kernel accumulates), when given.
template <int ITEMS>
__global__ __launch_bounds__(kRadixThreads) void k_radix_hist(const int32_t* __restrict__ idx,
                                                              const int32_t* __restrict__ src,
                                                              int64_t n, int shift, int bits,
                                                              int32_t* __restrict__ hist, int nb,
                                                              int32_t* __restrict__ zero,
                                                              int64_t nz, GroupKey gk) {
  __shared__ int32_t cnt[256];
  const int tid = threadIdx.x;
  for (int64_t i = (int64_t)blockIdx.x * kRadixThreads + tid; i < nz;
       i += (int64_t)gridDim.x * kRadixThreads)
    zero[i] = 0;
  const int mask = (1 << bits) - 1;
  cnt[tid] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * kRadixThreads * ITEMS;
#pragma unroll
  for (int r = 0; r < ITEMS; r++) {
    int64_t i = base + r * kRadixThreads + tid;
    if (i < n) {
      int32_t task = src ? src[i] : (int32_t)i;
      atomicAdd(&cnt[radix_digit(idx, task, shift, mask, gk)], 1);
    }
  }
  __syncthreads();
  if (tid <= mask) hist[(int64_t)tid * nb + blockIdx.x] = cnt[tid];
}

// Stable scatter.  Items of a tile are taken in task order r*256 + w*64 + l;
// an item's destination is base[digit, tile] + (same-digit items earlier in
// the tile).  Same-digit lanes of a wave are found with one ballot per key
// bit.  base[digit, tile] is the row-scanned histogram plus the exclusive
// scan of the digit totals (k_digit_scan first); or, with scan_self (single
// pass, few tiles), each block scans the raw histogram itself: its digit's
// earlier tiles plus all smaller digits.  The last pass also writes the
// inverse permutation.  Block nb, when launched, is the single pass's extra
// block: it writes the group offsets and counts (E <= 256 digits), then
// builds the tile list when asked, while the other blocks scatter.
template <int ITEMS>
__global__ __launch_bounds__(kRadixThreads) void k_radix_scatter(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ src, int64_t n, int shift,
    int bits, const int32_t* __restrict__ hist, const int32_t* __restrict__ digit_totals,
    int nb, int32_t* __restrict__ dst, int32_t* __restrict__ inv, int scan_self, int E,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, TileBuild tb, GroupKey gk) {
  __shared__ int32_t run[256];
  __shared__ int32_t wcnt[kRadixThreads / 64][256];
  __shared__ int32_t wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int mask = (1 << bits) - 1;
  int32_t start;
  if (scan_self) {
    int32_t tot = 0, pre = 0;
    if (tid <= mask)
      for (int b = 0; b < nb; b++) {
        const int32_t v = hist[(int64_t)tid * nb + b];
        tot += v;
        pre += b < (int)blockIdx.x ? v : 0;
      }
    int32_t unused;
    const int32_t dbase = block256_exclusive(tot, wsum, unused);
    start = dbase + pre;
    if (blockIdx.x == nb) {
      if (tid < E) {
        offsets[tid] = dbase;
        counts[tid] = tot;
      }
      if (tid == 0) offsets[E] = (int32_t)n;
      __syncthreads();
    }
  } else {
    start = tid <= mask && (int)blockIdx.x < nb ? hist[(int64_t)tid * nb + blockIdx.x] : 0;
    if (digit_totals) {
      int32_t unused;
      const int32_t tot = tid <= mask ? digit_totals[tid] : 0;
      const int32_t dbase = block256_exclusive(tot, wsum, unused);
      start += dbase;
      if (blockIdx.x == nb && offsets) {  // a single pass's extra block
        if (tid < E) {
          offsets[tid] = dbase;
          counts[tid] = tot;
        }
        if (tid == 0) offsets[E] = (int32_t)n;
        __syncthreads();
      }
    }
  }
  if (blockIdx.x == nb) {
    if (tb.tiles) build_tile_list(offsets, tb);
    return;
  }
  run[tid] = start;
#pragma unroll
  for (int ww = 0; ww < kRadixThreads / 64; ww++) wcnt[ww][tid] = 0;
  __syncthreads();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t base = (int64_t)blockIdx.x * kRadixThreads * ITEMS;
  for (int r = 0; r < ITEMS; r++) {
    const int64_t i = base + r * kRadixThreads + tid;
    const bool valid = i < n;
    int32_t task = 0;
    int dg = 0;
    if (valid) {
      task = src ? src[i] : (int32_t)i;
      dg = radix_digit(idx, task, shift, mask, gk);
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

// Small batches (E <= 256, n <= kSmallDispatch): the whole dispatch in one
// block of 1024 threads -- LDS histogram, scan (offsets, counts), then the
// stable scatter tile by tile in task order (in-wave ranks from ballots, as
// in k_radix_scatter), then the tile list when asked.  One launch instead
// of three: decode-sized batches are bound by launch latency.
constexpr int kSmallDispatch = 4096;

__global__ __launch_bounds__(1024) void k_dispatch_small(const int32_t* __restrict__ idx,
                                                         int64_t n, int E, int bits,
                                                         int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ perm,
                                                         int32_t* __restrict__ inv,
                                                         TileBuild tb, GroupKey gk) {
  constexpr int kPer = kSmallDispatch / 1024;  // tasks per thread
  __shared__ int32_t cnt[256];
  __shared__ int32_t run[256];
  __shared__ int32_t off[257];  // the offsets, for the tile list
  __shared__ int32_t wcnt[16][256];
  __shared__ int32_t wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int mask = (1 << bits) - 1;
  if (tid < 256) cnt[tid] = 0;
  for (int i = tid; i < 16 * 256; i += 1024) (&wcnt[0][0])[i] = 0;
  // this thread's tasks' digits, loaded once (task tid + 1024 r)
  int dgs[kPer];
#pragma unroll
  for (int r = 0; r < kPer; r++) {
    const int64_t i = tid + 1024 * r;
    dgs[r] = i < n ? (group_of(idx[i], gk) & mask) : 0;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kPer; r++)
    if (tid + 1024 * r < n) atomicAdd(&cnt[dgs[r]], 1);
  __syncthreads();
  // exclusive scan of the 256 digit counts by the first 4 waves
  if (tid < 256) {
    const int32_t v = cnt[tid];
    int32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t y = __shfl_up(x, o, kWave);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[w] = x;
    cnt[tid] = x - v;  // exclusive within the wave for now
  }
  __syncthreads();
  if (tid < 256) {
    int32_t pre = 0;
    for (int ww = 0; ww < w; ww++) pre += wsum[ww];
    run[tid] = cnt[tid] + pre;
    if (tid < E) {
      offsets[tid] = run[tid];
      off[tid] = run[tid];
    }
  }
  if (tid == 0) {
    offsets[E] = (int32_t)n;
    off[E] = (int32_t)n;
  }
  __syncthreads();
  for (int e = tid; e < E; e += 1024)
    counts[e] = (e + 1 < E ? run[e + 1] : (int32_t)n) - run[e];
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int r = 0; r < kPer; r++) {
    if (1024 * r >= n) break;
    const int64_t i = tid + 1024 * r;
    const bool valid = i < n;
    const int dg = dgs[r];
    uint64_t same = __ballot(valid);
    for (int b = 0; b < bits; b++) {
      const uint64_t bb = __ballot(valid && ((dg >> b) & 1));
      same &= ((dg >> b) & 1) ? bb : ~bb;
    }
    const int rank = __popcll(same & lt_mask);
    if (valid && rank == 0) wcnt[w][dg] = __popcll(same);
    __syncthreads();
    if (valid) {
      int32_t pos = run[dg] + rank;
      for (int ww = 0; ww < w; ww++) pos += wcnt[ww][dg];
      perm[pos] = (int32_t)i;
      inv[i] = pos;
    }
    __syncthreads();
    if (tid < 256) {
      int32_t add = 0;
#pragma unroll
      for (int ww = 0; ww < 16; ww++) {
        add += wcnt[ww][tid];
        wcnt[ww][tid] = 0;
      }
      run[tid] += add;
    }
    __syncthreads();
  }
  if (tb.tiles)
    build_tile_list(off, tb);
}

// offsets[e] = first sorted position whose expert is >= e, read off the
// sorted order: position p writes every e in (key(p-1), key(p)] (key(-1) =
// -1, key(n) = E), so each of offsets[0..E] is written exactly once.  The key
// is the id's low `bits` bits -- what the passes sorted on -- clamped to E,
// which keeps it non-decreasing along the order even for ids outside [0, E)
// (a caller error: such tasks end up past offsets[E], in no expert's group).
// counts (zeroed beforehand) gets, for the segment [a, b) of each expert,
// -a from its first position and +b from its last: integer adds, so the
// result does not depend on their order.
__global__ void k_segment_offsets(const int32_t* __restrict__ idx, const int32_t* __restrict__ perm,
                                  int64_t n, int E, int bits, int32_t* __restrict__ offsets,
                                  int32_t* __restrict__ counts, GroupKey gk) {
  const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (p > n) return;
  const int32_t mask = (int32_t)((1u << bits) - 1);
  auto key = [&](int64_t q) {
    const int32_t e = group_of(idx[perm[q]], gk) & mask;
    return e > E ? E : e;
  };
  const int lo = p > 0 ? key(p - 1) : -1;
  const int hi = p < n ? key(p) : E;
  for (int e = lo + 1; e <= hi; e++) offsets[e] = (int32_t)p;
  if (p < n && hi < E) {
    if (lo < hi) atomicAdd(&counts[hi], -(int32_t)p);
    const int nx = p + 1 < n ? key(p + 1) : E;
    if (nx > hi) atomicAdd(&counts[hi], (int32_t)(p + 1));
  }
}

// ------------------------------------------------------------------------

int64_t dispatch_scratch_ints(int64_t n, int E) {
  int passes = 0;
  while ((1ll << (8 * passes)) < E) passes++;
  if (passes == 0) passes = 1;
  const int64_t nb = cdiv(n, kRadixTile);
  // hist (256 * nb), the digit totals; multi-pass sorts add one temp array
  // of n
  return 256 * nb + 256 + (passes > 1 ? n : 0);
}

bool dispatch_builds_tiles(int64_t n, int E) { return n > 0 && E <= 256; }

hipError_t launch_dispatch(const int32_t* idx, int64_t n, int E_ids, int width, int32_t* counts,
                           int32_t* offsets, int32_t* perm, int32_t* inv_perm, int32_t* scratch,
                           hipStream_t st, const TileBuild* tb) {
  // E: the number of groups from here on
  const int E = (int)cdiv(E_ids, width);
  GroupKey gk;
  gk.width = width;
  gk.wshift = -1;
  for (int b = 0; b < 31; b++)
    if ((1 << b) == width) gk.wshift = b;
  int bits = 0;
  while ((1ll << bits) < E) bits++;
  if (bits == 0) bits = 1;  // one expert: a pass on a constant digit keeps task order
  if (n == 0) {
    hipLaunchKernelGGL(k_fill_i32, dim3((unsigned)cdiv(E, 256)), dim3(256), 0, st, counts, 0,
                       (int64_t)E);
    hipLaunchKernelGGL(k_fill_i32, dim3((unsigned)cdiv(E + 1, 256)), dim3(256), 0, st, offsets,
                       0, (int64_t)E + 1);
    return hipGetLastError();
  }
  if (bits <= 8 && n <= kSmallDispatch) {
    TileBuild none;
    none.tiles = nullptr;
    hipLaunchKernelGGL(k_dispatch_small, dim3(1), dim3(1024), 0, st, idx, n, E, bits, counts,
                       offsets, perm, inv_perm, tb ? *tb : none, gk);
    return hipGetLastError();
  }
  if (bits <= 8) {
    // one pass: histogram, scan (+ counts and offsets), stable scatter
    const int nb = (int)cdiv(n, kRadixTile);
    int32_t* hist = scratch;
    hipLaunchKernelGGL(k_radix_hist<kRadixItems>, dim3(nb), dim3(kRadixThreads), 0, st, idx,
                       (const int32_t*)nullptr, n, 0, bits, hist, nb, (int32_t*)nullptr,
                       (int64_t)0, gk);
    TileBuild none;
    none.tiles = nullptr;
    const bool build = tb && tb->tiles;
    // few tiles: every scatter block scans the histogram itself; otherwise
    // one block per digit scans its row of tiles first.  The extra block
    // writes offsets and counts, and builds the tile list (E <= 256 <= its
    // threads).
    const int scan_self = nb <= kSelfScanTiles;
    int32_t* totals = hist + 256 * (int64_t)nb;
    if (!scan_self)
      hipLaunchKernelGGL(k_digit_scan, dim3(1u << bits), dim3(256), 0, st, hist, nb, totals);
    hipLaunchKernelGGL(k_radix_scatter<kRadixItems>, dim3(nb + 1), dim3(kRadixThreads), 0, st,
                       idx, (const int32_t*)nullptr, n, 0, bits, hist,
                       scan_self ? (const int32_t*)nullptr : (const int32_t*)totals, nb, perm,
                       inv_perm, scan_self, E, counts, offsets, build ? *tb : none, gk);
    return hipGetLastError();
  }
  // many experts: 8-bit LSD passes (hist, per-digit scan, scatter), then
  // offsets and counts read off the sorted order
  const int nb = (int)cdiv(n, kRadixTile);
  int32_t* hist = scratch;
  int32_t* totals = scratch + 256 * (int64_t)nb;
  int32_t* tmp = totals + 256;
  const int passes = (bits + 7) / 8;
  const int32_t* src = nullptr;
  for (int p = 0; p < passes; p++) {
    const int shift = 8 * p;
    const int pb = bits - shift < 8 ? bits - shift : 8;
    const bool last = p == passes - 1;
    // ping-pong so that the last pass lands in perm
    int32_t* dst = ((passes - 1 - p) % 2) ? tmp : perm;
    // the first pass also zeroes counts, which the segment kernel accumulates
    hipLaunchKernelGGL(k_radix_hist<kRadixItems>, dim3(nb), dim3(kRadixThreads), 0, st, idx, src,
                       n, shift, pb, hist, nb, p == 0 ? counts : (int32_t*)nullptr,
                       p == 0 ? (int64_t)E : (int64_t)0, gk);
    hipLaunchKernelGGL(k_digit_scan, dim3(1u << pb), dim3(256), 0, st, hist, nb, totals);
    TileBuild none;
    none.tiles = nullptr;
    hipLaunchKernelGGL(k_radix_scatter<kRadixItems>, dim3(nb), dim3(kRadixThreads), 0, st, idx,
                       src, n, shift, pb, hist, (const int32_t*)totals, nb, dst,
                       last ? inv_perm : (int32_t*)nullptr, 0, E, (int32_t*)nullptr,
                       (int32_t*)nullptr, none, gk);
    src = dst;
  }
  hipLaunchKernelGGL(k_segment_offsets, dim3((unsigned)cdiv(n + 1, 256)), dim3(256), 0, st, idx,
                     perm, n, E, bits, offsets, counts, gk);
  return hipGetLastError();
}

}  // namespace moe
