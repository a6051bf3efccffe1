// Tile list of the expert GEMMs and its XCD schedule, built by one block (the
// tile builder kernel, the small dispatch, or an extra block of the dispatch
// scatter).
#pragma once

#include "kernels.h"

namespace moe {

// Tile list: routed experts e < E_ffn get ceil(count_e / BM) tiles of
// sorted positions; shared expert s gets ceil(T / BM) tiles of tokens.  Each
// tile's descriptor names its whole group: {group, first row, rows, first
// tile}.  The gated GEMM runs every tile; the down projection runs the
// routed tiles and those of shared expert 0, whose group there spans all
// shared experts' K.
//
// Then the XCD schedule: contiguous item ranges of about equal cost, one
// per XCD, over all items in the gated GEMM and over the routed items in
// the down projection (whose shared items, the longest, are dealt to the
// XCDs in equal shares by the kernel itself).  The expert GEMMs are bound
// by the rate at which a CU pulls operand bytes from L2, and a
// 256-row-path item reads its 256 weight rows whatever its height: timed
// per block, an item costs about a fixed base plus 1 per 64 rows of its
// variant (base 3 in the gated GEMM, 4 in the down projection, whose
// shorter K leaves the weight reads a larger share).  Tiles of the other
// paths have one size and cost 1.  XCD x starts at the first item whose
// cost prefix reaches x/8 of the total; then any range longer than its
// share of the launch's blocks per XCD is cut back (cap1, cap2), so no item
// is left without a block.  One block of blockDim.x threads, a multiple of
// 64 with E_ffn <= blockDim.x <= 1024.

// rows-dependent part of an item's cost, and the base of GEMM g
__device__ __forceinline__ int tile_units(int BM, int rows) {
  return BM == 256 ? (rows + 63) / 64 : 0;
}
__device__ __forceinline__ int tile_base(int BM, int g) { return BM == 256 ? 3 + g : 1; }

// Tiles [first, first + n) of one group, all of `full` rows but the last of
// `last` rows, starting at cost prefix P[g] in GEMM g with cost weight w[g]
// (1, or 0: not in that GEMM's ranges): writes every XCD boundary that falls
// in them into bnd[g].  The boundaries' targets tgt[g][x] = ceil(x total_g
// nn_g / 8) are in LDS.  A target t lands in tile i (prefix Pi, cost c) when
// Pi*nn < t <= (Pi+c)*nn, at item i*nn + ceil((t - Pi*nn) / c).
__device__ __forceinline__ void place_targets(int first, int n, int full, int last, int BM,
                                              const int64_t (&P)[2],
                                              const int64_t (*tgts)[kXcds], const int (&w)[2],
                                              int nn1, int nn2, int32_t (*bnd)[kXcds + 1]) {
  // rolled loops: the kernel runs once per layer call on a cold instruction
  // cache, so its code must stay small; offsets inside one group fit in 32
  // bits, so the divisions are 32-bit
#pragma unroll 1
  for (int g = 0; g < 2; g++) {
    if (w[g] == 0) continue;
    const uint32_t cf = (tile_units(BM, full) + tile_base(BM, g)) * w[g];
    const uint32_t cl = (tile_units(BM, last) + tile_base(BM, g)) * w[g];
    const uint32_t nn = g == 0 ? nn1 : nn2;
    const int64_t lo = P[g] * nn, hi = (P[g] + (int64_t)(n - 1) * cf + cl) * nn;
#pragma unroll 1
    for (int x = 1; x < kXcds; x++) {
      const int64_t tgt = tgts[g][x];
      if (tgt <= lo || tgt > hi) continue;
      // full tiles first, then the last one
      const uint32_t d = (uint32_t)(tgt - lo);  // in [1, hi - lo]
      uint32_t i = (d - 1) / (cf * nn);
      if (i > (uint32_t)(n - 1)) i = n - 1;
      const uint32_t c = i == (uint32_t)(n - 1) ? cl : cf;
      const uint32_t r = d - i * cf * nn;       // target minus the tile's prefix, >= 1
      bnd[g][x] = (int32_t)((first + i) * nn + (r + c - 1) / c);
    }
  }
}

// Builds the tile list and the schedule with the calling block's threads
// (offsets must be visible to the whole block).
__device__ __forceinline__ void build_tile_list(const int32_t* __restrict__ offsets,
                                                const TileBuild& tb) {
  __shared__ int32_t wtot[2][16];
  __shared__ int32_t bnd[2][kXcds + 1];
  __shared__ int64_t tgts[2][kXcds];
  const int E_ffn = tb.E_ffn, n_shared = tb.n_shared, BM = tb.BM;
  const int64_t T = tb.T;
  const int e = threadIdx.x, nthreads = blockDim.x, nwaves = nthreads >> 6;
  const int cnt = e < E_ffn ? offsets[e + 1] - offsets[e] : 0;
  const int nt = (cnt + BM - 1) / BM;
  const int last = cnt - (nt - 1) * BM;
  const int ce = nt ? (nt - 1) * tile_units(BM, BM) + tile_units(BM, last) : 0;
  // inclusive scans of (nt, ce) over the block: within each wave by
  // shuffles, then across the wave totals
  const int lane = e & 63, wv = e >> 6;
  int sn = nt, sc = ce;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int a = __shfl_up(sn, o, 64), b = __shfl_up(sc, o, 64);
    if (lane >= o) { sn += a; sc += b; }
  }
  if (lane == 63) { wtot[0][wv] = sn; wtot[1][wv] = sc; }
  if (e < 2 * (kXcds + 1)) bnd[e / (kXcds + 1)][e % (kXcds + 1)] = 0;  // targets of an empty list
  __syncthreads();
  // the waves' totals, one per lane: inclusive scan, then the lanes before
  // this wave's and the last
  int qn = lane < nwaves ? wtot[0][lane] : 0, qc = lane < nwaves ? wtot[1][lane] : 0;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) {
    const int a = __shfl_up(qn, o, 64), b = __shfl_up(qc, o, 64);
    if (lane >= o) { qn += a; qc += b; }
  }
  const int bn = wv ? __shfl(qn, wv - 1, 64) : 0, bc = wv ? __shfl(qc, wv - 1, 64) : 0;
  const int tn = __shfl(qn, nwaves - 1, 64), tc = __shfl(qc, nwaves - 1, 64);
  const int start = bn + sn - nt;              // exclusive prefix of tile counts
  const int cstart = bc + sc - ce;             // exclusive prefix of tile row units
  const int routed_total = tn;
  // routed costs per GEMM: row units + base per tile
  const int64_t routed_cost[2] = {tc + (int64_t)tile_base(BM, 0) * tn,
                                  tc + (int64_t)tile_base(BM, 1) * tn};
  if (e < E_ffn) {
    const int base = offsets[e];
    for (int i = 0; i < nt; i++) tb.tiles[start + i] = make_int4(e, base, cnt, start);
  }
  const int per_shared = (int)((T + BM - 1) / BM);
  const int shared_last = (int)(T - (int64_t)(per_shared - 1) * BM);
  for (int j = e; j < n_shared * per_shared; j += nthreads) {
    const int s = j / per_shared;
    tb.tiles[routed_total + j] = make_int4(E_ffn + s, 0, (int)T, routed_total + s * per_shared);
  }
  const int64_t su = per_shared ? (int64_t)(per_shared - 1) * tile_units(BM, BM) +
                                      tile_units(BM, shared_last) : 0;
  const int64_t cs[2] = {su + (int64_t)tile_base(BM, 0) * per_shared,
                         su + (int64_t)tile_base(BM, 1) * per_shared};
  // the down projection's ranges hold its routed items only
  const int64_t total[2] = {routed_cost[0] + n_shared * cs[0], routed_cost[1]};
  const int items[2] = {(routed_total + n_shared * per_shared) * tb.nn1,
                        routed_total * tb.nn2};
  if (e < 2) bnd[e][kXcds] = items[e];
  if (e < 2 * kXcds) {
    const int g = e / kXcds, x = e % kXcds;
    tgts[g][x] = (x * total[g] * (g == 0 ? tb.nn1 : tb.nn2) + kXcds - 1) / kXcds;
  }
  __syncthreads();
  if (e < E_ffn && nt > 0) {
    const int64_t P[2] = {cstart + (int64_t)tile_base(BM, 0) * start,
                          cstart + (int64_t)tile_base(BM, 1) * start};
    const int w[2] = {1, 1};
    place_targets(start, nt, BM, last, BM, P, tgts, w, tb.nn1, tb.nn2, bnd);
  }
  if (e < n_shared && per_shared > 0) {
    const int64_t P[2] = {routed_cost[0] + e * cs[0], 0};
    const int w[2] = {1, 0};
    place_targets(routed_total + e * per_shared, per_shared, BM, shared_last, BM, P, tgts, w,
                  tb.nn1, tb.nn2, bnd);
  }
  __syncthreads();
  if (e < 2) {
    // no range longer than the launch's blocks per XCD: cut the ranges
    // from the front, then push the boundaries up from the back (the total
    // is at most 8 caps, so both passes together leave every range <= cap)
    int32_t* b = bnd[e];
    const int cap = e == 0 ? tb.cap1 : tb.cap2;
#pragma unroll 1
    for (int x = 1; x < kXcds; x++) b[x] = min(b[x], b[x - 1] + cap);
#pragma unroll 1
    for (int x = kXcds - 1; x >= 1; x--) b[x] = max(b[x], b[x + 1] - cap);
#pragma unroll 1
    for (int x = 0; x <= kXcds; x++) tb.sched[1 + e * (kXcds + 1) + x] = b[x];
    if (e == 1) {
      // the down projection as 128-row halves: an XCD runs one 256-row item
      // per CU at a time, so with R items on its 32 CUs it takes ceil(R/32)
      // rounds, or ceil(2R/32) rounds of halves; a half takes about 0.62 of
      // an item (measured: the 128-row tile reads 1.5x the bytes per FLOP)
      int R = 0;
#pragma unroll 1
      for (int x = 0; x < kXcds; x++) R = max(R, b[x + 1] - b[x]);
      R += (n_shared ? per_shared * (int)tb.nn2 + kXcds - 1 : 0) / kXcds;
      const int r1 = (R + 31) / 32, r2 = (2 * R + 31) / 32;
      tb.sched[1 + 2 * (kXcds + 1)] = (BM == 256 && 62 * r2 < 95 * r1) ? 1 : 0;
    }
  }
  if (e == 0) tb.sched[0] = routed_total + n_shared * per_shared;
}

}  // namespace moe
