// Internal launchers of the gfx950 MoE kernels (not part of the C ABI).
#pragma once

#include "common.h"

namespace moe {

// Work schedule written by the tile builder, on device: [0] = number of M
// tiles; [1 + 9 g + x] = first work item of XCD x (x = 0..7) for GEMM g
// (g = 0: the gated GEMM, 1: the down projection), [1 + 9 g + 8] = number of
// work items.  A work item is one (M tile, N tile) pair, M-tile major.
constexpr int kXcds = 8;
// schedule: valid tiles, each GEMM's 9 XCD boundaries, then whether the
// down projection runs its items as two 128-row halves
constexpr int kSchedInts = 1 + 2 * (kXcds + 1) + 1;

struct GemmArgs {
  const int4* tiles;         // per M tile: {group, group's first row, group's rows, group's first tile}
  const int32_t* ntiles;     // device count of valid tiles (schedule entry 0)
  const int32_t* xcd_first;  // this GEMM's 9 XCD boundaries in the schedule
  int E_ffn;
  int64_t T;
  // A operand
  const void* a_x;         // GEMM1: x [T, d], rows gathered
  const int32_t* perm;     // GEMM1 routed rows: token = perm[p] / k
  int k;
  const void* a_routed;    // GEMM2: H rows of routed tasks [*, f]
  const void* a_shared;    // GEMM2: H of the shared experts [T, n_shared*f_shared]
  // B operand, [groups, N, K] each
  const void* b0_routed;
  const void* b1_routed;
  const void* b0_shared;
  const void* b1_shared;
  // C
  void* c_routed;
  void* c_shared;
  int N_routed, N_shared;  // output columns (of one shared group)
  int K_routed, K_shared;
  // Shared experts.  Gated GEMM: one group per expert s (B rows s*f_shared
  // on of the [n_shared f_shared, d] weights), writing columns s*f_shared
  // on of H [T, n_shared f_shared].  Down projection: one group (group s = 0)
  // with K = n_shared f_shared: expert s's K slice is its own [d, f_shared]
  // block, so the experts' sum comes out of one accumulation.  B row n of
  // shared group s starts at (s*N + n) * b_ld_shared; K element k lies in
  // slice k / k_seg_shared, whose block starts b_seg_shared elements after
  // the previous one; C row r of group s starts at r * c_ld_shared + s*N.
  int b_ld_shared;
  int k_seg_shared;
  int64_t b_seg_shared;
  int64_t c_ld_shared;
  int rev;                 // walk each XCD's item range from its end
  // items after the ranges' end (the down projection's shared group), dealt
  // to the XCDs in equal shares and run before their ranges; 0: none
  int shared_items;
  int n_ntiles;            // N tiles per M tile (set by the launcher)
  int bm;                  // rows per M tile (set by the launcher)
  // 256-row down projection: the tile builder may have it run every item as
  // two 128-row halves (its schedule entry after the XCD boundaries), for
  // which the launcher provides two blocks per item
  int halves_ok;
};

// Element offset of K column kcol of a shared-group B row, beyond kcol
// itself (0 unless the K slices are separate blocks)
__device__ __forceinline__ int64_t shared_kseg_delta(const GemmArgs& a, int kcol) {
  return (int64_t)(kcol / a.k_seg_shared) * (a.b_seg_shared - a.k_seg_shared);
}

struct CombineArgs {
  const void* x;
  const int32_t* idx;
  const float* gate;
  const int32_t* inv_perm;
  const void* y;
  const void* shared_y;
  void* out;
  const float* const_wc;
  const void* const_v;
  int64_t T;
  int d, k, E_ffn, n_shared;
  int zc_kind[MOE_MAX_ZC];
  int const_index[MOE_MAX_ZC];
};

// router.hip
int router_splits(int dtype, int64_t T, int NL, int K);
// One weight block of the router: logits[:, col_off + n] = x[:, x_off + K] .
// W[n]  (n < NL); ny is set by the launcher.  Up to two parts per launch
// (the product key's row and column keys); NL = 0 for an unused part.
struct RouterPart {
  const float* W;
  int NL, x_off, col_off, ny;
};
hipError_t launch_router_logits(int dtype, const void* x, int64_t T, int ldx, RouterPart p0,
                                RouterPart p1, int K, float* logits, int ldl, int splits,
                                hipStream_t st);
hipError_t launch_select_topk(const float* logits, int splits, int64_t T, int E, int E_ffn, int k,
                              float tau, const float* bias, const float* residual, int renorm,
                              int32_t* idx, float* gate, hipStream_t st);
// Softmax router logits before tau: sum of the K-split partials + bias (+
// gating residual), f32 [T, E]
hipError_t launch_logits_out(const float* part, int splits, int64_t T, int E, const float* bias,
                             const float* residual, float* out, hipStream_t st);
hipError_t launch_select_pk(const float* scores, int splits, int64_t T, int rows, int cols,
                            int krow, int kcol, int k, int32_t* idx, float* gate, hipStream_t st);

// dispatch.hip: tasks grouped by expert id / width (E groups below)
int64_t dispatch_scratch_ints(int64_t n, int E);
// whether launch_dispatch can build a tile list (it does when given one)
bool dispatch_builds_tiles(int64_t n, int E);
// Optional build of the expert GEMMs' tile list inside the dispatch scan
// (single-pass dispatch only; tiles == nullptr: none).
struct TileBuild {
  int4* tiles;
  int32_t* sched;
  int E_ffn, n_shared, BM, nn1, nn2;
  // longest XCD range of each GEMM: its blocks per XCD (gemm_blocks_per_xcd)
  // less the XCD's share of the down projection's shared items
  int cap1, cap2;
  int64_t T;
};
// E_ids expert ids in groups of `width`: counts / offsets get
// ceil(E_ids / width) (+1) entries
hipError_t launch_dispatch(const int32_t* idx, int64_t n, int E_ids, int width, int32_t* counts,
                           int32_t* offsets, int32_t* perm, int32_t* inv_perm, int32_t* scratch,
                           hipStream_t st,
                           const TileBuild* tb = nullptr);

// gemm.hip
int gemm_tile_rows(int dtype, int64_t tasks, int E_ffn);
int64_t gemm_max_tiles(int64_t T, int k, int E_ffn, int n_shared, int BM);
int gemm_n_ntiles(int dtype, bool swiglu, int N);
// Blocks per XCD of a GEMM launch over max_tiles tiles of nn items: the
// schedule never gives an XCD more items than this
int64_t gemm_blocks_per_xcd(int BM, int64_t max_tiles, int nn);
hipError_t launch_build_tiles(const TileBuild& tb, const int32_t* offsets, hipStream_t st);
hipError_t launch_grouped_gemm(int dtype, bool swiglu, int BM, const GemmArgs& a,
                               int64_t max_tiles, hipStream_t st);

// combine.hip
hipError_t launch_combine(int dtype, const CombineArgs& a, hipStream_t st);
hipError_t launch_atomic_h(int dtype, const void* x, const void* atom_u, const int32_t* idx,
                           const int32_t* perm, int64_t n, int k, int d, float* h,
                           hipStream_t st);
hipError_t launch_atomic_combine(int dtype, const void* atom_w, const int32_t* idx,
                                 const float* gate, const int32_t* inv_perm, const float* h,
                                 const void* shared_y, int n_shared, int64_t T, int k, int d,
                                 void* out, hipStream_t st);

}  // namespace moe
