// C ABI of the MoE layer library: argument validation, workspace carving and
// launch sequencing.  Every check runs before the first enqueue, so a
// rejected call writes nothing and makes no GPU call.
#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "kernels.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int elt_size(int dtype) { return dtype == MOE_BF16 ? 2 : 4; }

bool is_pk(const moe_dims* d) { return d->router_kind == MOE_ROUTER_PRODUCT_KEY; }

int32_t validate_dims(const moe_dims* d, int64_t T) {
  if (!d) return MOE_ERR_NULL;
  if (d->dtype != MOE_F32 && d->dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (T < 0) return MOE_ERR_SHAPE;
  if (d->d <= 0 || d->d % 64 != 0 || d->d > 8192) return MOE_ERR_SHAPE;
  if (d->k < 1 || d->k > MOE_MAX_K || d->k > d->E) return MOE_ERR_SHAPE;
  if (T * (int64_t)d->k > INT32_MAX) return MOE_ERR_SHAPE;
  if (T * (int64_t)d->d > ((int64_t)1 << 40)) return MOE_ERR_SHAPE;
  if (!(d->ffn_logit_scale == d->ffn_logit_scale) || isinf(d->ffn_logit_scale))
    return MOE_ERR_SHAPE;
  if (d->n_shared < 0 || d->n_shared > 64) return MOE_ERR_SHAPE;
  if (d->n_shared > 0 && (d->f_shared <= 0 || d->f_shared % 64 != 0)) return MOE_ERR_SHAPE;
  if (d->router_kind == MOE_ROUTER_SOFTMAX_TOPK) {
    if (d->E < 1 || d->E > MOE_MAX_E_SOFTMAX) return MOE_ERR_SHAPE;
    if (d->E_ffn < 0 || d->E_ffn > d->E || d->E - d->E_ffn > MOE_MAX_ZC) return MOE_ERR_SHAPE;
    for (int z = 0; z < d->E - d->E_ffn; z++)
      if (d->zc_kind[z] < MOE_ZC_ZERO || d->zc_kind[z] > MOE_ZC_CONST) return MOE_ERR_SHAPE;
    if (d->E_ffn > 0 && (d->f <= 0 || d->f % 64 != 0)) return MOE_ERR_SHAPE;
  } else if (d->router_kind == MOE_ROUTER_PRODUCT_KEY) {
    if (d->E_ffn != 0 || d->d % 128 != 0) return MOE_ERR_SHAPE;
    if (d->pk_rows < 1 || d->pk_cols < 1 || d->pk_rows > MOE_MAX_PK_SIDE ||
        d->pk_cols > MOE_MAX_PK_SIDE)
      return MOE_ERR_SHAPE;
    if ((int64_t)d->pk_rows * d->pk_cols != d->E) return MOE_ERR_SHAPE;
    if (d->pk_k_row < 1 || d->pk_k_row > d->pk_rows || d->pk_k_row > 64) return MOE_ERR_SHAPE;
    if (d->pk_k_col < 1 || d->pk_k_col > d->pk_cols || d->pk_k_col > 64) return MOE_ERR_SHAPE;
    if ((int64_t)d->pk_k_row * d->pk_k_col > MOE_MAX_PK_CAND) return MOE_ERR_SHAPE;
    if (d->k > d->pk_k_row * d->pk_k_col) return MOE_ERR_SHAPE;
  } else {
    return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

int n_const_of(const moe_dims* d) {
  int c = 0;
  if (d->router_kind != MOE_ROUTER_SOFTMAX_TOPK) return 0;
  for (int z = 0; z < d->E - d->E_ffn; z++) c += d->zc_kind[z] == MOE_ZC_CONST;
  return c;
}

// Dispatch groups: contiguous ranges of expert ids whose tasks are sorted
// together (OmniMoE page sec. 2.2, Grouping & Sorting): one expert each for
// FFN experts, one row of the expert grid for atomic experts.
int dispatch_width(const moe_dims* d) { return is_pk(d) ? d->pk_cols : 1; }
int dispatch_groups(const moe_dims* d) { return (int)cdiv(d->E, dispatch_width(d)); }

bool misaligned(const void* p) { return p && ((uintptr_t)p % 16) != 0; }

// Workspace layout (one figure for every entry point).
struct Layout {
  int64_t T, n;
  int NL, Kw, BM, splits;
  int64_t max_tiles;
  size_t logits, disp, tiles, ntiles, h, hs, idx, gate, counts, offsets, perm, inv, y, sy;
  size_t total;
};

Layout make_layout(const moe_dims* d, int64_t T) {
  Layout L;
  L.T = T;
  L.n = T * d->k;
  const int es = elt_size(d->dtype);
  if (is_pk(d)) {
    L.NL = d->pk_rows + d->pk_cols;
    L.Kw = d->d / 2;
  } else {
    L.NL = d->E;
    L.Kw = d->d;
  }
  L.splits = router_splits(d->dtype, T, is_pk(d) ? (d->pk_rows > d->pk_cols ? d->pk_rows : d->pk_cols) : d->E, L.Kw);
  L.BM = gemm_tile_rows(d->dtype, L.n, d->E_ffn);
  const int E_groups = is_pk(d) ? 0 : d->E_ffn;
  L.max_tiles = gemm_max_tiles(T, is_pk(d) ? 0 : d->k, E_groups, d->n_shared, L.BM);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align_up(bytes);
    return o;
  };
  L.logits = take((size_t)L.splits * T * L.NL * 4);
  L.disp = take((size_t)dispatch_scratch_ints(L.n, dispatch_groups(d)) * 4);
  L.tiles = take((size_t)L.max_tiles * sizeof(int4));
  L.ntiles = take(kSchedInts * 4);
  L.h = take(is_pk(d) ? 0 : (size_t)L.n * d->f * es);
  L.hs = take((size_t)d->n_shared * T * d->f_shared * es);
  L.idx = take((size_t)L.n * 4);
  L.gate = take((size_t)L.n * 4);
  L.counts = take((size_t)d->E * 4);
  L.offsets = take((size_t)(d->E + 1) * 4);
  L.perm = take((size_t)L.n * 4);
  L.inv = take((size_t)L.n * 4);
  L.y = take(is_pk(d) ? (size_t)L.n * 4 : (size_t)L.n * d->d * es);
  L.sy = take(d->n_shared ? (size_t)T * d->d * es : 0);  // the shared experts' sum
  L.total = off;
  return L;
}

template <typename P>
P at(void* ws, size_t off) {
  return reinterpret_cast<P>(reinterpret_cast<char*>(ws) + off);
}

int32_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

#define MOE_TRY(expr)                          \
  do {                                         \
    int32_t _s = hip_status(expr);             \
    if (_s != MOE_OK) return _s;               \
  } while (0)

int32_t check_weights(const moe_dims* d, const moe_weights* w, bool router, bool experts,
                      bool combine) {
  if (!w) return MOE_ERR_NULL;
  if (router && !w->router_w) return MOE_ERR_NULL;
  if (experts && !is_pk(d) && d->E_ffn > 0 && (!w->w_gate || !w->w_up || !w->w_down))
    return MOE_ERR_NULL;
  if (experts && d->n_shared > 0 && (!w->shared_gate || !w->shared_up || !w->shared_down))
    return MOE_ERR_NULL;
  if (experts && is_pk(d) && !w->atom_u) return MOE_ERR_NULL;
  if (combine && is_pk(d) && !w->atom_w) return MOE_ERR_NULL;
  if (combine && n_const_of(d) > 0 && (!w->const_wc || !w->const_v)) return MOE_ERR_NULL;
  if (router && is_pk(d) && w->router_residual) return MOE_ERR_UNSUPPORTED;
  const void* ps[] = {w->router_w, w->router_bias, w->w_gate, w->w_up, w->w_down,
                      w->shared_gate, w->shared_up, w->shared_down, w->const_wc, w->const_v,
                      w->atom_u, w->atom_w, w->router_residual};
  for (const void* p : ps)
    if (misaligned(p)) return MOE_ERR_SHAPE;
  return MOE_OK;
}

// ---------------------------------------------------------------- stages

int32_t do_route(const moe_dims* d, const moe_weights* w, const void* x, int64_t T, int32_t* idx,
                 float* gate, void* ws, const Layout& L, hipStream_t st) {
  float* logits = at<float*>(ws, L.logits);
  const float* W = w->router_w;
  const RouterPart none = {nullptr, 0, 0, 0, 0};
  if (!is_pk(d)) {
    const RouterPart all = {W, d->E, 0, 0, 0};
    MOE_TRY(launch_router_logits(d->dtype, x, T, d->d, all, none, d->d, logits, d->E, L.splits,
                                 st));
    MOE_TRY(launch_select_topk(logits, L.splits, T, d->E, d->E_ffn, d->k, d->ffn_logit_scale,
                               w->router_bias, w->router_residual, d->renorm, idx, gate, st));
  } else {
    const int K = L.Kw;
    const float* Wc = W + (size_t)d->pk_rows * K;
    const RouterPart rows = {W, d->pk_rows, 0, 0, 0};
    const RouterPart cols = {Wc, d->pk_cols, K, d->pk_rows, 0};
    MOE_TRY(launch_router_logits(d->dtype, x, T, d->d, rows, cols, K, logits, L.NL, L.splits,
                                 st));
    MOE_TRY(launch_select_pk(logits, L.splits, T, d->pk_rows, d->pk_cols, d->pk_k_row,
                             d->pk_k_col, d->k, idx, gate, st));
  }
  return MOE_OK;
}

// Items of the down projection's shared group (all shared experts' K in one
// group): dealt to the XCDs outside the cost-balanced ranges
int64_t down_shared_items(const moe_dims* d, int64_t T, const Layout& L) {
  return d->n_shared ? cdiv(T, L.BM) * gemm_n_ntiles(d->dtype, false, d->d) : 0;
}

// The expert GEMMs' tile list build for these dims (tiles == nullptr when
// the layer has no GEMM).
TileBuild tile_build(const moe_dims* d, int64_t T, void* ws, const Layout& L) {
  TileBuild tb;
  const int E_groups = is_pk(d) ? 0 : d->E_ffn;
  const int N1 = E_groups ? d->f : d->f_shared;
  tb.tiles = (E_groups > 0 || d->n_shared > 0) ? at<int4*>(ws, L.tiles) : nullptr;
  tb.sched = at<int32_t*>(ws, L.ntiles);
  tb.E_ffn = E_groups;
  tb.n_shared = d->n_shared;
  tb.BM = L.BM;
  tb.nn1 = gemm_n_ntiles(d->dtype, true, d->n_shared && d->f_shared > N1 ? d->f_shared : N1);
  tb.nn2 = gemm_n_ntiles(d->dtype, false, d->d);
  tb.cap1 = (int)gemm_blocks_per_xcd(L.BM, L.max_tiles, tb.nn1);
  tb.cap2 = (int)(gemm_blocks_per_xcd(L.BM, L.max_tiles, tb.nn2) -
                  cdiv(down_shared_items(d, T, L), kXcds));
  tb.T = T;
  return tb;
}

int32_t do_experts(const moe_dims* d, const moe_weights* w, const void* x, int64_t T,
                   const int32_t* idx, const int32_t* perm, const int32_t* offsets, void* y,
                   void* shared_y, void* ws, const Layout& L, hipStream_t st,
                   void* const* ev = nullptr, bool tiles_built = false) {
  auto mark = [&](int i) -> hipError_t {
    return ev ? hipEventRecord((hipEvent_t)ev[i], st) : hipSuccess;
  };
  const int E_groups = is_pk(d) ? 0 : d->E_ffn;
  const bool gemms = E_groups > 0 || d->n_shared > 0;
  int4* tiles = at<int4*>(ws, L.tiles);
  int32_t* ntiles = at<int32_t*>(ws, L.ntiles);
  const TileBuild tb = tile_build(d, T, ws, L);
  if (gemms && !tiles_built)
    MOE_TRY(launch_build_tiles(tb, offsets, st));
  MOE_TRY(mark(3));
  if (is_pk(d)) {
    MOE_TRY(launch_atomic_h(d->dtype, x, w->atom_u, idx, perm, L.n, d->k, d->d, (float*)y, st));
  }
  MOE_TRY(mark(4));
  void* H = at<void*>(ws, L.h);
  void* Hs = at<void*>(ws, L.hs);
  GemmArgs g1;
  memset(&g1, 0, sizeof(g1));
  g1.tiles = tiles;
  g1.ntiles = ntiles;
  g1.xcd_first = ntiles + 1;
  g1.E_ffn = E_groups;
  g1.T = T;
  g1.a_x = x;
  g1.perm = perm;
  g1.k = d->k;
  g1.b0_routed = w->w_gate;
  g1.b1_routed = w->w_up;
  g1.b0_shared = w->shared_gate;
  g1.b1_shared = w->shared_up;
  g1.c_routed = H;
  g1.c_shared = Hs;
  g1.N_routed = E_groups ? d->f : 0;
  // shared expert s: rows s*f_shared on of [n_shared f_shared, d], writing
  // columns s*f_shared on of H_shared [T, n_shared f_shared]
  g1.N_shared = d->n_shared ? d->f_shared : 0;
  g1.K_routed = d->d;
  g1.K_shared = d->d;
  g1.b_ld_shared = d->d;
  g1.k_seg_shared = d->d;
  g1.b_seg_shared = d->d;  // one K slice
  g1.c_ld_shared = (int64_t)d->n_shared * d->f_shared;
  if (gemms) MOE_TRY(launch_grouped_gemm(d->dtype, true, L.BM, g1, L.max_tiles, st));
  MOE_TRY(mark(5));
  GemmArgs g2 = g1;
  g2.xcd_first = ntiles + 1 + (kXcds + 1);
  g2.a_x = nullptr;
  g2.perm = nullptr;
  g2.a_routed = H;
  g2.a_shared = Hs;
  g2.b0_routed = w->w_down;
  g2.b1_routed = nullptr;
  g2.b0_shared = w->shared_down;
  g2.b1_shared = nullptr;
  g2.c_routed = is_pk(d) ? nullptr : y;
  g2.c_shared = shared_y;
  g2.N_routed = E_groups ? d->d : 0;
  // shared experts: one group, K concatenated; expert s's slice is its own
  // [d, f_shared] block, so the sum of the shared experts comes out of one
  // accumulation
  g2.N_shared = d->n_shared ? d->d : 0;
  g2.K_routed = E_groups ? d->f : 0;
  g2.K_shared = d->n_shared ? d->n_shared * d->f_shared : 0;
  g2.b_ld_shared = d->n_shared ? d->f_shared : 1;
  g2.k_seg_shared = d->n_shared ? d->f_shared : 1;
  g2.b_seg_shared = (int64_t)d->d * (d->n_shared ? d->f_shared : 1);
  g2.c_ld_shared = d->d;
  g2.shared_items = (int)down_shared_items(d, T, L);
  // ranges walked from their ends: timed faster for the down projection
  // (the MoE++-shaped layer, about 1.5 items per CU, gained 15-20 us)
  g2.rev = 1;
  if (gemms) MOE_TRY(launch_grouped_gemm(d->dtype, false, L.BM, g2, L.max_tiles, st));
  return MOE_OK;
}

int32_t do_combine(const moe_dims* d, const moe_weights* w, const void* x, int64_t T,
                   const int32_t* idx, const float* gate, const int32_t* inv, const void* y,
                   const void* shared_y, void* out, hipStream_t st) {
  if (is_pk(d)) {
    MOE_TRY(launch_atomic_combine(d->dtype, w->atom_w, idx, gate, inv, (const float*)y, shared_y,
                                  d->n_shared ? 1 : 0, T, d->k, d->d, out, st));
    return MOE_OK;
  }
  CombineArgs a;
  memset(&a, 0, sizeof(a));
  a.x = x;
  a.idx = idx;
  a.gate = gate;
  a.inv_perm = inv;
  a.y = y;
  a.shared_y = shared_y;
  a.out = out;
  a.const_wc = w->const_wc;
  a.const_v = w->const_v;
  a.T = T;
  a.d = d->d;
  a.k = d->k;
  a.E_ffn = d->E_ffn;
  a.n_shared = d->n_shared ? 1 : 0;  // shared_y holds the shared experts' sum
  int ci = 0;
  for (int z = 0; z < d->E - d->E_ffn; z++) {
    a.zc_kind[z] = d->zc_kind[z];
    a.const_index[z] = d->zc_kind[z] == MOE_ZC_CONST ? ci++ : -1;
  }
  MOE_TRY(launch_combine(d->dtype, a, st));
  return MOE_OK;
}

}  // namespace

// ================================================================ C ABI

extern "C" {

const char* moe_status_str(int32_t s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "null pointer";
    case MOE_ERR_SHAPE: return "bad shape, limit or alignment";
    case MOE_ERR_DTYPE: return "unsupported dtype";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_UNSUPPORTED: return "unsupported request";
    case MOE_ERR_HIP: return "HIP error";
    case MOE_ERR_SCRATCH: return "request exceeds the static scratch of moe_forward_noalloc";
    default: return "unknown status";
  }
}

int32_t moe_workspace_size(const moe_dims* dims, int64_t T, size_t* bytes) {
  if (!bytes) return MOE_ERR_NULL;
  int32_t s = validate_dims(dims, T);
  if (s != MOE_OK) return s;
  *bytes = make_layout(dims, T).total;
  return MOE_OK;
}

static int32_t check_ws(const Layout& L, void* ws, size_t ws_bytes) {
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (L.total > 0 && !ws) return MOE_ERR_NULL;
  if (misaligned(ws) || ((uintptr_t)ws % kAlign) != 0) return MOE_ERR_SHAPE;
  return MOE_OK;
}

int32_t moe_route(const moe_dims* dims, const moe_weights* w, const void* x, int64_t T,
                  int32_t* topk_idx, float* topk_gate, void* ws, size_t ws_bytes,
                  moe_stream stream) {
  int32_t s = validate_dims(dims, T);
  if (s != MOE_OK) return s;
  if ((s = check_weights(dims, w, true, false, false)) != MOE_OK) return s;
  if (T > 0 && (!x || !topk_idx || !topk_gate)) return MOE_ERR_NULL;
  if (misaligned(x)) return MOE_ERR_SHAPE;
  Layout L = make_layout(dims, T);
  if ((s = check_ws(L, ws, ws_bytes)) != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  return do_route(dims, w, x, T, topk_idx, topk_gate, ws, L, (hipStream_t)stream);
}

int32_t moe_router_logits(const moe_dims* dims, const moe_weights* w, const void* x, int64_t T,
                          float* logits, void* ws, size_t ws_bytes, moe_stream stream) {
  int32_t s = validate_dims(dims, T);
  if (s != MOE_OK) return s;
  if (is_pk(dims)) return MOE_ERR_UNSUPPORTED;
  if ((s = check_weights(dims, w, true, false, false)) != MOE_OK) return s;
  if (T > 0 && (!x || !logits)) return MOE_ERR_NULL;
  if (misaligned(x) || misaligned(logits)) return MOE_ERR_SHAPE;
  Layout L = make_layout(dims, T);
  if ((s = check_ws(L, ws, ws_bytes)) != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  const hipStream_t st = (hipStream_t)stream;
  float* part = at<float*>(ws, L.logits);
  const RouterPart all = {w->router_w, dims->E, 0, 0, 0};
  const RouterPart none = {nullptr, 0, 0, 0, 0};
  MOE_TRY(launch_router_logits(dims->dtype, x, T, dims->d, all, none, dims->d, part, dims->E,
                               L.splits, st));
  MOE_TRY(launch_logits_out(part, L.splits, T, dims->E, w->router_bias, w->router_residual,
                            logits, st));
  return MOE_OK;
}

int32_t moe_dispatch(const moe_dims* dims, const int32_t* topk_idx, int64_t T, int32_t* counts,
                     int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* ws,
                     size_t ws_bytes, moe_stream stream) {
  int32_t s = validate_dims(dims, T);
  if (s != MOE_OK) return s;
  if (!counts || !offsets) return MOE_ERR_NULL;
  if (T > 0 && (!topk_idx || !perm || !inv_perm)) return MOE_ERR_NULL;
  Layout L = make_layout(dims, T);
  if ((s = check_ws(L, ws, ws_bytes)) != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  MOE_TRY(launch_dispatch(topk_idx, L.n, dims->E, dispatch_width(dims), counts, offsets, perm,
                          inv_perm,
                          at<int32_t*>(ws, L.disp), (hipStream_t)stream));
  return MOE_OK;
}

int32_t moe_expert_ffn(const moe_dims* dims, const moe_weights* w, const void* x, int64_t T,
                       const int32_t* topk_idx, const int32_t* perm, const int32_t* offsets,
                       void* y, void* shared_y, void* ws, size_t ws_bytes, moe_stream stream) {
  int32_t s = validate_dims(dims, T);
  if (s != MOE_OK) return s;
  if ((s = check_weights(dims, w, false, true, false)) != MOE_OK) return s;
  if (T > 0 && (!x || !topk_idx || !perm || !offsets || !y)) return MOE_ERR_NULL;
  if (T > 0 && dims->n_shared > 0 && !shared_y) return MOE_ERR_NULL;
  if (misaligned(x) || misaligned(y) || misaligned(shared_y)) return MOE_ERR_SHAPE;
  Layout L = make_layout(dims, T);
  if ((s = check_ws(L, ws, ws_bytes)) != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  return do_experts(dims, w, x, T, topk_idx, perm, offsets, y, shared_y, ws, L,
                    (hipStream_t)stream);
}

int32_t moe_combine(const moe_dims* dims, const moe_weights* w, const void* x, int64_t T,
                    const int32_t* topk_idx, const float* topk_gate, const int32_t* inv_perm,
                    const void* y, const void* shared_y, void* out, moe_stream stream) {
  int32_t s = validate_dims(dims, T);
  if (s != MOE_OK) return s;
  if ((s = check_weights(dims, w, false, false, true)) != MOE_OK) return s;
  if (T > 0 && (!x || !topk_idx || !topk_gate || !inv_perm || !y || !out)) return MOE_ERR_NULL;
  if (T > 0 && dims->n_shared > 0 && !shared_y) return MOE_ERR_NULL;
  if (misaligned(x) || misaligned(y) || misaligned(shared_y) || misaligned(out))
    return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  return do_combine(dims, w, x, T, topk_idx, topk_gate, inv_perm, y, shared_y, out,
                    (hipStream_t)stream);
}

int32_t moe_forward_traced(const moe_dims* dims, const moe_weights* w, const void* x,
                           int64_t T, void* out, int32_t* topk_idx_opt, float* topk_gate_opt,
                           void* ws, size_t ws_bytes, moe_stream stream, void* const* events) {
  int32_t s = validate_dims(dims, T);
  if (s != MOE_OK) return s;
  if ((s = check_weights(dims, w, true, true, true)) != MOE_OK) return s;
  if (T > 0 && (!x || !out)) return MOE_ERR_NULL;
  if (misaligned(x) || misaligned(out)) return MOE_ERR_SHAPE;
  if (events)
    for (int i = 0; i <= MOE_N_PHASES; i++)
      if (!events[i]) return MOE_ERR_NULL;
  Layout L = make_layout(dims, T);
  if ((s = check_ws(L, ws, ws_bytes)) != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  hipStream_t st = (hipStream_t)stream;
  auto mark = [&](int i) -> hipError_t {
    return events ? hipEventRecord((hipEvent_t)events[i], st) : hipSuccess;
  };
  int32_t* idx = topk_idx_opt ? topk_idx_opt : at<int32_t*>(ws, L.idx);
  float* gate = topk_gate_opt ? topk_gate_opt : at<float*>(ws, L.gate);
  int32_t* counts = at<int32_t*>(ws, L.counts);
  int32_t* offsets = at<int32_t*>(ws, L.offsets);
  int32_t* perm = at<int32_t*>(ws, L.perm);
  int32_t* inv = at<int32_t*>(ws, L.inv);
  void* y = at<void*>(ws, L.y);
  void* sy = dims->n_shared ? at<void*>(ws, L.sy) : nullptr;
  MOE_TRY(mark(0));
  if ((s = do_route(dims, w, x, T, idx, gate, ws, L, st)) != MOE_OK) return s;
  MOE_TRY(mark(1));
  // a single-pass dispatch also builds the expert GEMMs' tile list
  const TileBuild tb = tile_build(dims, T, ws, L);
  const bool fused = tb.tiles && dispatch_builds_tiles(L.n, dispatch_groups(dims));
  MOE_TRY(launch_dispatch(idx, L.n, dims->E, dispatch_width(dims), counts, offsets, perm, inv,
                          at<int32_t*>(ws, L.disp), st, fused ? &tb : nullptr));
  MOE_TRY(mark(2));
  if ((s = do_experts(dims, w, x, T, idx, perm, offsets, y, sy, ws, L, st, events, fused)) !=
      MOE_OK)
    return s;
  MOE_TRY(mark(6));
  if ((s = do_combine(dims, w, x, T, idx, gate, inv, y, sy, out, st)) != MOE_OK) return s;
  MOE_TRY(mark(7));
  return MOE_OK;
}

int32_t moe_forward(const moe_dims* dims, const moe_weights* w, const void* x, int64_t T,
                    void* out, int32_t* topk_idx_opt, float* topk_gate_opt, void* ws,
                    size_t ws_bytes, moe_stream stream) {
  return moe_forward_traced(dims, w, x, T, out, topk_idx_opt, topk_gate_opt, ws, ws_bytes,
                            stream, nullptr);
}

}  // extern "C"

// ---------------------------------------------------------------- static scratch

namespace {

// The workspace of moe_forward_noalloc: one array in device memory, which
// the loader places on every GPU the library runs on and which stays there
// until the process ends.  Host code never uses the array's name as an
// address (on the host it is only a stand-in); it uses the device address
// that hipGetSymbolAddress returns on each device.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch, looked up on the first
// call on that device (with it current) and kept.
int32_t scratch_address(void** addr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *addr = p;
  return MOE_OK;
}

}  // namespace

extern "C" int32_t moe_forward_noalloc(const moe_dims* dims, const moe_weights* w,
                                       const void* x, int64_t T, void* out,
                                       int32_t* topk_idx_opt, float* topk_gate_opt,
                                       moe_stream stream) {
  // the same validation as moe_forward, then the size limit, all before
  // any HIP call
  int32_t s = validate_dims(dims, T);
  if (s != MOE_OK) return s;
  if ((s = check_weights(dims, w, true, true, true)) != MOE_OK) return s;
  if (T > 0 && (!x || !out)) return MOE_ERR_NULL;
  if (misaligned(x) || misaligned(out)) return MOE_ERR_SHAPE;
  if (make_layout(dims, T).total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
  if (T == 0) return MOE_OK;
  void* ws = nullptr;
  if ((s = scratch_address(&ws)) != MOE_OK) return s;
  // every region the pass reads is written earlier in the same pass (the
  // dispatch zeroes its own counters), so nothing needs clearing
  return moe_forward_traced(dims, w, x, T, out, topk_idx_opt, topk_gate_opt, ws,
                            (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}
