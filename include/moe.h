/*
 * moe.h -- C ABI of a forward pass of one sparse Mixture-of-Experts FFN
 * layer on AMD Instinct MI355X (gfx950).
 *
 * The layer (sources are web pages, cited by title and section):
 *   - router: per-token logits over E experts, top-k selection and softmax
 *     gates ("OmniMoE: An Efficient MoE by Orchestrating Atomic Experts at
 *     Scale", Technical Summary sec. 1, routing to N experts), or a
 *     Cartesian-product router over a grid of atomic experts (same page,
 *     sec. 2.2 "Cartesian Product Router");
 *   - MoE++ zero-computation experts: zero, copy and constant ("MoE++:
 *     Accelerating Mixture-of-Experts Methods with Zero-Computation
 *     Experts", "Approach"), with tau scaling the FFN experts' logits;
 *   - expert-centric dispatch: tasks collected, grouped by expert id and
 *     sorted by token inside a group (OmniMoE page, sec. 2.2 "Expert-Centric
 *     Scheduling", steps Task Collection and Grouping & Sorting);
 *   - the experts as a grouped GEMM (same passage, step Grouped GEMM); each
 *     FFN expert is a SwiGLU MLP W_down(silu(W_gate x) * (W_up x));
 *     atomic experts are E_i(x) = silu(x . u_i) w_i (OmniMoE page, sec. 2.1
 *     "Atomic Experts", "Dynamic Expert Assembly");
 *   - shared dense experts, always active (OmniMoE page, sec. 2.1 "Shared
 *     Dense MLP");
 *   - the weighted combine back to token order.
 *
 * Conventions for every entry point:
 *   - All tensor arguments are DEVICE pointers owned by the caller, row-major,
 *     densely packed.  The library never allocates, keeps no state between
 *     calls, and reads the two structs only during the call.
 *   - "layer dtype" (dims->dtype) is the type of x, out, the expert weights,
 *     const_v, the atomic tables and the expert outputs y / shared_y:
 *     MOE_F32 (float) or MOE_BF16 (bfloat16 bit patterns, uint16).  Router
 *     weights, router bias and const_wc are always float32.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and the call returns after enqueue.  Calls that share a workspace must
 *     not overlap.
 *   - Validation completes before anything is enqueued: on any error nothing
 *     is written and no GPU call is made.  T == 0 is a successful no-op.
 *   - Results are deterministic: no floating-point atomics anywhere.
 *   - NaN/Inf inputs give unspecified routing.
 *
 * Task numbering: task tau = t*k + j is token t's j-th choice (j ordered by
 * descending router score).  perm[p] is the task at sorted position p;
 * sorted order is (group, task id) ascending, a group being a contiguous
 * range of expert ids: one expert for softmax top-k routers, one row of the
 * expert grid (pk_cols ids, group = id / pk_cols) for product-key routers;
 * inv_perm[perm[p]] = p.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define MOE_OK              0
#define MOE_ERR_NULL        1  /* a required pointer is NULL                 */
#define MOE_ERR_SHAPE       2  /* dims inconsistent or outside the limits     */
#define MOE_ERR_DTYPE       3  /* dims->dtype is not MOE_F32 / MOE_BF16       */
#define MOE_ERR_WORKSPACE   4  /* ws_bytes smaller than moe_workspace_size    */
#define MOE_ERR_UNSUPPORTED 5  /* valid request this build does not implement */
#define MOE_ERR_HIP         6  /* a HIP launch reported an error              */
#define MOE_ERR_SCRATCH     7  /* moe_forward_noalloc: the pass needs more than
                                  MOE_NOALLOC_SCRATCH_BYTES of workspace     */

/* layer dtypes */
#define MOE_F32  0
#define MOE_BF16 1

/* router kinds */
#define MOE_ROUTER_SOFTMAX_TOPK 0  /* logits over E experts, top-k, softmax   */
#define MOE_ROUTER_PRODUCT_KEY  1  /* Cartesian-product router, atomic experts */

/* zero-computation expert kinds (MoE++ page, "Approach") */
#define MOE_ZC_ZERO  0  /* discards: contributes 0                        */
#define MOE_ZC_COPY  1  /* identity: contributes x                        */
#define MOE_ZC_CONST 2  /* a*x + b*v with [a,b] = softmax(W_c x)          */

/* limits of this build */
#define MOE_MAX_ZC        8     /* zero-computation experts                  */
#define MOE_MAX_K         64    /* top-k                                     */
#define MOE_MAX_E_SOFTMAX 256   /* experts of a softmax top-k router         */
#define MOE_MAX_PK_SIDE   1024  /* rows or columns of a product-key grid     */
#define MOE_MAX_PK_CAND   1024  /* pk_k_row * pk_k_col                        */

typedef void* moe_stream;  /* a hipStream_t */

/* Layer shape and options (host struct).
 *   d        model width; a multiple of 64 (of 128 for the product key,
 *            whose halves feed the row and column keys).
 *   E        routed experts, including zero-computation ones (product key:
 *            E = pk_rows * pk_cols atomic experts).
 *   E_ffn    SwiGLU experts are ids [0, E_ffn); ids [E_ffn, E) are
 *            zero-computation experts of kinds zc_kind[0 .. E-E_ffn).
 *            Product key: 0.
 *   k        experts per token, 1 <= k <= min(E, MOE_MAX_K).
 *   f        SwiGLU inner width of each routed expert; a multiple of 64.
 *   n_shared, f_shared   shared (always-on, unrouted, weight 1) SwiGLU
 *            experts and their inner width (a multiple of 64).
 *   renorm   nonzero: divide the k gates by their sum.
 *   ffn_logit_scale      tau: multiplies the FFN experts' logits (after the
 *            bias) before selection and softmax; 1.0 = none.
 *   router_kind          MOE_ROUTER_*.
 *   pk_rows, pk_cols, pk_k_row, pk_k_col   product-key grid and how many
 *            rows / columns are kept before the candidate top-k;
 *            k <= pk_k_row * pk_k_col.
 *   dtype    layer dtype, MOE_F32 or MOE_BF16. */
typedef struct moe_dims {
  int32_t d, E, E_ffn, k, f;
  int32_t n_shared, f_shared;
  int32_t renorm;
  float   ffn_logit_scale;
  int32_t router_kind;
  int32_t pk_rows, pk_cols, pk_k_row, pk_k_col;
  int32_t dtype;
  int32_t zc_kind[MOE_MAX_ZC];
} moe_dims;

/* Device pointers to the layer's parameters (host struct; unused ones may
 * be NULL).
 *   router_w     f32 [E, d]  (product key: [pk_rows + pk_cols, d/2]; rows
 *                first, keyed by x[:, :d/2]; then columns, keyed by x[:, d/2:])
 *   router_bias  f32 [E] or NULL; added to the logit before tau.
 *   w_gate, w_up [E_ffn, f, d];  w_down [E_ffn, d, f]
 *   shared_gate, shared_up [n_shared, f_shared, d]; shared_down [n_shared, d, f_shared]
 *   const_wc     f32 [n_const, 2, d];  const_v [n_const, d]  (n_const = number
 *                of MOE_ZC_CONST entries, in zc_kind order)
 *   atom_u, atom_w [E, d]  (the atomic experts' in- and out-vectors)
 *   router_residual  f32 [T, E] or NULL: a per-call input, not a parameter.
 *                The gating residual of the MoE++ page ("Approach": router
 *                scores carried over from the previous layer): the previous
 *                layer's logits (as moe_router_logits writes them), added
 *                to this layer's logits after the bias and before tau.
 *                Softmax router only (MOE_ERR_UNSUPPORTED with the product
 *                key); rows are tokens of this call. */
typedef struct moe_weights {
  const float* router_w;
  const float* router_bias;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  const void* shared_gate;
  const void* shared_up;
  const void* shared_down;
  const float* const_wc;
  const void* const_v;
  const void* atom_u;
  const void* atom_w;
  const float* router_residual;
} moe_weights;

/* Human-readable name of a status code (static string). */
const char* moe_status_str(int32_t status);

/* Bytes of device workspace `moe_route`, `moe_dispatch`, `moe_expert_ffn`
 * and `moe_forward` need for T tokens (the same figure serves all of them).
 * Writes *bytes; returns MOE_ERR_NULL / SHAPE / DTYPE on bad arguments. */
int32_t moe_workspace_size(const moe_dims* dims, int64_t T, size_t* bytes);

/* Routing (OmniMoE page sec. 1 and sec. 2.2 "Cartesian Product Router";
 * MoE++ page "Approach" for tau over FFN and zero-computation experts).
 *   x         [T, d] layer dtype.
 *   topk_idx  out: int32 [T, k], expert ids in descending score order, ties
 *             to the lower id.
 *   topk_gate out: f32 [T, k].
 * Softmax router: logit l_e = (x . R_e) + b_e (+ r_e, the gating residual
 * w->router_residual[t, e] when given), scaled by tau for e < E_ffn;
 * gates are softmax(l) over all E read at the chosen experts (renormalised
 * over the k when dims->renorm).  Product key: s_r = x[:d/2] . K_r,
 * s_c = x[d/2:] . K_c; top pk_k_row rows x top pk_k_col columns form the
 * candidates, scored s_r + s_c, id = row * pk_cols + col; the top k are kept
 * and their gates are the softmax over those k scores. */
int32_t moe_route(const moe_dims* dims, const moe_weights* w, const void* x,
                  int64_t T, int32_t* topk_idx, float* topk_gate,
                  void* ws, size_t ws_bytes, moe_stream stream);

/* The softmax router's logits before tau, for a next layer's gating
 * residual (MoE++ page "Approach"): logits[t, e] = (x . R_e) + b_e (+ the
 * residual w->router_residual[t, e] when given), f32 [T, E], the same
 * values moe_route selects on before scaling the FFN experts' by tau.
 * Product key: MOE_ERR_UNSUPPORTED.  Workspace as for moe_route. */
int32_t moe_router_logits(const moe_dims* dims, const moe_weights* w, const void* x,
                          int64_t T, float* logits, void* ws, size_t ws_bytes,
                          moe_stream stream);

/* Expert-centric dispatch (OmniMoE page sec. 2.2, Task Collection and
 * Grouping & Sorting: tasks grouped by contiguous ranges of expert ids,
 * sorted by token inside a group): a stable sort of the T*k task ids by
 * group.  G groups: G = E for softmax top-k routers (one expert each), G =
 * pk_rows for product-key routers (one row of the expert grid each).
 *   topk_idx  int32 [T, k] in; every id in [0, E).
 *   counts    out: int32 [E] buffer; entries 0..G-1 = tasks per group.
 *   offsets   out: int32 [E+1] buffer; entries 0..G = exclusive prefix sum
 *             of counts (offsets[G] = T*k).  Later entries are not written.
 *   perm      out: int32 [T*k] task id at each sorted position.
 *   inv_perm  out: int32 [T*k] sorted position of each task.
 * Zero-computation experts have the highest ids: their tasks form the tail
 * segments, which the expert stage skips.  Bit-exact and deterministic. */
int32_t moe_dispatch(const moe_dims* dims, const int32_t* topk_idx, int64_t T,
                     int32_t* counts, int32_t* offsets, int32_t* perm,
                     int32_t* inv_perm, void* ws, size_t ws_bytes,
                     moe_stream stream);

/* Expert stage (OmniMoE page sec. 2.2, step Grouped GEMM): every expert's
 * weights are read once per tile and reused by all tokens of its group.
 *   perm, offsets  from moe_dispatch on the same topk_idx.
 *   y         out.  SwiGLU layers: layer dtype [T*k, d]; row p (for
 *             p < offsets[E_ffn]) = FFN_e(x_t) of task perm[p]; rows of
 *             zero-computation tasks are not written.  Product key: float
 *             [T*k]; y[p] = silu(u_e . x_t) of task perm[p].
 *   shared_y  out: layer dtype [T, d], row t = the sum of the n_shared shared
 *             experts on token t (OmniMoE page sec. 2.1 "Shared Dense MLP";
 *             computed as one SwiGLU of width n_shared * f_shared, fp32
 *             accumulation, rounded once); may be NULL when n_shared == 0. */
int32_t moe_expert_ffn(const moe_dims* dims, const moe_weights* w,
                       const void* x, int64_t T, const int32_t* topk_idx,
                       const int32_t* perm, const int32_t* offsets, void* y,
                       void* shared_y, void* ws, size_t ws_bytes,
                       moe_stream stream);

/* Weighted combine back to token order, deterministic (fixed order, fp32):
 *   out_t = shared_y[t] + sum_{j<k} gate[t,j] * c_tj
 * with c_tj = y[inv_perm[t*k+j]] for FFN experts, 0 / x_t / a*x_t + b*v for
 * zero / copy / constant experts (MoE++ page, "Approach"), and
 * y[inv_perm[t*k+j]] * w_e for atomic experts (OmniMoE page sec. 2.1).
 *   out  layer dtype [T, d]; computed in fp32 and rounded once.
 *   shared_y may be NULL when n_shared == 0.
 * A constant expert's mixing weights [a, b] = softmax(W_c x_t) are computed
 * here, per token, in fp32. */
int32_t moe_combine(const moe_dims* dims, const moe_weights* w, const void* x,
                    int64_t T, const int32_t* topk_idx, const float* topk_gate,
                    const int32_t* inv_perm, const void* y,
                    const void* shared_y, void* out, moe_stream stream);

/* The whole layer: route -> dispatch -> experts -> combine, all on device,
 * no host synchronisation.  out: layer dtype [T, d].  topk_idx_opt /
 * topk_gate_opt (nullable) receive the routing when given. */
int32_t moe_forward(const moe_dims* dims, const moe_weights* w, const void* x,
                    int64_t T, void* out, int32_t* topk_idx_opt,
                    float* topk_gate_opt, void* ws, size_t ws_bytes,
                    moe_stream stream);

/* Number of phases moe_forward_traced marks with events. */
#define MOE_N_PHASES 7

/* moe_forward, plus timing marks for profiling the phases of the pass:
 * 0 route, 1 dispatch, 2 tile list of the expert GEMMs, 3 atomic-expert
 * activations (product-key layers), 4 gated GEMM + SiLU (grouped GEMM1,
 * routed and shared experts), 5 down projection (grouped GEMM2), 6 combine.
 *   events  NULL, or MOE_N_PHASES + 1 caller-created hipEvent_t handles;
 *           events[i] is recorded on `stream` just before phase i is
 *           enqueued and events[MOE_N_PHASES] after the last one, so
 *           hipEventElapsedTime(events[i], events[i+1]) is phase i's device
 *           time.  A phase with no work for the layer gets zero width.
 * Same arguments, results and errors as moe_forward otherwise; a failed
 * event record returns MOE_ERR_HIP. */
int32_t moe_forward_traced(const moe_dims* dims, const moe_weights* w,
                           const void* x, int64_t T, void* out,
                           int32_t* topk_idx_opt, float* topk_gate_opt,
                           void* ws, size_t ws_bytes, moe_stream stream,
                           void* const* events);

/* Static workspace of moe_forward_noalloc, per GPU: 64 MiB. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)

/* moe_forward without a caller workspace and without any allocation, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  The workspace is a
 * file-scope device array of MOE_NOALLOC_SCRATCH_BYTES that every GPU the
 * library runs on holds until the process ends; its device address is looked
 * up once per device, on the first call with that device current.  The
 * caller still passes x, out and the optional routing outputs; stream must
 * belong to the current device.
 *   Limit: a call whose moe_workspace_size(dims, T) exceeds
 *   MOE_NOALLOC_SCRATCH_BYTES returns MOE_ERR_SCRATCH before any GPU call
 *   (about 2,000 tokens of the MoE++-shaped layer, 1,200 of the
 *   DeepSeek-shaped one; a 16-token decode batch needs under 1 MiB).
 *   Concurrency: all calls on one GPU share its array, which keeps the last
 *   call's contents; calls that overlap on one GPU (other streams, other
 *   threads) race and must be serialised by the caller.
 * Arguments, results and other errors as moe_forward.  It calls no hipMalloc,
 * hipFree or other allocating routine. */
int32_t moe_forward_noalloc(const moe_dims* dims, const moe_weights* w, const void* x,
                            int64_t T, void* out, int32_t* topk_idx_opt,
                            float* topk_gate_opt, moe_stream stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
