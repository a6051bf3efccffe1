/* Ablation kernels kept outside the MoE layer library (libmoe_ablation.so).
 *
 * Token-centric atomic experts: the contrast to expert-centric scheduling
 * in "OmniMoE: An Efficient MoE by Orchestrating Atomic Experts at Scale",
 * sec. 2.2 (Expert-Centric Scheduling) and the scheduling ablation of its
 * sec. 4: every token gathers the in- and out-vectors of its own k atomic
 * experts directly, with no task grouping or sort.  Used only to measure
 * what the expert-centric path gains on this GPU; the layer library's
 * product-key path is the expert-centric one.
 */
#ifndef MOE_ABLATION_H
#define MOE_ABLATION_H

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* out[t] = sum_{j<k} topk_gate[t,j] * silu(u_e . x_t) * w_e, e =
 * topk_idx[t,j], fp32 accumulation in slot order j = 0..k-1, rounded once to
 * the layer dtype.
 *
 * dims: a product-key layer (router_kind MOE_ROUTER_PRODUCT_KEY) without
 *   shared experts (n_shared == 0), else MOE_ERR_UNSUPPORTED.
 * w: atom_u and atom_w, [pk_rows * pk_cols, d] in the layer dtype.
 * x [T, d] layer dtype; topk_idx int32 [T, k]; topk_gate fp32 [T, k] (as
 *   written by moe_route); out [T, d] layer dtype.  All device pointers,
 *   owned by the caller, 16-byte aligned.
 * Validation as in moe.h (shape, null, alignment errors; nothing is written
 * on error).  Asynchronous on `stream`; allocates nothing.
 */
int32_t moe_ablation_atomic_token_centric(const moe_dims* dims, const moe_weights* w,
                                          const void* x, int64_t T,
                                          const int32_t* topk_idx, const float* topk_gate,
                                          void* out, moe_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ABLATION_H */
