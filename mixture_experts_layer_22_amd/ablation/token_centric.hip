// Token-centric atomic experts, the scheduling contrast of "OmniMoE: An
// Efficient MoE by Orchestrating Atomic Experts at Scale" (sec. 2.2
// Expert-Centric Scheduling, sec. 4 scheduling ablation): each token reads
// the in- and out-vectors of its own k experts straight from the two global
// tables, with no task collection, grouping or sort.  Built as its own
// library (libmoe_ablation.so) so the layer library stays expert-centric;
// only the bench's ablation mode and its parity test call it.
#include "../../include/moe_ablation.h"
#include "../csrc/common.h"

namespace moe_ablation {

using moe::cdiv;
using moe::silu_f32;
using moe::wave_sum;

// 8 elements of the layer dtype, packed as loaded
template <typename T> struct Pack8;
template <> struct Pack8<uint16_t> {
  moe::u32x4 w;
  __device__ __forceinline__ void load(const uint16_t* p) {
    w = *reinterpret_cast<const moe::u32x4*>(p);
  }
  __device__ __forceinline__ float operator[](int i) const {
    return (i & 1) ? moe::hi_bf16(w[i >> 1]) : moe::lo_bf16(w[i >> 1]);
  }
};
template <> struct Pack8<float> {
  moe::f32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const moe::f32x4*>(p);
    b = *reinterpret_cast<const moe::f32x4*>(p + 4);
  }
  __device__ __forceinline__ float operator[](int i) const { return i < 4 ? a[i] : b[i - 4]; }
};

// One wave per token; lane owns 8-element units u = lane + 64 i (i < U).
// The k slots (expert, gate) are fetched one slot per lane; the u and w rows
// of CH slots are loaded before any is used.  h_j = silu(u_e . x_t) is a
// wave sum; out_t accumulates g_j h_j w_e in slot order.
template <typename T, int U>
__global__ __launch_bounds__(256) void k_token_centric(const T* __restrict__ x,
                                                      const T* __restrict__ au,
                                                      const T* __restrict__ aw,
                                                      const int32_t* __restrict__ idx,
                                                      const float* __restrict__ gate,
                                                      int64_t T_, int k, int d,
                                                      T* __restrict__ out) {
  constexpr int CH = U >= 4 ? 2 : 4;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T_) return;
  const int nu = d / 8;
  float xv[U][8], acc[U][8];
#pragma unroll
  for (int i = 0; i < U; i++) {
    const int u = lane + 64 * i;
    Pack8<T> p;
    if (u < nu) p.load(x + t * d + u * 8);
#pragma unroll
    for (int q = 0; q < 8; q++) {
      xv[i][q] = u < nu ? p[q] : 0.f;
      acc[i][q] = 0.f;
    }
  }
  int me = 0;
  float mg = 0.f;
  if (lane < k) {
    me = idx[t * k + lane];
    mg = gate[t * k + lane];
  }
  for (int j0 = 0; j0 < k; j0 += CH) {
    Pack8<T> ur[CH][U], wr[CH][U];
#pragma unroll
    for (int c = 0; c < CH; c++) {
      if (j0 + c < k) {
        const int64_t e = __builtin_amdgcn_readlane(me, j0 + c);
#pragma unroll
        for (int i = 0; i < U; i++) {
          const int u = lane + 64 * i;
          if (u < nu) {
            ur[c][i].load(au + e * d + u * 8);
            wr[c][i].load(aw + e * d + u * 8);
          }
        }
      }
    }
#pragma unroll
    for (int c = 0; c < CH; c++) {
      const int j = j0 + c;
      if (j >= k) break;
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < U; i++)
        if (lane + 64 * i < nu)
#pragma unroll
          for (int q = 0; q < 8; q++) s = fmaf(ur[c][i][q], xv[i][q], s);
      s = wave_sum(s);
      const float coef =
          __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mg), j)) * silu_f32(s);
#pragma unroll
      for (int i = 0; i < U; i++)
        if (lane + 64 * i < nu)
#pragma unroll
          for (int q = 0; q < 8; q++) acc[i][q] = fmaf(coef, wr[c][i][q], acc[i][q]);
    }
  }
#pragma unroll
  for (int i = 0; i < U; i++) {
    const int u = lane + 64 * i;
    if (u < nu) moe::Elt<T>::store8(out + t * d + u * 8, acc[i]);
  }
}

template <typename T>
static hipError_t launch(const moe_weights* w, const void* x, int64_t T_, const int32_t* idx,
                         const float* gate, int k, int d, void* out, hipStream_t st) {
  const int U = (int)cdiv(d, 512);
  const dim3 grid((unsigned)cdiv(T_, 4)), block(256);
  const T* xx = (const T*)x;
  const T* au = (const T*)w->atom_u;
  const T* aw = (const T*)w->atom_w;
  T* o = (T*)out;
  if (U <= 1)
    hipLaunchKernelGGL((k_token_centric<T, 1>), grid, block, 0, st, xx, au, aw, idx, gate, T_, k, d, o);
  else if (U <= 2)
    hipLaunchKernelGGL((k_token_centric<T, 2>), grid, block, 0, st, xx, au, aw, idx, gate, T_, k, d, o);
  else if (U <= 4)
    hipLaunchKernelGGL((k_token_centric<T, 4>), grid, block, 0, st, xx, au, aw, idx, gate, T_, k, d, o);
  else if (U <= 8)
    hipLaunchKernelGGL((k_token_centric<T, 8>), grid, block, 0, st, xx, au, aw, idx, gate, T_, k, d, o);
  else
    hipLaunchKernelGGL((k_token_centric<T, 16>), grid, block, 0, st, xx, au, aw, idx, gate, T_, k, d, o);
  return hipGetLastError();
}

static bool misaligned(const void* p) { return p && ((uintptr_t)p % 16) != 0; }

}  // namespace moe_ablation

extern "C" int32_t moe_ablation_atomic_token_centric(const moe_dims* dims, const moe_weights* w,
                                                     const void* x, int64_t T,
                                                     const int32_t* topk_idx,
                                                     const float* topk_gate, void* out,
                                                     moe_stream stream) {
  using namespace moe_ablation;
  if (!dims || !w) return MOE_ERR_NULL;
  if (dims->dtype != MOE_F32 && dims->dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (dims->router_kind != MOE_ROUTER_PRODUCT_KEY || dims->n_shared != 0)
    return MOE_ERR_UNSUPPORTED;
  if (T < 0 || dims->d <= 0 || dims->d % 64 != 0 || dims->d > 8192) return MOE_ERR_SHAPE;
  if (dims->k < 1 || dims->k > MOE_MAX_K || dims->k > dims->E) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (!x || !topk_idx || !topk_gate || !out || !w->atom_u || !w->atom_w) return MOE_ERR_NULL;
  if (misaligned(x) || misaligned(out) || misaligned(w->atom_u) || misaligned(w->atom_w))
    return MOE_ERR_SHAPE;
  const hipStream_t st = (hipStream_t)stream;
  const hipError_t e =
      dims->dtype == MOE_BF16
          ? launch<uint16_t>(w, x, T, topk_idx, topk_gate, dims->k, dims->d, out, st)
          : launch<float>(w, x, T, topk_idx, topk_gate, dims->k, dims->d, out, st);
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
