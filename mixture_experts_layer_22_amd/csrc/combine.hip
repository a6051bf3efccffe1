// Combine back to token order, and the atomic-expert stage.
//
// Combine: out_t = sum_s shared_s(x_t) + sum_{j<k} g_tj * c_tj, accumulated
// in fp32 in that fixed order and rounded once: a gather (one wave per
// token), so no atomics and a deterministic result.  c_tj is the expert
// output row of task t*k+j, or for MoE++ zero-computation experts ("MoE++:
// Accelerating Mixture-of-Experts Methods with Zero-Computation Experts",
// "Approach"): 0 (zero), x_t (copy), a*x_t + b*v with [a,b] = softmax(W_c x_t)
// (constant).
//
// Atomic experts ("OmniMoE: An Efficient MoE by Orchestrating Atomic Experts
// at Scale", sec. 2.1: E_i(x) = sigma(x w_in^T) w_out, all N experts kept in
// two global tables): the activation h = silu(u_e . x_t) is computed expert-
// centrically over the sorted task list (each u_e row read once and reused
// for the consecutive tasks of that expert, sec. 2.2 Grouped GEMM idea);
// the down projection gathers w_e rows per token and weights them by g*h.
#include "kernels.h"

namespace moe {

// ------------------------------------------------------------------------
// One wave per token; lane owns 8-element units u = lane + 64 i (i < U).
template <typename T, int U>
__global__ __launch_bounds__(256) void k_combine(CombineArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int d = a.d, nu = d / 8;
  float acc[U][8];
#pragma unroll
  for (int i = 0; i < U; i++)
#pragma unroll
    for (int q = 0; q < 8; q++) acc[i][q] = 0.f;

  const T* sy = reinterpret_cast<const T*>(a.shared_y);
  for (int s = 0; s < a.n_shared; s++) {
    const T* row = sy + ((int64_t)s * a.T + t) * d;
#pragma unroll
    for (int i = 0; i < U; i++) {
      const int u = lane + 64 * i;
      if (u < nu) {
        float v[8];
        Elt<T>::load8(row + u * 8, v);
#pragma unroll
        for (int q = 0; q < 8; q++) acc[i][q] += v[q];
      }
    }
  }
  const T* xrow = reinterpret_cast<const T*>(a.x) + t * d;
  const T* y = reinterpret_cast<const T*>(a.y);
  for (int j = 0; j < a.k; j++) {
    const int64_t task = t * a.k + j;
    const int e = a.idx[task];
    const float g = a.gate[task];
    if (e < a.E_ffn) {
      const T* row = y + (int64_t)a.inv_perm[task] * d;
#pragma unroll
      for (int i = 0; i < U; i++) {
        const int u = lane + 64 * i;
        if (u < nu) {
          float v[8];
          Elt<T>::load8(row + u * 8, v);
#pragma unroll
          for (int q = 0; q < 8; q++) acc[i][q] += g * v[q];
        }
      }
      continue;
    }
    const int z = e - a.E_ffn;
    const int kind = a.zc_kind[z];
    if (kind == MOE_ZC_ZERO) continue;
    if (kind == MOE_ZC_COPY) {
#pragma unroll
      for (int i = 0; i < U; i++) {
        const int u = lane + 64 * i;
        if (u < nu) {
          float v[8];
          Elt<T>::load8(xrow + u * 8, v);
#pragma unroll
          for (int q = 0; q < 8; q++) acc[i][q] += g * v[q];
        }
      }
      continue;
    }
    // constant expert
    const int ci = a.const_index[z];
    const float* wc0 = a.const_wc + (int64_t)ci * 2 * d;
    const float* wc1 = wc0 + d;
    const T* vrow = reinterpret_cast<const T*>(a.const_v) + (int64_t)ci * d;
    float xv[U][8];
    float pa = 0.f, pb = 0.f;
#pragma unroll
    for (int i = 0; i < U; i++) {
      const int u = lane + 64 * i;
      if (u < nu) {
        Elt<T>::load8(xrow + u * 8, xv[i]);
        float w0[8], w1[8];
        Elt<float>::load8(wc0 + u * 8, w0);
        Elt<float>::load8(wc1 + u * 8, w1);
#pragma unroll
        for (int q = 0; q < 8; q++) {
          pa = fmaf(w0[q], xv[i][q], pa);
          pb = fmaf(w1[q], xv[i][q], pb);
        }
      }
    }
    pa = wave_sum(pa);
    pb = wave_sum(pb);
    const float mx = fmaxf(pa, pb);
    const float ea = __expf(pa - mx), eb = __expf(pb - mx);
    const float ca = g * (ea / (ea + eb)), cb = g * (eb / (ea + eb));
#pragma unroll
    for (int i = 0; i < U; i++) {
      const int u = lane + 64 * i;
      if (u < nu) {
        float vv[8];
        Elt<T>::load8(vrow + u * 8, vv);
#pragma unroll
        for (int q = 0; q < 8; q++) acc[i][q] += ca * xv[i][q] + cb * vv[q];
      }
    }
  }
  T* orow = reinterpret_cast<T*>(a.out) + t * d;
#pragma unroll
  for (int i = 0; i < U; i++) {
    const int u = lane + 64 * i;
    if (u < nu) Elt<T>::store8(orow + u * 8, acc[i]);
  }
}

// ------------------------------------------------------------------------
// Atomic stage 1: h[p] = silu(u_e . x_t) for sorted task p (task perm[p] =
// t*k + j, e = idx[task]).  One wave walks kAtomChunk consecutive sorted
// tasks and keeps u_e in registers while the expert repeats.
constexpr int kAtomChunk = 8;

template <typename T, int U>
__global__ __launch_bounds__(256) void k_atomic_h(const T* __restrict__ x,
                                                 const T* __restrict__ atom_u,
                                                 const int32_t* __restrict__ idx,
                                                 const int32_t* __restrict__ perm, int64_t n,
                                                 int k, int d, float* __restrict__ h) {
  const int lane = threadIdx.x & 63;
  const int64_t p0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * kAtomChunk;
  if (p0 >= n) return;
  const int nu = d / 8;
  float uw[U][8];
  int cur_e = -1;
  for (int c = 0; c < kAtomChunk; c++) {
    const int64_t p = p0 + c;
    if (p >= n) break;
    const int32_t task = perm[p];
    const int e = idx[task];
    const int64_t tok = task / k;
    if (e != cur_e) {
      cur_e = e;
      const T* ur = atom_u + (int64_t)e * d;
#pragma unroll
      for (int i = 0; i < U; i++) {
        const int u = lane + 64 * i;
        if (u < nu) Elt<T>::load8(ur + u * 8, uw[i]);
      }
    }
    const T* xr = x + tok * d;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < U; i++) {
      const int u = lane + 64 * i;
      if (u < nu) {
        float xv[8];
        Elt<T>::load8(xr + u * 8, xv);
#pragma unroll
        for (int q = 0; q < 8; q++) s = fmaf(uw[i][q], xv[q], s);
      }
    }
    s = wave_sum(s);
    if (lane == 0) h[p] = silu_f32(s);
  }
}

// Atomic stage 2: out_t = sum_s shared + sum_j (g_tj * h_tj) w_e, one wave
// per token, slots in order, fp32.
template <typename T, int U>
__global__ __launch_bounds__(256) void k_atomic_combine(const T* __restrict__ atom_w,
                                                       const int32_t* __restrict__ idx,
                                                       const float* __restrict__ gate,
                                                       const int32_t* __restrict__ inv_perm,
                                                       const float* __restrict__ h,
                                                       const T* __restrict__ shared_y,
                                                       int n_shared, int64_t T_, int k, int d,
                                                       T* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T_) return;
  const int nu = d / 8;
  float acc[U][8];
#pragma unroll
  for (int i = 0; i < U; i++)
#pragma unroll
    for (int q = 0; q < 8; q++) acc[i][q] = 0.f;
  for (int s = 0; s < n_shared; s++) {
    const T* row = shared_y + ((int64_t)s * T_ + t) * d;
#pragma unroll
    for (int i = 0; i < U; i++) {
      const int u = lane + 64 * i;
      if (u < nu) {
        float v[8];
        Elt<T>::load8(row + u * 8, v);
#pragma unroll
        for (int q = 0; q < 8; q++) acc[i][q] += v[q];
      }
    }
  }
  for (int j = 0; j < k; j++) {
    const int64_t task = t * k + j;
    const float coef = gate[task] * h[inv_perm[task]];
    const T* wr = atom_w + (int64_t)idx[task] * d;
#pragma unroll
    for (int i = 0; i < U; i++) {
      const int u = lane + 64 * i;
      if (u < nu) {
        float v[8];
        Elt<T>::load8(wr + u * 8, v);
#pragma unroll
        for (int q = 0; q < 8; q++) acc[i][q] = fmaf(coef, v[q], acc[i][q]);
      }
    }
  }
  T* orow = out + t * d;
#pragma unroll
  for (int i = 0; i < U; i++) {
    const int u = lane + 64 * i;
    if (u < nu) Elt<T>::store8(orow + u * 8, acc[i]);
  }
}

// ------------------------------------------------------------------------
// launchers (U = units of 8 elements per lane = ceil(d / 512), d <= 8192)

template <typename T>
static hipError_t combine_t(const CombineArgs& a, hipStream_t st) {
  const int U = (int)cdiv(a.d, 512);
  dim3 grid((unsigned)cdiv(a.T, 4)), block(256);
  if (U <= 1) hipLaunchKernelGGL((k_combine<T, 1>), grid, block, 0, st, a);
  else if (U <= 2) hipLaunchKernelGGL((k_combine<T, 2>), grid, block, 0, st, a);
  else if (U <= 4) hipLaunchKernelGGL((k_combine<T, 4>), grid, block, 0, st, a);
  else if (U <= 8) hipLaunchKernelGGL((k_combine<T, 8>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((k_combine<T, 16>), grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_combine(int dtype, const CombineArgs& a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  return dtype == MOE_BF16 ? combine_t<uint16_t>(a, st) : combine_t<float>(a, st);
}

template <typename T>
static hipError_t atomic_h_t(const void* x, const void* u, const int32_t* idx,
                             const int32_t* perm, int64_t n, int k, int d, float* h,
                             hipStream_t st) {
  const int U = (int)cdiv(d, 512);
  dim3 grid((unsigned)cdiv(cdiv(n, kAtomChunk), 4)), block(256);
  const T* xx = (const T*)x;
  const T* uu = (const T*)u;
#define L(UU) hipLaunchKernelGGL((k_atomic_h<T, UU>), grid, block, 0, st, xx, uu, idx, perm, n, k, d, h)
  if (U <= 1) L(1);
  else if (U <= 2) L(2);
  else if (U <= 4) L(4);
  else if (U <= 8) L(8);
  else L(16);
#undef L
  return hipGetLastError();
}

hipError_t launch_atomic_h(int dtype, const void* x, const void* atom_u, const int32_t* idx,
                           const int32_t* perm, int64_t n, int k, int d, float* h,
                           hipStream_t st) {
  if (n == 0) return hipSuccess;
  return dtype == MOE_BF16 ? atomic_h_t<uint16_t>(x, atom_u, idx, perm, n, k, d, h, st)
                           : atomic_h_t<float>(x, atom_u, idx, perm, n, k, d, h, st);
}

template <typename T>
static hipError_t atomic_combine_t(const void* w, const int32_t* idx, const float* gate,
                                   const int32_t* inv, const float* h, const void* sy,
                                   int n_shared, int64_t T_, int k, int d, void* out,
                                   hipStream_t st) {
  const int U = (int)cdiv(d, 512);
  dim3 grid((unsigned)cdiv(T_, 4)), block(256);
  const T* ww = (const T*)w;
  const T* syy = (const T*)sy;
  T* oo = (T*)out;
#define L(UU) hipLaunchKernelGGL((k_atomic_combine<T, UU>), grid, block, 0, st, ww, idx, gate, inv, h, syy, n_shared, T_, k, d, oo)
  if (U <= 1) L(1);
  else if (U <= 2) L(2);
  else if (U <= 4) L(4);
  else if (U <= 8) L(8);
  else L(16);
#undef L
  return hipGetLastError();
}

hipError_t launch_atomic_combine(int dtype, const void* atom_w, const int32_t* idx,
                                 const float* gate, const int32_t* inv_perm, const float* h,
                                 const void* shared_y, int n_shared, int64_t T, int k, int d,
                                 void* out, hipStream_t st) {
  if (T == 0) return hipSuccess;
  return dtype == MOE_BF16
             ? atomic_combine_t<uint16_t>(atom_w, idx, gate, inv_perm, h, shared_y, n_shared, T,
                                          k, d, out, st)
             : atomic_combine_t<float>(atom_w, idx, gate, inv_perm, h, shared_y, n_shared, T, k,
                                       d, out, st);
}

}  // namespace moe
