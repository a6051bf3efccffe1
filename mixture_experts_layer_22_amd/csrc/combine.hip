// Combine back to token order, and the atomic-expert stage.
//
// Combine: out_t = shared(x_t) + sum_{j<k} g_tj * c_tj, accumulated in fp32
// in that fixed order and rounded once: a gather (one wave per token), so no
// atomics and a deterministic result.  shared(x_t) is the sum of the shared
// experts, which the down projection forms as one group (n_shared here is 0
// or 1 rows).  c_tj is the expert
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
// 8 layer-dtype elements kept packed in registers until they are used.
template <typename T> struct Raw8;
template <> struct Raw8<uint16_t> {
  u32x4 w;
  __device__ __forceinline__ void load(const uint16_t* p) { w = *reinterpret_cast<const u32x4*>(p); }
  __device__ __forceinline__ float operator[](int i) const {
    return (i & 1) ? hi_bf16(w[i >> 1]) : lo_bf16(w[i >> 1]);
  }
};
template <> struct Raw8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const f32x4*>(p);
    b = *reinterpret_cast<const f32x4*>(p + 4);
  }
  __device__ __forceinline__ float operator[](int i) const { return i < 4 ? a[i] : b[i - 4]; }
};

// s + a . b over 8 elements: bf16 pairs through v_dot2_f32_bf16 (both
// products exact, fp32 sums), fp32 through 8 FMAs in element order.  The
// pairs are taken from the whole 8-element vector with shufflevector: a bit
// cast of one 32-bit element of the packed vector to a bf16 pair is
// compiled as element 0 every time by this compiler.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot8(const Raw8<uint16_t>& a, const Raw8<uint16_t>& b, float s) {
  const bf16x8 x = __builtin_bit_cast(bf16x8, a.w), y = __builtin_bit_cast(bf16x8, b.w);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 0, 1),
                                      __builtin_shufflevector(y, y, 0, 1), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 2, 3),
                                      __builtin_shufflevector(y, y, 2, 3), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 4, 5),
                                      __builtin_shufflevector(y, y, 4, 5), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 6, 7),
                                      __builtin_shufflevector(y, y, 6, 7), s, false);
  return s;
}
__device__ __forceinline__ float dot8(const Raw8<float>& a, const Raw8<float>& b, float s) {
#pragma unroll
  for (int i = 0; i < 8; i++) s = fmaf(a[i], b[i], s);
  return s;
}

__device__ __forceinline__ int readlane_i(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// ------------------------------------------------------------------------
// One wave per token; lane owns 8-element units u = lane + 64 i (i < U).
// The k slots' (expert, gate, sorted position) are fetched one slot per
// lane, then expert rows are loaded CH slots at a time so that several row
// loads are in flight before any is consumed.
template <typename T, int U>
__global__ __launch_bounds__(256) void k_combine(CombineArgs a) {
  constexpr int CH = U >= 4 ? 2 : 4;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int d = a.d, nu = d / 8, k = a.k;
  float acc[U][8];
#pragma unroll
  for (int i = 0; i < U; i++)
#pragma unroll
    for (int q = 0; q < 8; q++) acc[i][q] = 0.f;

  int me = 0, mp = 0;
  float mg = 0.f;
  if (lane < k) {
    me = a.idx[t * k + lane];
    mg = a.gate[t * k + lane];
    mp = a.inv_perm[t * k + lane];
  }
  const T* sy = reinterpret_cast<const T*>(a.shared_y);
  for (int s = 0; s < a.n_shared; s++) {
    const T* row = sy + ((int64_t)s * a.T + t) * d;
#pragma unroll
    for (int i = 0; i < U; i++) {
      const int u = lane + 64 * i;
      if (u < nu) {
        Raw8<T> r;
        r.load(row + u * 8);
#pragma unroll
        for (int q = 0; q < 8; q++) acc[i][q] += r[q];
      }
    }
  }
  const T* xrow = reinterpret_cast<const T*>(a.x) + t * d;
  const T* y = reinterpret_cast<const T*>(a.y);
  for (int j0 = 0; j0 < k; j0 += CH) {
    Raw8<T> r[CH][U];
#pragma unroll
    for (int c = 0; c < CH; c++) {
      const int j = j0 + c;
      if (j < k) {
        const int e = readlane_i(me, j);
        if (e < a.E_ffn) {
          const T* row = y + (int64_t)readlane_i(mp, j) * d;
#pragma unroll
          for (int i = 0; i < U; i++) {
            const int u = lane + 64 * i;
            if (u < nu) r[c][i].load(row + u * 8);
          }
        }
      }
    }
#pragma unroll
    for (int c = 0; c < CH; c++) {
      const int j = j0 + c;
      if (j >= k) break;
      const int e = readlane_i(me, j);
      const float g = readlane_f(mg, j);
      if (e < a.E_ffn) {
#pragma unroll
        for (int i = 0; i < U; i++)
          if (lane + 64 * i < nu)
#pragma unroll
            for (int q = 0; q < 8; q++) acc[i][q] += g * r[c][i][q];
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
            Raw8<T> xv;
            xv.load(xrow + u * 8);
#pragma unroll
            for (int q = 0; q < 8; q++) acc[i][q] += g * xv[q];
          }
        }
        continue;
      }
      // constant expert: [a, b] = softmax(W_c x) over the whole row
      const int ci = a.const_index[z];
      const float* wc0 = a.const_wc + (int64_t)ci * 2 * d;
      const float* wc1 = wc0 + d;
      const T* vrow = reinterpret_cast<const T*>(a.const_v) + (int64_t)ci * d;
      float pa = 0.f, pb = 0.f;
#pragma unroll
      for (int i = 0; i < U; i++) {
        const int u = lane + 64 * i;
        if (u < nu) {
          Raw8<T> xv;
          xv.load(xrow + u * 8);
          float w0[8], w1[8];
          Elt<float>::load8(wc0 + u * 8, w0);
          Elt<float>::load8(wc1 + u * 8, w1);
#pragma unroll
          for (int q = 0; q < 8; q++) {
            pa = fmaf(w0[q], xv[q], pa);
            pb = fmaf(w1[q], xv[q], pb);
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
          Raw8<T> xv, vv;
          xv.load(xrow + u * 8);
          vv.load(vrow + u * 8);
#pragma unroll
          for (int q = 0; q < 8; q++) acc[i][q] += ca * xv[q] + cb * vv[q];
        }
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

// Small batches: one wave per (token, 512-element column slice), so a
// decode batch of 16 tokens runs 64 waves instead of 16 and every slot's row
// slice is loaded at once (up to 8 rows in flight per lane): the metadata
// and one round of row loads instead of one round per two slots.  Each
// output element takes the same additions in the same order as in
// k_combine, so both give identical results.  No constant experts (their
// coefficients need the whole row).
template <typename T>
__global__ __launch_bounds__(256) void k_combine_cols(CombineArgs a, int slices) {
  constexpr int CH = 8;
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t t = w / slices;
  if (t >= a.T) return;
  const int d = a.d, nu = d / 8, k = a.k;
  const int u = (int)(w - t * slices) * 64 + lane;
  const bool on = u < nu;
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; q++) acc[q] = 0.f;
  int me = 0, mp = 0;
  float mg = 0.f;
  if (lane < k) {
    me = a.idx[t * k + lane];
    mg = a.gate[t * k + lane];
    mp = a.inv_perm[t * k + lane];
  }
  const T* sy = reinterpret_cast<const T*>(a.shared_y);
  for (int s = 0; s < a.n_shared; s++) {
    if (on) {
      Raw8<T> r;
      r.load(sy + ((int64_t)s * a.T + t) * d + u * 8);
#pragma unroll
      for (int q = 0; q < 8; q++) acc[q] += r[q];
    }
  }
  const T* xrow = reinterpret_cast<const T*>(a.x) + t * d;
  const T* y = reinterpret_cast<const T*>(a.y);
  for (int j0 = 0; j0 < k; j0 += CH) {
    Raw8<T> r[CH];
#pragma unroll
    for (int c = 0; c < CH; c++) {
      const int j = j0 + c;
      if (j < k && on) {
        const int e = readlane_i(me, j);
        if (e < a.E_ffn) r[c].load(y + (int64_t)readlane_i(mp, j) * d + u * 8);
        else if (a.zc_kind[e - a.E_ffn] == MOE_ZC_COPY) r[c].load(xrow + u * 8);
      }
    }
#pragma unroll
    for (int c = 0; c < CH; c++) {
      const int j = j0 + c;
      if (j >= k) break;
      const int e = readlane_i(me, j);
      const float g = readlane_f(mg, j);
      if (e >= a.E_ffn && a.zc_kind[e - a.E_ffn] == MOE_ZC_ZERO) continue;
      if (on)
#pragma unroll
        for (int q = 0; q < 8; q++) acc[q] += g * r[c][q];
    }
  }
  if (on) Elt<T>::store8(reinterpret_cast<T*>(a.out) + t * d + u * 8, acc);
}

// ------------------------------------------------------------------------
// Atomic stage 1: h[p] = silu(u_e . x_t) for sorted task p (task perm[p] =
// t*k + j, e = idx[task]).  A wave takes 8 consecutive sorted tasks, 8
// lanes per task; lane s of a group loads units s, s+8, ... of both rows, so
// each load instruction reads 8 rows x 128 contiguous bytes and a lane has
// many loads in flight.
//
// The sorted order groups tasks by row of the expert grid and runs tokens
// in order inside a row, and each XCD walks one contiguous stretch of it:
// block b (on XCD b % 8) takes chunk i = b / 8 of XCD b % 8's stretch.  The
// blocks an XCD runs at once thus cover a few consecutive rows, whose u
// vectors (pk_cols of them) and tokens' x rows are read from HBM or the
// memory-side cache once and re-read from the XCD's L2; a token's several
// tasks in one row are adjacent and share their x row in one load.
constexpr int kAtomTasksPerWave = 8;
constexpr int kAtomTasksPerBlock = 4 * kAtomTasksPerWave;

template <typename T>
__global__ __launch_bounds__(256) void k_atomic_h(const T* __restrict__ x,
                                                 const T* __restrict__ atom_u,
                                                 const int32_t* __restrict__ idx,
                                                 const int32_t* __restrict__ perm, int64_t n,
                                                 int k, int d, float* __restrict__ h) {
  const int lane = threadIdx.x & 63, sub = lane & 7;
  // chunk of this block: XCD x owns chunks [x q + min(x, r), ..) of the
  // 8 q + r chunks (one more for the first r XCDs)
  const int64_t nblk = gridDim.x, q = nblk / kXcds, r = nblk % kXcds;
  const int64_t xcd = blockIdx.x % kXcds, i = blockIdx.x / kXcds;
  const int64_t chunk = xcd * q + (xcd < r ? xcd : r) + i;
  const int64_t p = chunk * kAtomTasksPerBlock + (threadIdx.x >> 6) * kAtomTasksPerWave +
                    (lane >> 3);
  const bool ok = p < n;
  const int32_t task = perm[ok ? p : n - 1];
  const int e = idx[task];
  const T* xr = x + (int64_t)(task / k) * d;
  const T* ur = atom_u + (int64_t)e * d;
  const int nu = d / 8;
  float s = 0.f;
#pragma unroll 8
  for (int u = sub; u < nu; u += 8) {
    Raw8<T> xv, uv;
    xv.load(xr + u * 8);
    uv.load(ur + u * 8);
    s = dot8(uv, xv, s);
  }
  s += __shfl_xor(s, 1, 64);
  s += __shfl_xor(s, 2, 64);
  s += __shfl_xor(s, 4, 64);
  if (ok && sub == 0) h[p] = silu_f32(s);
}

// Atomic stage 2: out_t = sum_s shared + sum_j (g_tj * h_tj) w_e, one wave
// per token, slots in order, fp32.  Slot metadata and coefficients are
// fetched one slot per lane; rows are loaded CH slots at a time.
template <typename T, int U>
__global__ __launch_bounds__(256) void k_atomic_combine(const T* __restrict__ atom_w,
                                                       const int32_t* __restrict__ idx,
                                                       const float* __restrict__ gate,
                                                       const int32_t* __restrict__ inv_perm,
                                                       const float* __restrict__ h,
                                                       const T* __restrict__ shared_y,
                                                       int n_shared, int64_t T_, int k, int d,
                                                       T* __restrict__ out) {
  constexpr int CH = U >= 4 ? 2 : (U == 2 ? 4 : 8);
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
        Raw8<T> r;
        r.load(row + u * 8);
#pragma unroll
        for (int q = 0; q < 8; q++) acc[i][q] += r[q];
      }
    }
  }
  int me = 0;
  float mc = 0.f;
  if (lane < k) {
    const int64_t task = t * k + lane;
    me = idx[task];
    mc = gate[task] * h[inv_perm[task]];
  }
  for (int j0 = 0; j0 < k; j0 += CH) {
    Raw8<T> r[CH][U];
#pragma unroll
    for (int c = 0; c < CH; c++) {
      const int j = j0 + c;
      if (j < k) {
        const T* wr = atom_w + (int64_t)readlane_i(me, j) * d;
#pragma unroll
        for (int i = 0; i < U; i++) {
          const int u = lane + 64 * i;
          if (u < nu) r[c][i].load(wr + u * 8);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < CH; c++) {
      const int j = j0 + c;
      if (j >= k) break;
      const float coef = readlane_f(mc, j);
#pragma unroll
      for (int i = 0; i < U; i++)
        if (lane + 64 * i < nu)
#pragma unroll
          for (int q = 0; q < 8; q++) acc[i][q] = fmaf(coef, r[c][i][q], acc[i][q]);
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

// batches of at most this many tokens use the column-slice kernel
constexpr int64_t kCombineColsTokens = 256;

template <typename T>
static hipError_t combine_t(const CombineArgs& a, hipStream_t st) {
  const int U = (int)cdiv(a.d, 512);
  bool consts = false;
  for (int z = 0; z < MOE_MAX_ZC; z++) consts |= a.zc_kind[z] == MOE_ZC_CONST;
  if (a.T <= kCombineColsTokens && !consts) {
    hipLaunchKernelGGL(k_combine_cols<T>, dim3((unsigned)cdiv(a.T * U, 4)), dim3(256), 0, st, a,
                       U);
    return hipGetLastError();
  }
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
  dim3 grid((unsigned)cdiv(n, kAtomTasksPerBlock)), block(256);
  hipLaunchKernelGGL((k_atomic_h<T>), grid, block, 0, st, (const T*)x, (const T*)u, idx, perm, n,
                     k, d, h);
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
