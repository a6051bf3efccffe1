// Router kernels: logits (fp32-exact dot products on bf16 MFMA, or plain
// fp32 FMA for fp32 layers) and the per-token selection (softmax top-k, or
// the Cartesian-product candidate search).
//
// Routing follows "OmniMoE: An Efficient MoE by Orchestrating Atomic Experts
// at Scale" (Technical Summary sec. 1: a router over N experts costs O(N d);
// sec. 2.2 "Cartesian Product Router": row and column logits over a 2-D
// expert grid, combined to score experts) and the MoE++ page ("Approach":
// one router over FFN and zero-computation experts, tau on the FFN ones).
#include "kernels.h"

namespace moe {

// ------------------------------------------------------------------------
// fp32 router weight -> three bf16 slices (hi + mid + lo == w exactly).
//
// hi keeps the top 8 significant bits of w (truncation), mid the next 8 of
// the exact remainder w - hi, and lo the remaining <= 8 bits, which bf16
// holds exactly.  A bf16 x times each slice is exact in fp32, so three bf16
// MFMA passes with fp32 accumulation give an fp32-accurate dot product at
// matrix-core rate.
__device__ __forceinline__ void split3(float v, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
  const uint32_t hb = __float_as_uint(v) & 0xffff0000u;
  const float r1 = v - __uint_as_float(hb);
  const uint32_t mb = __float_as_uint(r1) & 0xffff0000u;
  const float r2 = r1 - __uint_as_float(mb);
  hi = (uint16_t)(hb >> 16);
  mid = (uint16_t)(mb >> 16);
  lo = (uint16_t)(__float_as_uint(r2) >> 16);  // exact: <= 8 bits left
}

// ------------------------------------------------------------------------
// Partial logits over a K range:
//   part[z][t, col_off + n] = x[t, x_off + K_z] . W[n, K_z]   (n < NL)
// with K_z the z-th of gridDim.z equal K ranges (split K keeps enough
// blocks busy at small T; the selection kernel adds the partials in order z).
// bf16 x; fp32 W [NL, K].
//
// Block: MT tokens (64 with 4 waves, or 256 with 8) x 64 logits; wave w
// owns tokens w*MT/NW .. +MT/NW (MT/(16 NW) blocks of 16) and all 64 logits
// (four v_mfma_f32_16x16x32_bf16 tiles per token block).  Per 64-wide K
// chunk the block's 64 fp32 weight rows are read once, split into their
// three bf16 slices and staged in LDS (24 KB, double buffered), shared by
// the waves; x fragments go straight from global memory to registers, one
// chunk ahead.  The larger block re-splits the weights for 4x the tokens
// (the product-key layer, with many tokens and no split K).  K is permuted
// identically for both operands: lane (r = l%16, q = l/16) takes elements
// [16q, 16q+16) of the chunk, MFMA step h the half [16q + 8h, +8), so each x
// row is one 128-byte run.  The three slices accumulate into one fp32
// accumulator.
__device__ __forceinline__ int rl_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <int MT, int NW>
__global__ __launch_bounds__(64 * NW) void k_router_logits_bf16(
    const uint16_t* __restrict__ x, int64_t T, int ldx, RouterPart p0, RouterPart p1, int K,
    float* __restrict__ logits, int ldl, int64_t part_stride) {
  constexpr int NT = 64 * NW;
  constexpr int MB = MT / (16 * NW);  // token blocks of 16 per wave
  constexpr int BL = 1024 / NT;       // weight float4 loads per thread per chunk
  static_assert(MB >= 1 && MB * 16 * NW == MT && BL * NT == 1024, "router tile");
  // [buf][slice * 64 + logit][64 K] bf16, 16-byte chunks swizzled
  __shared__ __attribute__((aligned(16))) uint16_t bs[2][3 * 64 * 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t m0 = (int64_t)blockIdx.x * MT + wave * (MT / NW);
  // blockIdx.y: the first part's logit blocks, then the second's
  const bool second = (int)blockIdx.y >= p0.ny;
  const float* __restrict__ W = second ? p1.W : p0.W;
  const int NL = second ? p1.NL : p0.NL;
  const int x_off = second ? p1.x_off : p0.x_off;
  const int col_off = second ? p1.col_off : p0.col_off;
  const int n0 = ((int)blockIdx.y - (second ? p0.ny : 0)) * 64;
  const int kc = K / gridDim.z;
  const int kbeg = blockIdx.z * kc, nch = kc / 64;
  const int r = lane & 15, q = lane >> 4;
  const uint16_t* ap[MB];
#pragma unroll
  for (int mb = 0; mb < MB; mb++) {
    int64_t am = m0 + mb * 16 + r;
    if (am >= T) am = T - 1;  // clamped rows feed only outputs that are not stored
    ap[mb] = x + am * (int64_t)ldx + x_off + kbeg + q * 16;
  }

  // B loader: 64 rows x 16 float4 = 1024 float4, BL per thread; float4 i
  // of this thread is row id/16, K elements 4(id%16) .. +3
  // Rows past NL load a valid row (unconditional loads) but are neither
  // split nor stored: their logits are never written, and a router of
  // fewer than 64 experts skips most of the splitting.
  const float* bsrc[BL];
  int bdst[BL];
  bool bok[BL];
#pragma unroll
  for (int i = 0; i < BL; i++) {
    const int id = tid + NT * i;
    const int nl = id >> 4, k4 = (id & 15) * 4;
    bok[i] = n0 + nl < NL;
    const int n = n0 + nl < NL ? n0 + nl : NL - 1;
    bsrc[i] = W + (int64_t)n * K + kbeg + k4;
    bdst[i] = nl * 64 + (((k4 >> 3) ^ rl_swz(nl)) * 8) + (k4 & 7);  // slice 0 position
  }
  f32x4 breg[BL];
  auto bload = [&](int c) {
#pragma unroll
    for (int i = 0; i < BL; i++) breg[i] = *reinterpret_cast<const f32x4*>(bsrc[i] + c * 64);
  };
  auto bstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < BL; i++) {
      if (!bok[i]) continue;
      uint16_t h[4], m[4], l[4];
#pragma unroll
      for (int e = 0; e < 4; e++) split3(breg[i][e], h[e], m[e], l[e]);
      auto pack = [](const uint16_t (&v)[4]) {
        return make_uint2((uint32_t)v[0] | ((uint32_t)v[1] << 16),
                          (uint32_t)v[2] | ((uint32_t)v[3] << 16));
      };
      // rows of slice p are p*64 + nl: same swizzle, offset p * 64 rows
      *reinterpret_cast<uint2*>(&bs[buf][bdst[i]]) = pack(h);
      *reinterpret_cast<uint2*>(&bs[buf][64 * 64 + bdst[i]]) = pack(m);
      *reinterpret_cast<uint2*>(&bs[buf][2 * 64 * 64 + bdst[i]]) = pack(l);
    }
  };

  f32x4 acc[MB][4];
#pragma unroll
  for (int mb = 0; mb < MB; mb++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[mb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // x fragments of chunk c + 1 are loaded while chunk c multiplies
  u32x4 a0[MB], a1[MB];
#pragma unroll
  for (int mb = 0; mb < MB; mb++) {
    a0[mb] = *reinterpret_cast<const u32x4*>(ap[mb]);
    a1[mb] = *reinterpret_cast<const u32x4*>(ap[mb] + 8);
  }
  bload(0);
  bstore(0);
  __syncthreads();
  for (int c = 0; c < nch; c++) {
    const int buf = c & 1;
    u32x4 an0[MB], an1[MB];
#pragma unroll
    for (int mb = 0; mb < MB; mb++) {
      an0[mb] = a0[mb];
      an1[mb] = a1[mb];
    }
    if (c + 1 < nch) {
#pragma unroll
      for (int mb = 0; mb < MB; mb++) {
        an0[mb] = *reinterpret_cast<const u32x4*>(ap[mb] + (c + 1) * 64);
        an1[mb] = *reinterpret_cast<const u32x4*>(ap[mb] + (c + 1) * 64 + 8);
      }
      bload(c + 1);
    }
#pragma unroll
    for (int p = 0; p < 3; p++)
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int row = p * 64 + j * 16 + r;
        const int sw = rl_swz(row);
        const u32x4 b0 = *reinterpret_cast<const u32x4*>(&bs[buf][row * 64 + (((2 * q) ^ sw) * 8)]);
        const u32x4 b1 = *reinterpret_cast<const u32x4*>(&bs[buf][row * 64 + (((2 * q + 1) ^ sw) * 8)]);
#pragma unroll
        for (int mb = 0; mb < MB; mb++) {
          acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, a0[mb]), __builtin_bit_cast(bf16x8, b0), acc[mb][j], 0, 0, 0);
          acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, a1[mb]), __builtin_bit_cast(bf16x8, b1), acc[mb][j], 0, 0, 0);
        }
      }
    if (c + 1 < nch) bstore(buf ^ 1);
#pragma unroll
    for (int mb = 0; mb < MB; mb++) {
      a0[mb] = an0[mb];
      a1[mb] = an1[mb];
    }
    __syncthreads();
  }
  // lane holds C[4 q + e][16 j + r] of each of its token blocks
  float* out = logits + blockIdx.z * part_stride;
#pragma unroll
  for (int mb = 0; mb < MB; mb++)
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int n = n0 + 16 * j + r;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int64_t m = m0 + mb * 16 + 4 * q + e;
        if (m < T && n < NL) out[m * ldl + col_off + n] = acc[mb][j][e];
      }
    }
}

// fp32 layers: one thread per logit, four interleaved fp32 partial sums.
__global__ void k_router_logits_f32(const float* __restrict__ x, int64_t T, int ldx, int x_off,
                                    const float* __restrict__ W, int NL, int K,
                                    float* __restrict__ logits, int ldl, int col_off) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * NL) return;
  int64_t t = i / NL;
  int n = (int)(i % NL);
  const float* a = x + t * ldx + x_off;
  const float* b = W + (int64_t)n * K;
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
  for (int kk = 0; kk < K; kk += 4) {
    s0 = fmaf(a[kk], b[kk], s0);
    s1 = fmaf(a[kk + 1], b[kk + 1], s1);
    s2 = fmaf(a[kk + 2], b[kk + 2], s2);
    s3 = fmaf(a[kk + 3], b[kk + 3], s3);
  }
  logits[t * ldl + col_off + n] = (s0 + s1) + (s2 + s3);
}

// ------------------------------------------------------------------------
// Sum of the K-split partials of one logit, in split order.  All loads are
// issued before the first add (a load-add chain would pay the memory
// latency once per split).
constexpr int kMaxRouterSplits = 16;
__device__ __forceinline__ float sum_parts(const float* p, int nparts, int64_t stride) {
  if (nparts == 1) return p[0];  // no K split: skips 2 x 15 uniform branches per logit
  float v[kMaxRouterSplits];
#pragma unroll
  for (int z = 0; z < kMaxRouterSplits; z++) v[z] = z < nparts ? p[z * stride] : 0.f;
  float l = v[0];
#pragma unroll
  for (int z = 1; z < kMaxRouterSplits; z++)
    if (z < nparts) l += v[z];
  return l;
}

// Softmax top-k selection, one wave per token.  V = values per lane
// (E <= 64 V).  Logit l = fl32(dot + bias), plus the gating residual r of
// the MoE++ page ("Approach": router scores carried over from the previous
// layer) when given, then fl32(tau * l) for FFN experts.  Order (-l, e);
// gates = softmax over all E at the chosen ones, optionally renormalised
// over the k.
template <int V>
__global__ __launch_bounds__(256) void k_select_topk(const float* __restrict__ logits, int nparts,
                                                    int64_t part_stride, int64_t T,
                                                    int E, int E_ffn, int k, float tau,
                                                    const float* __restrict__ bias,
                                                    const float* __restrict__ residual, int renorm,
                                                    int32_t* __restrict__ idx_out,
                                                    float* __restrict__ gate_out) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + t * E;
  float v[V];
#pragma unroll
  for (int i = 0; i < V; i++) {
    int e = lane + 64 * i;
    float l = -INFINITY;
    if (e < E) {
      l = sum_parts(row + e, nparts, part_stride);
      if (bias) l = l + bias[e];
      if (residual) l = l + residual[t * E + e];
      if (e < E_ffn) l = tau * l;
    }
    v[i] = l;
  }
  float m = v[0];
#pragma unroll
  for (int i = 1; i < V; i++) m = fmaxf(m, v[i]);
  m = wave_max(m);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < V; i++)
    if (lane + 64 * i < E) s += __expf(v[i] - m);
  s = wave_sum(s);
  uint32_t taken = 0;
  float my_val = 0.f;
  int my_idx = 0;
  float gsum = 0.f;
  for (int j = 0; j < k; j++) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < V; i++) {
      int e = lane + 64 * i;
      bool ok = e < E && !((taken >> i) & 1u);
      if (ok && (v[i] > bv || bi == 0x7fffffff)) { bv = v[i]; bi = e; }
    }
    wave_argmax(bv, bi);
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    float g = __expf(bv - m) / s;
    gsum += g;
    if (lane == j) { my_val = g; my_idx = bi; }
  }
  if (lane < k) {
    float g = renorm ? my_val / gsum : my_val;
    idx_out[t * k + lane] = my_idx;
    gate_out[t * k + lane] = g;
  }
}

// ------------------------------------------------------------------------
// Wave-wide selection helpers.  A wave holds up to 64 V (key, id) pairs, V
// per lane (slot i of lane l).  Keys are fp32 scores mapped to uint32 so
// that unsigned order is score order; empty slots hold key 0, which no
// score maps to, so they never count.  Ids are unique.  Rank order is (key
// descending, id ascending); NaN scores are not supported.

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t b = f == 0.f ? 0u : __float_as_uint(f);  // -0 ranks as +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// keys >= c over the wave
template <int V>
__device__ __forceinline__ int count_ge(const uint32_t (&key)[V], uint32_t c) {
  int n = 0;
#pragma unroll
  for (int i = 0; i < V; i++) n += __popcll(__ballot(key[i] >= c));
  return n;
}

// Threshold search of wave_select: the largest th with at least K keys
// >= th, found bit by bit (a key prefix is kept while at least K keys reach
// it).  Stops early once exactly K keys reach the prefix: those K are then
// the answer whatever the lower bits.  K >= 1 and at least K non-empty
// slots, so th > 0.
template <int V>
__device__ __forceinline__ uint32_t select_threshold(const uint32_t (&key)[V], int K) {
  uint32_t th = 0;
  for (int b = 31; b >= 0; b--) {
    const uint32_t cand = th | (1u << b);
    const int cnt = count_ge<V>(key, cand);
    if (cnt >= K) th = cand;
    if (cnt == K) break;
  }
  return th;
}

// Marks in sel (bit i = slot i) the K best pairs given the threshold th of
// select_threshold: every key above th is taken, and the keys equal to th
// are taken by ascending id until K are.
template <int V>
__device__ __forceinline__ uint32_t select_at(const uint32_t (&key)[V], const int (&id)[V], int K,
                                             uint32_t th) {
  uint32_t sel = 0, eq = 0;
  int gt = 0, neq = 0;
#pragma unroll
  for (int i = 0; i < V; i++) {
    if (key[i] > th) sel |= 1u << i;
    if (key[i] == th) eq |= 1u << i;
    gt += __popcll(__ballot(key[i] > th));
    neq += __popcll(__ballot(key[i] == th));
  }
  int need = K - gt;
  if (need >= neq) return sel | eq;
  // more ties than places: smallest ids first
  for (; need > 0; need--) {
    int best = 0x7fffffff, slot = -1;
#pragma unroll
    for (int i = 0; i < V; i++)
      if (((eq >> i) & 1u) && id[i] < best) { best = id[i]; slot = i; }
    const int m = wave_reduce_dpp(best, [](int a, int b) { return a < b ? a : b; });
    if (slot >= 0 && best == m) {
      sel |= 1u << slot;
      eq &= ~(1u << slot);
    }
  }
  return sel;
}

template <int V>
__device__ __forceinline__ uint32_t wave_select(const uint32_t (&key)[V], const int (&id)[V],
                                                int K) {
  return select_at<V>(key, id, K, select_threshold<V>(key, K));
}

// Position of each selected pair in [0, K): slots in order, lanes in order.
template <int V>
__device__ __forceinline__ void wave_positions(uint32_t sel, int (&pos)[V]) {
  const int lane = threadIdx.x & 63;
  int base = 0;
#pragma unroll
  for (int i = 0; i < V; i++) {
    const uint64_t m = __ballot((sel >> i) & 1u);
    pos[i] = base + __popcll(m & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
    base += __popcll(m);
  }
}

// Value of lane l ^ M: DPP quad permutations for M = 1, 2 (no LDS trip),
// ds_swizzle's xor mode inside 32 lanes for M = 4 .. 16, ds_bpermute for 32.
template <int M>
__device__ __forceinline__ int lane_xor(int v) {
  if constexpr (M == 1) return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
  else if constexpr (M == 2) return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);  // [2,3,0,1]
  else if constexpr (M < 32) return __builtin_amdgcn_ds_swizzle(v, 0x1F | (M << 10));
  else return __shfl_xor(v, M, kWave);
}

// One compare-exchange step of a bitonic sort, best first within blocks
// of SIZE lanes whose SIZE-bit is clear (the other blocks sort reversed)
template <int SIZE, int STRIDE>
__device__ __forceinline__ void bitonic_step(uint32_t& key, int& id, int lane) {
  const uint32_t ok = (uint32_t)lane_xor<STRIDE>((int)key);
  const int oi = lane_xor<STRIDE>(id);
  const bool first = key > ok || (key == ok && id < oi);
  const bool keep = (((lane & STRIDE) == 0) == ((lane & SIZE) == 0)) ? first : !first;
  if (!keep) { key = ok; id = oi; }
}

template <int SIZE>
__device__ __forceinline__ void bitonic_merge(uint32_t& key, int& id, int lane) {
  if constexpr (SIZE >= 64) bitonic_step<SIZE, 32>(key, id, lane);
  if constexpr (SIZE >= 32) bitonic_step<SIZE, 16>(key, id, lane);
  if constexpr (SIZE >= 16) bitonic_step<SIZE, 8>(key, id, lane);
  if constexpr (SIZE >= 8) bitonic_step<SIZE, 4>(key, id, lane);
  if constexpr (SIZE >= 4) bitonic_step<SIZE, 2>(key, id, lane);
  bitonic_step<SIZE, 1>(key, id, lane);
}

// Sorts one (key, id) pair per lane, best first, over lanes 0..n-1 (n <=
// 64; lanes n.. hold pads: key 0, id INT_MAX).  n <= 32 sorts each half of
// the wave on its own, which leaves lanes 0..31 in order.
__device__ __forceinline__ void wave_sort(uint32_t& key, int& id, int n) {
  const int lane = threadIdx.x & 63;
  bitonic_merge<2>(key, id, lane);
  bitonic_merge<4>(key, id, lane);
  bitonic_merge<8>(key, id, lane);
  bitonic_merge<16>(key, id, lane);
  bitonic_merge<32>(key, id, lane);
  if (n > 32) bitonic_merge<64>(key, id, lane);
}

// ------------------------------------------------------------------------
// Cartesian-product selection, one wave per token.
//   scores: [T, rows + cols] (row scores first).
//   1. top-krow rows, top-kcol columns by (-score, index);
//   2. candidates (a, b): sigma = fl32(s_r + s_c), id = row * cols + col;
//   3. top-k candidates by (-sigma, id); gates = softmax over the k sigmas.
// V = values per lane (max(rows, cols, krow*kcol) <= 64 V); krow, kcol, k
// <= 64.
template <int V>
__global__ __launch_bounds__(256) void k_select_pk(const float* __restrict__ scores, int nparts,
                                                  int64_t part_stride, int64_t T,
                                                  int rows, int cols, int krow, int kcol, int k,
                                                  int32_t* __restrict__ idx_out,
                                                  float* __restrict__ gate_out) {
  __shared__ float sel_val[4][2][64];
  __shared__ int sel_idx[4][2][64];
  __shared__ uint32_t top_key[4][64];
  __shared__ int top_id[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= T) return;
  const float* srow = scores + t * (int64_t)(rows + cols);
  // step 1: rows and columns, their two threshold searches in one loop
  float v2[2][V];
  uint32_t key2[2][V];
  int id2[2][V];
#pragma unroll
  for (int side = 0; side < 2; side++) {
    const int n = side ? cols : rows;
    const float* s = srow + (side ? rows : 0);
#pragma unroll
    for (int i = 0; i < V; i++) {
      const int e = lane + 64 * i;
      float sc = -INFINITY;
      if (e < n) sc = sum_parts(s + e, nparts, part_stride);
      v2[side][i] = sc;
      key2[side][i] = e < n ? order_key(sc) : 0u;
      id2[side][i] = e;
    }
  }
  // two plain searches: the scalar unit (shared by the CU's SIMDs) is the
  // bound here, and one loop per side carries far less loop control than
  // one loop interleaving both
  const uint32_t th2[2] = {select_threshold<V>(key2[0], krow), select_threshold<V>(key2[1], kcol)};
#pragma unroll
  for (int side = 0; side < 2; side++) {
    const uint32_t sel = select_at<V>(key2[side], id2[side], side ? kcol : krow, th2[side]);
    int pos[V];
    wave_positions<V>(sel, pos);
#pragma unroll
    for (int i = 0; i < V; i++)
      if ((sel >> i) & 1u) {
        sel_val[wave][side][pos[i]] = v2[side][i];
        sel_idx[wave][side][pos[i]] = id2[side][i];
      }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  // step 2: candidate scores
  const int nc = krow * kcol;
  uint32_t key[V];
  int id[V];
#pragma unroll
  for (int i = 0; i < V; i++) {
    const int c = lane + 64 * i;
    if (c < nc) {
      const int a = c / kcol, b = c - a * kcol;
      key[i] = order_key(sel_val[wave][0][a] + sel_val[wave][1][b]);
      id[i] = sel_idx[wave][0][a] * cols + sel_idx[wave][1][b];
    } else {
      key[i] = 0u;
      id[i] = 0x7fffffff;
    }
  }
  // step 3: the k best candidates, gathered in lanes 0..k-1 and sorted
  const uint32_t sel = wave_select<V>(key, id, k);
  int pos[V];
  wave_positions<V>(sel, pos);
#pragma unroll
  for (int i = 0; i < V; i++)
    if ((sel >> i) & 1u) {
      top_key[wave][pos[i]] = key[i];
      top_id[wave][pos[i]] = id[i];
    }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  uint32_t mk = lane < k ? top_key[wave][lane] : 0u;
  int mi = lane < k ? top_id[wave][lane] : 0x7fffffff;
  wave_sort(mk, mi, k);
  // back to fp32 scores; gates = softmax over the k (the first is the max)
  const uint32_t bits = (mk & 0x80000000u) ? (mk & 0x7fffffffu) : ~mk;
  const float sv = __uint_as_float(bits);
  const float top = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                                  __builtin_bit_cast(int, sv)));
  const float e = lane < k ? __expf(sv - top) : 0.f;
  // the sum in rank order (lane broadcasts through scalar registers)
  float gsum = 0.f;
  for (int j = 0; j < k; j++)
    gsum += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, e), j));
  if (lane < k) {
    idx_out[t * k + lane] = mi;
    gate_out[t * k + lane] = e / gsum;
  }
}

// ------------------------------------------------------------------------
// launchers

int router_splits(int dtype, int64_t T, int NL, int K) {
  if (dtype != MOE_BF16) return 1;
  const int64_t blocks = cdiv(T, 64) * cdiv(NL, 64);
  int S = 1;
  while (S < kMaxRouterSplits && blocks * S < 512 && K % (64 * 2 * S) == 0) S *= 2;
  return S;
}

hipError_t launch_router_logits(int dtype, const void* x, int64_t T, int ldx, RouterPart p0,
                                RouterPart p1, int K, float* logits, int ldl, int splits,
                                hipStream_t st) {
  if (T == 0) return hipSuccess;
  p0.ny = (int)cdiv(p0.NL, 64);
  p1.ny = (int)cdiv(p1.NL, 64);
  if (p0.ny + p1.ny == 0) return hipSuccess;
  if (dtype == MOE_BF16) {
    // 256-token blocks of 8 waves when they alone give every CU a block:
    // the weights' split is then shared by 4x the tokens, and two waves per
    // SIMD overlap one's MFMAs with the other's splitting and loads
    const int ny = p0.ny + p1.ny;
    if (splits == 1 && cdiv(T, 256) * ny >= 256) {
      dim3 grid((unsigned)cdiv(T, 256), (unsigned)ny, 1);
      hipLaunchKernelGGL((k_router_logits_bf16<256, 8>), grid, dim3(512), 0, st,
                         (const uint16_t*)x, T, ldx, p0, p1, K, logits, ldl, (int64_t)T * ldl);
    } else {
      dim3 grid((unsigned)cdiv(T, 64), (unsigned)ny, (unsigned)splits);
      hipLaunchKernelGGL((k_router_logits_bf16<64, 4>), grid, dim3(256), 0, st,
                         (const uint16_t*)x, T, ldx, p0, p1, K, logits, ldl, (int64_t)T * ldl);
    }
  } else {
    for (const RouterPart& p : {p0, p1})
      if (p.NL > 0)
        hipLaunchKernelGGL(k_router_logits_f32, dim3((unsigned)cdiv(T * p.NL, 256)), dim3(256),
                           0, st, (const float*)x, T, ldx, p.x_off, p.W, p.NL, K, logits, ldl,
                           p.col_off);
  }
  return hipGetLastError();
}

hipError_t launch_select_topk(const float* logits, int splits, int64_t T, int E, int E_ffn, int k,
                              float tau, const float* bias, const float* residual, int renorm,
                              int32_t* idx, float* gate, hipStream_t st) {
  if (T == 0) return hipSuccess;
  dim3 grid((unsigned)cdiv(T, 4)), block(256);
  int V = (int)cdiv(E, 64);
#define SEL(VV) hipLaunchKernelGGL(k_select_topk<VV>, grid, block, 0, st, logits, splits, \
                                   (int64_t)T * E, T, E, E_ffn, k, tau, bias, residual, renorm, \
                                   idx, gate)
  if (V <= 1) SEL(1);
  else if (V <= 2) SEL(2);
  else SEL(4);
#undef SEL
  return hipGetLastError();
}

// Router logits before tau (for a next layer's gating residual): the same
// fl32 sums k_select_topk forms, in the same order, written out.
__global__ __launch_bounds__(256) void k_logits_out(const float* __restrict__ part, int nparts,
                                                   int64_t part_stride, int64_t n, int E,
                                                   const float* __restrict__ bias,
                                                   const float* __restrict__ residual,
                                                   float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float l = sum_parts(part + i, nparts, part_stride);
  if (bias) l = l + bias[i % E];
  if (residual) l = l + residual[i];
  out[i] = l;
}

hipError_t launch_logits_out(const float* part, int splits, int64_t T, int E, const float* bias,
                             const float* residual, float* out, hipStream_t st) {
  const int64_t n = T * E;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_logits_out, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, st, part, splits,
                     n, n, E, bias, residual, out);
  return hipGetLastError();
}

hipError_t launch_select_pk(const float* scores, int splits, int64_t T, int rows, int cols,
                            int krow, int kcol, int k, int32_t* idx, float* gate, hipStream_t st) {
  if (T == 0) return hipSuccess;
  int64_t mx = rows;
  if (cols > mx) mx = cols;
  if ((int64_t)krow * kcol > mx) mx = (int64_t)krow * kcol;
  int V = (int)cdiv(mx, 64);
  dim3 grid((unsigned)cdiv(T, 4)), block(256);
#define SEL(VV) hipLaunchKernelGGL(k_select_pk<VV>, grid, block, 0, st, scores, splits, \
                                   (int64_t)T * (rows + cols), T, rows, cols, krow, kcol, k, idx, \
                                   gate)
  if (V <= 1) SEL(1);
  else if (V <= 2) SEL(2);
  else if (V <= 4) SEL(4);
  else if (V <= 8) SEL(8);
  else SEL(16);
#undef SEL
  return hipGetLastError();
}

}  // namespace moe
