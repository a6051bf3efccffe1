// Shared device helpers for the gfx950 MoE kernels (wave64, CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16 bits

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// low / high bf16 of a packed dword as float
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Load 8 consecutive layer-dtype elements as floats (16 B bf16 / 32 B f32).
template <typename T> struct Elt;
template <> struct Elt<uint16_t> {
  __device__ __forceinline__ static void load8(const uint16_t* p, float v[8]) {
    u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; i++) { v[2 * i] = lo_bf16(w[i]); v[2 * i + 1] = hi_bf16(w[i]); }
  }
  __device__ __forceinline__ static void store8(uint16_t* p, const float v[8]) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; i++) w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    *reinterpret_cast<u32x4*>(p) = w;
  }
  __device__ __forceinline__ static float load1(const uint16_t* p) { return bf16_to_f32(*p); }
  __device__ __forceinline__ static void store1(uint16_t* p, float v) { *p = f32_to_bf16(v); }
};
template <> struct Elt<float> {
  __device__ __forceinline__ static void load8(const float* p, float v[8]) {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; i++) { v[i] = a[i]; v[4 + i] = b[i]; }
  }
  __device__ __forceinline__ static void store8(float* p, const float v[8]) {
    f32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; i++) { a[i] = v[i]; b[i] = v[4 + i]; }
    *reinterpret_cast<f32x4*>(p) = a;
    *reinterpret_cast<f32x4*>(p + 4) = b;
  }
  __device__ __forceinline__ static float load1(const float* p) { return *p; }
  __device__ __forceinline__ static void store1(float* p, float v) { *p = v; }
};

// ------------------------------------------------------------ wave reduce

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Cross-lane reductions with DPP: xor 1 and xor 2 inside quads, rotations
// by 4 and 8 inside rows of 16 lanes, then the four row results read into
// scalars.  Every lane returns the wave-wide result.
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce_dpp(T v, Op op) {
  static_assert(sizeof(T) == 4, "32-bit values");
  int b = __builtin_bit_cast(int, v);
  b = __builtin_bit_cast(int, op(v, __builtin_bit_cast(T, __builtin_amdgcn_update_dpp(b, b, 0xB1, 0xF, 0xF, false))));
  b = __builtin_bit_cast(int, op(__builtin_bit_cast(T, b), __builtin_bit_cast(T, __builtin_amdgcn_update_dpp(b, b, 0x4E, 0xF, 0xF, false))));
  b = __builtin_bit_cast(int, op(__builtin_bit_cast(T, b), __builtin_bit_cast(T, __builtin_amdgcn_update_dpp(b, b, 0x124, 0xF, 0xF, false))));
  b = __builtin_bit_cast(int, op(__builtin_bit_cast(T, b), __builtin_bit_cast(T, __builtin_amdgcn_update_dpp(b, b, 0x128, 0xF, 0xF, false))));
  const T r0 = __builtin_bit_cast(T, __builtin_amdgcn_readlane(b, 0));
  const T r1 = __builtin_bit_cast(T, __builtin_amdgcn_readlane(b, 16));
  const T r2 = __builtin_bit_cast(T, __builtin_amdgcn_readlane(b, 32));
  const T r3 = __builtin_bit_cast(T, __builtin_amdgcn_readlane(b, 48));
  return op(op(r0, r1), op(r2, r3));
}

// (value, index) argmax across the wave: larger value wins, ties go to the
// smaller index.  Every lane returns the winner.  NaN values are not
// supported (routing of NaN inputs is unspecified).
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  const float m = wave_reduce_dpp(v, [](float a, float b) { return fmaxf(a, b); });
  const int cand = (v == m) ? i : 0x7fffffff;
  i = wave_reduce_dpp(cand, [](int a, int b) { return a < b ? a : b; });
  v = m;
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + __expf(-z)); }

__host__ __device__ constexpr inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace moe
