// Grouped GEMMs of the expert stage ("OmniMoE: An Efficient MoE by
// Orchestrating Atomic Experts at Scale", Technical Summary sec. 2.2, step
// Grouped GEMM: a block of expert weights is loaded once and reused across
// all tokens of the expert's group).
//
//   GEMM1 (+ fused SiLU gate):  H = silu(X_e W_gate,e^T) * (X_e W_up,e^T)
//   GEMM2:                      Y = H_e W_down,e^T
//
// X_e rows are gathered from x through the dispatch permutation while the
// A tile is loaded.  Shared experts are extra groups whose rows are all
// tokens in order.  For GEMM1 the B tile holds W_gate rows and the same
// columns' W_up rows, and each wave's fragments pair gate and up columns, so
// silu(g)*u is formed in registers and H is written once, in bf16.
//
// Three kernels: k_gemm_dl (bf16 items of up to 256 rows: 8 waves,
// v_mfma_f32_16x16x32_bf16, 64-wide K tiles in a 20-slot direct-to-LDS
// ring; the main path), k_grouped_gemm_bf16 (decode-sized groups: 32-row
// tiles, v_mfma_f32_32x32x16_bf16, K tiles of 64 in one LDS buffer with the
// next staged in registers, 16-byte chunk c of a 128-byte row at
// c ^ (row & 7)), and k_grouped_gemm_f32 (fp32 layers, plain FMA).
#include <type_traits>

#include "kernels.h"
#include "tiles.h"

namespace moe {


template <bool SWIGLU>
struct TileCtx {
  bool shared;
  int e;      // expert index inside its table
  int64_t r0; // first row in the group's row space
  int nr;     // valid rows
  int N, K;
};

// Tile descriptors describe the tile's group: {group, first row, rows, first
// tile}; M tile g of the group covers rows [g*bm, min((g+1)*bm, rows)).
template <bool SWIGLU>
__device__ __forceinline__ TileCtx<SWIGLU> tile_ctx(const GemmArgs& a, int4 t, int g) {
  TileCtx<SWIGLU> c;
  c.shared = t.x >= a.E_ffn;
  c.e = c.shared ? t.x - a.E_ffn : t.x;
  c.r0 = (int64_t)t.y + (int64_t)g * a.bm;
  c.nr = t.z - g * a.bm < a.bm ? t.z - g * a.bm : a.bm;
  c.N = c.shared ? a.N_shared : a.N_routed;
  c.K = c.shared ? a.K_shared : a.K_routed;
  return c;
}

// A row source (element pointer) of local row i, or nullptr when out of range
template <typename T, bool SWIGLU>
__device__ __forceinline__ const T* a_row(const GemmArgs& a, const TileCtx<SWIGLU>& c, int i) {
  if (i >= c.nr) return nullptr;
  const int64_t r = c.r0 + i;
  if (SWIGLU) {
    int64_t tok = c.shared ? r : (int64_t)(a.perm[r] / a.k);
    return reinterpret_cast<const T*>(a.a_x) + tok * c.K;
  }
  if (c.shared)
    return reinterpret_cast<const T*>(a.a_shared) + r * c.K;  // one shared group here
  return reinterpret_cast<const T*>(a.a_routed) + r * c.K;
}

// B row source of tile row j (0 <= j < BN), or nullptr past N
template <typename T, bool SWIGLU, int BN>
__device__ __forceinline__ const T* b_row(const GemmArgs& a, const TileCtx<SWIGLU>& c, int n0,
                                          int j) {
  const void* base;
  int n;
  if (SWIGLU) {
    const bool up = j >= BN / 2;
    n = n0 + (up ? j - BN / 2 : j);
    base = c.shared ? (up ? a.b1_shared : a.b0_shared) : (up ? a.b1_routed : a.b0_routed);
  } else {
    n = n0 + j;
    base = c.shared ? a.b0_shared : a.b0_routed;
  }
  if (n >= c.N) return nullptr;
  if (c.shared) return reinterpret_cast<const T*>(base) + ((int64_t)c.e * c.N + n) * a.b_ld_shared;
  return reinterpret_cast<const T*>(base) + ((int64_t)c.e * c.N + n) * c.K;
}

template <typename T, bool SWIGLU>
__device__ __forceinline__ T* c_row(const GemmArgs& a, const TileCtx<SWIGLU>& c, int i) {
  const int64_t r = c.r0 + i;
  if (c.shared) return reinterpret_cast<T*>(a.c_shared) + r * a.c_ld_shared + (int64_t)c.e * c.N;
  return reinterpret_cast<T*>(a.c_routed) + r * c.N;
}

// ------------------------------------------------------------------------
// Block -> (M tile, N tile).  Workgroups go to the 8 XCDs round-robin
// (block b runs on XCD b % 8, and each XCD runs its blocks in order), and
// each XCD has its own L2.  The work items are listed M-tile major (the N
// tiles of one M tile are consecutive: they share the gathered A rows;
// consecutive M tiles of one expert share its weights) and cut into 8
// contiguous ranges of about equal cost, range x going to the blocks of XCD
// x.  In the down projection the shared group's items, which run over all
// shared experts' K and are the longest, follow the ranges: XCD x first
// takes its equal share of them, items [x S/8, (x+1) S/8), so every XCD
// starts its long items first and no XCD ends on a run of them; then its
// range, walked from the end when a.rev is set.  Blocks past both exit.
__device__ __forceinline__ bool work_item(const GemmArgs& a, int& m_tile, int& n_tile,
                                          int& half) {
  const int b = blockIdx.x;
  const int x = b % kXcds;
  int j = b / kXcds;
  // halves: consecutive blocks of an XCD take the two halves of one item
  half = 0;
  if (a.halves_ok && a.xcd_first[kXcds + 1]) {
    half = 1 + (j & 1);
    j >>= 1;
  }
  int w;
  const int s0 = (int)((int64_t)x * a.shared_items / kXcds);
  const int s1 = (int)((int64_t)(x + 1) * a.shared_items / kXcds);
  if (j < s1 - s0) {
    w = a.xcd_first[kXcds] + s0 + j;
  } else {
    j -= s1 - s0;
    const int first = a.xcd_first[x], end = a.xcd_first[x + 1];
    if (first + j >= end) return false;
    w = a.rev ? end - 1 - j : first + j;
  }
  m_tile = w / a.n_ntiles;
  n_tile = w - m_tile * a.n_ntiles;
  return true;
}

// ------------------------------------------------------------------------
// bf16 MFMA grouped GEMM.  WM x WN waves, each FM x FN 32x32 fragments.
template <int WM, int WN, int FM, int FN, bool SWIGLU>
__global__ __launch_bounds__(WM * WN * 64) void k_grouped_gemm_bf16(GemmArgs args) {
  constexpr int NT = WM * WN * 64;
  constexpr int BM = WM * FM * 32;
  constexpr int BN = WN * FN * 32;
  constexpr int BNO = SWIGLU ? BN / 2 : BN;  // output columns per tile
  constexpr int BK = 64;
  constexpr int CA = BM * 8 / NT;  // 16-byte chunks per thread per K tile
  constexpr int CB = BN * 8 / NT;
  static_assert(CA >= 1 && CB >= 1 && (NT / 8) % 8 == 0, "tile shape");
  static_assert(!SWIGLU || FN % 2 == 0, "gate/up pairs");

  // one LDS buffer (36 KB): the next K tile waits in registers, and four
  // blocks fit a CU, so a decode-sized GEMM's items run in one wave with
  // twice the loads in flight of a double-buffered LDS ring
  __shared__ __attribute__((aligned(16))) uint16_t lds_a[BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t lds_b[BN * BK];

  int tile_id, n_tile, half;
  if (!work_item(args, tile_id, n_tile, half)) return;
  (void)half;  // whole items only
  const int4 tl = args.tiles[tile_id];
  const TileCtx<SWIGLU> c = tile_ctx<SWIGLU>(args, tl, tile_id - tl.w);
  const int n0 = n_tile * BNO;
  if (n0 >= c.N) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // loader: this thread's rows are (tid >> 3) + (NT/8) i, chunk tid & 7
  const int lrow = tid >> 3;
  const int lchunk = tid & 7;
  const int lphys = (lchunk ^ (lrow & 7)) * 8;
  const uint16_t* ap[CA];
  const uint16_t* bp[CB];
#pragma unroll
  for (int i = 0; i < CA; i++) ap[i] = a_row<uint16_t, SWIGLU>(args, c, lrow + (NT / 8) * i);
#pragma unroll
  for (int i = 0; i < CB; i++) bp[i] = b_row<uint16_t, SWIGLU, BN>(args, c, n0, lrow + (NT / 8) * i);

  // A group of one M tile reads each weight row once: its weight loads are
  // non-temporal (streamed past the caches: measured 7.0-7.2 against
  // 6.2-6.3 TB/s for plain loads); a taller group's other M tiles read the
  // same rows again, so those stay cached
  const bool stream_b = tl.z <= BM;
  u32x4 ra[CA], rb[CB];
  auto gload = [&](int kt, auto nt) {
    const int col = kt * BK + lchunk * 8;
    const int64_t bcol = col + (c.shared ? shared_kseg_delta(args, kt * BK) : 0);
#pragma unroll
    for (int i = 0; i < CA; i++)
      ra[i] = ap[i] ? *reinterpret_cast<const u32x4*>(ap[i] + col) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < CB; i++) {
      const u32x4* p = reinterpret_cast<const u32x4*>(bp[i] + bcol);
      if constexpr (decltype(nt)::value)
        rb[i] = bp[i] ? __builtin_nontemporal_load(p) : u32x4{0, 0, 0, 0};
      else
        rb[i] = bp[i] ? *p : u32x4{0, 0, 0, 0};
    }
  };
  auto load_tile = [&](int kt) {
    if (stream_b) gload(kt, std::true_type{});
    else gload(kt, std::false_type{});
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < CA; i++)
      *reinterpret_cast<u32x4*>(&lds_a[(lrow + (NT / 8) * i) * BK + lphys]) = ra[i];
#pragma unroll
    for (int i = 0; i < CB; i++)
      *reinterpret_cast<u32x4*>(&lds_b[(lrow + (NT / 8) * i) * BK + lphys]) = rb[i];
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; i++)
#pragma unroll
    for (int j = 0; j < FN; j++) acc[i][j] = f32x16{};

  // fragment row bases inside the tile
  int brow[FN];
#pragma unroll
  for (int fn = 0; fn < FN; fn++) {
    if (SWIGLU) {
      const int half = FN / 2;
      brow[fn] = (fn < half) ? (wn * half + fn) * 32 : BN / 2 + (wn * half + fn - half) * 32;
    } else {
      brow[fn] = (wn * FN + fn) * 32;
    }
  }
  const int frow = lane & 31;
  const int fsw = lane & 7;
  const int fhalf = lane >> 5;

  const int nk = c.K / BK;
  load_tile(0);
  sstore();
  __syncthreads();
  for (int kt = 0; kt < nk; kt++) {
    if (kt + 1 < nk) load_tile(kt + 1);
#pragma unroll
    for (int s = 0; s < BK / 16; s++) {
      const int ch = ((2 * s + fhalf) ^ fsw) * 8;
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int fm = 0; fm < FM; fm++)
        af[fm] = *reinterpret_cast<const bf16x8*>(
            &lds_a[((wm * FM + fm) * 32 + frow) * BK + ch]);
#pragma unroll
      for (int fn = 0; fn < FN; fn++)
        bfr[fn] = *reinterpret_cast<const bf16x8*>(&lds_b[(brow[fn] + frow) * BK + ch]);
#pragma unroll
      for (int fm = 0; fm < FM; fm++)
#pragma unroll
        for (int fn = 0; fn < FN; fn++)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[fm], bfr[fn], acc[fm][fn], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      __syncthreads();  // every wave is done with tile kt
      sstore();
    }
    __syncthreads();
  }

  // epilogue: lane holds C[8(j/4) + 4(l/32) + j%4][l%32] of each fragment
  const int ccol = lane & 31;
#pragma unroll
  for (int fm = 0; fm < FM; fm++) {
#pragma unroll
    for (int j = 0; j < 16; j++) {
      const int row = (wm * FM + fm) * 32 + 8 * (j >> 2) + 4 * fhalf + (j & 3);
      if (row >= c.nr) continue;
      uint16_t* out = c_row<uint16_t, SWIGLU>(args, c, row);
      if (SWIGLU) {
        const int half = FN / 2;
#pragma unroll
        for (int fn = 0; fn < half; fn++) {
          const int col = n0 + (wn * half + fn) * 32 + ccol;
          const float g = acc[fm][fn][j], u = acc[fm][fn + half][j];
          if (col < c.N) out[col] = f32_to_bf16(silu_f32(g) * u);
        }
      } else {
#pragma unroll
        for (int fn = 0; fn < FN; fn++) {
          const int col = n0 + (wn * FN + fn) * 32 + ccol;
          if (col < c.N) out[col] = f32_to_bf16(acc[fm][fn][j]);
        }
      }
    }
  }
}

// ------------------------------------------------------------------------
// bf16 MFMA grouped GEMM, BMT x 256 (B rows) tiles, direct-to-LDS pipeline.
//
// Global -> LDS copies use global_load_lds_dwordx4 (no staging registers):
// lane i of a wave lands 16 bytes at LDS base + 16 i, so a swizzled LDS
// layout comes from permuting the lanes' source addresses.
//
// Eight waves, two per SIMD, each owning BMT/2 rows x 64 B rows (128
// accumulator registers).  On CDNA4 the 32x32x16 MFMA shape stalls the
// vector-memory path that feeds LDS while it runs, and one wave per SIMD
// cannot issue MFMAs while its own copy instructions wait to issue; the
// 16x16x32 shape with two waves per SIMD keeps the copies and the MFMAs
// overlapped (measured: the same copy + MFMA mix runs in 0.7x the time).
//
// Rows past the group's end (A) or past N (B) are pointed at a valid row:
// their products only reach output rows / columns that are not stored.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

__device__ __forceinline__ void dl_copy16(const uint16_t* g, uint16_t* l) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)g, (lds_void_t*)l, 16, 0, 0);
}

// s_waitcnt vmcnt(N) (gfx9 encoding; expcnt and lgkmcnt left at their max)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (((N >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8));
}

constexpr int kGemmLdsElems = 81920;  // 160 KB: all of the CU's LDS

constexpr int kGemmThreads = 512;
constexpr int kGroupWindow = 32;  // blocks an XCD runs at once (one per CU)
constexpr int kMinChunkN = 4;     // N tiles of a group walked together, at least

// Epilogue.  With the weight fragment as the MFMA's first operand, lane l of
// acc[fm][fn] holds output row wm*BMT/2 + fm*16 + l%16 and the 4 output
// columns brow(fn) + 4(l/16) .. +3 (for the gated GEMM, the gate block fn
// and the up block fn+2 cover the same columns).  The bf16 tile (BMT x BNO,
// at most 128 KB) is staged in the idle K stages, then written out as whole
// rows with 16-byte stores.  In LDS a row is BNO/4 slots of 8 bytes (4
// columns); slot s of row r sits at s ^ (r & 31).
template <int BMT, bool SWIGLU, int FM, int FN>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& args, const TileCtx<SWIGLU>& c,
                                              int n0, uint16_t* lds, const f32x4 (&acc)[FM][FN],
                                              int wm, int wn) {
  constexpr int BNO = SWIGLU ? 128 : 256;
  constexpr int SLOTS = BNO / 4;
  constexpr int CPR = BNO / 8;
  static_assert(BMT * BNO <= kGemmLdsElems, "epilogue staging");
  const int tid = threadIdx.x, lane = tid & 63;
  const int frow = lane & 15, fq = lane >> 4;
  uint2* s8 = reinterpret_cast<uint2*>(lds);
  __syncthreads();  // every wave is past its last fragment read
#pragma unroll
  for (int fm = 0; fm < FM; fm++) {
    const int row = wm * (BMT / 2) + fm * 16 + frow;
    uint2* srow = s8 + row * SLOTS;
    if (SWIGLU) {
#pragma unroll
      for (int fn = 0; fn < 2; fn++) {
        const int slot = (wn * 32 + fn * 16) / 4 + fq;
        float h[4];
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const float gt = acc[fm][fn][e], up = acc[fm][fn + 2][e];
          h[e] = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up;
        }
        srow[slot ^ (row & 31)] = make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
      }
    } else {
#pragma unroll
      for (int fn = 0; fn < FN; fn++) {
        const int slot = (wn * 64 + fn * 16) / 4 + fq;
        srow[slot ^ (row & 31)] = make_uint2(pack_bf16x2(acc[fm][fn][0], acc[fm][fn][1]),
                                             pack_bf16x2(acc[fm][fn][2], acc[fm][fn][3]));
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // one fragment row at a time
  }
  __syncthreads();
  // 16-byte chunk j of row r is slots 2j, 2j+1: one aligned 16-byte read at
  // slot 2j ^ (r & 30), halves swapped when r is odd
  const int nrows = c.nr < BMT ? c.nr : BMT;
  const bool full_cols = n0 + BNO <= c.N;
#pragma unroll 4
  for (int i = tid; i < nrows * CPR; i += kGemmThreads) {
    const int r = i / CPR, j = i - (i / CPR) * CPR;
    const int col = n0 + 8 * j;
    if (!full_cols && col >= c.N) continue;
    const uint4 v = *reinterpret_cast<const uint4*>(s8 + r * SLOTS + ((2 * j) ^ (r & 30)));
    const uint4 w = (r & 1) ? make_uint4(v.z, v.w, v.x, v.y) : v;
    *reinterpret_cast<uint4*>(c_row<uint16_t, SWIGLU>(args, c, r) + col) = w;
  }
}

// vmcnt(n) for a wave-uniform n in [0, 20]
__device__ __forceinline__ void wait_vmcnt_n(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 9: wait_vmcnt<9>(); break;
    case 10: wait_vmcnt<10>(); break;
    case 11: wait_vmcnt<11>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 13: wait_vmcnt<13>(); break;
    case 14: wait_vmcnt<14>(); break;
    case 15: wait_vmcnt<15>(); break;
    case 16: wait_vmcnt<16>(); break;
    case 17: wait_vmcnt<17>(); break;
    case 18: wait_vmcnt<18>(); break;
    case 19: wait_vmcnt<19>(); break;
    default: wait_vmcnt<20>(); break;
  }
}

// The tile's K loop with 64-wide K tiles: every LDS row holds 128 bytes of
// K, so each copy instruction moves 8 whole 128-byte rows (full cache lines)
// rather than 16 half lines.  The LDS is a ring of 20 slots of 64 rows
// (8 KB); K tile t takes S = BMT/64 + 4 consecutive slots of the ring (its
// A rows, then its B rows), so 20/S tiles are resident or in flight: 2.5 at
// 256 rows, 4 at 64 rows.  One slot is one copy instruction per wave (wave w
// moves rows 8w .. 8w+7 of it).  Copies are numbered in ring order; tile t's
// are numbers [tS, (t+1)S).  A K tile is two K steps of 32 (one MFMA each);
// the barrier comes once per K tile, in its second step: it publishes tile
// t+1 and frees tile t's slots, which then take copies 20 + tS ..
// 20 + (t+1)S - 1, issued over that step's MFMA rows.  16-byte chunk c of
// row r sits at c ^ ((r >> 1) & 7): a fragment read (16 rows, one chunk
// each) and a copy (8 rows x 8 chunks) touch every bank once per 16 lanes.
template <int BMT, bool SWIGLU>
__device__ __forceinline__ void gemm_tile_ring(const GemmArgs& args, const TileCtx<SWIGLU>& c,
                                               int n0, uint16_t* lds) {
  constexpr int BN = 256, BK = 64, SROWS = 64;
  constexpr int SLOT = SROWS * BK;           // elements per slot (8 KB)
  constexpr int NSLOT = kGemmLdsElems / SLOT;
  constexpr int SA = BMT / SROWS, SB = BN / SROWS;
  constexpr int S = SA + SB;                 // slots per K tile
  constexpr int AHEAD = NSLOT - 2 * S;       // copies still in flight at a steady barrier
  constexpr int NW = kGemmThreads / 64;
  constexpr int FM = BMT / 32, FN = 4;
  constexpr int CPR = (S + FM - 1) / FM;     // copies per MFMA row after the barrier
  static_assert(NSLOT == 20 && BMT % SROWS == 0 && AHEAD >= 0 && NW * 8 == SROWS, "ring");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  auto swz = [](int r) { return (r >> 1) & 7; };

  // source of this wave's copy of slot j of a tile (rows 8 wave .. +7 of
  // the slot); the lane's 16 bytes are logical chunk (lane & 7) ^ swz(row)
  // of its row's 128-byte K slice.  Rows past the group's end or past N
  // point at a valid row.
  const uint16_t* src[S];
#pragma unroll
  for (int j = 0; j < S; j++) {
    const int rr = 8 * wave + (lane >> 3);
    const int chunk = (lane & 7) ^ swz(rr);
    const uint16_t* p;
    if (j < SA) {
      p = a_row<uint16_t, SWIGLU>(args, c, j * SROWS + rr);
      if (!p) p = a_row<uint16_t, SWIGLU>(args, c, 0);
    } else {
      const int r = (j - SA) * SROWS + rr;
      p = b_row<uint16_t, SWIGLU, BN>(args, c, n0, r);
      if (!p) p = b_row<uint16_t, SWIGLU, BN>(args, c, n0, SWIGLU && r >= BN / 2 ? BN / 2 : 0);
    }
    src[j] = p + chunk * 8;
  }
  // shared group of the down projection: K slices in separate blocks (the
  // delta is 0 elsewhere)
  const int64_t seg_step = c.shared ? args.b_seg_shared - args.k_seg_shared : 0;
  const int seg_tiles = c.shared ? args.k_seg_shared / BK : 1;
  const int nk = c.K / BK;
  // copy number q (tile q / S, slot q % S) into ring slot q % NSLOT
  auto copy_q = [&](int tq, int j, int pos) {
    const int64_t bdel = (j >= SA && seg_step) ? (int64_t)(tq / seg_tiles) * seg_step : 0;
    dl_copy16(src[j] + tq * BK + bdel, lds + pos * SLOT + 8 * wave * BK);
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; i++)
#pragma unroll
    for (int j = 0; j < FN; j++) acc[i][j] = f32x4{};

  int brow[FN];
#pragma unroll
  for (int fn = 0; fn < FN; fn++)
    brow[fn] = SWIGLU ? (fn < 2 ? wn * 32 + fn * 16 : BN / 2 + wn * 32 + (fn - 2) * 16)
                      : wn * 64 + fn * 16;
  const int frow = lane & 15;
  const int fch0 = ((lane >> 4) ^ swz(frow)) * 8;        // K step 0 of a tile
  const int fch1 = ((4 + (lane >> 4)) ^ swz(frow)) * 8;  // K step 1

  bf16x8 afr[FM];
  bf16x8 bfr[FN];
  auto ring = [](int p) { return p >= NSLOT ? p - NSLOT : p; };
  // pt: ring slot of tile t's slot 0
  auto read_a = [&](int pt, int fch, int fm) {
    const int row = wm * (BMT / 2) + fm * 16;  // wave-uniform; + frow
    const int pos = ring(pt + row / SROWS);
    afr[fm] = *reinterpret_cast<const bf16x8*>(lds + pos * SLOT + (row % SROWS + frow) * BK + fch);
  };
  auto read_b = [&](int pt, int fch, int fn) {
    const int pos = ring(pt + SA + brow[fn] / SROWS);
    bfr[fn] = *reinterpret_cast<const bf16x8*>(lds + pos * SLOT +
                                               (brow[fn] % SROWS + frow) * BK + fch);
  };
  auto mfma_row = [&](int fm) {
#pragma unroll
    for (int fn = 0; fn < FN; fn++)
      acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[fn], afr[fm], acc[fm][fn], 0, 0, 0);
  };

  // One K step: row 0 multiplies first; in a tile's second step the barrier
  // follows (this wave's copies of tile t+1 landed, its reads of tile t
  // done, then everyone's).  Rows 1.. issue the copy batch the barrier
  // allowed (tile t's copies t*S .. , qbase = 20 + t*S, into ring slots
  // from pfree) and read the next step's fragments (ring slot np of its
  // tile, chunk offset nfch).
  auto kstep = [&](bool bar, bool more, bool copy, int t, int np, int nfch, int pfree,
                   int wait_n) {
    mfma_row(0);
    __builtin_amdgcn_sched_barrier(0);
    if (bar) {
      wait_vmcnt_n(wait_n);
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's reads are done
      __builtin_amdgcn_s_barrier();
    }
#pragma unroll
    for (int fm = 1; fm <= FM; fm++) {
      if (fm < FM) mfma_row(fm);
      if (copy) {
#pragma unroll
        for (int i = (fm - 1) * CPR; i < fm * CPR && i < S; i++) {
          const int tq = t + (NSLOT + i) / S;  // copy 20 + t*S + i
          if (tq < nk) copy_q(tq, (NSLOT + i) % S, ring(pfree + i));
        }
      }
      if (more) {
        if (fm == 1) read_a(np, nfch, 0);
        if (fm < FM) read_a(np, nfch, fm);
        if (fm == FM)
#pragma unroll
          for (int fn = 0; fn < FN; fn++) read_b(np, nfch, fn);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // prologue: copies 0 .. min(20, nk S) - 1 (slots in ring order, except
  // that tile 0 issues its weight slots before its gathered rows, whose
  // addresses wait on the row-index load), tile 0 published, its first
  // step's fragments in registers
  const int pro = nk * S < NSLOT ? nk * S : NSLOT;
#pragma unroll
  for (int q = 0; q < NSLOT; q++) {
    const int j = q < S ? (q < SB ? SA + q : q - SB) : q % S;
    if (q < pro) copy_q(q / S, j, q < S ? j : q);
  }
  wait_vmcnt_n(pro - S);
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int fm = 0; fm < FM; fm++) read_a(0, fch0, fm);
#pragma unroll
  for (int fn = 0; fn < FN; fn++) read_b(0, fch0, fn);

  int t = 0, pt = 0;  // pt: ring slot of tile t's first slot
  // steady state: every copy of the batch exists (20 + (t+1) S <= nk S)
  for (; NSLOT + (t + 1) * S <= nk * S; t++) {
    const int pn = ring(pt + S);
    kstep(false, true, false, t, pt, fch1, 0, 0);
    kstep(true, true, true, t, pn, fch0, pt, AHEAD);
    pt = pn;
  }
  // drain: copies past the last tile are skipped
  for (; t < nk; t++) {
    const int pn = ring(pt + S);
    kstep(false, true, false, t, pt, fch1, 0, 0);
    const bool last = t + 1 >= nk;
    // copies issued before this barrier: min(20 + t S, nk S); needed: (t+2) S
    const int issued = NSLOT + t * S < nk * S ? NSLOT + t * S : nk * S;
    kstep(!last, !last, !last, t, pn, fch0, pt, issued - (t + 2) * S);
    pt = pn;
  }

  gemm_epilogue<BMT, SWIGLU, FM, FN>(args, c, n0, lds, acc, wm, wn);
}

// A tile runs the variant of 64, 128, 192 or 256 rows that covers its valid
// rows, so the last tile of a group (and the small groups of the long tail
// of expert loads) wastes at most 63 rows of MFMA work.
template <bool SWIGLU>
__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm_dl(GemmArgs args) {
  __shared__ __attribute__((aligned(1024))) uint16_t lds[kGemmLdsElems];
  int tile_id, n_tile, half;
  if (!work_item(args, tile_id, n_tile, half)) return;
  // Inside its group the item list is walked N chunk by N chunk: a chunk
  // holds all G M tiles of the group times about 32/G N tiles, at least 4,
  // so the ~32 blocks an XCD runs at once share both their gathered rows and
  // their weight tiles in L2 (a group with many N tiles walked M-tile major
  // would have them all read different weights; in a group of 16 M tiles,
  // 8 M x 4 N tiles at once read fewer distinct tiles than 16 x 2, timed
  // 8-10 us faster on the DeepSeek-shaped gated GEMM).
  const int4 tl = args.tiles[tile_id];
  const int nn = args.n_ntiles;
  const int G = (tl.z + args.bm - 1) / args.bm;
  const int u = (tile_id - tl.w) * nn + n_tile;  // M-major index inside the group
  int gw = (kGroupWindow + G - 1) / G;
  gw = gw < kMinChunkN ? kMinChunkN : gw;
  gw = gw > nn ? nn : gw;
  const int chunk = u / (G * gw);
  const int cw = nn - chunk * gw < gw ? nn - chunk * gw : gw;  // the last chunk may be narrower
  const int v = u - chunk * G * gw;
  const int g = v / cw;
  n_tile = chunk * gw + (v - g * cw);
  TileCtx<SWIGLU> c = tile_ctx<SWIGLU>(args, tl, g);
  const int n0 = n_tile * (SWIGLU ? 128 : 256);
  if (n0 >= c.N) return;
  if (half) {  // rows [0, 128) or [128, 256) of the item
    if (half == 2) {
      c.r0 += 128;
      c.nr -= 128;
    } else if (c.nr > 128) {
      c.nr = 128;
    }
    if (c.nr <= 0) return;
  }
  if (c.nr > 192)
    gemm_tile_ring<256, SWIGLU>(args, c, n0, lds);
  else if (c.nr > 128)
    gemm_tile_ring<192, SWIGLU>(args, c, n0, lds);
  else if (c.nr > 64)
    gemm_tile_ring<128, SWIGLU>(args, c, n0, lds);
  else
    gemm_tile_ring<64, SWIGLU>(args, c, n0, lds);
}

// ------------------------------------------------------------------------
// fp32 layers: 32-row x 64-column output tiles on plain FMA.  K advances in
// chunks of 32 staged through LDS (A 32 x 32, B 64 x 32; for the gated GEMM
// the gate and up rows of the 64 columns); thread (r = tid / 8, c = tid % 8)
// accumulates row r, columns c, c+8, ..., c+56.
template <bool SWIGLU>
__global__ __launch_bounds__(256) void k_grouped_gemm_f32(GemmArgs args) {
  constexpr int KC = 32;
  constexpr int NB = SWIGLU ? 128 : 64;   // B rows staged per chunk
  __shared__ float sa[32][KC + 1];
  __shared__ float sb[NB][KC + 1];
  int tile_id, n_tile, half;
  if (!work_item(args, tile_id, n_tile, half)) return;
  (void)half;  // whole items only
  const int4 tl = args.tiles[tile_id];
  const TileCtx<SWIGLU> c = tile_ctx<SWIGLU>(args, tl, tile_id - tl.w);
  const int n0 = n_tile * 64;
  if (n0 >= c.N) return;
  const int tid = threadIdx.x;
  const int r = tid >> 3, cc = tid & 7;
  float acc[8], acc2[8];
#pragma unroll
  for (int j = 0; j < 8; j++) { acc[j] = 0.f; acc2[j] = 0.f; }
  // loader: A row tid/8 (4 floats at (tid%8)*4); B rows tid/8 + 32 q
  const float* arow = a_row<float, SWIGLU>(args, c, r);
  const float* brow[NB / 32];
#pragma unroll
  for (int q = 0; q < NB / 32; q++) {
    const int j = r + 32 * q;  // 0 .. NB-1
    const float* p = SWIGLU ? b_row<float, SWIGLU, 128>(args, c, n0, j)
                            : b_row<float, SWIGLU, 64>(args, c, n0, j);
    brow[q] = p;
  }
  for (int k0 = 0; k0 < c.K; k0 += KC) {
    {
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (arow) v = *reinterpret_cast<const f32x4*>(arow + k0 + cc * 4);
#pragma unroll
      for (int e = 0; e < 4; e++) sa[r][cc * 4 + e] = v[e];
    }
    const int64_t bk0 = k0 + (c.shared ? shared_kseg_delta(args, k0) : 0);
#pragma unroll
    for (int q = 0; q < NB / 32; q++) {
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (brow[q]) v = *reinterpret_cast<const f32x4*>(brow[q] + bk0 + cc * 4);
#pragma unroll
      for (int e = 0; e < 4; e++) sb[r + 32 * q][cc * 4 + e] = v[e];
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < KC; kk++) {
      const float av = sa[r][kk];
#pragma unroll
      for (int j = 0; j < 8; j++) {
        acc[j] = fmaf(av, sb[cc + 8 * j][kk], acc[j]);
        if (SWIGLU) acc2[j] = fmaf(av, sb[64 + cc + 8 * j][kk], acc2[j]);
      }
    }
    __syncthreads();
  }
  if (r >= c.nr) return;
  float* out = c_row<float, SWIGLU>(args, c, r);
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const int n = n0 + cc + 8 * j;
    if (n < c.N) out[n] = SWIGLU ? silu_f32(acc[j]) * acc2[j] : acc[j];
  }
}

// ------------------------------------------------------------------------
// Tile list and XCD schedule (the builder itself is in tiles.h, shared with
// the dispatch scan, which builds them in the same launch for a forward).
__global__ __launch_bounds__(1024) void k_build_tiles(const int32_t* __restrict__ offsets,
                                                      TileBuild tb) {
  build_tile_list(offsets, tb);
}

// ------------------------------------------------------------------------
// launchers

int gemm_tile_rows(int dtype, int64_t tasks, int E_ffn) {
  if (dtype != MOE_BF16) return 32;
  // small groups (decode-sized batches): 32-row tiles; otherwise 256
  return (E_ffn > 0 && tasks / E_ffn < 64) ? 32 : 256;
}

int64_t gemm_max_tiles(int64_t T, int k, int E_ffn, int n_shared, int BM) {
  return cdiv(T * k, BM) + E_ffn + n_shared * cdiv(T, BM);
}

int gemm_n_ntiles(int dtype, bool swiglu, int N) {
  // output columns per tile: fp32 64; bf16 256 B rows = 128 gated / 256 plain
  const int bno = dtype == MOE_F32 ? 64 : (swiglu ? 128 : 256);
  return N > 0 ? (int)cdiv(N, bno) : 1;
}

int64_t gemm_blocks_per_xcd(int BM, int64_t max_tiles, int nn) {
  // enough for an XCD's share of the items: a range holds about 1/8 of the
  // cost, and on the 256-row path an item costs 4 to 7 (elsewhere 1); the
  // schedule clamps any range that would hold more
  const int64_t W = max_tiles * nn;
  return (BM == 256 ? cdiv(7 * W, 4 * kXcds) : cdiv(W, kXcds)) + 2;
}

hipError_t launch_build_tiles(const TileBuild& tb, const int32_t* offsets, hipStream_t st) {
  hipLaunchKernelGGL(k_build_tiles, dim3(1), dim3(1024), 0, st, offsets, tb);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(int dtype, bool swiglu, int BM, const GemmArgs& a_in,
                               int64_t max_tiles, hipStream_t st) {
  GemmArgs a = a_in;
  const int Nmax = a.N_routed > a.N_shared ? a.N_routed : a.N_shared;
  if (max_tiles == 0 || Nmax == 0) return hipSuccess;
  a.n_ntiles = gemm_n_ntiles(dtype, swiglu, Nmax);
  a.bm = BM;
  a.halves_ok = (dtype == MOE_BF16 && BM == 256 && !swiglu) ? 1 : 0;
  const unsigned grid = (unsigned)(gemm_blocks_per_xcd(BM, max_tiles, a.n_ntiles) * kXcds *
                                   (a.halves_ok ? 2 : 1));
  if (dtype == MOE_F32) {
    if (swiglu)
      hipLaunchKernelGGL(k_grouped_gemm_f32<true>, dim3(grid), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(k_grouped_gemm_f32<false>, dim3(grid), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  if (BM == 256) {
    if (swiglu)
      hipLaunchKernelGGL((k_gemm_dl<true>), dim3(grid), dim3(kGemmThreads), 0, st, a);
    else
      hipLaunchKernelGGL((k_gemm_dl<false>), dim3(grid), dim3(kGemmThreads), 0, st, a);
  } else {
    if (swiglu)
      hipLaunchKernelGGL((k_grouped_gemm_bf16<1, 4, 1, 2, true>), dim3(grid), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((k_grouped_gemm_bf16<1, 4, 1, 2, false>), dim3(grid), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace moe
