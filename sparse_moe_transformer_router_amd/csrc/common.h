// Device-side helpers shared by the libmoe kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
// Round to nearest even (gfx950 v_cvt_pk_bf16_f32).
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

// tanh form of GELU: 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))).
__device__ __forceinline__ float gelu_tanh(float z) {
  const float c = 0.7978845608028654f;  // sqrt(2/pi)
  float inner = c * (z + 0.044715f * z * z * z);
  return 0.5f * z * (1.0f + tanhf(inner));
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// s_waitcnt vmcnt(N) with the other counters unconstrained.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// s_waitcnt lgkmcnt(0).
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4):
// lane l's 16 bytes at gsrc land at lds + 16 l (lds is the same for every
// lane).  Issued from inline asm, so the compiler does not see it: when it
// tracks such copies itself it cannot tell the slots of a copy ring apart,
// and makes LDS reads that follow a copy wait for every copy in flight,
// which drains the ring on each k-tile.  Callers order the ring with
// wait_vmem and a barrier.  The low 32 bits of a generic LDS address are the
// LDS offset; M0 takes it, and one wait state separates that write from the
// copy.
__device__ __forceinline__ void lds_copy16(const void* gsrc, const void* lds) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gsrc), "s"(m0)
               : "memory", "m0");
}

// s_barrier that the compiler may not move memory accesses across.
__device__ __forceinline__ void block_barrier() {
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Row tiles of a grouped GEMM.  Expert e owns rows [offsets[e], offsets[e+1])
// of the expert-sorted slot order; it is cut into ceil(count / bm) tiles of
// bm rows.  Tiles are numbered expert by expert in ascending order.  One wave
// scans the per-expert tile counts (each lane takes a run of consecutive
// experts) and can then map a tile number to its expert and row range.  Every
// lane of the calling wave gets the same answers.  Requires E <= 4 * 64.
struct RowTileScan {
  int cnt[4];     // this lane's experts' tile counts
  int base;       // this lane's first expert
  int excl, incl; // exclusive / inclusive prefix of the lanes' totals
  int total;      // tiles over all experts
};

__device__ __forceinline__ void row_tile_scan(const int32_t* __restrict__ offsets, int E, int bm,
                                              RowTileScan& s) {
  const int lane = lane_id();
  const int per = (E + kWave - 1) / kWave;  // experts per lane (<= 4)
  s.base = lane * per;
  int local = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = s.base + j;
    int c = 0;
    if (j < per && e < E) c = (offsets[e + 1] - offsets[e] + bm - 1) / bm;
    s.cnt[j] = c;
    local += c;
  }
  int incl = local;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += t;
  }
  s.incl = incl;
  s.excl = incl - local;
  s.total = __shfl(incl, kWave - 1, kWave);
}

// Tile `tile` (< s.total) -> expert and row range.
__device__ __forceinline__ void row_tile_lookup(const RowTileScan& s,
                                                const int32_t* __restrict__ offsets, int bm,
                                                int tile, int& e_out, int& row0, int& row1) {
  const int lane = lane_id();
  const unsigned long long hit = __ballot(tile >= s.excl && tile < s.incl);
  const int owner = __ffsll((long long)hit) - 1;
  int e_found = 0, t_in = 0;
  if (lane == owner) {
    int rem = tile - s.excl;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (rem >= 0 && rem < s.cnt[j]) { e_found = s.base + j; t_in = rem; }
      rem -= s.cnt[j];
    }
  }
  e_out = __shfl(e_found, owner, kWave);
  t_in = __shfl(t_in, owner, kWave);
  row0 = offsets[e_out] + t_in * bm;
  row1 = min(row0 + bm, offsets[e_out + 1]);
}

// Work item `item` of a grouped GEMM with NT column tiles -> expert, row
// range and column tile, numbered expert by expert and, within an expert,
// column tile by column tile with the expert's row tiles fastest: the row
// tiles that stream the same weight slab are neighbours, so they run on one
// XCD at about the same time and share the slab through its L2.  (Item i lies
// in expert e's range exactly when tile i / NT is one of e's tiles.)
__device__ __forceinline__ void weight_major_item(const RowTileScan& s,
                                                  const int32_t* __restrict__ offsets, int bm,
                                                  int item, int NT, int& e, int& row0,
                                                  int& row1, int& nt) {
  const int tile = item / NT;
  row_tile_lookup(s, offsets, bm, tile, e, row0, row1);
  const int first = tile - (row0 - offsets[e]) / bm;  // the expert's first tile
  const int re = (offsets[e + 1] - offsets[e] + bm - 1) / bm;
  const int local = item - first * NT;
  nt = local / re;
  row0 = offsets[e] + (local % re) * bm;
  row1 = min(row0 + bm, offsets[e + 1]);
}

// Work items are numbered in the order of the caller (stream_item: the
// column groups of a row tile fastest; the tiled GEMMs: weight_major_item).
// Block b of a 1-D grid runs on XCD b % 8 (workgroups go round-robin to the eight
// XCDs); each XCD takes a contiguous range of the real items, so that items
// sharing gathered rows or a weight slab run on one XCD at about the same time
// and share its L2.  Blocks past an XCD's range get -1.  Needs gridDim.x >=
// n_items.
__device__ __forceinline__ int xcd_item(int b, int n_items) {
  const int x = b % 8, l = b / 8;
  const int q = n_items / 8, r = n_items % 8;
  const int cnt = q + (x < r ? 1 : 0);
  return l < cnt ? x * q + min(x, r) + l : -1;
}

// The block's work item: row tile (of at most bm rows of one expert, or of
// the tokens when ident) and column group cg of CG, from the XCD-aware
// mapping of xcd_item over the real number of items, so that the column
// groups of a row tile (which read the same activation rows) share one XCD's
// L2.  1-D grid of at least (row tile bound) * CG blocks.
__device__ __forceinline__ bool stream_item(bool ident, int rows, const int32_t* offsets, int E,
                                            int bm, int CG, int& e, int& row0, int& row1,
                                            int& cg) {
  RowTileScan sc;
  int R;
  if (ident) {
    R = (rows + bm - 1) / bm;
  } else {
    row_tile_scan(offsets, E, bm, sc);
    R = sc.total;
  }
  const int item = xcd_item(blockIdx.x, R * CG);
  if (item < 0) return false;
  const int rt = item / CG;
  cg = item % CG;
  if (ident) {
    e = 0;
    row0 = rt * bm;
    row1 = min(row0 + bm, rows);
  } else {
    row_tile_lookup(sc, offsets, bm, rt, e, row0, row1);
  }
  // the same for every lane: scalar registers, scalar branches
  e = __builtin_amdgcn_readfirstlane(e);
  row0 = __builtin_amdgcn_readfirstlane(row0);
  row1 = __builtin_amdgcn_readfirstlane(row1);
  cg = __builtin_amdgcn_readfirstlane(cg);
  return true;
}

// Upper bound on the number of bm-row tiles over all groups (host side): a
// tile holds at least one row, each group has at most bm - 1 rows of
// padding, and a group (an expert) holds at most T rows.  The grids of the
// grouped kernels are this bound times their column tiles; blocks past the
// real items exit at once (at 1 token: 8 row tiles, not the 60 of the first
// two terms).
inline int tile_count_bound(bool ident, int rows, int T, int E, int bm) {
  if (ident) return (rows + bm - 1) / bm;
  long long n = ((long long)rows + (long long)E * (bm - 1)) / bm;
  n = n < (long long)E * ((T + bm - 1) / bm) ? n : (long long)E * ((T + bm - 1) / bm);
  n = n < rows ? n : rows;
  return (int)n;
}

// Returns false if `tile` is past the last tile.
__device__ __forceinline__ bool find_row_tile(const int32_t* __restrict__ offsets, int E,
                                              int bm, int tile, int& e_out, int& row0,
                                              int& row1) {
  RowTileScan s;
  row_tile_scan(offsets, E, bm, s);
  if (tile >= s.total) return false;
  row_tile_lookup(s, offsets, bm, tile, e_out, row0, row1);
  return true;
}

}  // namespace moe
