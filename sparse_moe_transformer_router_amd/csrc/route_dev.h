// Device helpers of the routing step shared by the router and dispatch
// kernels: wave-wide DPP reductions, the per-token top-K selection and the
// per-chunk stable ranking of token-slots by expert.
#pragma once

#include "common.h"

namespace moe {

// Order-preserving map from fp32 to uint32 (larger float -> larger key).
// -0 is folded into +0 first, so IEEE-equal values get equal keys.
__device__ __forceinline__ uint32_t float_key(float f) {
  const uint32_t b = __float_as_uint(f + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xf, false);
}

// Maximum of v over the 64 lanes, returned to every lane (row shifts within
// 16-lane rows, then row broadcasts 15 and 31; lane 63 ends with the result).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0x111, 0xf>(0u, v));
  v = max(v, dpp_u32<0x112, 0xf>(0u, v));
  v = max(v, dpp_u32<0x114, 0xf>(0u, v));
  v = max(v, dpp_u32<0x118, 0xf>(0u, v));
  v = max(v, dpp_u32<0x142, 0xa>(0u, v));
  v = max(v, dpp_u32<0x143, 0xc>(0u, v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Top-K of one token's E (<= 256) fp32 logits, by one wave.  Experts are taken
// in descending logit order, equal logits going to the lower index; the
// weights are softmax restricted to the chosen experts,
// w_k = z_k / sum_j z_j with z = exp(l - max l), times per_expert_scale.
// (Equal, in exact arithmetic, to renormalising the full softmax over the K.)
// Writes idx_out[0..K) and w_out[0..K); if sidx is not null also sidx[0..K).
// Value of v in lane src (src the same in every lane): v_readlane, no LDS
// round trip.
__device__ __forceinline__ float lane_value(float v, int src) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

__device__ __forceinline__ void wave_topk(const float* __restrict__ lg, int E, int K,
                                          const float* __restrict__ pes,
                                          int32_t* __restrict__ idx_out,
                                          float* __restrict__ w_out, int* sidx) {
  const int lane = lane_id();
  float l[4];
  uint32_t key[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + kWave * j;
    l[j] = e < E ? lg[e] : 0.0f;
    key[j] = e < E ? float_key(l[j]) : 0u;  // 0 = not a candidate
  }
  const uint32_t kmax = wave_max_u32(max(max(key[0], key[1]), max(key[2], key[3])));
  // the largest logit, read back from the lane that holds it
  float lmax = 0.0f;
  {
    int src = 0, jj = 0;
#pragma unroll
    for (int j = 3; j >= 0; --j) {
      const unsigned long long b = __ballot(key[j] == kmax);
      if (b) { src = __ffsll((long long)b) - 1; jj = j; }
    }
    float mine = l[0];
#pragma unroll
    for (int j = 1; j < 4; ++j) if (j == jj) mine = l[j];
    lmax = lane_value(mine, src);
  }
  int my_e = 0;
  float my_z = 0.0f;
  for (int k = 0; k < K; ++k) {
    const uint32_t m = wave_max_u32(max(max(key[0], key[1]), max(key[2], key[3])));
    // lowest expert index holding the maximum: first j with a hit, lowest lane
    int win = -1;
#pragma unroll
    for (int j = 3; j >= 0; --j) {
      const unsigned long long b = __ballot(key[j] == m);
      if (b) win = (__ffsll((long long)b) - 1) + kWave * j;
    }
    const int wl = win & (kWave - 1), wj = win / kWave;
    float lv = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j == wj && lane == wl) { lv = l[j]; key[j] = 0u; }
    lv = lane_value(lv, wl);
    if (lane == k) { my_e = win; my_z = expf(lv - lmax); }
  }
  float q = 0.0f;
  for (int k = 0; k < K; ++k) q = q + lane_value(my_z, k);
  if (lane < K) {
    idx_out[lane] = my_e;
    w_out[lane] = (my_z / q) * pes[my_e];
    if (sidx) sidx[lane] = my_e;
  }
}

// ---------------------------------------------------------------------------
// Stable grouping of token-slots by expert (used by the dispatch kernels).
// A chunk of 1024 slots is handled by one 16-wave block.
// ---------------------------------------------------------------------------
constexpr int kChunkSlots = 1024;
constexpr int kChunkWaves = kChunkSlots / kWave;  // 16
constexpr int kMaxE = 256;

// Rank of this lane's expert among the lanes below it holding the same
// expert, the size of its group and whether it is the group's last lane.
// Invalid lanes take part in no group.
__device__ __forceinline__ void wave_match_rank(int e, bool valid, int& rank, int& group_count,
                                                bool& last) {
  const int lane = lane_id();
  unsigned long long m = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const bool bit = (e >> b) & 1;
    const unsigned long long bb = __ballot(bit);
    m &= bit ? bb : ~bb;
  }
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  rank = __popcll(m & below);
  group_count = __popcll(m);
  const unsigned long long above = (lane == kWave - 1) ? 0ull : (m >> (lane + 1));
  last = valid && above == 0ull;
}

// Per-chunk ranking by the 1024 threads of a block: returns the slot's rank
// within the chunk among slots of the same expert (slot order), and leaves in
// totals[e] the chunk's count of expert e.  wave_base is scratch.
__device__ __forceinline__ int chunk_rank(int e, bool valid, int E,
                                          int (*wave_base)[kMaxE], int* totals) {
  const int tid = threadIdx.x, wave = tid / kWave;
  for (int i = tid; i < kChunkWaves * kMaxE; i += kChunkSlots) (&wave_base[0][0])[i] = 0;
  __syncthreads();
  int rank, cnt;
  bool last;
  wave_match_rank(e, valid, rank, cnt, last);
  if (last) wave_base[wave][e] = cnt;
  __syncthreads();
  if (tid < E) {
    int run = 0;
    for (int w = 0; w < kChunkWaves; ++w) {
      const int c = wave_base[w][tid];
      wave_base[w][tid] = run;
      run += c;
    }
    totals[tid] = run;
  }
  __syncthreads();
  return valid ? wave_base[wave][e] + rank : 0;
}

// Exclusive scan of counts[0..E) into offsets[0..E] by one wave (E <= 256).
__device__ __forceinline__ void wave_offsets(const int* counts, int E, int32_t* offsets) {
  const int lane = lane_id();
  int c[4], local = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane * 4 + j;
    c[j] = e < E ? counts[e] : 0;
    local += c[j];
  }
  int incl = local;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += t;
  }
  int run = incl - local;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane * 4 + j;
    if (e < E) offsets[e] = run;
    run += c[j];
  }
  if (lane == kWave - 1) offsets[E] = incl;
}

// Dispatch of one lone chunk (T*K <= 1024) by a 1024-thread block: expert
// of slot tid is e (valid when tid < S).  Writes counts, offsets and the
// stable slot permutation.
__device__ __forceinline__ void dispatch_lone_chunk(int e, bool valid, int E,
                                                    int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ sorted_slots,
                                                    int (*wave_base)[kMaxE], int* totals,
                                                    int* offs) {
  const int r = chunk_rank(e, valid, E, wave_base, totals);
  if (threadIdx.x < kWave) wave_offsets(totals, E, offs);
  __syncthreads();
  if (valid) sorted_slots[offs[e] + r] = threadIdx.x;
  if (threadIdx.x < E) counts[threadIdx.x] = totals[threadIdx.x];
  if (threadIdx.x <= E) offsets[threadIdx.x] = offs[threadIdx.x];
}

}  // namespace moe
