// Dispatch: groups the T*K token-slots by expert, the gather side of the
// experts' sparse loop (Gemma4TextExperts' data-dependent gather / scatter on
// the page "Porting a 128-expert MoE (Gemma-4 26B-A4B) to AWS Inferentia2",
// section "The architecture: a dual-path FFN nobody warned me about").
//
// Integer-only.  The order within an expert is the slot order (stable), so
// the result is unique.  No atomics decide a position: ranks come from wave
// ballots and prefix sums.
//
// Slots are cut into chunks of 1024 (one 16-wave block each).  Inside a
// wave, a slot's rank among equal experts is the popcount of the lanes below
// it that carry the same expert (found with 8 ballots over the bits of the
// expert id).  Per-wave counts are scanned across the block's waves; per-block
// counts are scanned across blocks by a single-block kernel, which also forms
// the expert offsets.  A lone chunk (T*K <= 1024, every decode batch) runs all
// of it in one kernel.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kChunkSlots = 1024;
constexpr int kWaves = kChunkSlots / kWave;  // 16
constexpr int kMaxE = 256;

// Rank of this lane's expert among the lanes below it holding the same
// expert, and whether this lane is the last of its group.  Invalid lanes
// (valid == false) take part in no group.
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

// Per-chunk work shared by both paths: fills wave_base[w][e] (exclusive scan
// over the chunk's waves of each expert's count), block totals in
// totals[e], and returns the slot's rank within the chunk among equal
// experts.  Must be called by all 1024 threads.
__device__ __forceinline__ int chunk_rank(const int32_t* __restrict__ topk_idx, int S, int E,
                                          int chunk, int (*wave_base)[kMaxE], int* totals,
                                          int& e_out, bool& valid_out) {
  const int tid = threadIdx.x, wave = tid / kWave;
  for (int i = tid; i < kWaves * kMaxE; i += kChunkSlots) (&wave_base[0][0])[i] = 0;
  __syncthreads();
  const int s = chunk * kChunkSlots + tid;
  const bool valid = s < S;
  const int e = valid ? topk_idx[s] : 0;
  int rank, cnt;
  bool last;
  wave_match_rank(e, valid, rank, cnt, last);
  if (last) wave_base[wave][e] = cnt;
  __syncthreads();
  if (tid < E) {
    int run = 0;
    for (int w = 0; w < kWaves; ++w) {
      const int c = wave_base[w][tid];
      wave_base[w][tid] = run;
      run += c;
    }
    totals[tid] = run;
  }
  __syncthreads();
  e_out = e;
  valid_out = valid;
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

__global__ __launch_bounds__(kChunkSlots) void dispatch_single_kernel(
    const int32_t* __restrict__ topk_idx, int S, int E, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slots) {
  __shared__ int wave_base[kWaves][kMaxE];
  __shared__ int totals[kMaxE];
  __shared__ int offs[kMaxE + 1];
  int e;
  bool valid;
  const int r = chunk_rank(topk_idx, S, E, 0, wave_base, totals, e, valid);
  if (threadIdx.x < kWave) wave_offsets(totals, E, offs);
  __syncthreads();
  if (valid) sorted_slots[offs[e] + r] = threadIdx.x;
  if (threadIdx.x < E) counts[threadIdx.x] = totals[threadIdx.x];
  if (threadIdx.x <= E) offsets[threadIdx.x] = offs[threadIdx.x];
}

__global__ __launch_bounds__(kChunkSlots) void dispatch_rank_kernel(
    const int32_t* __restrict__ topk_idx, int S, int E, int32_t* __restrict__ blk_counts,
    int32_t* __restrict__ local_rank) {
  __shared__ int wave_base[kWaves][kMaxE];
  __shared__ int totals[kMaxE];
  int e;
  bool valid;
  const int r = chunk_rank(topk_idx, S, E, blockIdx.x, wave_base, totals, e, valid);
  if (valid) local_rank[blockIdx.x * kChunkSlots + threadIdx.x] = r;
  if (threadIdx.x < E) blk_counts[(size_t)blockIdx.x * E + threadIdx.x] = totals[threadIdx.x];
}

// One block: per expert, exclusive scan of the chunk counts (in place), the
// expert totals and offsets.
__global__ __launch_bounds__(kMaxE) void dispatch_scan_kernel(int nblk, int E,
                                                              int32_t* __restrict__ blk_counts,
                                                              int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ offsets) {
  __shared__ int totals[kMaxE];
  const int e = threadIdx.x;
  if (e < E) {
    int run = 0;
    for (int b = 0; b < nblk; ++b) {
      const int c = blk_counts[(size_t)b * E + e];
      blk_counts[(size_t)b * E + e] = run;
      run += c;
    }
    totals[e] = run;
    counts[e] = run;
  }
  __syncthreads();
  if (threadIdx.x < kWave) wave_offsets(totals, E, offsets);
}

__global__ __launch_bounds__(kChunkSlots) void dispatch_scatter_kernel(
    const int32_t* __restrict__ topk_idx, int S, int E, const int32_t* __restrict__ blk_base,
    const int32_t* __restrict__ local_rank, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_slots) {
  const int s = blockIdx.x * kChunkSlots + threadIdx.x;
  if (s >= S) return;
  const int e = topk_idx[s];
  sorted_slots[offsets[e] + blk_base[(size_t)blockIdx.x * E + e] + local_rank[s]] = s;
}

}  // namespace

int dispatch_num_blocks(int S) { return (S + kChunkSlots - 1) / kChunkSlots; }

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s) {
  const int S = a.T * a.K;
  const int nblk = dispatch_num_blocks(S);
  if (nblk <= 1) {
    hipLaunchKernelGGL(dispatch_single_kernel, dim3(1), dim3(kChunkSlots), 0, s, a.topk_idx, S,
                       a.E, a.counts, a.offsets, a.sorted_slots);
  } else {
    hipLaunchKernelGGL(dispatch_rank_kernel, dim3(nblk), dim3(kChunkSlots), 0, s, a.topk_idx, S,
                       a.E, a.ws_blk_counts, a.ws_local_rank);
    hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(kMaxE), 0, s, nblk, a.E,
                       a.ws_blk_counts, a.counts, a.offsets);
    hipLaunchKernelGGL(dispatch_scatter_kernel, dim3(nblk), dim3(kChunkSlots), 0, s, a.topk_idx,
                       S, a.E, a.ws_blk_counts, a.ws_local_rank, a.offsets, a.sorted_slots);
  }
  return hipGetLastError();
}

}  // namespace moe
