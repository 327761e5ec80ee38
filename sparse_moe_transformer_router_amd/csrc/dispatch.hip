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
// it that carry the same expert (8 ballots over the bits of the expert id).
// Per-wave counts are scanned across the block's waves; per-block counts are
// scanned across blocks by a single-block kernel, which also forms the expert
// offsets.  A lone chunk (T*K <= 1024, every decode batch) runs all of it in
// one kernel; the router can also run that lone-chunk dispatch itself, right
// after its top-K (see the router kernels).  An expert id outside [0, E) in a
// caller's topk_idx is dropped: its slot joins no group and is not listed.
#include "launch.h"
#include "route_dev.h"

namespace moe {
namespace {

__global__ __launch_bounds__(kChunkSlots) void dispatch_single_kernel(
    const int32_t* __restrict__ topk_idx, int S, int E, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slots) {
  __shared__ int wave_base[kChunkWaves][kMaxE];
  __shared__ int totals[kMaxE];
  __shared__ int offs[kMaxE + 1];
  // an expert id outside [0, E) takes part in no group (it is dropped)
  const int e0 = (int)threadIdx.x < S ? topk_idx[threadIdx.x] : -1;
  const bool valid = (unsigned)e0 < (unsigned)E;
  const int e = valid ? e0 : 0;
  dispatch_lone_chunk(e, valid, E, counts, offsets, sorted_slots, wave_base, totals, offs);
}

__global__ __launch_bounds__(kChunkSlots) void dispatch_rank_kernel(
    const int32_t* __restrict__ topk_idx, int S, int E, int32_t* __restrict__ blk_counts,
    int32_t* __restrict__ local_rank) {
  __shared__ int wave_base[kChunkWaves][kMaxE];
  __shared__ int totals[kMaxE];
  const int s = blockIdx.x * kChunkSlots + threadIdx.x;
  const int e0 = s < S ? topk_idx[s] : -1;
  const bool valid = (unsigned)e0 < (unsigned)E;  // ids outside [0, E) are dropped
  const int e = valid ? e0 : 0;
  const int r = chunk_rank(e, valid, E, wave_base, totals);
  if (valid) local_rank[s] = r;
  if ((int)threadIdx.x < E) blk_counts[(size_t)blockIdx.x * E + threadIdx.x] = totals[threadIdx.x];
}

// One block: per expert, exclusive scan of the chunk counts (in place), the
// expert totals and offsets.  A thread's counts are loaded 8 chunks at a time
// before they are added: one load round trip per chunk had cost 9.5 us at
// 32 chunks (4096 tokens at top-8).
constexpr int kScanBatch = 8;
__global__ __launch_bounds__(kMaxE) void dispatch_scan_kernel(int nblk, int E,
                                                              int32_t* __restrict__ blk_counts,
                                                              int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ offsets) {
  __shared__ int totals[kMaxE];
  const int e = threadIdx.x;
  if (e < E) {
    int run = 0;
    for (int b0 = 0; b0 < nblk; b0 += kScanBatch) {
      int c[kScanBatch];
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j)
        c[j] = b0 + j < nblk ? blk_counts[(size_t)(b0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) {
        if (b0 + j < nblk) blk_counts[(size_t)(b0 + j) * E + e] = run;
        run += c[j];
      }
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
  if ((unsigned)e >= (unsigned)E) return;
  sorted_slots[offsets[e] + blk_base[(size_t)blockIdx.x * E + e] + local_rank[s]] = s;
}

// Slot layout of the all-experts form ("Porting a 128-expert MoE (Gemma-4
// 26B-A4B) to AWS Inferentia2", section "The traceable trick: compute all
// experts, mask to top-8"): every expert takes every token, slot t * E + e,
// expert e's rows in token order, each slot weighted by the token's routing
// weight for e, or 0 when e is not among its top-K.  One thread per slot.
__global__ __launch_bounds__(256) void dense_mask_kernel(
    int T, int E, int K, const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_w,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slots,
    float* __restrict__ w_dense) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i <= E) offsets[i] = (int32_t)(i * T);
  if (i >= (long long)T * E) return;
  const int t = (int)(i / E), e = (int)(i % E);
  float w = 0.0f;
  for (int k = 0; k < K; ++k)
    if (topk_idx[(size_t)t * K + k] == e) w = topk_w[(size_t)t * K + k];
  w_dense[i] = w;
  sorted_slots[(size_t)e * T + t] = (int32_t)i;
}

}  // namespace

hipError_t launch_dense_mask(int T, int E, int K, const int32_t* topk_idx, const float* topk_w,
                             int32_t* offsets, int32_t* sorted_slots, float* w_dense,
                             hipStream_t s) {
  const long long n = (long long)T * E > E + 1 ? (long long)T * E : E + 1;
  hipLaunchKernelGGL(dense_mask_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, T, E,
                     K, topk_idx, topk_w, offsets, sorted_slots, w_dense);
  return hipGetLastError();
}

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
