// Router of the Gemma-4 26B-A4B mixture-of-experts block (Gemma4TextRouter on
// the page "Porting a 128-expert MoE (Gemma-4 26B-A4B) to AWS Inferentia2",
// section "The architecture: a dual-path FFN nobody warned me about"): an
// RMSNorm of its own, a scale, the H -> E projection, softmax in fp32, top-K,
// renormalisation over the K, times per_expert_scale.
//
// Routing must come out bit-identical on any IEEE fp32 machine, so every
// reduction over H follows one fixed order: 64-element chunks, each a fused
// multiply-add chain in ascending index from +0, the chunk results added in
// ascending chunk order from +0.  Division and square root are the correctly
// rounded ones (HIP's default for sqrtf and '/'), and contraction is off in
// this file so that products written separately stay separate.
//
// Three kernels:
//   router_prep   one wave per token: the inverse RMS of x (and, with a
//                 pre-norm gain, of v = x * r0 * gain), in the fixed order;
//   router_logits the projection.  Small batches: a wave takes a few
//                 (token, expert) pairs and its lane c owns chunk c of every
//                 pair; the chunk results meet in LDS and one lane per pair
//                 adds them in order.  Large batches: a block takes 64 tokens
//                 x 32 experts, lane = token, so every lane runs whole chunks
//                 while the expert weights are read as LDS broadcasts;
//   router_topk   one wave per token: softmax, top-K selection with the
//                 lowest-index tie break, renormalisation, per-expert scale.
#include "common.h"
#include "launch.h"

#pragma clang fp contract(off)

namespace moe {
namespace {

constexpr int kChunk = 64;

__device__ __forceinline__ void load8(const float* p, float v[8]) {
  const float4* q = reinterpret_cast<const float4*>(p);
  float4 a = q[0], b = q[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ void load8(const bf16* p, float v[8]) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  v[0] = __uint_as_float(u.x << 16); v[1] = __uint_as_float(u.x & 0xffff0000u);
  v[2] = __uint_as_float(u.y << 16); v[3] = __uint_as_float(u.y & 0xffff0000u);
  v[4] = __uint_as_float(u.z << 16); v[5] = __uint_as_float(u.z & 0xffff0000u);
  v[6] = __uint_as_float(u.w << 16); v[7] = __uint_as_float(u.w & 0xffff0000u);
}

// Sum of squares of one 64-element chunk, as one fma chain from +0.
template <typename XT>
__device__ __forceinline__ float chunk_sumsq(const XT* p) {
  float part = 0.0f;
#pragma unroll
  for (int i = 0; i < kChunk; i += 8) {
    float v[8];
    load8(p + i, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) part = __builtin_fmaf(v[j], v[j], part);
  }
  return part;
}

// Inverse RMS from the chunk partial sums held in LDS: sum in chunk order,
// then 1 / sqrt(sum / H + eps), each operation rounded once.
__device__ __forceinline__ float inv_rms_from_parts(const float* sp, int nc, int H, float eps) {
  float total = 0.0f;
  for (int c = 0; c < nc; ++c) total = total + sp[c];
  float mean = total / (float)H;
  return 1.0f / sqrtf(mean + eps);
}

template <typename XT>
__global__ __launch_bounds__(256) void router_prep_kernel(int T, int H, float eps,
                                                          const XT* __restrict__ x,
                                                          const float* __restrict__ pre_gain,
                                                          float* __restrict__ r0_out,
                                                          float* __restrict__ r_out) {
  __shared__ float parts[4][256];
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int t = blockIdx.x * 4 + wave;
  const bool active = t < T;
  const int nc = H / kChunk;
  const XT* xr = x + (size_t)(active ? t : 0) * H;
  float* sp = parts[wave];

  if (active)
    for (int c = lane; c < nc; c += kWave) sp[c] = chunk_sumsq(xr + c * kChunk);
  __syncthreads();
  float r0 = 0.0f;
  if (active && lane == 0) r0 = inv_rms_from_parts(sp, nc, H, eps);
  r0 = __shfl(r0, 0, kWave);
  if (pre_gain == nullptr) {
    if (active && lane == 0) r_out[t] = r0;
    return;
  }
  __syncthreads();
  // second norm on v = (x * r0) * gain
  if (active) {
    for (int c = lane; c < nc; c += kWave) {
      float part = 0.0f;
      for (int i = 0; i < kChunk; i += 8) {
        float v[8], g[8];
        load8(xr + c * kChunk + i, v);
        load8(pre_gain + c * kChunk + i, g);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float vv = (v[j] * r0) * g[j];
          part = __builtin_fmaf(vv, vv, part);
        }
      }
      sp[c] = part;
    }
  }
  __syncthreads();
  if (active && lane == 0) {
    r0_out[t] = r0;
    r_out[t] = inv_rms_from_parts(sp, nc, H, eps);
  }
}

// Router input element after both norms: vhat = (v * r) * scale with
// v = x, or v = (x * r0) * gain under a pre-norm.
__device__ __forceinline__ float router_vhat(float x, bool pre, float r0, float g, float r,
                                             float s) {
  float v = pre ? (x * r0) * g : x;
  return (v * r) * s;
}

// Small batches: TPW tokens x EPW experts per wave; lane c owns chunk c
// (requires H / 64 <= 64).
template <typename XT, int TPW, int EPW>
__global__ __launch_bounds__(256) void router_logits_pairs_kernel(
    int T, int H, int E, const XT* __restrict__ x, const float* __restrict__ pre_gain,
    const float* __restrict__ r0v, const float* __restrict__ rv,
    const float* __restrict__ scale, const float* __restrict__ W, float* __restrict__ logits) {
  constexpr int P = TPW * EPW;
  __shared__ float parts[4][P][kWave + 1];
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int gw = blockIdx.x * 4 + wave;
  const int n_eg = (E + EPW - 1) / EPW;
  const int tg = gw / n_eg, eg = gw % n_eg;
  const bool active = tg * TPW < T;
  const int nc = H / kChunk;
  const bool pre = pre_gain != nullptr;

  float acc[TPW][EPW];
#pragma unroll
  for (int a = 0; a < TPW; ++a)
#pragma unroll
    for (int b = 0; b < EPW; ++b) acc[a][b] = 0.0f;

  if (active && lane < nc) {
    const XT* xr[TPW];
    float rt[TPW], r0t[TPW];
#pragma unroll
    for (int a = 0; a < TPW; ++a) {
      int t = min(tg * TPW + a, T - 1);
      xr[a] = x + (size_t)t * H;
      rt[a] = rv[t];
      r0t[a] = pre ? r0v[t] : 0.0f;
    }
    const float* wr[EPW];
#pragma unroll
    for (int b = 0; b < EPW; ++b) wr[b] = W + (size_t)min(eg * EPW + b, E - 1) * H;
    const int h0 = lane * kChunk;
    for (int i = 0; i < kChunk; i += 8) {
      float s[8], g[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      load8(scale + h0 + i, s);
      if (pre) load8(pre_gain + h0 + i, g);
      float vh[TPW][8];
#pragma unroll
      for (int a = 0; a < TPW; ++a) {
        float xv[8];
        load8(xr[a] + h0 + i, xv);
#pragma unroll
        for (int j = 0; j < 8; ++j) vh[a][j] = router_vhat(xv[j], pre, r0t[a], g[j], rt[a], s[j]);
      }
#pragma unroll
      for (int b = 0; b < EPW; ++b) {
        float wv[8];
        load8(wr[b] + h0 + i, wv);
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int a = 0; a < TPW; ++a) acc[a][b] = __builtin_fmaf(vh[a][j], wv[j], acc[a][b]);
      }
    }
#pragma unroll
    for (int a = 0; a < TPW; ++a)
#pragma unroll
      for (int b = 0; b < EPW; ++b) parts[wave][a * EPW + b][lane] = acc[a][b];
  }
  __syncthreads();
  if (active && lane < P) {
    const int a = lane / EPW, b = lane % EPW;
    const int t = tg * TPW + a, e = eg * EPW + b;
    if (t < T && e < E) {
      float total = 0.0f;
      for (int c = 0; c < nc; ++c) total = total + parts[wave][lane][c];
      logits[(size_t)t * E + e] = total;
    }
  }
}

// Large batches: 64 tokens (lane = token) x 32 experts (8 per wave) per block.
template <typename XT>
__global__ __launch_bounds__(256) void router_logits_tiled_kernel(
    int T, int H, int E, const XT* __restrict__ x, const float* __restrict__ pre_gain,
    const float* __restrict__ r0v, const float* __restrict__ rv,
    const float* __restrict__ scale, const float* __restrict__ W, float* __restrict__ logits) {
  __shared__ float wl[kChunk][32];
  __shared__ float sl[kChunk], gl[kChunk];
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 32;
  const int t = t0 + lane;
  const bool tv = t < T;
  const int tc = tv ? t : T - 1;
  const bool pre = pre_gain != nullptr;
  const float r = rv[tc];
  const float r0 = pre ? r0v[tc] : 0.0f;
  const XT* xr = x + (size_t)tc * H;
  const int nc = H / kChunk;

  float total[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) total[j] = 0.0f;

  for (int c = 0; c < nc; ++c) {
    float xv[kChunk];
#pragma unroll
    for (int i = 0; i < kChunk; i += 8) load8(xr + c * kChunk + i, xv + i);
    __syncthreads();  // the previous chunk's LDS reads are done
    {
      const int ei = threadIdx.x / 8, ks = (threadIdx.x % 8) * 8;
      const int e = e0 + ei;
      float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (e < E) load8(W + (size_t)e * H + c * kChunk + ks, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) wl[ks + j][ei] = v[j];
      if (threadIdx.x < kChunk) sl[threadIdx.x] = scale[c * kChunk + threadIdx.x];
      else if (threadIdx.x < 2 * kChunk)
        gl[threadIdx.x - kChunk] = pre ? pre_gain[c * kChunk + threadIdx.x - kChunk] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kChunk; ++k) xv[k] = router_vhat(xv[k], pre, r0, gl[k], r, sl[k]);
    float part[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) part[j] = 0.0f;
#pragma unroll
    for (int k = 0; k < kChunk; ++k) {
      const float4* wp = reinterpret_cast<const float4*>(&wl[k][wave * 8]);
      float4 wa = wp[0], wb = wp[1];
      part[0] = __builtin_fmaf(xv[k], wa.x, part[0]);
      part[1] = __builtin_fmaf(xv[k], wa.y, part[1]);
      part[2] = __builtin_fmaf(xv[k], wa.z, part[2]);
      part[3] = __builtin_fmaf(xv[k], wa.w, part[3]);
      part[4] = __builtin_fmaf(xv[k], wb.x, part[4]);
      part[5] = __builtin_fmaf(xv[k], wb.y, part[5]);
      part[6] = __builtin_fmaf(xv[k], wb.z, part[6]);
      part[7] = __builtin_fmaf(xv[k], wb.w, part[7]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) total[j] = total[j] + part[j];
  }
  if (tv) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = e0 + wave * 8 + j;
      if (e < E) logits[(size_t)t * E + e] = total[j];
    }
  }
}

// One wave per token: softmax over E (<= 256) logits, top-K by logit with
// ties to the lower index, weights z_k / sum_j z_j * per_expert_scale.
__global__ __launch_bounds__(256) void router_topk_kernel(int T, int E, int K,
                                                          const float* __restrict__ logits,
                                                          const float* __restrict__ pes,
                                                          int32_t* __restrict__ idx,
                                                          float* __restrict__ w) {
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;  // no block barrier below
  float l[4], z[4];
  bool taken[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + kWave * j;
    taken[j] = e >= E;
    l[j] = taken[j] ? -INFINITY : logits[(size_t)t * E + e];
  }
  float m = wave_max(fmaxf(fmaxf(l[0], l[1]), fmaxf(l[2], l[3])));
#pragma unroll
  for (int j = 0; j < 4; ++j) z[j] = taken[j] ? 0.0f : expf(l[j] - m);

  int my_idx = 0;
  float my_z = 0.0f;
  for (int k = 0; k < K; ++k) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + kWave * j;
      if (!taken[j] && (l[j] > bv || (l[j] == bv && e < bi))) { bv = l[j]; bi = e; }
    }
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
      float ov = __shfl_xor(bv, o, kWave);
      int oi = __shfl_xor(bi, o, kWave);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    const int owner = bi & (kWave - 1), slot = bi / kWave;
    float zw = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (lane == owner && j == slot) { taken[j] = true; zw = z[j]; }
    zw = __shfl(zw, owner, kWave);
    if (lane == k) { my_idx = bi; my_z = zw; }
  }
  float q = 0.0f;
  for (int k = 0; k < K; ++k) q = q + __shfl(my_z, k, kWave);
  if (lane < K) {
    idx[(size_t)t * K + lane] = my_idx;
    w[(size_t)t * K + lane] = (my_z / q) * pes[my_idx];
  }
}

template <typename XT>
hipError_t launch_router_t(const RouterArgs& a, hipStream_t s) {
  const XT* x = static_cast<const XT*>(a.x);
  const int nc = a.H / kChunk;
  hipLaunchKernelGGL(router_prep_kernel<XT>, dim3((a.T + 3) / 4), dim3(256), 0, s, a.T, a.H,
                     a.eps, x, a.pre_gain, a.ws_r0, a.ws_r);
  if (nc <= kWave && a.T < 8) {
    const int waves = a.T * ((a.E + 3) / 4);
    hipLaunchKernelGGL((router_logits_pairs_kernel<XT, 1, 4>), dim3((waves + 3) / 4), dim3(256),
                       0, s, a.T, a.H, a.E, x, a.pre_gain, a.ws_r0, a.ws_r, a.router_scale,
                       a.router_w, a.ws_logits);
  } else if (nc <= kWave && a.T <= 256) {
    const int waves = ((a.T + 3) / 4) * ((a.E + 3) / 4);
    hipLaunchKernelGGL((router_logits_pairs_kernel<XT, 4, 4>), dim3((waves + 3) / 4), dim3(256),
                       0, s, a.T, a.H, a.E, x, a.pre_gain, a.ws_r0, a.ws_r, a.router_scale,
                       a.router_w, a.ws_logits);
  } else {
    hipLaunchKernelGGL(router_logits_tiled_kernel<XT>, dim3((a.T + 63) / 64, (a.E + 31) / 32),
                       dim3(256), 0, s, a.T, a.H, a.E, x, a.pre_gain, a.ws_r0, a.ws_r,
                       a.router_scale, a.router_w, a.ws_logits);
  }
  hipLaunchKernelGGL(router_topk_kernel, dim3((a.T + 3) / 4), dim3(256), 0, s, a.T, a.E, a.K,
                     a.ws_logits, a.per_expert_scale, a.topk_idx, a.topk_w);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router(const RouterArgs& a, hipStream_t s) {
  return a.x_bf16 ? launch_router_t<bf16>(a, s) : launch_router_t<float>(a, s);
}

}  // namespace moe
