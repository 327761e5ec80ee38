// Combine, pre-norms and the layer epilogue of the Gemma-4 26B-A4B dual-path
// feed-forward layer (the diagram in "Porting a 128-expert MoE (Gemma-4
// 26B-A4B) to AWS Inferentia2", section "The architecture: a dual-path FFN
// nobody warned me about"; the final multiply by layer_scalar is described
// in "Porting Gemma-4 (2B / 4B / 12B) to AWS Inferentia2", section 4.6).
//
// combine        out[t] = sum_k y[t,k] (k ascending, fp32, no atomics) + addend[t]
// prenorm        xd = RMSNorm_pre(x), xm = RMSNorm_pre2(x) in one pass over x
// block epilogue o = RMSNorm_post(RMSNorm_post1(dn) + RMSNorm_post2(sum_k y[t,k]));
//                out = (o + x) * layer_scalar
// All bandwidth-bound: 16-byte vector accesses, one block per token row for
// the norms, fp32 arithmetic.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void ld8(const float* p, float v[8]) {
  const float4* q = reinterpret_cast<const float4*>(p);
  float4 a = q[0], b = q[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void ld8(const bf16* p, float v[8]) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  v[0] = __uint_as_float(u.x << 16); v[1] = __uint_as_float(u.x & 0xffff0000u);
  v[2] = __uint_as_float(u.y << 16); v[3] = __uint_as_float(u.y & 0xffff0000u);
  v[4] = __uint_as_float(u.z << 16); v[5] = __uint_as_float(u.z & 0xffff0000u);
  v[6] = __uint_as_float(u.w << 16); v[7] = __uint_as_float(u.w & 0xffff0000u);
}
__device__ __forceinline__ void st8(float* p, const float v[8]) {
  float4* q = reinterpret_cast<float4*>(p);
  q[0] = make_float4(v[0], v[1], v[2], v[3]);
  q[1] = make_float4(v[4], v[5], v[6], v[7]);
}
__device__ __forceinline__ void st8(bf16* p, const float v[8]) {
  bf16x8 b;
#pragma unroll
  for (int i = 0; i < 8; ++i) b[i] = (bf16)v[i];
  *reinterpret_cast<bf16x8*>(p) = b;
}

// acc[j] += y_t[k][c + j] for k = 0 .. K-1 in ascending order (the
// combine's fixed order; y_t points at token t's K slot rows of length H).
// The loads of up to 8 slots are issued before their adds, so K slots cost
// about K / 8 memory round trips instead of K.
template <typename YT>
__device__ __forceinline__ void sum_slots(const YT* __restrict__ y_t, int K, int H, int c,
                                          float acc[8]) {
  for (int k0 = 0; k0 < K; k0 += 8) {
    float v[8][8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      if (k0 + kk < K) ld8(y_t + (size_t)(k0 + kk) * H + c, v[kk]);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      if (k0 + kk < K) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] += v[kk][j];
      }
  }
}

template <typename YT, typename OT>
__global__ __launch_bounds__(kThreads) void combine_kernel(int T, int H, int K,
                                                           const YT* __restrict__ y,
                                                           const OT* __restrict__ addend,
                                                           OT* __restrict__ out) {
  const int per_row = H / 8;
  const long long n = (long long)T * per_row;
  for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (long long)gridDim.x * kThreads) {
    const int t = (int)(i / per_row), c = (int)(i % per_row) * 8;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    sum_slots(y + (size_t)t * K * H, K, H, c, acc);
    if (addend) {
      float v[8];
      ld8(addend + (size_t)t * H + c, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] += v[j];
    }
    st8(out + (size_t)t * H + c, acc);
  }
}

__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int wave = threadIdx.x / kWave, lane = lane_id();
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float s = 0.0f;
#pragma unroll
  for (int w = 0; w < kThreads / kWave; ++w) s += red[w];
  return s;
}

// xd = x / rms(x) * g_pre, xm = x / rms(x) * g_pre2 (one block per token).
template <typename XT>
__global__ __launch_bounds__(kThreads) void prenorm_kernel(int H, float eps,
                                                           const XT* __restrict__ x,
                                                           const float* __restrict__ g_pre,
                                                           const float* __restrict__ g_pre2,
                                                           XT* __restrict__ xd,
                                                           XT* __restrict__ xm) {
  __shared__ float red[kThreads / kWave];
  const int t = blockIdx.x;
  const XT* xr = x + (size_t)t * H;
  float ss = 0.0f;
  for (int c = threadIdx.x * 8; c < H; c += kThreads * 8) {
    float v[8];
    ld8(xr + c, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) ss += v[j] * v[j];
  }
  const float r = 1.0f / sqrtf(block_sum(ss, red) / (float)H + eps);
  for (int c = threadIdx.x * 8; c < H; c += kThreads * 8) {
    float v[8], g1[8], g2[8], o1[8], o2[8];
    ld8(xr + c, v);
    ld8(g_pre + c, g1);
    ld8(g_pre2 + c, g2);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      o1[j] = v[j] * r * g1[j];
      o2[j] = v[j] * r * g2[j];
    }
    st8(xd + (size_t)t * H + c, o1);
    st8(xm + (size_t)t * H + c, o2);
  }
}

// One block per token; the MoE sum and the dense row are kept in LDS
// (dynamic shared memory of 2 * H floats).
template <typename YT, typename XT>
__global__ __launch_bounds__(kThreads) void block_epilogue_kernel(
    int H, int K, float eps, float layer_scalar, const YT* __restrict__ y,
    const YT* __restrict__ dn, const XT* __restrict__ x, const float* __restrict__ g_post1,
    const float* __restrict__ g_post2, const float* __restrict__ g_post, XT* __restrict__ out,
    float* __restrict__ ffn_out) {
  extern __shared__ float row[];
  float* ms = row;      // [H] sum_k y
  float* ds = row + H;  // [H] dense
  __shared__ float red[kThreads / kWave];
  const int t = blockIdx.x;
  float ssm = 0.0f, ssd = 0.0f;
  for (int c = threadIdx.x * 8; c < H; c += kThreads * 8) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0}, d[8];
    ld8(dn + (size_t)t * H + c, d);
    sum_slots(y + (size_t)t * K * H, K, H, c, acc);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      ssm += acc[j] * acc[j];
      ssd += d[j] * d[j];
    }
    st8(ms + c, acc);
    st8(ds + c, d);
  }
  const float rm = 1.0f / sqrtf(block_sum(ssm, red) / (float)H + eps);
  const float rd = 1.0f / sqrtf(block_sum(ssd, red) / (float)H + eps);
  float sss = 0.0f;
  for (int c = threadIdx.x * 8; c < H; c += kThreads * 8) {
    float m[8], d[8], g1[8], g2[8];
    ld8(ms + c, m);
    ld8(ds + c, d);
    ld8(g_post1 + c, g1);
    ld8(g_post2 + c, g2);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      m[j] = d[j] * rd * g1[j] + m[j] * rm * g2[j];
      sss += m[j] * m[j];
    }
    st8(ms + c, m);
  }
  const float rs = 1.0f / sqrtf(block_sum(sss, red) / (float)H + eps);
  for (int c = threadIdx.x * 8; c < H; c += kThreads * 8) {
    float m[8], g[8], xv[8], o[8];
    ld8(ms + c, m);
    ld8(g_post + c, g);
    ld8(x + (size_t)t * H + c, xv);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      m[j] = m[j] * rs * g[j];
      o[j] = (m[j] + xv[j]) * layer_scalar;
    }
    st8(out + (size_t)t * H + c, o);
    if (ffn_out) st8(ffn_out + (size_t)t * H + c, m);
  }
}

int grid_for(long long n) {
  long long b = (n + kThreads - 1) / kThreads;
  return (int)(b < 8192 ? (b < 1 ? 1 : b) : 8192);
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  const int grid = grid_for((long long)a.T * (a.H / 8));
  if (a.act_bf16) {
    if (a.y_bf16)
      hipLaunchKernelGGL((combine_kernel<bf16, bf16>), dim3(grid), dim3(kThreads), 0, s, a.T, a.H,
                         a.K, static_cast<const bf16*>(a.y), static_cast<const bf16*>(a.addend),
                         static_cast<bf16*>(a.out));
    else
      hipLaunchKernelGGL((combine_kernel<float, bf16>), dim3(grid), dim3(kThreads), 0, s, a.T,
                         a.H, a.K, static_cast<const float*>(a.y),
                         static_cast<const bf16*>(a.addend), static_cast<bf16*>(a.out));
  } else {
    hipLaunchKernelGGL((combine_kernel<float, float>), dim3(grid), dim3(kThreads), 0, s, a.T,
                       a.H, a.K, static_cast<const float*>(a.y),
                       static_cast<const float*>(a.addend), static_cast<float*>(a.out));
  }
  return hipGetLastError();
}

hipError_t launch_prenorm(const PreNormArgs& a, hipStream_t s) {
  if (a.bf16)
    hipLaunchKernelGGL(prenorm_kernel<bf16>, dim3(a.T), dim3(kThreads), 0, s, a.H, a.eps,
                       static_cast<const bf16*>(a.x), a.g_pre, a.g_pre2, static_cast<bf16*>(a.xd),
                       static_cast<bf16*>(a.xm));
  else
    hipLaunchKernelGGL(prenorm_kernel<float>, dim3(a.T), dim3(kThreads), 0, s, a.H, a.eps,
                       static_cast<const float*>(a.x), a.g_pre, a.g_pre2,
                       static_cast<float*>(a.xd), static_cast<float*>(a.xm));
  return hipGetLastError();
}

hipError_t launch_block_epilogue(const EpilogueArgs& a, hipStream_t s) {
  const size_t lds = 2 * (size_t)a.H * sizeof(float);
  if (a.act_bf16) {
    if (a.y_bf16)
      hipLaunchKernelGGL((block_epilogue_kernel<bf16, bf16>), dim3(a.T), dim3(kThreads), lds, s,
                         a.H, a.K, a.eps, a.layer_scalar, static_cast<const bf16*>(a.y),
                         static_cast<const bf16*>(a.dn), static_cast<const bf16*>(a.x),
                         a.g_post1, a.g_post2, a.g_post, static_cast<bf16*>(a.out), a.ffn_out);
    else
      hipLaunchKernelGGL((block_epilogue_kernel<float, bf16>), dim3(a.T), dim3(kThreads), lds, s,
                         a.H, a.K, a.eps, a.layer_scalar, static_cast<const float*>(a.y),
                         static_cast<const float*>(a.dn), static_cast<const bf16*>(a.x),
                         a.g_post1, a.g_post2, a.g_post, static_cast<bf16*>(a.out), a.ffn_out);
  } else {
    hipLaunchKernelGGL((block_epilogue_kernel<float, float>), dim3(a.T), dim3(kThreads), lds, s,
                       a.H, a.K, a.eps, a.layer_scalar, static_cast<const float*>(a.y),
                       static_cast<const float*>(a.dn), static_cast<const float*>(a.x),
                       a.g_post1, a.g_post2, a.g_post, static_cast<float*>(a.out), a.ffn_out);
  }
  return hipGetLastError();
}

}  // namespace moe
