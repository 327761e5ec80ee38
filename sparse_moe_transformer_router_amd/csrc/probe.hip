// Measurement probes: the achievable HBM read rate and bf16 MFMA rate of the
// part, the two ceilings the path's kernels are compared against besides the
// published peaks.  Not part of the path; built as libmoe_probe.so.
//
// Both kernels produce a checkable result so that the work cannot be dropped
// and a test can confirm it ran: the read probe XORs every 32-bit word of the
// buffer (one word per block), the MFMA probe multiplies all-ones fragments,
// so every accumulator lane ends at 16 * iterations exactly.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "moe_probe.h"

namespace {

constexpr int kReadThreads = 256;
constexpr int kReadBlocks = 256 * 8;
constexpr int kReadUnroll = 4;
constexpr int kStep = kReadThreads * 2;  // 16-byte units a block reads per step

// Each block streams one contiguous chunk of the buffer (so the blocks in
// flight spread over all memory channels), a lane taking 32 contiguous bytes
// per step (four lanes use a whole 128-byte line at once), kReadUnroll steps
// of loads issued before their results are used.
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(
    const uint4* __restrict__ p, long long n16, uint32_t* __restrict__ block_xor) {
  uint32_t acc = 0;
  const long long per = (n16 + gridDim.x - 1) / gridDim.x;
  const long long chunk = (per + kStep - 1) / kStep * kStep;
  const long long begin = (long long)blockIdx.x * chunk;
  const long long end = min(begin + chunk, n16);
  long long i = begin + 2 * threadIdx.x;
  for (; i + (kReadUnroll - 1) * kStep + 1 < end; i += kReadUnroll * kStep) {
    uint4 v[kReadUnroll][2];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      v[u][0] = p[i + u * kStep];
      v[u][1] = p[i + u * kStep + 1];
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc ^= v[u][j].x ^ v[u][j].y ^ v[u][j].z ^ v[u][j].w;
  }
  for (; i < end; i += kStep) {
    const uint4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
    if (i + 1 < end) {
      const uint4 b = p[i + 1];
      acc ^= b.x ^ b.y ^ b.z ^ b.w;
    }
  }
  __shared__ uint32_t red[kReadThreads];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = kReadThreads / 2; s > 0; s /= 2) {
    if ((int)threadIdx.x < s) red[threadIdx.x] ^= red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) block_xor[blockIdx.x] = red[0];
}

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
constexpr int kMfmaAcc = 8;

__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* __restrict__ out) {
  bf16x8_t a;
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = (__bf16)1.0f;
  f32x16_t acc[kMfmaAcc];
#pragma unroll
  for (int j = 0; j < kMfmaAcc; ++j)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[j][q] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kMfmaAcc; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, acc[j], 0, 0, 0);
  }
  // Every lane of every accumulator holds 16 * iters; the per-wave value is
  // taken from lane 0 of accumulator 0 after checking the others agree.
  float v = acc[0][0];
  bool same = true;
#pragma unroll
  for (int j = 0; j < kMfmaAcc; ++j)
#pragma unroll
    for (int q = 0; q < 16; ++q) same = same && acc[j][q] == v;
  if ((threadIdx.x & 63) == 0)
    out[blockIdx.x * 4 + threadIdx.x / 64] = same ? v : -1.0f;
}

}  // namespace

extern "C" {

int moe_probe_read_blocks(void) { return kReadBlocks; }

int moe_probe_stream_read(const void* buf, long long bytes, uint32_t* block_xor, void* stream) {
  if (!buf || !block_xor || bytes <= 0 || bytes % 16 != 0) return -1;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0) return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(moe_probe_read_blocks()), dim3(kReadThreads),
                     0, static_cast<hipStream_t>(stream), static_cast<const uint4*>(buf),
                     bytes / 16, block_xor);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

long long moe_probe_mfma_flops(int blocks, int iters) {
  return (long long)blocks * 4 * iters * kMfmaAcc * (2LL * 32 * 32 * 16);
}

int moe_probe_mfma(int blocks, int iters, float* out, void* stream) {
  if (!out || blocks <= 0 || blocks > (1 << 20) || iters <= 0 || iters > (1 << 20)) return -1;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), iters, out);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
