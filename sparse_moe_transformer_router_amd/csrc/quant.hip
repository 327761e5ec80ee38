// int8 per-channel symmetric weights: the int8-expert variant on the page
// "Porting a 128-expert MoE (Gemma-4 26B-A4B) to AWS Inferentia2", section
// "Can it run on a smaller box? Yes, no, and "deeper than it looks"".  A
// channel is one output row of an [out, in] weight: s = max |w| / 127, codes
// q = round-half-to-even(w / s) clamped to [-127, 127] (both divisions
// correctly rounded fp32); a row of zeros gets s = 0 and q = 0.  One wave per
// row: the maximum is exact in any order, so codes and scales come out the
// same on any IEEE machine.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void quantize_rows_kernel(long long rows, int cols,
                                                            const bf16* __restrict__ w,
                                                            int8_t* __restrict__ q,
                                                            float* __restrict__ scale) {
  const long long r = (long long)blockIdx.x * 4 + threadIdx.x / kWave;
  if (r >= rows) return;  // whole wave
  const int lane = lane_id();
  const bf16* wr = w + r * cols;
  float amax = 0.0f;
  for (int c = 8 * lane; c < cols; c += 8 * kWave) {
    const uint4 u = *reinterpret_cast<const uint4*>(wr + c);
    const uint32_t p[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      amax = fmaxf(amax, fabsf(__uint_as_float(p[i] << 16)));
      amax = fmaxf(amax, fabsf(__uint_as_float(p[i] & 0xffff0000u)));
    }
  }
  amax = wave_max(amax);
  const float s = amax / 127.0f;
  if (lane == 0) scale[r] = s;
  int8_t* qr = q + r * cols;
  for (int c = 8 * lane; c < cols; c += 8 * kWave) {
    const uint4 u = *reinterpret_cast<const uint4*>(wr + c);
    const uint32_t p[4] = {u.x, u.y, u.z, u.w};
    uint32_t out[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t bits = (i & 1) ? (p[i / 2] & 0xffff0000u) : (p[i / 2] << 16);
      float v = 0.0f;
      if (s > 0.0f) v = rintf(__uint_as_float(bits) / s);
      v = fminf(fmaxf(v, -127.0f), 127.0f);
      out[i / 4] |= ((uint32_t)(int32_t)v & 0xffu) << (8 * (i % 4));
    }
    *reinterpret_cast<uint2*>(qr + c) = make_uint2(out[0], out[1]);
  }
}

}  // namespace

hipError_t launch_quantize_rows(long long rows, int cols, const void* w, int8_t* q, float* scale,
                                hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_rows_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s,
                     rows, cols, static_cast<const bf16*>(w), q, scale);
  return hipGetLastError();
}

}  // namespace moe
