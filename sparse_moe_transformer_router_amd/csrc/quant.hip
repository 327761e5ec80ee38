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
#include "wformat.h"

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

// E4M3 per output channel (OCP 8-bit floating point, the format of
// wformat.h): s = max |w| / 448 and code = e4m3_encode(w / s) (wformat.h),
// the division correctly rounded fp32; a row of zeros gets s = 0 and codes 0.
__global__ __launch_bounds__(256) void quantize_fp8_kernel(long long rows, int cols,
                                                           const bf16* __restrict__ w,
                                                           uint8_t* __restrict__ q,
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
  const float s = amax / 448.0f;
  if (lane == 0) scale[r] = s;
  uint8_t* qr = q + r * cols;
  for (int c = 8 * lane; c < cols; c += 8 * kWave) {
    const uint4 u = *reinterpret_cast<const uint4*>(wr + c);
    const uint32_t p[4] = {u.x, u.y, u.z, u.w};
    uint32_t out[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = __uint_as_float((i & 1) ? (p[i / 2] & 0xffff0000u) : (p[i / 2] << 16));
      const uint32_t code = s > 0.0f ? e4m3_encode(x / s) : 0u;
      out[i / 4] |= code << (8 * (i % 4));
    }
    *reinterpret_cast<uint2*>(qr + c) = make_uint2(out[0], out[1]);
  }
}

// E2M1 code of a magnitude a (< 8) on the grid 0, 0.5, 1, 1.5, 2, 3, 4, 6:
// the decision points are the midpoints, each tie going to the code with
// mantissa bit 0; past 6 the code saturates at 6.
__device__ __forceinline__ uint32_t e2m1_code(float a) {
  if (a <= 0.25f) return 0;
  if (a < 0.75f) return 1;
  if (a <= 1.25f) return 2;
  if (a < 1.75f) return 3;
  if (a <= 2.5f) return 4;
  if (a < 3.5f) return 5;
  if (a <= 5.0f) return 6;
  return 7;
}

// MXFP4 (OCP Microscaling): each block of 32 consecutive weights of a row
// gets the E8M0 scale 2^shared with shared = floor(log2 max |w|) - 2 (2 is
// E2M1's largest exponent), clamped to [-127, 127]; the elements are the
// E2M1 codes of |w| / 2^shared with the sign bit w < 0, two per byte, the even
// element in the low nibble.  A block of zeros gets scale code 0 and zero
// codes.  One wave per row, one lane per block.
__global__ __launch_bounds__(256) void quantize_mxfp4_kernel(long long rows, int cols,
                                                             const bf16* __restrict__ w,
                                                             uint8_t* __restrict__ q,
                                                             uint8_t* __restrict__ scale) {
  const long long r = (long long)blockIdx.x * 4 + threadIdx.x / kWave;
  if (r >= rows) return;  // whole wave
  const int nb = cols / 32;
  for (int b = lane_id(); b < nb; b += kWave) {
    const uint4* src = reinterpret_cast<const uint4*>(w + r * cols + 32 * b);
    uint32_t p[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 u = src[i];
      p[4 * i] = u.x;
      p[4 * i + 1] = u.y;
      p[4 * i + 2] = u.z;
      p[4 * i + 3] = u.w;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      amax = fmaxf(amax, fabsf(__uint_as_float(p[i] << 16)));
      amax = fmaxf(amax, fabsf(__uint_as_float(p[i] & 0xffff0000u)));
    }
    uint32_t e8 = 0;
    int shared = 0;
    if (amax > 0.0f) {
      int ex;
      (void)frexpf(amax, &ex);  // floor(log2 amax) = ex - 1, exactly
      shared = min(max(ex - 1 - 2, -127), 127);
      e8 = (uint32_t)(shared + 127);
    }
    uint32_t out[4] = {0u, 0u, 0u, 0u};
    if (amax > 0.0f) {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const uint32_t bits = (i & 1) ? (p[i / 2] & 0xffff0000u) : (p[i / 2] << 16);
        const float x = __uint_as_float(bits);
        const uint32_t code = e2m1_code(ldexpf(fabsf(x), -shared)) | (x < 0.0f ? 8u : 0u);
        out[i / 8] |= code << (4 * (i % 8));
      }
    }
    *reinterpret_cast<uint4*>(q + r * (cols / 2) + 16 * b) =
        make_uint4(out[0], out[1], out[2], out[3]);
    scale[r * nb + b] = (uint8_t)e8;
  }
}

// Codes back to fp32 with the expert kernels' widening (wformat.h), times
// the channel scale for int8 and E4M3 (one rounding of the exact product).
// One thread per 16 weights.
template <typename WQ>
__global__ __launch_bounds__(256) void dequantize_kernel(long long rows, int cols,
                                                         const WQ* __restrict__ q,
                                                         const void* __restrict__ scale,
                                                         float* __restrict__ out) {
  typedef WFmt<WQ> F;
  const long long g = (long long)blockIdx.x * 256 + threadIdx.x;
  const int per_row = cols / 16;
  if (g >= rows * per_row) return;
  const long long r = g / per_row;
  const int k = 16 * (int)(g % per_row);
  const uint8_t* srow = nullptr;
  if constexpr (F::kBlockScale) srow = static_cast<const uint8_t*>(scale) + r * (cols / 32);
  WRaw<WQ> raw;
  raw.load16(wrow(q, r * cols), k, srow);
  const W16 f = raw.widen(0);
  float sc = 1.0f;
  if constexpr (F::kChannelScale) sc = static_cast<const float*>(scale)[r];
  float v[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t word = (i < 4) ? (&f.u[0].x)[i] : (&f.u[1].x)[i - 4];
    v[2 * i] = __uint_as_float(word << 16) * sc;
    v[2 * i + 1] = __uint_as_float(word & 0xffff0000u) * sc;
  }
  float4* o = reinterpret_cast<float4*>(out + r * cols + k);
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
}

}  // namespace

hipError_t launch_quantize_fp8(long long rows, int cols, const void* w, uint8_t* q, float* scale,
                               hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_fp8_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, rows,
                     cols, static_cast<const bf16*>(w), q, scale);
  return hipGetLastError();
}

hipError_t launch_quantize_mxfp4(long long rows, int cols, const void* w, uint8_t* q,
                                 uint8_t* scale, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_mxfp4_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s,
                     rows, cols, static_cast<const bf16*>(w), q, scale);
  return hipGetLastError();
}

hipError_t launch_dequantize(WFormat f, long long rows, int cols, const void* q,
                             const void* scale, float* out, hipStream_t s) {
  const long long n = rows * (cols / 16);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  switch (f) {
    case WFormat::kInt8:
      hipLaunchKernelGGL(dequantize_kernel<int8_t>, grid, dim3(256), 0, s, rows, cols,
                         static_cast<const int8_t*>(q), scale, out);
      break;
    case WFormat::kFP8:
      hipLaunchKernelGGL(dequantize_kernel<fp8e4m3>, grid, dim3(256), 0, s, rows, cols,
                         static_cast<const fp8e4m3*>(q), scale, out);
      break;
    case WFormat::kMXFP4:
      hipLaunchKernelGGL(dequantize_kernel<fp4x2>, grid, dim3(256), 0, s, rows, cols,
                         static_cast<const fp4x2*>(q), scale, out);
      break;
    case WFormat::kBF16:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_quantize_rows(long long rows, int cols, const void* w, int8_t* q, float* scale,
                                hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_rows_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s,
                     rows, cols, static_cast<const bf16*>(w), q, scale);
  return hipGetLastError();
}

}  // namespace moe
