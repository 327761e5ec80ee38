// Storage formats of expert weights below bf16, and their exact widening to
// bf16 for the matrix cores.  The page "Porting a 128-expert MoE (Gemma-4
// 26B-A4B) to AWS Inferentia2" weighs int8 per-channel experts (section "Can
// it run on a smaller box? Yes, no, and "deeper than it looks"") and the
// 8-bit and 4-bit floating-point options (section "The fp4 rabbit hole (two
// of them, both dead ends)").  The floating-point formats are those of the
// OCP standards:
//
//   fp8e4m3  one E4M3 code per weight (sign, 4 exponent bits with bias 7, 3
//            mantissa bits, no infinities, largest finite 448), with one fp32
//            scale per output channel applied after the dot product;
//   fp4x2    two E2M1 codes per byte (the even element in the low nibble), 32
//            consecutive weights along the contraction sharing one E8M0
//            scale 2^(e - 127) (MXFP4).
//
// Every code widens to bf16 exactly: int8 codes need 7 significant bits,
// E4M3 values 4, and E2M1 values times a power of two 2 (while the product
// stays in bf16's normal range, i.e. block scales above 2^-125).
#pragma once

#include "common.h"

namespace moe {

struct fp8e4m3 {
  uint8_t b;
};
struct fp4x2 {
  uint8_t b;
};

// Per-format layout facts.  kPerUnit: weights per stored unit; kChannelScale:
// one fp32 scale per output channel (after the k-sum); kBlockScale: one E8M0
// scale per 32 weights along the contraction (folded into the widening);
// kLaneK: weights of one row a lane loads at a time, 32 bytes as stored in
// every format, so that four lanes cover one 128-byte line of the row.
template <typename WQ> struct WFmt {
  static constexpr int kPerUnit = 1, kLaneK = 16;
  static constexpr bool kChannelScale = false, kBlockScale = false;
};
template <> struct WFmt<int8_t> {
  static constexpr int kPerUnit = 1, kLaneK = 32;
  static constexpr bool kChannelScale = true, kBlockScale = false;
};
template <> struct WFmt<fp8e4m3> {
  static constexpr int kPerUnit = 1, kLaneK = 32;
  static constexpr bool kChannelScale = true, kBlockScale = false;
};
template <> struct WFmt<fp4x2> {
  static constexpr int kPerUnit = 2, kLaneK = 64;
  static constexpr bool kChannelScale = false, kBlockScale = true;
};

// E4M3 code nearest to v (OCP 8-bit floating point: half-way cases to the
// even mantissa; magnitudes at or past 448 take 448); the sign bit is v < 0.  The rounding works in the value's binade: its
// exponent E and 3 fraction bits rint((|v| / 2^E - 1) * 8) (exact scalings),
// a carry into the next binade when that gives 8, and below 2^-6 the
// subnormal grid rint(|v| * 2^9).
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const float a = fabsf(v);
  uint32_t code;
  if (a >= 448.0f) {
    code = 0x7E;
  } else if (a < 0.015625f) {
    code = (uint32_t)rintf(a * 512.0f);  // 0..8; 8 is the smallest normal, code 0x08
  } else {
    int ex;
    (void)frexpf(a, &ex);  // a = f * 2^ex, f in [0.5, 1)
    int E = ex - 1;
    uint32_t m = (uint32_t)rintf((ldexpf(a, -E) - 1.0f) * 8.0f);
    if (m == 8) {
      m = 0;
      ++E;
    }
    code = ((uint32_t)(E + 7) << 3) | m;
    if (code > 0x7E) code = 0x7E;
  }
  return code | (v < 0.0f ? 0x80u : 0u);
}


typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 keep4(uint4 q, bool v) {
  return make_uint4(v ? q.x : 0u, v ? q.y : 0u, v ? q.z : 0u, v ? q.w : 0u);
}

__device__ __forceinline__ uint32_t bf16x2_bits(bf16x2_v v) {
  return __builtin_bit_cast(uint32_t, v);
}

// E8M0 scale code -> 2^(e - 127) in fp32 (code 0 is the subnormal 2^-127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  return e != 0 ? __uint_as_float(e << 23) : __uint_as_float(0x00400000u);
}

// Four int8 codes (one word, element 0 in the low byte) -> four bf16 in two
// words (element 0 in the low half).
__device__ __forceinline__ void int8x4_to_bf16(uint32_t word, uint32_t& lo, uint32_t& hi) {
  uint32_t o[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int b0 = 2 * m;
    const float a = (float)((int32_t)(word << (24 - 8 * b0)) >> 24);
    const float b = (float)((int32_t)(word << (16 - 8 * b0)) >> 24);
    o[m] = (__float_as_uint(b) & 0xffff0000u) | (__float_as_uint(a) >> 16);
  }
  lo = o[0];
  hi = o[1];
}

// Four E4M3 codes (one word, element 0 in the low byte) -> four bf16.
__device__ __forceinline__ void fp8x4_to_bf16(uint32_t word, uint32_t& lo, uint32_t& hi) {
  lo = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, false));
  hi = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, true));
}

// Eight E2M1 codes (one word, element 0 in the low nibble) times `scale` (a
// power of two) -> eight bf16 in four words.
__device__ __forceinline__ void fp4x8_to_bf16(uint32_t word, float scale, uint32_t (&o)[4]) {
  o[0] = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 0));
  o[1] = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 1));
  o[2] = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 2));
  o[3] = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 3));
}

// 16 consecutive weights of one row as bf16 (two uint4: elements 0..7, 8..15).
union W16 {
  uint4 u[2];
  bf16x8 v[2];
};

// One lane's kLaneK weights of one row (32 bytes), held raw (as stored) from
// their load to their use.  load(row, k, srow, full): row points at the
// weight row's first unit, k is the element index of the first weight (a
// multiple of kLaneK), srow the row's block scales (fp4x2 only); full is
// false when only the first half of the span lies inside the row (fp4x2
// only: a contraction that is a multiple of 32 but not of 64), and the
// second half is then loaded from the first half's address and must be
// dropped with mask().  The loads are unconditional and nothing reads their
// registers until the weights are used, so a ring of them stays in flight.
// mask(v, full) zeroes the span unless v, and its second half unless full
// (selects; called at the point of use).  widen(u) gives weights
// [16 u, 16 u + 16) of the span as bf16 (u < kLaneK / 16).  load16(row, k,
// srow) loads only weights [k, k + 16) (k a multiple of 16), as sub-group 0.
template <typename WQ> struct WRaw;
template <> struct WRaw<bf16> {
  W16 f;
  __device__ __forceinline__ void load(const bf16* row, int k, const uint8_t*, bool) {
    const uint4* q = reinterpret_cast<const uint4*>(row + k);
    f.u[0] = q[0];
    f.u[1] = q[1];
  }
  __device__ __forceinline__ void load16(const bf16* row, int k, const uint8_t* srow) {
    load(row, k, srow, true);
  }
  __device__ __forceinline__ void mask(bool v, bool) {
    f.u[0] = keep4(f.u[0], v);
    f.u[1] = keep4(f.u[1], v);
  }
  __device__ __forceinline__ W16 widen(int) const { return f; }
};
template <> struct WRaw<int8_t> {
  uint4 q[2];
  __device__ __forceinline__ void load(const int8_t* row, int k, const uint8_t*, bool) {
    const uint4* p = reinterpret_cast<const uint4*>(row + k);
    q[0] = p[0];
    q[1] = p[1];
  }
  __device__ __forceinline__ void load16(const int8_t* row, int k, const uint8_t*) {
    q[0] = *reinterpret_cast<const uint4*>(row + k);
  }
  __device__ __forceinline__ void mask(bool v, bool) {
    q[0] = keep4(q[0], v);
    q[1] = keep4(q[1], v);
  }
  __device__ __forceinline__ W16 widen(int u) const {
    W16 f;
    int8x4_to_bf16(q[u].x, f.u[0].x, f.u[0].y);
    int8x4_to_bf16(q[u].y, f.u[0].z, f.u[0].w);
    int8x4_to_bf16(q[u].z, f.u[1].x, f.u[1].y);
    int8x4_to_bf16(q[u].w, f.u[1].z, f.u[1].w);
    return f;
  }
};
template <> struct WRaw<fp8e4m3> {
  uint4 q[2];
  __device__ __forceinline__ void load(const fp8e4m3* row, int k, const uint8_t*, bool) {
    const uint4* p = reinterpret_cast<const uint4*>(row + k);
    q[0] = p[0];
    q[1] = p[1];
  }
  __device__ __forceinline__ void load16(const fp8e4m3* row, int k, const uint8_t*) {
    q[0] = *reinterpret_cast<const uint4*>(row + k);
  }
  __device__ __forceinline__ void mask(bool v, bool) {
    q[0] = keep4(q[0], v);
    q[1] = keep4(q[1], v);
  }
  __device__ __forceinline__ W16 widen(int u) const {
    W16 f;
    fp8x4_to_bf16(q[u].x, f.u[0].x, f.u[0].y);
    fp8x4_to_bf16(q[u].y, f.u[0].z, f.u[0].w);
    fp8x4_to_bf16(q[u].z, f.u[1].x, f.u[1].y);
    fp8x4_to_bf16(q[u].w, f.u[1].z, f.u[1].w);
    return f;
  }
};
template <> struct WRaw<fp4x2> {
  uint4 q[2];
  float scale[2];  // of weights [0, 32) and [32, 64) of the span
  __device__ __forceinline__ void load(const fp4x2* row, int k, const uint8_t* srow, bool full) {
    const uint4* p = reinterpret_cast<const uint4*>(row + k / 2);
    const int h = full ? 1 : 0;  // the second half re-reads the first when past the end
    q[0] = p[0];
    q[1] = p[h];
    scale[0] = e8m0_to_f32(srow[k / 32]);
    scale[1] = e8m0_to_f32(srow[k / 32 + h]);
  }
  __device__ __forceinline__ void mask(bool v, bool full) {
    q[0] = keep4(q[0], v);
    q[1] = keep4(q[1], v && full);
  }
  __device__ __forceinline__ void load16(const fp4x2* row, int k, const uint8_t* srow) {
    const uint2 w = *reinterpret_cast<const uint2*>(row + k / 2);
    q[0] = make_uint4(w.x, w.y, 0, 0);
    scale[0] = e8m0_to_f32(srow[k / 32]);
  }
  __device__ __forceinline__ W16 widen(int u) const {
    const uint4& w = q[u / 2];
    const uint32_t lo = (u & 1) ? w.z : w.x, hi = (u & 1) ? w.w : w.y;
    W16 f;
    uint32_t o[4];
    fp4x8_to_bf16(lo, scale[u / 2], o);
    f.u[0] = make_uint4(o[0], o[1], o[2], o[3]);
    fp4x8_to_bf16(hi, scale[u / 2], o);
    f.u[1] = make_uint4(o[0], o[1], o[2], o[3]);
    return f;
  }
};

// First stored unit of the weight row that starts at element `elem`.
template <typename WQ>
__device__ __forceinline__ const WQ* wrow(const WQ* base, long long elem) {
  return base + elem / WFmt<WQ>::kPerUnit;
}

}  // namespace moe
