// Experts on the 8-bit / 4-bit matrix cores: the E4M3 and MXFP4 expert
// weights of the low-precision options on the page "Porting a 128-expert MoE
// (Gemma-4 26B-A4B) to AWS Inferentia2" (section "The fp4 rabbit hole (two of
// them, both dead ends)"), multiplied in their own formats by gfx950's scaled
// matrix instructions (v_mfma_scale_f32_*_f8f6f4), with no widening of the
// weight stream.  The activations enter those products as MXFP8: E4M3
// elements with one E8M0 scale per 32 consecutive values along the
// contraction, the block structure of the MXFP4 weights (the OCP
// Microscaling format); the expert input x is quantized so before gate_up
// (a kernel of its own), the gated product h in gate_up's epilogue, from its
// fp32 value.
//
// Operand layout of v_mfma_scale_f32_16x16x128_f8f6f4 (checked on the part
// against a host model): lane l holds row (or column) l % 16 and lane group
// g = l / 16; an 8-bit operand's 32 bytes are k = 16g .. 16g + 15 followed
// by k = 64 + 16g .. 64 + 16g + 15; a 4-bit operand's 16 bytes are k = 32g
// .. 32g + 31, the even k in the low nibble; the lane's scale byte (byte 0
// of its scale operand) covers k = 32g .. 32g + 31 of its row, whatever the
// data layout.  For the 32x32x64 form: row l % 32, group g = l / 32, an
// 8-bit operand's bytes k = 16g .. 16g + 15 then 32 + 16g .. 32 + 16g + 15,
// a 4-bit operand's k = 32g .. 32g + 31.
#include <initializer_list>
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "wformat.h"

namespace moe {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// Operand format codes of the scaled matrix instructions.
constexpr int kOpFp8 = 0, kOpFp4 = 4;
constexpr uint32_t kUnitScale = 127;  // E8M0 code of 1.0

// ---------------------------------------------------------------------------
// MXFP8 quantization of bf16 rows (cols % 32 == 0): one thread per 32-value
// block.  shared = floor(log2 max |v|) - 8 (E4M3's largest exponent),
// clamped to [-127, 127]; element = e4m3_encode(v / 2^shared), exact
// scaling; a block of zeros gets scale code 0 and zero codes.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mx8_quantize_kernel(long long nblocks, int cols,
                                                           const bf16* __restrict__ in,
                                                           uint8_t* __restrict__ q,
                                                           uint8_t* __restrict__ e8) {
  const long long b = (long long)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  const int nb = cols / 32;
  const long long r = b / nb, c0 = (b % nb) * 32;
  const uint4* src = reinterpret_cast<const uint4*>(in + r * cols + c0);
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
  uint32_t code8 = 0, out[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (amax > 0.0f) {
    int ex;
    (void)frexpf(amax, &ex);  // floor(log2 amax) = ex - 1, exactly
    const int shared = min(max(ex - 1 - 8, -127), 127);
    code8 = (uint32_t)(shared + 127);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t bits = (i & 1) ? (p[i / 2] & 0xffff0000u) : (p[i / 2] << 16);
      out[i / 4] |= e4m3_encode(ldexpf(__uint_as_float(bits), -shared)) << (8 * (i % 4));
    }
  }
  uint4* dst = reinterpret_cast<uint4*>(q + r * cols + c0);
  dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
  dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
  e8[b] = (uint8_t)code8;
}

// MXFP8 codes back to fp32 values: e4m3(code) * 2^(e8 - 127), exact (the
// product of an E4M3 value and a power of two down to 2^-136 is an fp32
// number).  One thread per 32-value block.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t ex = (c >> 3) & 15u, m = c & 7u;
  float v = ex == 0 ? (float)m * 0.001953125f  // m / 8 * 2^-6
                    : __uint_as_float(((ex + 120u) << 23) | (m << 20));
  return (c & 0x80u) ? -v : v;
}

__global__ __launch_bounds__(256) void mx8_dequantize_kernel(long long nblocks, int cols,
                                                             const uint8_t* __restrict__ q,
                                                             const uint8_t* __restrict__ e8,
                                                             float* __restrict__ out) {
  const long long b = (long long)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  const int nb = cols / 32;
  const long long r = b / nb, c0 = (b % nb) * 32;
  const float sc = e8m0_to_f32(e8[b]);
  const uint8_t* src = q + r * cols + c0;
  float* dst = out + r * cols + c0;
#pragma unroll
  for (int i = 0; i < 32; ++i) dst[i] = e4m3_value(src[i]) * sc;
}

// One lane's operand of a 128-k block as loaded.  o0 / o1: byte offsets
// (within the row) of its two 16-byte halves (8-bit formats) or of its one
// half (4-bit), already clamped into the row.
template <int OP>
__device__ __forceinline__ i32x8 ld_op(const uint8_t* row, int o0, int o1) {
  const uint4 a = *reinterpret_cast<const uint4*>(row + o0);
  uint4 b = make_uint4(0, 0, 0, 0);
  if constexpr (OP == kOpFp8) b = *reinterpret_cast<const uint4*>(row + o1);
  return i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

// Zeroes the halves of an operand that lie past the contraction (v0 / v1:
// whether each half lies inside it).  Applied where the operand is used, in
// the k-blocks that reach past the end only, so that no load is waited for
// before its k-block's matrix instructions.
__device__ __forceinline__ i32x8 keep_op(i32x8 v, bool v0, bool v1) {
  return i32x8{v0 ? v[0] : 0, v0 ? v[1] : 0, v0 ? v[2] : 0, v0 ? v[3] : 0,
               v1 ? v[4] : 0, v1 ? v[5] : 0, v1 ? v[6] : 0, v1 ? v[7] : 0};
}

// Byte offsets and validity of lane group g's share of 128-k block kb of a
// row of Kd values (8-bit operands: two 16-byte halves; 4-bit: one).
template <int OP>
__device__ __forceinline__ void op_span(int kb, int g, int Kd, int& o0, int& o1, bool& v0,
                                        bool& v1) {
  const int k0 = kb * 128;
  if constexpr (OP == kOpFp8) {
    const int a = k0 + 16 * g, b = k0 + 64 + 16 * g;
    v0 = a + 16 <= Kd;
    v1 = b + 16 <= Kd;
    o0 = v0 ? a : 0;
    o1 = v1 ? b : 0;
  } else {
    const int a = k0 + 32 * g;  // values
    v0 = a + 32 <= Kd;
    v1 = false;
    o0 = v0 ? a / 2 : 0;
    o1 = 0;
  }
}

__device__ __forceinline__ f32x4 mfma_mx(i32x8 a, uint32_t sa, i32x8 b, uint32_t sb, f32x4 c,
                                         std::integral_constant<int, kOpFp8>) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, kOpFp8, kOpFp8, 0, (int)sa, 0,
                                                          (int)sb);
}
__device__ __forceinline__ f32x4 mfma_mx(i32x8 a, uint32_t sa, i32x8 b, uint32_t sb, f32x4 c,
                                         std::integral_constant<int, kOpFp4>) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, kOpFp8, kOpFp4, 0, (int)sa, 0,
                                                          (int)sb);
}

// Weight formats of this path: E4M3 codes with an fp32 scale per output row
// (the scaled instruction gets a unit scale, the row scale multiplies the
// k-sum), or MXFP4 codes with their E8M0 block scales.
template <int OP> struct MxWeights {
  static constexpr int kPerByte = OP == kOpFp4 ? 2 : 1;
  static constexpr bool kChannelScale = OP == kOpFp8;
};

// Scale staging of the decode kernels (MXFP4 weights, SU > 0): the E8M0
// scale rows of a block's weight rows go to LDS once, in SU-byte pieces (SU
// divides the row length and every row's offset), up to kStgPieces pieces
// per thread, all loaded before the ring's first operand loads.  The k-loop
// then loads the weight codes alone; their scale bytes come from LDS.
// Loaded in the k-loop, one byte per lane, the weight scales were as many
// loads as the weight codes.
constexpr int kStgPieces = 8;
template <int SU>
using StgPiece = typename std::conditional<SU == 8, uint2, unsigned short>::type;

// ---------------------------------------------------------------------------
// Decode sizes: the weights streamed once per 16 * MB-row tile of an expert.
// gate_up: one block = one row tile x NC groups of 16 gate + 16 up columns;
// WK waves split the contraction H in 128-k blocks.  Each lane loads its
// weight spans straight into registers, NS - 1 k-blocks ahead of the
// matrix instructions.  Loads are unconditional (addresses clamped into
// their rows) and issued in ring order, and the spans past the contraction
// are zeroed where they are used, in the tail k-blocks only, so that each
// step waits for its own slot alone (a condition around a load, or a value
// masked right after it, made the compiler drain the whole ring there).
// ---------------------------------------------------------------------------
template <int OP, int WK, int MB, int NS, int NC, int SU>
__global__ __launch_bounds__(64 * WK) void gate_up_mx_kernel(
    int H, int N, int E, int K, int rows, const uint8_t* __restrict__ xq,
    const uint8_t* __restrict__ xs, const uint8_t* __restrict__ wg,
    const uint8_t* __restrict__ wu, long long w_stride, const void* __restrict__ sg,
    const void* __restrict__ su, long long s_stride, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_slots, uint8_t* __restrict__ hq,
    uint8_t* __restrict__ hs) {
  typedef MxWeights<OP> W;
  static_assert(NS >= 2, "the load ring needs two slots or more");
  static_assert(NC % 2 == 0, "a 32-column MXFP8 block of h spans two column groups");
  static_assert(SU == 0 || (OP == kOpFp4 && (SU == 2 || SU == 8)), "scale staging: MXFP4 only");
  __shared__ f32x4 red[WK][MB][NC][2][kWave];
  // staged weight scale rows: gate rows 16 c + r, up rows 16 NC + 16 c + r,
  // nsb bytes each
  extern __shared__ __align__(16) uint8_t sst[];
  int e, row0, row1, cg;
  const int CG = (N + 16 * NC - 1) / (16 * NC);
  if (!stream_item(false, rows, offsets, E, 16 * MB, CG, e, row0, row1, cg)) return;
  const int lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int fr = lane % 16, g = lane / 16;
  const int n0 = cg * 16 * NC + fr;  // column of group c: n0 + 16 c
  const int rowb = H / W::kPerByte, nsb = H / 32;  // bytes and scale bytes per weight row
  const uint8_t* grow[NC];
  const uint8_t* urow[NC];
  const uint8_t* gsc[NC];
  const uint8_t* usc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const long long n = min(n0 + 16 * c, N - 1);
    grow[c] = wg + (e * w_stride + n * H) / W::kPerByte;
    urow[c] = wu + (e * w_stride + n * H) / W::kPerByte;
    gsc[c] = usc[c] = nullptr;
    if constexpr (!W::kChannelScale) {
      gsc[c] = static_cast<const uint8_t*>(sg) + e * s_stride + n * nsb;
      usc[c] = static_cast<const uint8_t*>(su) + e * s_stride + n * nsb;
    }
  }
  const int nmb = (row1 - row0 + 15) / 16;
  const uint8_t* arow[MB];
  const uint8_t* asc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int r = row0 + 16 * mb + fr, rr = r < row1 ? r : row0;
    const long long tok = sorted_slots[rr] / K;
    arow[mb] = xq + tok * H;
    asc[mb] = xs + tok * nsb;
  }
  (void)rowb;
  const int KB = (H + 127) / 128;
  // The waves split the contraction in whole 128-byte lines of the weight
  // rows: an MXFP4 line holds two 128-weight blocks, and a line split between
  // two waves was read from HBM twice (gate_up read 1.11x its bytes).
  constexpr int KL = OP == kOpFp4 ? 2 : 1;  // k-blocks per line
  const int KBL = (KB + KL - 1) / KL;
  const int kb0 = min(KL * (wave * KBL / WK), KB), kb1 = min(KL * ((wave + 1) * KBL / WK), KB);

  constexpr int NRW = 32 * NC;  // staged rows: 16 NC gate rows, then 16 NC up rows
  StgPiece<SU == 0 ? 2 : SU> stv[SU > 0 ? kStgPieces : 1];
  const int ppr = SU > 0 ? nsb / (SU > 0 ? SU : 1) : 1, npc = NRW * ppr;
  if constexpr (SU > 0) {
    // every piece is loaded and later stored unconditionally (the index
    // clamped; surplus threads repeat the last piece), so that no wait lands
    // before the ring's loads
#pragma unroll
    for (int i = 0; i < kStgPieces; ++i) {
      const int j = min((int)threadIdx.x + i * 64 * WK, npc - 1), r = j / ppr;
      const bool up = r >= 16 * NC;
      const long long n = min(cg * 16 * NC + (up ? r - 16 * NC : r), N - 1);
      const uint8_t* src = static_cast<const uint8_t*>(up ? su : sg) + e * s_stride + n * nsb;
      stv[i] = *reinterpret_cast<const StgPiece<SU>*>(src + (j - r * ppr) * SU);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  f32x4 accg[MB][NC], accu[MB][NC];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int c = 0; c < NC; ++c) accg[mb][c] = accu[mb][c] = f32x4{0, 0, 0, 0};
  i32x8 ra[NS][MB], rg[NS][NC], ru[NS][NC];
  uint32_t sa[NS][MB], sgw[NS][NC], suw[NS][NC];
  int kbs[NS];  // the k-block each ring slot holds
  auto load_w = [&](int kb, int slot) {
    int o0, o1;
    bool v0, v1;
    kbs[slot] = kb;
    op_span<kOpFp8>(kb, g, H, o0, o1, v0, v1);
    const int sb = min(kb * 4 + g, nsb - 1);  // natural 32-block of this lane
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      ra[slot][mb] = ld_op<kOpFp8>(arow[mb], o0, o1);
      sa[slot][mb] = asc[mb][sb];
    }
    op_span<OP>(kb, g, H, o0, o1, v0, v1);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      rg[slot][c] = ld_op<OP>(grow[c], o0, o1);
      ru[slot][c] = ld_op<OP>(urow[c], o0, o1);
    }
  };
  // the weight scales (from LDS when staged)
  auto load_s = [&](int kb, int slot) {
    const int sb = min(kb * 4 + g, nsb - 1);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if constexpr (W::kChannelScale) {
        sgw[slot][c] = suw[slot][c] = kUnitScale;
      } else if constexpr (SU > 0) {
        sgw[slot][c] = sst[(16 * c + fr) * nsb + sb];
        suw[slot][c] = sst[(16 * NC + 16 * c + fr) * nsb + sb];
      } else {
        sgw[slot][c] = gsc[c][sb];
        suw[slot][c] = usc[c][sb];
      }
    }
  };
  auto load = [&](int kb, int slot) {
    load_w(kb, slot);
    load_s(kb, slot);
  };
  // CHECKED: the slot's k-block may reach past H (only in the tail loop).
  auto step = [&](int slot, auto checked) {
    if (decltype(checked)::value && (kbs[slot] + 1) * 128 > H) {  // uniform
      int o0, o1;
      bool v0, v1;
      op_span<kOpFp8>(kbs[slot], g, H, o0, o1, v0, v1);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) ra[slot][mb] = keep_op(ra[slot][mb], v0, v1);
      op_span<OP>(kbs[slot], g, H, o0, o1, v0, v1);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        rg[slot][c] = keep_op(rg[slot][c], v0, v1);
        ru[slot][c] = keep_op(ru[slot][c], v0, v1);
      }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        if (mb == 0 || mb < nmb) {
          accg[mb][c] = mfma_mx(ra[slot][mb], sa[slot][mb], rg[slot][c], sgw[slot][c],
                                accg[mb][c], std::integral_constant<int, OP>{});
          accu[mb][c] = mfma_mx(ra[slot][mb], sa[slot][mb], ru[slot][c], suw[slot][c],
                                accu[mb][c], std::integral_constant<int, OP>{});
        }
  };
  // The ring's first NS - 1 slots, loaded unconditionally: a wave with
  // fewer k-blocks loads a valid one again and never uses it.  (Loads under
  // a condition make the waits after them count as if none had been issued.)
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) {
    const int kbp = max(min(kb0 + s, kb1 - 1), 0);
    if constexpr (SU > 0) load_w(kbp, s);
    else load(kbp, s);
    __builtin_amdgcn_sched_barrier(0);  // slots issued in order
  }
  if constexpr (SU > 0) {
#pragma unroll
    for (int i = 0; i < kStgPieces; ++i) {
      const int j = min((int)threadIdx.x + i * 64 * WK, npc - 1), r = j / ppr;
      *reinterpret_cast<StgPiece<SU>*>(sst + r * nsb + (j - r * ppr) * SU) = stv[i];
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) load_s(max(min(kb0 + s, kb1 - 1), 0), s);
  }
  int kb = kb0;
  // steady state: every load of the unrolled NS steps lies inside the range,
  // and every k-block it loads lies wholly inside H, so no operand is masked
  // and each step waits only for its own slot
  const int kbf = min(kb1, H / 128);
  for (; kb + 2 * NS - 2 < kbf; kb += NS) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      load(kb + s + NS - 1, (s + NS - 1) % NS);
      __builtin_amdgcn_sched_barrier(0);
      step(s, std::false_type{});
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  for (; kb < kb1; kb += NS) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (kb + s >= kb1) break;
      if (kb + s + NS - 1 < kb1) load(kb + s + NS - 1, (s + NS - 1) % NS);
      step(s, std::true_type{});
    }
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      red[wave][mb][c][0][lane] = accg[mb][c];
      red[wave][mb][c][1][lane] = accu[mb][c];
    }
  __syncthreads();
  if (wave != 0) return;
  // h = GELU(gate) * up in fp32, then MXFP8 per 32 columns straight from
  // fp32: column groups 2j and 2j + 1 form one 32-column block; its maximum
  // over the 16 lanes of a lane group (one row each) comes from xor shuffles.
  const int nsh = N / 32;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    if (mb >= nmb) break;
#pragma unroll
    for (int c2 = 0; c2 < NC; c2 += 2) {
      f32x4 hv[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = c2 + j, n = n0 + 16 * c;
        f32x4 gv = red[0][mb][c][0][lane], uv = red[0][mb][c][1][lane];
#pragma unroll
        for (int w = 1; w < WK; ++w) {
          gv += red[w][mb][c][0][lane];
          uv += red[w][mb][c][1][lane];
        }
        if constexpr (W::kChannelScale) {
          const int nn = min(n, N - 1);
          gv *= static_cast<const float*>(sg)[(size_t)e * s_stride + nn];
          uv *= static_cast<const float*>(su)[(size_t)e * s_stride + nn];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) hv[j][r] = gelu_tanh(gv[r]) * uv[r];
      }
      const int blk0 = n0 - fr + 16 * c2;  // first column of the 32-column block
      if (blk0 >= N) break;                // uniform: the block lies past the last column
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float m = fmaxf(fabsf(hv[0][r]), fabsf(hv[1][r]));
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
        uint32_t code8 = 0, q0 = 0, q1 = 0;
        if (m > 0.0f) {
          int ex;
          (void)frexpf(m, &ex);
          const int shared = min(max(ex - 1 - 8, -127), 127);
          code8 = (uint32_t)(shared + 127);
          q0 = e4m3_encode(ldexpf(hv[0][r], -shared));
          q1 = e4m3_encode(ldexpf(hv[1][r], -shared));
        }
        const int row = row0 + 16 * mb + 4 * g + r;
        if (row < row1) {
          uint8_t* dst = hq + (size_t)row * N + blk0 + fr;
          dst[0] = (uint8_t)q0;
          dst[16] = (uint8_t)q1;
          if (fr == 0) hs[(size_t)row * nsh + blk0 / 32] = (uint8_t)code8;
        }
      }
    }
  }
}

// down: one block = one row tile x WN waves of NC groups of 16 output
// columns (the contraction, the expert width, is short and is not split).
// A = the tile's rows of h in MXFP8 (expert-sorted order).
// Activation staging of the decode down kernel (AL): the tile's rows of h
// (MXFP8 codes, row pitch N + 16 bytes, and their E8M0 scales) go to LDS once
// per block, in up to kAlCodePieces 16-byte and kAlScalePieces 2-byte pieces
// per thread; the block's waves, which take different output columns, then
// read their A operands from LDS instead of each loading them.
constexpr int kAlCodePieces = 4, kAlScalePieces = 1;

template <int OP, int WN, int MB, int NS, int NC, int SU, bool AL, typename YT>
__global__ __launch_bounds__(64 * WN) void down_mx_kernel(
    int H, int N, int E, int rows, const uint8_t* __restrict__ hq, const uint8_t* __restrict__ hs,
    const uint8_t* __restrict__ wd, long long w_stride, const void* __restrict__ sd,
    long long s_stride, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_slots, const float* __restrict__ topk_w,
    YT* __restrict__ y) {
  typedef MxWeights<OP> W;
  static_assert(NS >= 2, "the load ring needs two slots or more");
  static_assert(SU == 0 || (OP == kOpFp4 && (SU == 2 || SU == 8)), "scale staging: MXFP4 only");
  // staged weight scale rows: row 16 NC w + 16 c + r is wave w's column
  // group c, lane row r; nsb bytes each
  extern __shared__ __align__(16) uint8_t sst[];
  int e, row0, row1, cg;
  const int CG = (H + 16 * WN * NC - 1) / (16 * WN * NC);
  if (!stream_item(false, rows, offsets, E, 16 * MB, CG, e, row0, row1, cg)) return;
  const int lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int fr = lane % 16, g = lane / 16;
  const int n0 = (cg * WN + wave) * 16 * NC + fr;  // output column of group c: n0 + 16 c
  const int nsb = N / 32;
  const uint8_t* brow[NC];
  const uint8_t* bsc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const long long n = min(n0 + 16 * c, H - 1);
    brow[c] = wd + (e * w_stride + n * N) / W::kPerByte;
    bsc[c] = nullptr;
    if constexpr (!W::kChannelScale)
      bsc[c] = static_cast<const uint8_t*>(sd) + e * s_stride + n * nsb;
  }
  const int nmb = (row1 - row0 + 15) / 16;
  // Output slot and routing weight of this lane's rows (rows past the tile
  // clamp to its last row): the slots loaded first, the weights before the
  // k-loop, so that neither waits at the end.  In the epilogue each store
  // had waited for its slot and then its weight, re-loaded for every column
  // group.
  int oslot[MB][4];
  float ow[MB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) oslot[mb][r] = sorted_slots[min(row0 + 16 * mb + 4 * g + r, row1 - 1)];
  const uint8_t* arow[MB];
  const uint8_t* asc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int r = row0 + 16 * mb + fr, rr = r < row1 ? r : row0;
    arow[mb] = hq + (long long)rr * N;
    asc[mb] = hs + (long long)rr * nsb;
  }
  const int KB = (N + 127) / 128;
  constexpr int NRW = 16 * WN * NC;  // staged rows
  StgPiece<SU == 0 ? 2 : SU> stv[SU > 0 ? kStgPieces : 1];
  const int ppr = SU > 0 ? nsb / (SU > 0 ? SU : 1) : 1, npc = NRW * ppr;
  if constexpr (SU > 0) {
    // unconditional loads and stores, as in gate_up
#pragma unroll
    for (int i = 0; i < kStgPieces; ++i) {
      const int j = min((int)threadIdx.x + i * 64 * WN, npc - 1), r = j / ppr;
      const long long n = min(cg * 16 * WN * NC + r, H - 1);
      const uint8_t* src = static_cast<const uint8_t*>(sd) + e * s_stride + n * nsb;
      stv[i] = *reinterpret_cast<const StgPiece<SU>*>(src + (j - r * ppr) * SU);
    }
  }
  // activation rows of the tile in LDS (AL): codes at alq (pitch N + 16),
  // scales at als (pitch nsb), after the weight-scale rows
  const int apitch = N + 16, arows = 16 * MB;
  uint8_t* alq = sst + (SU > 0 ? (NRW * nsb + 15) / 16 * 16 : 0);
  uint8_t* als = alq + arows * apitch;
  const int cpr = N / 16, spr = nsb / 2;  // code and scale pieces per row
  const int nrow = row1 - row0;
  uint4 acv[AL ? kAlCodePieces : 1];
  unsigned short asv[AL ? kAlScalePieces : 1];
  if constexpr (AL) {
    // unconditional: rows past the tile load its first row (never used)
#pragma unroll
    for (int i = 0; i < kAlCodePieces; ++i) {
      const int j = min((int)threadIdx.x + i * 64 * WN, arows * cpr - 1), r = j / cpr;
      acv[i] = *reinterpret_cast<const uint4*>(hq + (long long)(row0 + (r < nrow ? r : 0)) * N +
                                               (j - r * cpr) * 16);
    }
#pragma unroll
    for (int i = 0; i < kAlScalePieces; ++i) {
      const int j = min((int)threadIdx.x + i * 64 * WN, arows * spr - 1), r = j / spr;
      asv[i] = *reinterpret_cast<const unsigned short*>(
          hs + (long long)(row0 + (r < nrow ? r : 0)) * nsb + (j - r * spr) * 2);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  f32x4 acc[MB][NC];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[mb][c] = f32x4{0, 0, 0, 0};
  i32x8 ra[NS][MB], rb[NS][NC];
  uint32_t sa[NS][MB], sb[NS][NC];
  int kbs[NS];  // the k-block each ring slot holds
  // the weights, and the activations unless they are staged
  auto load_w = [&](int kb, int slot) {
    int o0, o1;
    bool v0, v1;
    kbs[slot] = kb;
    if constexpr (!AL) {
      op_span<kOpFp8>(kb, g, N, o0, o1, v0, v1);
      const int s8 = min(kb * 4 + g, nsb - 1);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        ra[slot][mb] = ld_op<kOpFp8>(arow[mb], o0, o1);
        sa[slot][mb] = asc[mb][s8];
      }
    }
    op_span<OP>(kb, g, N, o0, o1, v0, v1);
#pragma unroll
    for (int c = 0; c < NC; ++c) rb[slot][c] = ld_op<OP>(brow[c], o0, o1);
  };
  // the staged activations (AL), from LDS
  auto load_a = [&](int kb, int slot) {
    if constexpr (AL) {
      int o0, o1;
      bool v0, v1;
      op_span<kOpFp8>(kb, g, N, o0, o1, v0, v1);
      const int s8 = min(kb * 4 + g, nsb - 1);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const uint8_t* ar = alq + (16 * mb + fr) * apitch;
        const uint4 x0 = *reinterpret_cast<const uint4*>(ar + o0);
        const uint4 x1 = *reinterpret_cast<const uint4*>(ar + o1);
        ra[slot][mb] = i32x8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                             (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        sa[slot][mb] = als[(16 * mb + fr) * nsb + s8];
      }
    }
  };
  // the weight scales (from LDS when staged)
  auto load_s = [&](int kb, int slot) {
    const int s8 = min(kb * 4 + g, nsb - 1);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if constexpr (W::kChannelScale) sb[slot][c] = kUnitScale;
      else if constexpr (SU > 0) sb[slot][c] = sst[(16 * NC * wave + 16 * c + fr) * nsb + s8];
      else sb[slot][c] = bsc[c][s8];
    }
  };
  auto load = [&](int kb, int slot) {
    load_w(kb, slot);
    load_a(kb, slot);
    load_s(kb, slot);
  };
  // CHECKED: the slot's k-block may reach past N (only in the tail loop).
  auto step = [&](int slot, auto checked) {
    if (decltype(checked)::value && (kbs[slot] + 1) * 128 > N) {  // uniform
      int o0, o1;
      bool v0, v1;
      op_span<kOpFp8>(kbs[slot], g, N, o0, o1, v0, v1);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) ra[slot][mb] = keep_op(ra[slot][mb], v0, v1);
      op_span<OP>(kbs[slot], g, N, o0, o1, v0, v1);
#pragma unroll
      for (int c = 0; c < NC; ++c) rb[slot][c] = keep_op(rb[slot][c], v0, v1);
    }
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        if (mb == 0 || mb < nmb)
          acc[mb][c] = mfma_mx(ra[slot][mb], sa[slot][mb], rb[slot][c], sb[slot][c], acc[mb][c],
                               std::integral_constant<int, OP>{});
  };
  // the ring's first slots, unconditionally (as in gate_up); with staging,
  // their weight loads go out before the staged pieces are stored
  constexpr bool STAGED = SU > 0 || AL;
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) {
    if constexpr (STAGED) load_w(min(s, KB - 1), s);
    else load(min(s, KB - 1), s);
    __builtin_amdgcn_sched_barrier(0);  // slots issued in order
  }
  if constexpr (STAGED) {
    if constexpr (SU > 0) {
#pragma unroll
      for (int i = 0; i < kStgPieces; ++i) {
        const int j = min((int)threadIdx.x + i * 64 * WN, npc - 1), r = j / ppr;
        *reinterpret_cast<StgPiece<SU>*>(sst + r * nsb + (j - r * ppr) * SU) = stv[i];
      }
    }
    if constexpr (AL) {
#pragma unroll
      for (int i = 0; i < kAlCodePieces; ++i) {
        const int j = min((int)threadIdx.x + i * 64 * WN, arows * cpr - 1), r = j / cpr;
        *reinterpret_cast<uint4*>(alq + r * apitch + (j - r * cpr) * 16) = acv[i];
      }
#pragma unroll
      for (int i = 0; i < kAlScalePieces; ++i) {
        const int j = min((int)threadIdx.x + i * 64 * WN, arows * spr - 1), r = j / spr;
        *reinterpret_cast<unsigned short*>(als + r * nsb + (j - r * spr) * 2) = asv[i];
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) {
      load_a(min(s, KB - 1), s);
      load_s(min(s, KB - 1), s);
    }
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) ow[mb][r] = topk_w[oslot[mb][r]];
  int kb = 0;
  // steady state as in gate_up: k-blocks wholly inside N, nothing masked
  const int kbf = N / 128;
  for (; kb + 2 * NS - 2 < kbf; kb += NS) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      load(kb + s + NS - 1, (s + NS - 1) % NS);
      __builtin_amdgcn_sched_barrier(0);
      step(s, std::false_type{});
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  for (; kb < KB; kb += NS) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (kb + s >= KB) break;
      if (kb + s + NS - 1 < KB) load(kb + s + NS - 1, (s + NS - 1) % NS);
      step(s, std::true_type{});
    }
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int n = n0 + 16 * c;
    const bool nvalid = n < H;
    float chs = 1.0f;
    if constexpr (W::kChannelScale)
      if (nvalid) chs = static_cast<const float*>(sd)[(size_t)e * s_stride + n];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (mb >= nmb) break;
      const f32x4 v = acc[mb][c] * chs;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + 16 * mb + 4 * g + r;
        if (row >= row1 || !nvalid) continue;
        y[(size_t)oslot[mb][r] * H + n] = from_f32<YT>(ow[mb][r] * v[r]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Prefill sizes: grouped GEMM tiles of 256 rows x 256 output columns
// (gate_up: 128 gate + the matching 128 up columns), 64-long k-tiles, on
// v_mfma_scale_f32_32x32x64_f8f6f4.  8 waves (2 x 4), each a 128 x 64
// sub-tile.  Every k-tile of A (MXFP8 rows: 64 bytes) and B (weight rows: 64
// bytes in E4M3, 32 in MXFP4) goes global -> LDS directly (global_load_lds,
// 16 bytes per lane) into a ring of NSTAGE stages; a stage is refilled as
// soon as the barrier of the next k-tile has passed.  LDS lines are 64 bytes
// (an MXFP4 line holds two weight rows); chunk c of line L sits at position
// c ^ ((L >> 2) & 3).  The tile's E8M0 scales (A rows, and MXFP4 weight
// rows) are staged in LDS past the ring once per tile.  A wave reads the
// next k-tile's B fragments first, then, after the instructions that last use
// each A fragment, that fragment's successor, so only B is double-buffered.
// gate_up's epilogue stages h = GELU(gate) * up in fp32 in LDS and a thread
// per (row, 32-column block) writes its MXFP8 codes and scale; down's stages
// the rows and writes each slot's output times its routing weight.
// ---------------------------------------------------------------------------
constexpr int MXBM = 256, MXGN = 256, MXGK = 64;
constexpr int kMxDnStageRows = 128, kMxDnStride = MXGN + 4;  // floats
constexpr int kMxGuStride = MXGN / 2 + 4;                     // floats

template <int OPB>
struct MxTile {
  static constexpr int RB = OPB == kOpFp4 ? 32 : 64;  // bytes of a B row per k-tile
  static constexpr int ALINES = MXBM, BLINES = MXGN * RB / 64, LINES = ALINES + BLINES;
  static constexpr int SB = LINES * 64;               // stage bytes
};

__device__ __forceinline__ int mswz(int line, int c) { return c ^ ((line >> 2) & 3); }

template <bool GU, int OPB, int NSTAGE>
struct MxLds {
  typedef MxTile<OPB> T;
  static constexpr int ring = NSTAGE * T::SB;
  // scale bytes: A rows then (MXFP4) B rows, nsb per row; placed past the ring
  static constexpr int scales(int nsb) { return (OPB == kOpFp4 ? 2 : 1) * 256 * nsb; }
  static constexpr int stage_out = GU ? MXBM * kMxGuStride * 4 : kMxDnStageRows * kMxDnStride * 4;
  static constexpr int slots(int nsb) {
    return ring + scales(nsb) > stage_out ? ring + scales(nsb) : stage_out;
  }
  // the tile's A row indices (gathered token or sorted row) past everything
  static constexpr int tok(int nsb) { return slots(nsb) + (GU ? 0 : MXBM * 8); }
  static constexpr int total(int nsb) { return tok(nsb) + MXBM * 4; }
};

template <bool GU, int OPB, int NSTAGE, typename YT>
__global__ __launch_bounds__(512, 1) void grouped_mx_kernel(
    int Kd, int Nout, int E, int K, int rows, int NT, const uint8_t* __restrict__ A,
    const uint8_t* __restrict__ As, const uint8_t* __restrict__ W0,
    const uint8_t* __restrict__ W1, long long w_stride, const void* __restrict__ S0,
    const void* __restrict__ S1, long long s_stride, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_slots, const float* __restrict__ topk_w,
    uint8_t* __restrict__ hq, uint8_t* __restrict__ hs, YT* __restrict__ yout) {
  typedef MxTile<OPB> TL;
  typedef MxLds<GU, OPB, NSTAGE> LD;
  typedef MxWeights<OPB> W;
  constexpr int WM = 2, WN = 4, NW = WM * WN;
  constexpr int WR = MXBM / WM, WC = MXGN / WN, TM = WR / 32, TN = WC / 32;
  constexpr int LPW = TL::LINES / 16 / NW;
  static_assert(LPW * NW * 16 == TL::LINES, "copies cover a stage");
  static_assert(!GU || TN == 2, "a gate_up wave takes one gate and one up sub-tile");
  extern __shared__ __align__(16) unsigned char smem[];
  const int nsb = Kd / 32;

  int e = 0, row0, row1, nt;
  {
    RowTileScan sc;
    row_tile_scan(offsets, E, MXBM, sc);
    const int item = xcd_item(blockIdx.x, sc.total * NT);
    if (item < 0) return;  // uniform over the block
    weight_major_item(sc, offsets, MXBM, item, NT, e, row0, row1, nt);
  }
  const int lane = lane_id(), wave = threadIdx.x / kWave, tid = threadIdx.x;
  const int wm = wave / WN, wn = wave % WN;
  const int nbase = GU ? nt * (MXGN / 2) : nt * MXGN;
  uint8_t* sA = smem + LD::ring;
  uint8_t* sBs = sA + 256 * nsb;
  int* row_slot = reinterpret_cast<int*>(smem + LD::slots(nsb));
  float* row_w = reinterpret_cast<float*>(row_slot + MXBM);
  int* rtok = reinterpret_cast<int*>(smem + LD::tok(nsb));
  // A row r of the tile (rows past the tile re-read row0: outputs dropped)
  if (tid < MXBM) {
    int gr = row0 + tid;
    if (gr >= row1) gr = row0;
    rtok[tid] = GU ? sorted_slots[gr] / K : gr;
  }
  // B row n of the tile: its column in the weight matrix (its row there), the
  // gate or up half for gate_up; byte offsets within the expert's weights
  const uint8_t* wbase = W0 + e * w_stride / W::kPerByte;
  const uint8_t* sbase0 = nullptr;
  if constexpr (!W::kChannelScale) sbase0 = static_cast<const uint8_t*>(S0) + e * s_stride;
  const long long up_off = GU ? (long long)(W1 - W0) : 0;  // bytes from gate to up rows
  const long long sup_off =
      GU && !W::kChannelScale ? static_cast<const uint8_t*>(S1) - static_cast<const uint8_t*>(S0)
                              : 0;
  auto bcol = [&](int n, bool& up) {
    up = GU && n >= MXGN / 2;
    int col = nbase + n - (up ? MXGN / 2 : 0);
    return col < Nout ? col : 0;  // past the last column: a valid row, output dropped
  };
  auto boffs = [&](int n) -> unsigned {
    bool up;
    const int col = bcol(n, up);
    return (unsigned)((up ? up_off : 0) + (long long)col * Kd / W::kPerByte);
  };
  __syncthreads();

  // the tile's scale rows into LDS, two bytes at a time (nsb is even), in
  // batches of 8 loads per thread
  {
    const int h2 = nsb / 2, tot = MXBM * h2;
    constexpr int BT = 8;
    for (int i0 = tid; i0 < tot; i0 += 512 * BT) {
      uint16_t va[BT], vb[BT];
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        const int i = i0 + 512 * b;
        const int r = i < tot ? i / h2 : 0, c = i < tot ? i % h2 : 0;
        va[b] = reinterpret_cast<const uint16_t*>(As + (long long)rtok[r] * nsb)[c];
        vb[b] = 0;
        if constexpr (!W::kChannelScale) {
          bool up;
          const int col = bcol(r, up);
          vb[b] = reinterpret_cast<const uint16_t*>(sbase0 + (up ? sup_off : 0) +
                                                     (long long)col * nsb)[c];
        }
      }
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        const int i = i0 + 512 * b;
        if (i < tot) {
          reinterpret_cast<uint16_t*>(sA)[i] = va[b];
          if constexpr (!W::kChannelScale) reinterpret_cast<uint16_t*>(sBs)[i] = vb[b];
        }
      }
    }
  }
  if constexpr (!GU) {
    if (tid < MXBM) {
      const int row = row0 + tid;
      int slot = 0;
      float w = 0.0f;
      if (row < row1) {
        slot = sorted_slots[row];
        w = topk_w[slot];
      }
      row_slot[tid] = slot;
      row_w[tid] = w;
    }
  }

  // copy j of this lane: LDS line 16 q + lane / 4 of a stage, position lane % 4
  // Copy j of wave w fills lines 16 q .. 16 q + 15 with q = j * NW + w, so
  // that copy j is of A lines for every wave or of B lines for every wave
  // (the A lines are a multiple of 16 * NW).
  static_assert(TL::ALINES % (16 * NW) == 0, "copy j is of one kind in every wave");
  constexpr int JA = TL::ALINES / (16 * NW);  // copies j < JA are of A lines
  // byte offsets of this lane's copy sources: from A (32 bits: A has at most
  // 2^32 bytes) or from the expert's weights (wbase)
  unsigned src[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int q = j * NW + wave;
    const int line = 16 * q + lane / 4;
    const int lc = mswz(line, lane % 4);  // logical chunk this lane fetches
    if (j < JA) {
      src[j] = (unsigned)rtok[line] * (unsigned)Kd + lc * 16;
    } else {
      const int bl = line - TL::ALINES;
      if constexpr (OPB == kOpFp4) src[j] = boffs(2 * bl + (lc >> 1)) + (lc & 1) * 16;
      else src[j] = boffs(bl) + lc * 16;
    }
  }
  const int nk = Kd / MXGK;
  auto copy = [&](int kt, int j) {
    const int ktc = kt < nk ? kt : nk - 1;  // past the end: the last tile again
    const int q = j * NW + wave;
    const int kstep = j < JA || OPB != kOpFp4 ? MXGK : MXGK / 2;
    const uint8_t* base = j < JA ? A : wbase;
#if defined(__HIP_DEVICE_COMPILE__)
    lds_copy16(base + src[j] + (unsigned)(ktc * kstep), smem + (kt % NSTAGE) * TL::SB + q * 1024);
#endif
  };

  // fragment addresses within a stage
  const int fr = lane % 32, g = lane / 32;
  // An 8-bit operand's two chunks g and 2 + g sit 32 bytes apart after the
  // swizzle (the swizzle flips only the low two chunk bits): offset ^ 32.
  // Rows of the wave's sub-tiles: A (wm * WR + 32 i + fr), B as below; the
  // swizzle term (r >> 2) & 3 is the same for rows 32 apart.
  const int ar0 = wm * WR + fr;
  const int aoff = ar0 * 64 + mswz(ar0, g) * 16;  // + i * 32 * 64 for sub-tile i
  int boff[TN], browl[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    int n;
    if (GU) n = (j == 0 ? 0 : MXGN / 2) + wn * (WC / 2) + fr;
    else n = wn * WC + j * 32 + fr;
    browl[j] = n;
    if constexpr (OPB == kOpFp4) {
      const int line = TL::ALINES + n / 2;
      boff[j] = line * 64 + mswz(line, (n % 2) * 2 + g) * 16;
    } else {
      const int line = TL::ALINES + n;
      boff[j] = line * 64 + mswz(line, g) * 16;
    }
  }
  int nv;  // 32-row sub-tiles of this wave holding rows of the tile (uniform)
  {
    const int left = row1 - row0 - wm * WR;
    nv = left <= 0 ? 0 : min(TM, (left + 31) / 32);
    nv = __builtin_amdgcn_readfirstlane(nv);
  }

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
  i32x8 fa[TM], fb[2][TN];
  uint32_t sa[TM], sb[2][TN];
  auto ld16 = [&](const unsigned char* st, int off) {
    return *reinterpret_cast<const uint4*>(st + off);
  };
  auto rd_a = [&](const unsigned char* st, int kt, int i) {
    const int o = aoff + i * 32 * 64;
    const uint4 x = ld16(st, o), y = ld16(st, o ^ 32);
    fa[i] = i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
    sa[i] = sA[(ar0 + 32 * i) * nsb + 2 * kt + g];
  };
  auto rd_b = [&](const unsigned char* st, int kt, int j, int buf) {
    const uint4 x = ld16(st, boff[j]);
    uint4 y = make_uint4(0, 0, 0, 0);
    if constexpr (OPB == kOpFp8) y = ld16(st, boff[j] ^ 32);
    fb[buf][j] = i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w,
                       (int)y.x, (int)y.y, (int)y.z, (int)y.w};
    sb[buf][j] = W::kChannelScale ? kUnitScale : (uint32_t)sBs[browl[j] * nsb + 2 * kt + g];
  };
  auto mma = [&](int i, int j, int buf) {
    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
        fa[i], fb[buf][j], acc[i][j], kOpFp8, OPB, 0, (int)sa[i], 0, (int)sb[buf][j]);
  };

  {
#pragma unroll
    for (int st = 0; st < NSTAGE; ++st)
#pragma unroll
      for (int j = 0; j < LPW; ++j) copy(st, j);
    wait_vmem<(NSTAGE - 1) * LPW>();
    __syncthreads();  // tile 0 landed everywhere; the scale rows are in LDS
#pragma unroll
    for (int i = 0; i < TM; ++i) rd_a(smem, 0, i);
#pragma unroll
    for (int j = 0; j < TN; ++j) rd_b(smem, 0, j, 0);
    wait_lds();
    // iteration kt: B of tile kt in buffer `cur`
    auto iter = [&](int kt, auto cur_tag) {
      constexpr int cur = decltype(cur_tag)::value, nxt = 1 - cur;
      const bool more = __builtin_amdgcn_readfirstlane(kt + 1 < nk ? 1 : 0) != 0;
      wait_vmem<(NSTAGE - 2) * LPW>();   // tile kt+1 landed (this wave's copies)
      block_barrier();                   // ... everyone's; tile kt's slot is free
      __builtin_amdgcn_sched_barrier(0);
      const unsigned char* sn = smem + ((kt + 1) % NSTAGE) * TL::SB;
      if (more) {
#pragma unroll
        for (int j = 0; j < TN; ++j) rd_b(sn, kt + 1, j, nxt);
      }
#pragma unroll
      for (int j = 0; j < LPW; ++j) copy(kt + NSTAGE, j);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        if (i < nv) {  // uniform: sub-tiles past the group's rows skip their products
#pragma unroll
          for (int j = 0; j < TN; ++j) mma(i, j, cur);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (more) rd_a(sn, kt + 1, i);
        __builtin_amdgcn_sched_barrier(0);
      }
      wait_lds();
    };
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      iter(kt, std::integral_constant<int, 0>{});
      iter(kt + 1, std::integral_constant<int, 1>{});
    }
    if (kt < nk) iter(kt, std::integral_constant<int, 0>{});
    wait_vmem<0>();
  }

  __syncthreads();  // every wave is done with the ring and the scale rows
  if constexpr (GU) {
    // h = GELU(gate * s_g) * (up * s_u) in fp32, staged row-major in LDS
    float* stg = reinterpret_cast<float*>(smem);
    const int n = nbase + wn * (WC / 2) + fr;
    float cg = 1.0f, cu = 1.0f;
    if constexpr (W::kChannelScale) {
      const int nn = min(n, Nout - 1);
      cg = static_cast<const float*>(S0)[e * s_stride + nn];
      cu = static_cast<const float*>(S1)[e * s_stride + nn];
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if (i >= nv) break;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int r = wm * WR + i * 32 + 8 * (q / 4) + 4 * g + (q % 4);
        stg[r * kMxGuStride + wn * (WC / 2) + fr] =
            gelu_tanh(acc[i][0][q] * cg) * (acc[i][1][q] * cu);
      }
    }
    __syncthreads();
    // one thread per (row, 32-column block): 256 rows x 4 blocks
    const int nsh = Nout / 32;
#pragma unroll
    for (int it = 0; it < MXBM * 4 / 512; ++it) {
      const int k = tid + it * 512;
      const int r = k / 4, b = k % 4;
      const int col = nbase + 32 * b;
      if (row0 + r >= row1 || col >= Nout) continue;
      const float* v = stg + r * kMxGuStride + 32 * b;
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(v[i]));
      uint32_t code8 = 0, out[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (m > 0.0f) {
        int ex;
        (void)frexpf(m, &ex);
        const int shared = min(max(ex - 1 - 8, -127), 127);
        code8 = (uint32_t)(shared + 127);
#pragma unroll
        for (int i = 0; i < 32; ++i) out[i / 4] |= e4m3_encode(ldexpf(v[i], -shared)) << (8 * (i % 4));
      }
      uint4* dst = reinterpret_cast<uint4*>(hq + (size_t)(row0 + r) * Nout + col);
      dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
      dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
      hs[(size_t)(row0 + r) * nsh + col / 32] = (uint8_t)code8;
    }
  } else {
    float* stg = reinterpret_cast<float*>(smem);
    constexpr int CH = MXGN / 4;  // chunks of 4 fp32 per row
#pragma unroll
    for (int pass = 0; pass < MXBM / kMxDnStageRows; ++pass) {
      if (wm * WR / kMxDnStageRows == pass) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          if (i >= nv) break;
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
              const int r = wm * WR - pass * kMxDnStageRows + i * 32 + 8 * (q / 4) + 4 * g + (q % 4);
              stg[r * kMxDnStride + wn * WC + j * 32 + fr] = acc[i][j][q];
            }
        }
      }
      __syncthreads();
#pragma unroll
      for (int it = 0; it < kMxDnStageRows * CH / 512; ++it) {
        const int k = tid + it * 512;
        const int rl = k / CH, ch = k % CH;
        const int r = pass * kMxDnStageRows + rl;
        const int col = nbase + ch * 4;
        if (row0 + r < row1 && col < Nout) {
          float4 cs = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
          if constexpr (W::kChannelScale)
            cs = *reinterpret_cast<const float4*>(static_cast<const float*>(S0) +
                                                  e * s_stride + col);
          const float sc = row_w[r];
          const float4 v = *reinterpret_cast<const float4*>(stg + rl * kMxDnStride + ch * 4);
          YT* dst = yout + (size_t)row_slot[r] * Nout + col;
          const float o[4] = {sc * (v.x * cs.x), sc * (v.y * cs.y), sc * (v.z * cs.z),
                              sc * (v.w * cs.w)};
          if constexpr (std::is_same<YT, float>::value) {
            // streaming stores, as in the bf16 tiled down: read once, by the combine
            const f32x4 ov = {o[0], o[1], o[2], o[3]};
            __builtin_nontemporal_store(ov, reinterpret_cast<f32x4*>(dst));
          } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) dst[u] = from_f32<YT>(o[u]);
          }
        }
      }
      __syncthreads();
    }
  }
}

template <bool GU, int OPB, int NSTAGE, typename YT>
hipError_t launch_grouped_mx(int Kd, int Nout, const MxArgs& a, int NT, const uint8_t* A,
                             const uint8_t* As, const uint8_t* W0, const uint8_t* W1,
                             long long w_stride, const void* S0, const void* S1,
                             long long s_stride, hipStream_t s) {
  auto kf = grouped_mx_kernel<GU, OPB, NSTAGE, YT>;
  const int lds = MxLds<GU, OPB, NSTAGE>::total(Kd / 32);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  static int attr_set = 0;  // the largest size set so far
  if (lds > attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kf),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    attr_set = lds;
  }
  const int RT = tile_count_bound(false, a.rows, a.T, a.E, MXBM);
  hipLaunchKernelGGL(kf, dim3(RT * NT), dim3(512), lds, s, Kd, Nout, a.E, a.K, a.rows, NT, A, As,
                     W0, W1, w_stride, S0, S1, s_stride, a.offsets, a.sorted_slots, a.topk_w,
                     a.hq, a.hs, static_cast<YT*>(a.y));
  return hipGetLastError();
}

template <int OP>
hipError_t launch_mx_tiled(const MxArgs& a, hipStream_t s) {
  const long long I = a.I, H = a.H;
  const int pb = MxWeights<OP>::kPerByte;
  const uint8_t* gq = static_cast<const uint8_t*>(a.gate_up_q);
  const void* gs = a.gate_up_s;
  const void* us;
  long long gss, dss;
  if constexpr (OP == kOpFp8) {
    us = static_cast<const float*>(gs) + I;
    gss = 2 * I;
    dss = H;
  } else {
    us = static_cast<const uint8_t*>(gs) + I * (H / 32);
    gss = 2 * I * (H / 32);
    dss = H * (I / 32);
  }
  constexpr int NSG = OP == kOpFp4 ? 4 : 4;
  hipError_t e = launch_grouped_mx<true, OP, NSG, float>(
      a.H, a.I, a, (a.I + MXGN / 2 - 1) / (MXGN / 2), a.xq, a.xs, gq, gq + I * H / pb, 2 * I * H,
      gs, us, gss, s);
  if (e != hipSuccess) return e;
  const uint8_t* dq = static_cast<const uint8_t*>(a.down_q);
  const int NTd = (a.H + MXGN - 1) / MXGN;
  if (a.y_bf16)
    return launch_grouped_mx<false, OP, 4, bf16>(a.I, a.H, a, NTd, a.hq, a.hs, dq, dq, H * I,
                                                 a.down_s, a.down_s, dss, s);
  return launch_grouped_mx<false, OP, 4, float>(a.I, a.H, a, NTd, a.hq, a.hs, dq, dq, H * I,
                                                a.down_s, a.down_s, dss, s);
}

// Piece size of the scale staging (8 or 2 bytes; 0: none): it must divide
// the row length nsb and every base address and stride in `align`, and the
// nrows rows must fit kStgPieces pieces per thread of the block.
int stage_unit(long long nsb, int nrows, int nthreads, std::initializer_list<uintptr_t> align) {
  for (int u : {8, 2}) {
    bool ok = nsb % u == 0 && nrows * (nsb / u) <= (long long)kStgPieces * nthreads;
    for (uintptr_t v : align) ok = ok && v % u == 0;
    if (ok) return u;
  }
  return 0;
}

template <int OP, int WK, int MB, int NS, int NC>
void launch_gu_mx(const MxArgs& a, hipStream_t s) {
  const long long cgs = (a.I + 16 * NC - 1) / (16 * NC);
  dim3 grid((unsigned)(tile_count_bound(false, a.rows, a.T, a.E, 16 * MB) * cgs));
  const long long I = a.I, H = a.H;
  const uint8_t* gq = static_cast<const uint8_t*>(a.gate_up_q);
  const int pb = MxWeights<OP>::kPerByte;
  const uint8_t* uq = gq + I * H / pb;
  const void* gs = a.gate_up_s;
  const void* us;
  long long ss;
  if constexpr (OP == kOpFp8) {
    us = static_cast<const float*>(gs) + I;
    ss = 2 * I;
  } else {
    us = static_cast<const uint8_t*>(gs) + I * (H / 32);
    ss = 2 * I * (H / 32);
  }
  auto go = [&](auto su_tag) {
    constexpr int SU = decltype(su_tag)::value;
    const size_t lds = SU > 0 ? (size_t)(32 * NC) * (H / 32) : 0;
    hipLaunchKernelGGL((gate_up_mx_kernel<OP, WK, MB, NS, NC, SU>), grid, dim3(64 * WK), lds, s,
                       a.H, a.I, a.E, a.K, a.rows, a.xq, a.xs, gq, uq, 2 * I * H, gs, us, ss,
                       a.offsets, a.sorted_slots, a.hq, a.hs);
  };
  if constexpr (OP == kOpFp4) {
    const int su = stage_unit(H / 32, 32 * NC, 64 * WK,
                              {(uintptr_t)gs, (uintptr_t)us, (uintptr_t)ss});
    if (su == 8) return go(std::integral_constant<int, 8>{});
    if (su == 2) return go(std::integral_constant<int, 2>{});
  }
  go(std::integral_constant<int, 0>{});
}

template <int OP, int WN, int MB, int NS, int NC, typename YT>
void launch_dn_mx(const MxArgs& a, hipStream_t s) {
  const long long cgs = (a.H + 16 * WN * NC - 1) / (16 * WN * NC);
  dim3 grid((unsigned)(tile_count_bound(false, a.rows, a.T, a.E, 16 * MB) * cgs));
  const long long I = a.I, H = a.H;
  const long long ss = OP == kOpFp8 ? H : H * (I / 32);
  // the tile's activation rows staged in LDS when they fit the pieces
  const long long nsb = I / 32;
  const bool al = 16LL * MB * (I / 16) <= (long long)kAlCodePieces * 64 * WN &&
                  16LL * MB * (nsb / 2) <= (long long)kAlScalePieces * 64 * WN && nsb % 2 == 0 &&
                  (uintptr_t)a.hs % 2 == 0;
  auto go = [&](auto su_tag, auto al_tag) {
    constexpr int SU = decltype(su_tag)::value;
    constexpr bool AL = decltype(al_tag)::value;
    size_t lds = SU > 0 ? ((size_t)(16 * WN * NC) * nsb + 15) / 16 * 16 : 0;
    if (AL) lds += (size_t)16 * MB * (I + 16) + (size_t)16 * MB * nsb;
    hipLaunchKernelGGL((down_mx_kernel<OP, WN, MB, NS, NC, SU, AL, YT>), grid, dim3(64 * WN), lds,
                       s, a.H, a.I, a.E, a.rows, a.hq, a.hs,
                       static_cast<const uint8_t*>(a.down_q), H * I, a.down_s, ss, a.offsets,
                       a.sorted_slots, a.topk_w, static_cast<YT*>(a.y));
  };
  auto go_al = [&](auto su_tag) {
    if (al) go(su_tag, std::true_type{});
    else go(su_tag, std::false_type{});
  };
  if constexpr (OP == kOpFp4) {
    const int su = stage_unit(I / 32, 16 * WN * NC, 64 * WN, {(uintptr_t)a.down_s, (uintptr_t)ss});
    if (su == 8) return go_al(std::integral_constant<int, 8>{});
    if (su == 2) return go_al(std::integral_constant<int, 2>{});
  }
  go_al(std::integral_constant<int, 0>{});
}

// Configurations from a sweep at 1 / 8 / 64 / 256 tokens (26B shapes):
// MXFP4 gate_up 2 waves x 2 column groups x ring depth 3 (16-row tiles up to
// 128 tokens, 32-row past), down 4 waves x 2 column groups x depth 2; E4M3
// gate_up 4 waves x 2 groups x depth 2, down 2 waves x 1 group x depth 2 up
// to 16 tokens and 4 waves x 1 group past (16-row tiles, whose activation
// rows are staged in LDS: 256 tokens 82 -> 71 us).
template <int OP>
void launch_mx_stream(const MxArgs& a, hipStream_t s) {
  const bool small = a.T <= 128;
  if constexpr (OP == kOpFp4) {
    if (small) launch_gu_mx<OP, 2, 1, 3, 2>(a, s);
    else launch_gu_mx<OP, 2, 2, 3, 2>(a, s);
    if (a.y_bf16) launch_dn_mx<OP, 4, 1, 2, 2, bf16>(a, s);
    else launch_dn_mx<OP, 4, 1, 2, 2, float>(a, s);
  } else {
    if (small) launch_gu_mx<OP, 4, 1, 2, 2>(a, s);
    else launch_gu_mx<OP, 4, 2, 2, 2>(a, s);
    if (a.T <= 16) {
      if (a.y_bf16) launch_dn_mx<OP, 2, 1, 2, 1, bf16>(a, s);
      else launch_dn_mx<OP, 2, 1, 2, 1, float>(a, s);
    } else {
      if (a.y_bf16) launch_dn_mx<OP, 4, 1, 2, 1, bf16>(a, s);
      else launch_dn_mx<OP, 4, 1, 2, 1, float>(a, s);
    }
  }
}

}  // namespace

hipError_t launch_mx8_quantize(long long rows, int cols, const void* in, uint8_t* q,
                               uint8_t* e8, hipStream_t s) {
  const long long nb = rows * (cols / 32);
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL(mx8_quantize_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, s, nb,
                     cols, static_cast<const bf16*>(in), q, e8);
  return hipGetLastError();
}

hipError_t launch_mx8_dequantize(long long rows, int cols, const uint8_t* q, const uint8_t* e8,
                                 float* out, hipStream_t s) {
  const long long nb = rows * (cols / 32);
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL(mx8_dequantize_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, s,
                     nb, cols, q, e8, out);
  return hipGetLastError();
}

bool mx_uses_stream_kernels(int T, int rows, int E) { return T <= 256 && rows <= 16 * E; }

hipError_t launch_expert_ffn_mx(const MxArgs& a, hipStream_t s) {
  hipError_t e = launch_mx8_quantize(a.T, a.H, a.x, a.xq, a.xs, s);
  if (e != hipSuccess) return e;
  if (mx_uses_stream_kernels(a.T, a.rows, a.E)) {
    if (a.fmt == WFormat::kFP8) launch_mx_stream<kOpFp8>(a, s);
    else launch_mx_stream<kOpFp4>(a, s);
    return hipGetLastError();
  }
  return a.fmt == WFormat::kFP8 ? launch_mx_tiled<kOpFp8>(a, s) : launch_mx_tiled<kOpFp4>(a, s);
}

bool mx_tiled_supported(int H, int I) {
  return H % MXGK == 0 && I % MXGK == 0 &&
         MxLds<true, kOpFp4, 4>::total(H / 32) <= 160 * 1024 &&
         MxLds<true, kOpFp8, 4>::total(H / 32) <= 160 * 1024 &&
         MxLds<false, kOpFp4, 4>::total(I / 32) <= 160 * 1024 &&
         MxLds<false, kOpFp8, 4>::total(I / 32) <= 160 * 1024;
}

}  // namespace moe
