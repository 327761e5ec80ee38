// Decode-sized grouped expert GEMMs (few rows per expert): weight streaming.
//
// At decode batch sizes an expert sees a handful of rows, so the two expert
// GEMMs are bound by reading each touched expert's weights from HBM once
// (gate_up [2I, H] and down [H, I] of the page "Porting a 128-expert MoE
// (Gemma-4 26B-A4B) to AWS Inferentia2", section "The architecture: a
// dual-path FFN nobody warned me about").  These kernels keep the weight
// operand out of LDS: per 64-wide k-block every lane loads 32 contiguous
// bytes of one weight row straight into registers (four lanes cover a
// 128-byte line) and feeds them to v_mfma_f32_16x16x32_bf16 as two
// 8-element operands; the activation rows (at most 16 * MB per tile, resident
// in L2) are loaded the same way.  Loads run NS k-blocks ahead of the MFMAs
// (a register ring).  A block's waves split the contraction; their partial
// sums meet in LDS and are added in wave order (deterministic), then the
// epilogue applies GELU-tanh(gate) * up (gate_up) or the routing weight and
// the slot scatter (down).
//
// k mapping: in k-block kb, lane l (row or column l % 16, group g = l / 16)
// holds k = 64 kb + 16 g + [0, 16); MFMA j of the block uses its elements
// [8 j, 8 j + 8).  A and B use the same mapping, so the two MFMAs of a block
// sum over all of its k.  Contraction lengths are multiples of 32, so a
// lane's 16-element group is either wholly inside or wholly past the end.
//
// Measured on the 26B-A4B decode shapes (64 tokens, ~125 experts touched):
// gate_up streams at ~5.8 TB/s and down at ~4.8 TB/s, against ~6.0 TB/s for
// a plain streaming read on the same part; wider per-lane loads, deeper
// register rings and non-temporal loads measured no better or worse.
#include "common.h"
#include "launch.h"
#include "wformat.h"

namespace moe {
namespace {

constexpr int kKB = 64;  // k per block

typedef W16 Frag;  // 16 bf16 activations of one row

__device__ __forceinline__ void ld_frag(Frag& f, const bf16* p) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int i = 0; i < 2; ++i) f.u[i] = q[i];
}

__device__ __forceinline__ void zero_frag(Frag& f) {
#pragma unroll
  for (int i = 0; i < 2; ++i) f.u[i] = make_uint4(0, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bool stream_tile(bool ident, int rows, const int32_t* offsets, int E,
                                            int bm, int& e, int& row0, int& row1) {
  if (ident) {
    e = 0;
    row0 = blockIdx.x * bm;
    row1 = min(row0 + bm, rows);
    return row0 < rows;
  }
  return find_row_tile(offsets, E, bm, blockIdx.x, e, row0, row1);
}

// gate_up: one block = one row tile (<= 16 * MB rows) x 16 gate + 16 up
// columns; its WK waves split H.
template <typename WQ, int WK, int MB, int NS>
__global__ __launch_bounds__(64 * WK) void gate_up_stream_kernel(
    int H, int N, int E, int K, int rows, int ident, const bf16* __restrict__ x,
    const WQ* __restrict__ wg, const WQ* __restrict__ wu, long long w_stride,
    const void* __restrict__ sg, const void* __restrict__ su, long long s_stride,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_slots,
    bf16* __restrict__ h) {
  typedef WFmt<WQ> F;
  __shared__ f32x4 red[WK][MB][2][kWave];
  int e, row0, row1;
  if (!stream_tile(ident, rows, offsets, E, 16 * MB, e, row0, row1)) return;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int fr = lane % 16, fg = lane / 16;
  const int n = blockIdx.y * 16 + fr;
  const bool nvalid = n < N;
  const long long wel = (long long)e * w_stride + (long long)(nvalid ? n : 0) * H;
  const WQ* gp = wrow(wg, wel);
  const WQ* up = wrow(wu, wel);
  const uint8_t* gsr = nullptr;
  const uint8_t* usr = nullptr;
  if constexpr (F::kBlockScale) {
    const long long sel = (long long)e * s_stride + (long long)(nvalid ? n : 0) * (H / 32);
    gsr = static_cast<const uint8_t*>(sg) + sel;
    usr = static_cast<const uint8_t*>(su) + sel;
  }
  const int nmb = (row1 - row0 + 15) / 16;  // active 16-row blocks (uniform)
  const bf16* ap[MB];
  bool av[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int r = row0 + 16 * mb + fr;
    av[mb] = r < row1;
    const int tok = av[mb] ? (ident ? r : sorted_slots[r] / K) : 0;
    ap[mb] = x + (size_t)tok * H + 16 * fg;
  }
  const int KB = (H + kKB - 1) / kKB;
  const int kb0 = wave * KB / WK, kb1 = (wave + 1) * KB / WK;

  f32x4 accg[MB], accu[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    accg[mb] = f32x4{0, 0, 0, 0};
    accu[mb] = f32x4{0, 0, 0, 0};
  }
  WRaw<WQ> bg[NS], bu[NS];
  Frag ba[NS][MB];
  auto load = [&](int kb, WRaw<WQ>& g, WRaw<WQ>& u, Frag (&a)[MB]) {
    const int k = kb * kKB;
    const bool kv = k + 16 * fg < H;
    if (nvalid && kv) {
      g.load(gp, k + 16 * fg, gsr);
      u.load(up, k + 16 * fg, usr);
    } else {
      g.zero();
      u.zero();
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (mb < nmb && av[mb] && kv) ld_frag(a[mb], ap[mb] + k);
      else zero_frag(a[mb]);
    }
  };
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (kb0 + s < kb1) load(kb0 + s, bg[s], bu[s], ba[s]);
  for (int kb = kb0; kb < kb1; kb += NS) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (kb + s >= kb1) break;
      const int kl = kb + s + NS - 1;
      if (kl < kb1) load(kl, bg[(s + NS - 1) % NS], bu[(s + NS - 1) % NS], ba[(s + NS - 1) % NS]);
      const Frag fgt = bg[s].widen(), fup = bu[s].widen();
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          if (mb < nmb) {
            accg[mb] = mfma16(ba[s][mb].v[j], fgt.v[j], accg[mb]);
            accu[mb] = mfma16(ba[s][mb].v[j], fup.v[j], accu[mb]);
          }
    }
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    red[wave][mb][0][lane] = accg[mb];
    red[wave][mb][1][lane] = accu[mb];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    if (mb >= nmb) break;
    f32x4 g = red[0][mb][0][lane], u = red[0][mb][1][lane];
#pragma unroll
    for (int w = 1; w < WK; ++w) {
      g += red[w][mb][0][lane];
      u += red[w][mb][1][lane];
    }
    if constexpr (F::kChannelScale) {
      if (nvalid) {
        g *= static_cast<const float*>(sg)[(size_t)e * s_stride + n];
        u *= static_cast<const float*>(su)[(size_t)e * s_stride + n];
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = row0 + 16 * mb + 4 * fg + r;
      if (row < row1 && nvalid) h[(size_t)row * N + n] = (bf16)(gelu_tanh(g[r]) * u[r]);
    }
  }
}

// down: one block = one row tile x 16 * WN output columns; WK waves split
// the contraction (the intermediate width N).
template <typename WQ, int WN, int WK, int MB, int NS, typename YT>
__global__ __launch_bounds__(64 * WN * WK) void down_stream_kernel(
    int H, int N, int E, int rows, int ident, const bf16* __restrict__ hbuf,
    const WQ* __restrict__ wd, long long w_stride, const void* __restrict__ sd,
    long long s_stride, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_slots, const float* __restrict__ topk_w,
    YT* __restrict__ y) {
  typedef WFmt<WQ> F;
  __shared__ f32x4 red[WK > 1 ? WN * WK : 1][MB][kWave];
  int e, row0, row1;
  if (!stream_tile(ident, rows, offsets, E, 16 * MB, e, row0, row1)) return;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int wn = wave % WN, wk = wave / WN;
  const int fr = lane % 16, fg = lane / 16;
  const int n = blockIdx.y * 16 * WN + 16 * wn + fr;
  const bool nvalid = n < H;
  const WQ* bp = wrow(wd, (long long)e * w_stride + (long long)(nvalid ? n : 0) * N);
  const uint8_t* bsr = nullptr;
  if constexpr (F::kBlockScale)
    bsr = static_cast<const uint8_t*>(sd) + (long long)e * s_stride +
          (long long)(nvalid ? n : 0) * (N / 32);
  const int nmb = (row1 - row0 + 15) / 16;
  const bf16* ap[MB];
  bool av[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int r = row0 + 16 * mb + fr;
    av[mb] = r < row1;
    ap[mb] = hbuf + (size_t)(av[mb] ? r : 0) * N + 16 * fg;
  }
  const int KB = (N + kKB - 1) / kKB;
  const int kb0 = wk * KB / WK, kb1 = (wk + 1) * KB / WK;

  f32x4 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0, 0, 0, 0};
  WRaw<WQ> bb[NS];
  Frag ba[NS][MB];
  auto load = [&](int kb, WRaw<WQ>& b, Frag (&a)[MB]) {
    const int k = kb * kKB;
    const bool kv = k + 16 * fg < N;
    if (nvalid && kv) b.load(bp, k + 16 * fg, bsr);
    else b.zero();
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (mb < nmb && av[mb] && kv) ld_frag(a[mb], ap[mb] + k);
      else zero_frag(a[mb]);
    }
  };
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (kb0 + s < kb1) load(kb0 + s, bb[s], ba[s]);
  for (int kb = kb0; kb < kb1; kb += NS) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (kb + s >= kb1) break;
      const int kl = kb + s + NS - 1;
      if (kl < kb1) load(kl, bb[(s + NS - 1) % NS], ba[(s + NS - 1) % NS]);
      const Frag fb = bb[s].widen();
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          if (mb < nmb) acc[mb] = mfma16(ba[s][mb].v[j], fb.v[j], acc[mb]);
    }
  }
  if constexpr (WK > 1) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) red[wave][mb][lane] = acc[mb];
    __syncthreads();
    if (wk != 0) return;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      acc[mb] = red[wn][mb][lane];
#pragma unroll
      for (int w = 1; w < WK; ++w) acc[mb] += red[wn + w * WN][mb][lane];
    }
  }
  float chs = 1.0f;
  if constexpr (F::kChannelScale)
    if (nvalid) chs = static_cast<const float*>(sd)[(size_t)e * s_stride + n];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    if (mb >= nmb) break;
    if constexpr (F::kChannelScale) acc[mb] *= chs;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = row0 + 16 * mb + 4 * fg + r;
      if (row >= row1 || !nvalid) continue;
      const int slot = ident ? row : sorted_slots[row];
      const float sc = ident ? 1.0f : topk_w[slot];
      y[(size_t)slot * H + n] = from_f32<YT>(sc * acc[mb][r]);
    }
  }
}

int tile_bound(bool ident, int rows, int T, int E, int bm) {
  if (ident) return (rows + bm - 1) / bm;
  long long a = ((long long)rows + (long long)E * (bm - 1)) / bm;
  long long b = (long long)E * ((T + bm - 1) / bm);
  return (int)(a < b ? a : b);
}

template <typename WQ, int WK, int MB, int NS>
void launch_gu(const GateUpArgs& a, hipStream_t s) {
  dim3 grid(tile_bound(a.ident, a.rows, a.T, a.E, 16 * MB), (a.N + 15) / 16);
  hipLaunchKernelGGL((gate_up_stream_kernel<WQ, WK, MB, NS>), grid, dim3(64 * WK), 0, s, a.H, a.N,
                     a.E, a.K, a.rows, (int)a.ident, static_cast<const bf16*>(a.x),
                     static_cast<const WQ*>(a.w_gate), static_cast<const WQ*>(a.w_up), a.w_stride,
                     a.s_gate, a.s_up, a.s_stride,
                     a.offsets, a.sorted_slots, static_cast<bf16*>(a.h));
}

template <typename WQ, int WN, int WK, int MB, int NS, typename YT>
void launch_dn(const DownArgs& a, hipStream_t s) {
  dim3 grid(tile_bound(a.ident, a.rows, a.T, a.E, 16 * MB), (a.H + 16 * WN - 1) / (16 * WN));
  hipLaunchKernelGGL((down_stream_kernel<WQ, WN, WK, MB, NS, YT>), grid, dim3(64 * WN * WK), 0, s,
                     a.H, a.N, a.E, a.rows, (int)a.ident, static_cast<const bf16*>(a.h),
                     static_cast<const WQ*>(a.w_down), a.w_stride,
                     a.s_down, a.s_stride, a.offsets, a.sorted_slots,
                     a.topk_w, static_cast<YT*>(a.y));
}

template <typename YT>
void launch_dn_t(const DownArgs& a, hipStream_t s) {
  switch (a.w_fmt) {
    case WFormat::kInt8: launch_dn<int8_t, 2, 2, 1, 2, YT>(a, s); return;
    case WFormat::kFP8: launch_dn<fp8e4m3, 2, 2, 1, 2, YT>(a, s); return;
    case WFormat::kMXFP4: launch_dn<fp4x2, 2, 2, 1, 2, YT>(a, s); return;
    case WFormat::kBF16: break;
  }
  if (a.T <= 8) launch_dn<bf16, 2, 2, 1, 2, YT>(a, s);
  else launch_dn<bf16, 4, 1, 1, 2, YT>(a, s);
}

}  // namespace

// Weight streaming pays while every expert's row group is a few 16-row
// tiles: at most 64 tokens and, for the expert groups, at most 16 rows per
// expert on average (the top-K layout of 64 tokens has 4; the all-experts
// layout has T, and takes the tiled GEMMs).
bool use_stream_kernels(int T, int rows, int E, bool ident) {
  return T <= 64 && (ident || rows <= 16 * E);
}

// The dense branch (ident) at <= 64 tokens takes 32-row tiles (its weights
// are streamed once per tile, the second time mostly from L2); its down
// projection splits the contraction over 4 waves to keep enough loads in
// flight.
hipError_t launch_gate_up_stream(const GateUpArgs& a, hipStream_t s) {
  switch (a.w_fmt) {
    case WFormat::kInt8: launch_gu<int8_t, 4, 1, 2>(a, s); break;
    case WFormat::kFP8: launch_gu<fp8e4m3, 4, 1, 2>(a, s); break;
    case WFormat::kMXFP4: launch_gu<fp4x2, 4, 1, 2>(a, s); break;
    case WFormat::kBF16:
      if (a.ident) launch_gu<bf16, 8, 2, 2>(a, s);
      else launch_gu<bf16, 8, 1, 3>(a, s);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_down_stream(const DownArgs& a, hipStream_t s) {
  if (a.ident && a.w_fmt == WFormat::kBF16) {
    if (a.y_bf16) launch_dn<bf16, 2, 4, 2, 2, bf16>(a, s);
    else launch_dn<bf16, 2, 4, 2, 2, float>(a, s);
  } else if (a.y_bf16) {
    launch_dn_t<bf16>(a, s);
  } else {
    launch_dn_t<float>(a, s);
  }
  return hipGetLastError();
}

}  // namespace moe
