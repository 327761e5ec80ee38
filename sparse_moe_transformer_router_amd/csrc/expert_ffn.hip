// Grouped expert GEMMs: the compute of Gemma4TextExperts on the page
// "Porting a 128-expert MoE (Gemma-4 26B-A4B) to AWS Inferentia2" (section
// "The architecture: a dual-path FFN nobody warned me about"): fused
// gate_up_proj [E, 2I, H] and down_proj [E, H, I] per expert, with the tanh
// form of GELU ("Porting Gemma-4 (2B / 4B / 12B) to AWS Inferentia2",
// section 4.5) applied to the gate and multiplied by the up projection.
//
// Rows are the expert-sorted token-slots from the dispatch: expert e owns
// rows [offsets[e], offsets[e+1]).  A block takes one row tile of one expert
// (found from the offsets by one wave, no tile list needed) and one column
// tile.  The dense MLP of the layer runs through the same kernels as a single
// group whose rows are the tokens themselves.
//
// bf16 path: v_mfma_f32_16x16x32_bf16 with fp32 accumulation; A rows are
// gathered from the token matrix while they are staged into LDS; weight tiles
// are double-buffered in LDS.  gate_up's epilogue applies GELU(gate) * up and
// rounds h to bf16; down's epilogue multiplies each row by its routing weight
// and writes it to the slot-major output.
// fp32 path (debug): the same tiling idea on the vector ALUs in fp32.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

// ---------------------------------------------------------------------------
// bf16 MFMA kernels
// ---------------------------------------------------------------------------
constexpr int kBK = 64;
constexpr int kPitch = kBK + 8;  // LDS row pitch in bf16 (144 B: conflict-free 16 B reads)

struct RowTile {
  int e, row0, row1;
};

__device__ __forceinline__ bool get_row_tile(bool ident, int rows, const int32_t* offsets, int E,
                                             int bm, RowTile& rt) {
  if (ident) {
    rt.e = 0;
    rt.row0 = blockIdx.x * bm;
    rt.row1 = min(rt.row0 + bm, rows);
    return rt.row0 < rows;
  }
  return find_row_tile(offsets, E, bm, blockIdx.x, rt.e, rt.row0, rt.row1);
}

__device__ __forceinline__ uint4 ld16(const bf16* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(bf16* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds_frag(const bf16* base, int row, int k) {
  return *reinterpret_cast<const bf16x8*>(base + row * kPitch + k);
}

// gate_up: tile 64 rows x (64 gate + 64 up) columns, 4 waves in 2 x 2, each
// wave 32 rows x (32 gate + 32 up).
__global__ __launch_bounds__(256) void gate_up_bf16_kernel(
    int H, int N, int E, int K, int rows, int ident, const bf16* __restrict__ x,
    const bf16* __restrict__ wg, const bf16* __restrict__ wu, long long w_stride,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_slots,
    bf16* __restrict__ h) {
  constexpr int BM = 64, BN = 64;
  __shared__ bf16 As[2][BM * kPitch];
  __shared__ bf16 Gs[2][BN * kPitch];
  __shared__ bf16 Us[2][BN * kPitch];

  RowTile rt;
  if (!get_row_tile(ident, rows, offsets, E, BM, rt)) return;
  const int n0 = blockIdx.y * BN;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int wm = wave / 2, wn = wave % 2;

  // staging assignment: row tid/4, 16 elements at (tid%4)*16
  const int lr = tid / 4, lk = (tid % 4) * 16;
  const int arow = rt.row0 + lr;
  const bool avalid = arow < rt.row1;
  const bf16* ap = x;
  if (avalid) {
    const int tok = ident ? arow : sorted_slots[arow] / K;
    ap = x + (size_t)tok * H + lk;
  }
  const int wrow = n0 + lr;
  const bool wvalid = wrow < N;
  const bf16* gp = wg + (size_t)rt.e * w_stride + (size_t)(wvalid ? wrow : 0) * H + lk;
  const bf16* up = wu + (size_t)rt.e * w_stride + (size_t)(wvalid ? wrow : 0) * H + lk;
  const uint4 zero = make_uint4(0, 0, 0, 0);

  uint4 ra[2], rg[2], ru[2];
  auto gload = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      ra[j] = avalid ? ld16(ap + k0 + j * 8) : zero;
      rg[j] = wvalid ? ld16(gp + k0 + j * 8) : zero;
      ru[j] = wvalid ? ld16(up + k0 + j * 8) : zero;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      st16(&As[buf][lr * kPitch + lk + j * 8], ra[j]);
      st16(&Gs[buf][lr * kPitch + lk + j * 8], rg[j]);
      st16(&Us[buf][lr * kPitch + lk + j * 8], ru[j]);
    }
  };

  f32x4 accg[2][2], accu[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      accg[i][j] = f32x4{0, 0, 0, 0};
      accu[i][j] = f32x4{0, 0, 0, 0};
    }

  const int nk = H / kBK;
  gload(0);
  lstore(0);
  __syncthreads();
  const int fr = lane % 16, fk = (lane / 16) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * kBK);
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 32) {
      bf16x8 a[2], g[2], u[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = lds_frag(As[buf], wm * 32 + i * 16 + fr, kk + fk);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        g[j] = lds_frag(Gs[buf], wn * 32 + j * 16 + fr, kk + fk);
        u[j] = lds_frag(Us[buf], wn * 32 + j * 16 + fr, kk + fk);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          accg[i][j] = mfma16(a[i], g[j], accg[i][j]);
          accu[i][j] = mfma16(a[i], u[j], accu[i][j]);
        }
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue: D[(lane/16)*4 + r][lane%16] of each 16x16 sub-tile
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = rt.row0 + wm * 32 + i * 16 + (lane / 16) * 4 + r;
        const int col = n0 + wn * 32 + j * 16 + (lane % 16);
        if (row < rt.row1 && col < N)
          h[(size_t)row * N + col] = (bf16)(gelu_tanh(accg[i][j][r]) * accu[i][j][r]);
      }
}

// down: tile 64 rows x 128 columns, 4 waves in 2 x 2, each wave 32 x 64.
template <typename YT>
__global__ __launch_bounds__(256) void down_bf16_kernel(
    int H, int N, int E, int rows, int ident, const bf16* __restrict__ hbuf,
    const bf16* __restrict__ wd, long long w_stride, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_slots, const float* __restrict__ topk_w,
    YT* __restrict__ y) {
  constexpr int BM = 64, BN = 128;
  __shared__ bf16 As[2][BM * kPitch];
  __shared__ bf16 Bs[2][BN * kPitch];

  RowTile rt;
  if (!get_row_tile(ident, rows, offsets, E, BM, rt)) return;
  const int n0 = blockIdx.y * BN;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int wm = wave / 2, wn = wave % 2;

  const int lr = tid / 4, lk = (tid % 4) * 16;
  const int arow = rt.row0 + lr;
  const bool avalid = arow < rt.row1;
  const bf16* ap = hbuf + (size_t)(avalid ? arow : 0) * N + lk;
  // weight rows: this thread stages rows lr and lr + 64
  const bf16* bp[2];
  bool bvalid[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + lr + j * 64;
    bvalid[j] = n < H;
    bp[j] = wd + (size_t)rt.e * w_stride + (size_t)(bvalid[j] ? n : 0) * N + lk;
  }
  const uint4 zero = make_uint4(0, 0, 0, 0);

  uint4 ra[2], rb[2][2];
  auto gload = [&](int k0) {
    const bool kv = k0 + lk < N;  // N % 32 == 0: a 16-wide segment is all in or all out
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      ra[j] = (avalid && kv) ? ld16(ap + k0 + j * 8) : zero;
#pragma unroll
      for (int q = 0; q < 2; ++q) rb[q][j] = (bvalid[q] && kv) ? ld16(bp[q] + k0 + j * 8) : zero;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      st16(&As[buf][lr * kPitch + lk + j * 8], ra[j]);
#pragma unroll
      for (int q = 0; q < 2; ++q) st16(&Bs[buf][(lr + q * 64) * kPitch + lk + j * 8], rb[q][j]);
    }
  };

  f32x4 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

  const int nk = (N + kBK - 1) / kBK;
  gload(0);
  lstore(0);
  __syncthreads();
  const int fr = lane % 16, fk = (lane / 16) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * kBK);
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 32) {
      bf16x8 a[2], b[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = lds_frag(As[buf], wm * 32 + i * 16 + fr, kk + fk);
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = lds_frag(Bs[buf], wn * 64 + j * 16 + fr, kk + fk);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(a[i], b[j], acc[i][j]);
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = rt.row0 + wm * 32 + i * 16 + (lane / 16) * 4 + r;
      if (row >= rt.row1) continue;
      const int slot = ident ? row : sorted_slots[row];
      const float sc = ident ? 1.0f : topk_w[slot];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + wn * 64 + j * 16 + (lane % 16);
        if (col < H) y[(size_t)slot * H + col] = from_f32<YT>(sc * acc[i][j][r]);
      }
    }
}

// ---------------------------------------------------------------------------
// fp32 kernels (debug path)
// ---------------------------------------------------------------------------
constexpr int kFT = 32;  // rows per tile and k-tile

// gate_up fp32: tile 32 rows x 32 (gate, up) columns; thread = 2 rows x 2 cols.
__global__ __launch_bounds__(256) void gate_up_f32_kernel(
    int H, int N, int E, int K, int rows, int ident, const float* __restrict__ x,
    const float* __restrict__ wg, const float* __restrict__ wu, long long w_stride,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_slots,
    float* __restrict__ h) {
  __shared__ float As[kFT][kFT + 1], Gs[kFT][kFT + 1], Us[kFT][kFT + 1];
  RowTile rt;
  if (!get_row_tile(ident, rows, offsets, E, kFT, rt)) return;
  const int n0 = blockIdx.y * kFT;
  const int tid = threadIdx.x;
  const int tr = tid / 16, tc = tid % 16;
  float ag[2][2] = {{0, 0}, {0, 0}}, au[2][2] = {{0, 0}, {0, 0}};
  for (int k0 = 0; k0 < H; k0 += kFT) {
    for (int i = tid; i < kFT * kFT; i += 256) {
      const int r = i / kFT, k = i % kFT;
      const int arow = rt.row0 + r;
      float av = 0.0f;
      if (arow < rt.row1) {
        const int tok = ident ? arow : sorted_slots[arow] / K;
        av = x[(size_t)tok * H + k0 + k];
      }
      As[r][k] = av;
      const int n = n0 + r;
      const size_t wo = (size_t)rt.e * w_stride + (size_t)n * H + k0 + k;
      Gs[r][k] = n < N ? wg[wo] : 0.0f;
      Us[r][k] = n < N ? wu[wo] : 0.0f;
    }
    __syncthreads();
    for (int k = 0; k < kFT; ++k) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          ag[a][b] = fmaf(As[2 * tr + a][k], Gs[2 * tc + b][k], ag[a][b]);
          au[a][b] = fmaf(As[2 * tr + a][k], Us[2 * tc + b][k], au[a][b]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int row = rt.row0 + 2 * tr + a, col = n0 + 2 * tc + b;
      if (row < rt.row1 && col < N) h[(size_t)row * N + col] = gelu_tanh(ag[a][b]) * au[a][b];
    }
}

// down fp32: tile 32 rows x 64 columns; thread = 2 rows x 4 cols.
__global__ __launch_bounds__(256) void down_f32_kernel(
    int H, int N, int E, int rows, int ident, const float* __restrict__ hbuf,
    const float* __restrict__ wd, long long w_stride, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_slots, const float* __restrict__ topk_w,
    float* __restrict__ y) {
  __shared__ float As[kFT][kFT + 1], Bs[2 * kFT][kFT + 1];
  RowTile rt;
  if (!get_row_tile(ident, rows, offsets, E, kFT, rt)) return;
  const int n0 = blockIdx.y * 2 * kFT;
  const int tid = threadIdx.x;
  const int tr = tid / 16, tc = tid % 16;
  float acc[2][4] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
  for (int k0 = 0; k0 < N; k0 += kFT) {
    for (int i = tid; i < kFT * kFT; i += 256) {
      const int r = i / kFT, k = i % kFT;
      const int arow = rt.row0 + r;
      As[r][k] = arow < rt.row1 ? hbuf[(size_t)arow * N + k0 + k] : 0.0f;
    }
    for (int i = tid; i < 2 * kFT * kFT; i += 256) {
      const int r = i / kFT, k = i % kFT;
      const int n = n0 + r;
      Bs[r][k] = n < H ? wd[(size_t)rt.e * w_stride + (size_t)n * N + k0 + k] : 0.0f;
    }
    __syncthreads();
    for (int k = 0; k < kFT; ++k) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = fmaf(As[2 * tr + a][k], Bs[4 * tc + b][k], acc[a][b]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int row = rt.row0 + 2 * tr + a;
    if (row >= rt.row1) continue;
    const int slot = ident ? row : sorted_slots[row];
    const float sc = ident ? 1.0f : topk_w[slot];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int col = n0 + 4 * tc + b;
      if (col < H) y[(size_t)slot * H + col] = sc * acc[a][b];
    }
  }
}

// Upper bound on the number of row tiles over all groups.
int row_tile_bound(bool ident, int rows, int T, int E, int bm) {
  if (ident) return (rows + bm - 1) / bm;
  long long a = ((long long)rows + (long long)E * (bm - 1)) / bm;
  long long b = (long long)E * ((T + bm - 1) / bm);
  return (int)(a < b ? a : b);
}

}  // namespace

hipError_t launch_gate_up(const GateUpArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  if (a.bf16 && use_stream_kernels(a.T, a.ident)) return launch_gate_up_stream(a, s);
  if (a.bf16) {
    dim3 grid(row_tile_bound(a.ident, a.rows, a.T, a.E, 64), (a.N + 63) / 64);
    hipLaunchKernelGGL(gate_up_bf16_kernel, grid, dim3(256), 0, s, a.H, a.N, a.E, a.K, a.rows,
                       (int)a.ident, static_cast<const bf16*>(a.x),
                       static_cast<const bf16*>(a.w_gate), static_cast<const bf16*>(a.w_up),
                       a.w_stride, a.offsets, a.sorted_slots, static_cast<bf16*>(a.h));
  } else {
    dim3 grid(row_tile_bound(a.ident, a.rows, a.T, a.E, kFT), (a.N + kFT - 1) / kFT);
    hipLaunchKernelGGL(gate_up_f32_kernel, grid, dim3(256), 0, s, a.H, a.N, a.E, a.K, a.rows,
                       (int)a.ident, static_cast<const float*>(a.x),
                       static_cast<const float*>(a.w_gate), static_cast<const float*>(a.w_up),
                       a.w_stride, a.offsets, a.sorted_slots, static_cast<float*>(a.h));
  }
  return hipGetLastError();
}

hipError_t launch_down(const DownArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  if (a.bf16 && use_stream_kernels(a.T, a.ident)) return launch_down_stream(a, s);
  if (a.bf16) {
    dim3 grid(row_tile_bound(a.ident, a.rows, a.T, a.E, 64), (a.H + 127) / 128);
    const bf16* hb = static_cast<const bf16*>(a.h);
    const bf16* wd = static_cast<const bf16*>(a.w_down);
    if (a.y_bf16)
      hipLaunchKernelGGL(down_bf16_kernel<bf16>, grid, dim3(256), 0, s, a.H, a.N, a.E, a.rows,
                         (int)a.ident, hb, wd, a.w_stride, a.offsets, a.sorted_slots, a.topk_w,
                         static_cast<bf16*>(a.y));
    else
      hipLaunchKernelGGL(down_bf16_kernel<float>, grid, dim3(256), 0, s, a.H, a.N, a.E, a.rows,
                         (int)a.ident, hb, wd, a.w_stride, a.offsets, a.sorted_slots, a.topk_w,
                         static_cast<float*>(a.y));
  } else {
    dim3 grid(row_tile_bound(a.ident, a.rows, a.T, a.E, kFT), (a.H + 2 * kFT - 1) / (2 * kFT));
    hipLaunchKernelGGL(down_f32_kernel, grid, dim3(256), 0, s, a.H, a.N, a.E, a.rows,
                       (int)a.ident, static_cast<const float*>(a.h),
                       static_cast<const float*>(a.w_down), a.w_stride, a.offsets,
                       a.sorted_slots, a.topk_w, static_cast<float*>(a.y));
  }
  return hipGetLastError();
}

}  // namespace moe
