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
// bf16 path at prefill sizes (decode sizes use the weight-streaming kernels):
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation on 128 x 128 block tiles;
// A rows are gathered from the token matrix while they are staged into LDS;
// A and weight tiles are double-buffered in LDS.  gate_up's epilogue applies
// GELU(gate) * up and rounds h to bf16; down's epilogue multiplies each row by
// its routing weight and writes it to the slot-major output.
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

// Blocks are dealt to the 8 XCDs round-robin (block b runs on XCD b % 8);
// give each XCD a contiguous range of work items so that neighbouring items
// (row tiles of the same expert on the same column tile, which read the same
// weight slab) run on one XCD at about the same time and share its L2.
__device__ __forceinline__ int xcd_item(int b, int nb) {
  const int q = nb / 8, r = nb % 8, x = b % 8;
  return x * q + min(x, r) + b / 8;
}

constexpr int TBM = 128, TBK = 64, TP = TBK + 8;  // LDS pitch in bf16 (144 B)

__device__ __forceinline__ void ld64(uint4 (&r)[4], const bf16* p, bool valid) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = valid ? *reinterpret_cast<const uint4*>(p + 8 * i) : make_uint4(0, 0, 0, 0);
}
__device__ __forceinline__ void st64(bf16* p, const uint4 (&r)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(p + 8 * i) = r[i];
}

// gate_up, prefill sizes: block tile 128 rows x (64 gate + 64 up) columns,
// BK = 64, double-buffered LDS; 4 waves in 2 x 2, each 64 rows x (32 gate +
// 32 up).  Work item = (column tile, row tile), row tiles fastest.
__global__ __launch_bounds__(256, 2) void gate_up_tiled_kernel(
    int H, int N, int E, int K, int rows, int ident, int RT, const bf16* __restrict__ x,
    const bf16* __restrict__ wg, const bf16* __restrict__ wu, long long w_stride,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_slots,
    bf16* __restrict__ h) {
  __shared__ bf16 As[2][TBM * TP];
  __shared__ bf16 Bs[2][TBM * TP];  // rows [0,64) gate, [64,128) up
  const int item = xcd_item(blockIdx.x, gridDim.x);
  const int nt = item / RT, rti = item % RT;
  RowTile rt;
  if (ident) {
    rt.e = 0;
    rt.row0 = rti * TBM;
    rt.row1 = min(rt.row0 + TBM, rows);
    if (rt.row0 >= rows) return;
  } else if (!find_row_tile(offsets, E, TBM, rti, rt.e, rt.row0, rt.row1)) {
    return;
  }
  const int n0 = nt * 64;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int wm = wave / 2, wn = wave % 2;

  // staging: thread -> row tid / 2, 32 k at (tid % 2) * 32, for A and for B
  const int sr = tid / 2, sk = (tid % 2) * 32;
  const int arow = rt.row0 + sr;
  const bool av = arow < rt.row1;
  const bf16* ap = x + (size_t)(av ? (ident ? arow : sorted_slots[arow] / K) : 0) * H + sk;
  const int bn = n0 + (sr & 63);
  const bool bv = bn < N;
  const bf16* bp = (sr < 64 ? wg : wu) + (size_t)rt.e * w_stride + (size_t)(bv ? bn : 0) * H + sk;

  f32x4 accg[4][2], accu[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      accg[i][j] = f32x4{0, 0, 0, 0};
      accu[i][j] = f32x4{0, 0, 0, 0};
    }
  uint4 ra[4], rb[4];
  const int nk = H / TBK;
  ld64(ra, ap, av);
  ld64(rb, bp, bv);
  st64(&As[0][sr * TP + sk], ra);
  st64(&Bs[0][sr * TP + sk], rb);
  __syncthreads();
  const int fr = lane % 16, fk = (lane / 16) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) {
      ld64(ra, ap + (kt + 1) * TBK, av);
      ld64(rb, bp + (kt + 1) * TBK, bv);
    }
    const bf16* A = As[buf];
    const bf16* B = Bs[buf];
#pragma unroll
    for (int kk = 0; kk < TBK; kk += 32) {
      bf16x8 a[4], g[2], u[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = lds_frag(A, wm * 64 + i * 16 + fr, kk + fk);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        g[j] = lds_frag(B, wn * 32 + j * 16 + fr, kk + fk);
        u[j] = lds_frag(B, 64 + wn * 32 + j * 16 + fr, kk + fk);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          accg[i][j] = mfma16(a[i], g[j], accg[i][j]);
          accu[i][j] = mfma16(a[i], u[j], accu[i][j]);
        }
    }
    if (kt + 1 < nk) {
      st64(&As[buf ^ 1][sr * TP + sk], ra);
      st64(&Bs[buf ^ 1][sr * TP + sk], rb);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = rt.row0 + wm * 64 + i * 16 + (lane / 16) * 4 + r;
        const int col = n0 + wn * 32 + j * 16 + (lane % 16);
        if (row < rt.row1 && col < N)
          h[(size_t)row * N + col] = (bf16)(gelu_tanh(accg[i][j][r]) * accu[i][j][r]);
      }
}

// down, prefill sizes: block tile 128 rows x 128 columns, BK = 64; 4 waves in
// 2 x 2, each 64 x 64.  The contraction length N is a multiple of 32; a
// 32-wide half past the end is staged as zeros.
template <typename YT>
__global__ __launch_bounds__(256, 2) void down_tiled_kernel(
    int H, int N, int E, int rows, int ident, int RT, const bf16* __restrict__ hbuf,
    const bf16* __restrict__ wd, long long w_stride, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_slots, const float* __restrict__ topk_w,
    YT* __restrict__ y) {
  __shared__ bf16 As[2][TBM * TP];
  __shared__ bf16 Bs[2][TBM * TP];
  const int item = xcd_item(blockIdx.x, gridDim.x);
  const int nt = item / RT, rti = item % RT;
  RowTile rt;
  if (ident) {
    rt.e = 0;
    rt.row0 = rti * TBM;
    rt.row1 = min(rt.row0 + TBM, rows);
    if (rt.row0 >= rows) return;
  } else if (!find_row_tile(offsets, E, TBM, rti, rt.e, rt.row0, rt.row1)) {
    return;
  }
  const int n0 = nt * 128;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int wm = wave / 2, wn = wave % 2;
  const int sr = tid / 2, sk = (tid % 2) * 32;
  const int arow = rt.row0 + sr;
  const bool av = arow < rt.row1;
  const bf16* ap = hbuf + (size_t)(av ? arow : 0) * N + sk;
  const int bn = n0 + sr;
  const bool bv = bn < H;
  const bf16* bp = wd + (size_t)rt.e * w_stride + (size_t)(bv ? bn : 0) * N + sk;

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0, 0, 0, 0};
  uint4 ra[4], rb[4];
  const int nk = (N + TBK - 1) / TBK;
  ld64(ra, ap, av && sk < N);
  ld64(rb, bp, bv && sk < N);
  st64(&As[0][sr * TP + sk], ra);
  st64(&Bs[0][sr * TP + sk], rb);
  __syncthreads();
  const int fr = lane % 16, fk = (lane / 16) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) {
      const bool kv = (kt + 1) * TBK + sk < N;
      ld64(ra, ap + (kt + 1) * TBK, av && kv);
      ld64(rb, bp + (kt + 1) * TBK, bv && kv);
    }
    const bf16* A = As[buf];
    const bf16* B = Bs[buf];
#pragma unroll
    for (int kk = 0; kk < TBK; kk += 32) {
      bf16x8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = lds_frag(A, wm * 64 + i * 16 + fr, kk + fk);
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = lds_frag(B, wn * 64 + j * 16 + fr, kk + fk);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(a[i], b[j], acc[i][j]);
    }
    if (kt + 1 < nk) {
      st64(&As[buf ^ 1][sr * TP + sk], ra);
      st64(&Bs[buf ^ 1][sr * TP + sk], rb);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = rt.row0 + wm * 64 + i * 16 + (lane / 16) * 4 + r;
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
    const int RT = row_tile_bound(a.ident, a.rows, a.T, a.E, TBM);
    const int NT = (a.N + 63) / 64;
    hipLaunchKernelGGL(gate_up_tiled_kernel, dim3(RT * NT), dim3(256), 0, s, a.H, a.N, a.E, a.K,
                       a.rows, (int)a.ident, RT, static_cast<const bf16*>(a.x),
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
    const int RT = row_tile_bound(a.ident, a.rows, a.T, a.E, TBM);
    dim3 grid(RT * ((a.H + 127) / 128));
    const bf16* hb = static_cast<const bf16*>(a.h);
    const bf16* wd = static_cast<const bf16*>(a.w_down);
    if (a.y_bf16)
      hipLaunchKernelGGL(down_tiled_kernel<bf16>, grid, dim3(256), 0, s, a.H, a.N, a.E, a.rows,
                         (int)a.ident, RT, hb, wd, a.w_stride, a.offsets, a.sorted_slots,
                         a.topk_w, static_cast<bf16*>(a.y));
    else
      hipLaunchKernelGGL(down_tiled_kernel<float>, grid, dim3(256), 0, s, a.H, a.N, a.E, a.rows,
                         (int)a.ident, RT, hb, wd, a.w_stride, a.offsets, a.sorted_slots,
                         a.topk_w, static_cast<float*>(a.y));
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
