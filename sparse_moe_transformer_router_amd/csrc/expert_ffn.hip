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
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation on 256 x 256 block tiles
// of 16 waves; A rows are gathered from the token matrix by the per-lane
// source addresses of direct global -> LDS copies into a 4-stage ring shared
// with the weight tiles.  gate_up's epilogue applies GELU(gate) * up and
// rounds h to bf16; down's epilogue multiplies each row by its routing weight
// and writes it to the slot-major output; both leave through LDS-staged rows.
// fp32 path (debug): the same tiling idea on the vector ALUs in fp32.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace moe {
namespace {

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

// ---------------------------------------------------------------------------
// bf16 grouped GEMM, prefill sizes
// ---------------------------------------------------------------------------
// Block tile: BM (256 or 128) rows x 256 output columns (gate_up: 128 gate
// columns and the matching 128 up columns), k-tile 32.  Each k-tile of A (gathered rows) and B
// (weight rows) goes global -> LDS directly (global_load_lds, 16 B per lane)
// into a ring of NSTAGE stages of 32 KB.  A stage is refilled as soon as the
// barrier in the middle of its k-tile has passed (its last fragments were
// read in the first half), so up to NSTAGE - 1 tiles are in flight while one
// is consumed, and a tile is requested 2.5 k-tiles before it is needed.  An
// LDS row is 64 B (32 k values); the 16-B chunk c of row r is stored at position c ^ ((r >> 2) & 3), which keeps the fragment reads of
// v_mfma_f32_32x32x16_bf16 free of bank conflicts.  WM x WN waves each own a
// (BM / WM) x (256 / WN) sub-tile.  In a fixed issue order, a wave reads the
// fragments of the next half k-tile and issues its share of the next
// global -> LDS copies between its MFMAs, so that LDS and memory latency hide
// behind the matrix pipe; one barrier per k-tile.
constexpr int GN = 256, GK = 32;
template <int BM>
constexpr int stage_bytes() { return (BM + GN) * GK * 2; }
// Epilogue staging (the ring's LDS, free after the main loop): down stages
// 128 rows x 256 fp32 per pass, gate_up all BM rows x 128 bf16 at once; rows
// are padded by 16 B.  The down tile's row slots and weights sit past both.
constexpr int kDnStageRows = 128, kDnStride = GN + 4;     // floats
constexpr int kGuStride = GN / 2 + 8;                     // bf16
template <bool GU, int BM, int NSTAGE>
constexpr int slots_offset() {
  return NSTAGE * stage_bytes<BM>() > kDnStageRows * kDnStride * 4 ? NSTAGE * stage_bytes<BM>()
                                                                    : kDnStageRows * kDnStride * 4;
}
template <bool GU, int BM, int NSTAGE>
constexpr int gemm_lds_bytes() {
  return GU ? NSTAGE * stage_bytes<BM>() : slots_offset<GU, BM, NSTAGE>() + BM * 8;
}

__device__ __forceinline__ int gswz(int r, int c) { return c ^ ((r >> 2) & 3); }


// GU: h[row] = GELU(A[row] . W0[n]) * (A[row] . W1[n]) for the block's 128
// columns n, A row = token of the slot (or the row itself when ident).
// !GU: y[slot] = w[slot] * (h[row] . W0[n]) for the block's 256 columns n.
template <bool GU, int BM, int WM, int WN, int NSTAGE, typename YT>
__global__ __launch_bounds__(64 * WM * WN, 1) void grouped_gemm_kernel(
    int Kd, int Nout, int E, int K, int rows, int ident, int NT, const bf16* __restrict__ A,
    const bf16* __restrict__ W0, const bf16* __restrict__ W1, long long w_stride,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_slots,
    const float* __restrict__ topk_w, bf16* __restrict__ hout, YT* __restrict__ yout) {
  constexpr int SB = stage_bytes<BM>();
  constexpr int NW = WM * WN, ROWS = BM + GN, LPW = ROWS / 16 / NW;
  constexpr int WR = BM / WM, WC = GN / WN, TM = WR / 32, TN = WC / 32;
  constexpr int NF = TM + TN, NMF = TM * TN;
  static_assert(LPW * NW * 16 == ROWS && NF <= NMF && LPW <= NMF, "tile shape");
  static_assert(!GU || TN % 2 == 0, "gate_up waves need gate/up column pairs");
  static_assert(NSTAGE >= 3 && gemm_lds_bytes<GU, BM, NSTAGE>() <= 160 * 1024, "LDS");
  static_assert(!GU || BM * kGuStride * 2 <= NSTAGE * SB, "gate_up staging fits the ring");
  static_assert(GU || BM % kDnStageRows == 0, "down staging passes");
  static_assert((BM * (GN / 16)) % (64 * NW) == 0 && (kDnStageRows * (GN / 4)) % (64 * NW) == 0,
                "epilogue store loops cover the staged rows exactly");
  extern __shared__ __align__(16) unsigned char smem[];

  int e = 0, row0, row1, nt;
  {
    RowTileScan sc;
    int R;
    if (ident) {
      R = (rows + BM - 1) / BM;
    } else {
      row_tile_scan(offsets, E, BM, sc);
      R = sc.total;
    }
    const int item = xcd_item(blockIdx.x, R * NT);
    if (item < 0) return;  // uniform over the block
    const int rt = item / NT;
    nt = item % NT;
    if (ident) {
      row0 = rt * BM;
      row1 = min(row0 + BM, rows);
    } else {
      row_tile_lookup(sc, offsets, BM, rt, e, row0, row1);
    }
  }
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int wm = wave / WN, wn = wave % WN;
  const int nbase = GU ? nt * (GN / 2) : nt * GN;
  // down: output slot and routing weight of each of the tile's rows, fetched
  // now (behind the main loop) into LDS past the ring, for the epilogue
  int* row_slot = reinterpret_cast<int*>(smem + slots_offset<GU, BM, NSTAGE>());
  float* row_w = reinterpret_cast<float*>(row_slot + BM);
  if constexpr (!GU) {
    if (threadIdx.x < BM) {
      const int row = row0 + threadIdx.x;
      int slot = row;
      float w = 1.0f;
      if (!ident && row < row1) {
        slot = sorted_slots[row];
        w = topk_w[slot];
      }
      row_slot[threadIdx.x] = slot;
      row_w[threadIdx.x] = w;
    }
  }

  // Copy q of a stage fills LDS rows 16 q .. 16 q + 15; lane -> row 16 q +
  // lane / 4, position lane % 4.  This lane's LPW copies per k-tile:
  const bf16* src[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int q = wave * LPW + j;
    const int r = 16 * q + lane / 4;
    const int c = gswz(r, lane % 4);
    const bf16* p;
    if (r < BM) {
      int gr = row0 + r;
      if (gr >= row1) gr = row0;  // past the tile: re-read a valid row, output dropped
      const int arow = GU && !ident ? sorted_slots[gr] / K : gr;
      p = A + (size_t)arow * Kd;
    } else {
      const int br = r - BM;
      int n;
      const bf16* base;
      if (GU) {
        n = nbase + br % (GN / 2);
        base = br < GN / 2 ? W0 : W1;
      } else {
        n = nbase + br;
        base = W0;
      }
      if (n >= Nout) n = 0;  // past the last column: valid row, output dropped
      p = base + (size_t)e * w_stride + (size_t)n * Kd;
    }
    src[j] = p + c * 8;
  }
  const int nk = Kd / GK;
  // One copy per (k-tile, j); past the last k-tile the last tile is copied
  // again into the (free) ring slot, so that every k-tile issues the same
  // number of copies and the vmcnt waits below are constants.
  auto copy = [&](int kt, int j) {
    const int ktc = kt < nk ? kt : nk - 1;
    const int q = wave * LPW + j;
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(src[j] + ktc * GK,
                                     (void*)(smem + (kt % NSTAGE) * SB + q * 1024), 16,
                                     0, 0);
#endif
  };

  // Fragment byte offsets within a stage, per k16 half s: A sub-tiles 0..TM-1,
  // then B sub-tiles (gate_up: gate halves first, then up).
  const int fr = lane % 32, fq = lane / 32;
  int off[2][NF];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = wm * WR + i * 32 + fr;
      off[s][i] = r * 64 + gswz(r, 2 * s + fq) * 16;
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      int r;
      if (GU) {
        constexpr int half = TN / 2;
        r = BM + (j < half ? 0 : GN / 2) + wn * (WC / 2) + (j % half) * 32 + fr;
      } else {
        r = BM + wn * WC + j * 32 + fr;
      }
      off[s][TM + j] = r * 64 + gswz(r, 2 * s + fq) * 16;
    }
  }
  // 32-row sub-tiles of this wave that hold rows of the tile (wave-uniform).
  int nv;
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
  bf16x8 f0[NF], f1[NF];
  auto rd = [&](const unsigned char* st, int s, int f, bf16x8 (&fr_)[NF]) {
    fr_[f] = *reinterpret_cast<const bf16x8*>(st + off[s][f]);
  };

  auto mainloop = [&](auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    auto mf = [&](int m, bf16x8 (&c)[NF]) {
      const int i = m / TN, j = m % TN;
      if (FULL || i < nv)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(c[i], c[TM + j], acc[i][j], 0, 0, 0);
    };
#pragma unroll
    for (int s = 0; s < NSTAGE; ++s)
#pragma unroll
      for (int j = 0; j < LPW; ++j) copy(s, j);
    wait_vmem<(NSTAGE - 1) * LPW>();
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int f = 0; f < NF; ++f) rd(smem, 0, f, f0);
    wait_lds();
    __builtin_amdgcn_sched_barrier(0);
    for (int kt = 0; kt < nk; ++kt) {
      const unsigned char* st = smem + (kt % NSTAGE) * SB;
      const unsigned char* sn = smem + ((kt + 1) % NSTAGE) * SB;
      // first half: MFMAs on f0, reads of this tile's second-half fragments
#pragma unroll
      for (int m = 0; m < NMF; ++m) {
        if (m < NF) rd(st, 1, m, f1);
        mf(m, f0);
        __builtin_amdgcn_sched_barrier(0);
      }
      wait_lds();
      // tile kt+1 has landed for every wave; after the barrier no wave reads
      // tile kt any more, so its ring slot takes tile kt+NSTAGE
      wait_vmem<(NSTAGE - 2) * LPW>();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      // second half: MFMAs on f1, reads of tile kt+1's first-half fragments,
      // copies of tile kt+NSTAGE
#pragma unroll
      for (int m = 0; m < NMF; ++m) {
        if (m < NF) rd(sn, 0, m, f0);
        mf(m, f1);
        if (m >= NMF - LPW) copy(kt + NSTAGE, m - (NMF - LPW));
        __builtin_amdgcn_sched_barrier(0);
      }
      wait_lds();
    }
    wait_vmem<0>();
  };
  if (nv == TM)
    mainloop(std::true_type{});
  else
    mainloop(std::false_type{});

  // Epilogue through LDS: the accumulators go to a row-major staging tile
  // in the ring's LDS, then whole rows leave in 16-B stores (the accumulator
  // layout alone gives 2- or 4-B stores scattered over two rows each; those
  // took ~10% of gate_up's and ~20% of down's time).
  __syncthreads();  // every wave is done with the ring
  const int tid = threadIdx.x;
  constexpr int NT_ = 64 * NW;
  if constexpr (GU) {
    constexpr int half = TN / 2;
    bf16* stg = reinterpret_cast<bf16*>(smem);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if (i >= nv) break;
#pragma unroll
      for (int j = 0; j < half; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int r = wm * WR + i * 32 + 8 * (q / 4) + 4 * fq + (q % 4);
          const int c = wn * (WC / 2) + j * 32 + fr;
          stg[r * kGuStride + c] = (bf16)(gelu_tanh(acc[i][j][q]) * acc[i][j + half][q]);
        }
    }
    __syncthreads();
    // BM rows x 16 chunks of 8 bf16; Nout is a multiple of 32, so a chunk is
    // wholly inside or past the last column.
    constexpr int CH = (GN / 2) / 8;
#pragma unroll
    for (int it = 0; it < BM * CH / NT_; ++it) {
      const int k = tid + it * NT_;
      const int r = k / CH, ch = k % CH;
      const int col = nbase + ch * 8;
      if (row0 + r < row1 && col < Nout)
        *reinterpret_cast<uint4*>(hout + (size_t)(row0 + r) * Nout + col) =
            *reinterpret_cast<const uint4*>(stg + r * kGuStride + ch * 8);
    }
  } else {
    float* stg = reinterpret_cast<float*>(smem);
    constexpr int CH = GN / 4;  // chunks of 4 fp32 per row
#pragma unroll
    for (int pass = 0; pass < BM / kDnStageRows; ++pass) {
      if (wm * WR / kDnStageRows == pass) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          if (i >= nv) break;
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
              const int r = wm * WR - pass * kDnStageRows + i * 32 + 8 * (q / 4) + 4 * fq + (q % 4);
              stg[r * kDnStride + wn * WC + j * 32 + fr] = acc[i][j][q];
            }
        }
      }
      __syncthreads();
#pragma unroll
      for (int it = 0; it < kDnStageRows * CH / NT_; ++it) {
        const int k = tid + it * NT_;
        const int rl = k / CH, ch = k % CH;
        const int r = pass * kDnStageRows + rl;
        const int col = nbase + ch * 4;
        if (row0 + r < row1 && col < Nout) {
          const float sc = row_w[r];
          const float4 v = *reinterpret_cast<const float4*>(stg + rl * kDnStride + ch * 4);
          YT* dst = yout + (size_t)row_slot[r] * Nout + col;
          if constexpr (std::is_same<YT, float>::value) {
            *reinterpret_cast<float4*>(dst) = make_float4(sc * v.x, sc * v.y, sc * v.z, sc * v.w);
          } else {
            dst[0] = from_f32<YT>(sc * v.x);
            dst[1] = from_f32<YT>(sc * v.y);
            dst[2] = from_f32<YT>(sc * v.z);
            dst[3] = from_f32<YT>(sc * v.w);
          }
        }
      }
      __syncthreads();
    }
  }
}

// Configurations (256-row tiles): gate_up and down both 16 waves (4 x 4), 4
// stages.  gate_up with 8 waves (4 x 2) and 5 stages was 3-6% slower (4096
// skewed, 2048 and 8192 tokens): with 16 waves a partial row tile still keeps
// one wave on every SIMD.  128-row tiles measured slower on every shape tried
// (groups of ~128 rows at 2048 tokens included): the per-barrier MFMA count
// halves, and weights are read from HBM once per tile either way.

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

namespace {

template <bool GU, int BM, int WM, int WN, int NSTAGE, typename YT>
hipError_t launch_grouped(int Kd, int Nout, int E, int K, int rows, bool ident, int RT, int NT,
                          const bf16* A, const bf16* W0, const bf16* W1, long long w_stride,
                          const int32_t* offsets, const int32_t* sorted_slots,
                          const float* topk_w, bf16* hout, YT* yout, hipStream_t s,
                          hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr) {
  auto kf = grouped_gemm_kernel<GU, BM, WM, WN, NSTAGE, YT>;
  const int lds = gemm_lds_bytes<GU, BM, NSTAGE>();  // ring or staging (+ row slots, weights)
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kf), hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  launch_maybe_timed(kf, dim3(RT * NT), dim3(64 * WM * WN), lds, s, ev_start, ev_stop, Kd, Nout, E,
                     K, rows, (int)ident, NT, A, W0, W1, w_stride, offsets, sorted_slots, topk_w,
                     hout, yout);
  return hipSuccess;
}

template <typename YT>
hipError_t launch_down_tiled(const DownArgs& a, hipStream_t s) {
  const int NT = (a.H + GN - 1) / GN;
  const bf16* hb = static_cast<const bf16*>(a.h);
  const bf16* wd = static_cast<const bf16*>(a.w_down);
  YT* y = static_cast<YT*>(a.y);
  return launch_grouped<false, 256, 4, 4, 4, YT>(
      a.N, a.H, a.E, a.K, a.rows, a.ident, row_tile_bound(a.ident, a.rows, a.T, a.E, 256), NT, hb,
      wd, wd, a.w_stride, a.offsets, a.sorted_slots, a.topk_w, nullptr, y, s);
}

}  // namespace

hipError_t launch_gate_up(const GateUpArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  if (a.bf16 && use_stream_kernels(a.T, a.rows, a.E, a.ident)) return launch_gate_up_stream(a, s);
  if (a.bf16) {
    const int NT = (a.N + GN / 2 - 1) / (GN / 2);
    const bf16* x = static_cast<const bf16*>(a.x);
    const bf16* wg = static_cast<const bf16*>(a.w_gate);
    const bf16* wu = static_cast<const bf16*>(a.w_up);
    bf16* h = static_cast<bf16*>(a.h);
    const hipError_t e = launch_grouped<true, 256, 4, 4, 4, float>(
          a.H, a.N, a.E, a.K, a.rows, a.ident, row_tile_bound(a.ident, a.rows, a.T, a.E, 256), NT,
          x, wg, wu, a.w_stride, a.offsets, a.sorted_slots, nullptr, h, nullptr, s, a.ev_start,
          a.ev_stop);
    if (e != hipSuccess) return e;
  } else {
    dim3 grid(row_tile_bound(a.ident, a.rows, a.T, a.E, kFT), (a.N + kFT - 1) / kFT);
    launch_maybe_timed(gate_up_f32_kernel, grid, dim3(256), 0, s, a.ev_start, a.ev_stop, a.H, a.N,
                       a.E, a.K, a.rows, (int)a.ident, static_cast<const float*>(a.x),
                       static_cast<const float*>(a.w_gate), static_cast<const float*>(a.w_up),
                       a.w_stride, a.offsets, a.sorted_slots, static_cast<float*>(a.h));
  }
  return hipGetLastError();
}

hipError_t launch_down(const DownArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  if (a.bf16 && use_stream_kernels(a.T, a.rows, a.E, a.ident)) return launch_down_stream(a, s);
  if (a.bf16) {
    const hipError_t e = a.y_bf16 ? launch_down_tiled<bf16>(a, s) : launch_down_tiled<float>(a, s);
    if (e != hipSuccess) return e;
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
