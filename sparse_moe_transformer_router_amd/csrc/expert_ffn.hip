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
// tile; the row tiles of an expert that read the same weight slab are
// consecutive work items.  The dense MLP of the layer runs through the same
// kernels as a single group whose rows are the tokens themselves.
//
// bf16 path at prefill sizes (decode sizes use the weight-streaming kernels):
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation on 256 x 256 block tiles
// of 16 waves (bf16 gate_up over expert groups of 256 rows or more on
// average: 8 waves); A rows are gathered from the token matrix by the per-lane
// source addresses of direct global -> LDS copies into a ring shared with the
// weight tiles (gate_up: 5 stages in bf16, 6 for 8-bit codes, 4 for MXFP4;
// down: 4).  gate_up's epilogue applies GELU(gate) * up and
// rounds h to bf16; down's epilogue multiplies each row by its routing weight
// and writes it to the slot-major output; both leave through LDS-staged rows.
// Weights stored as int8, E4M3 or MXFP4 take the same kernels past the
// decode sizes, widened exactly to bf16 after their LDS reads.
// fp32 path (debug): the same tiling idea on the vector ALUs in fp32.
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "wformat.h"

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
// Grouped GEMM on the bf16 matrix cores, prefill sizes
// ---------------------------------------------------------------------------
// Block tile: BM (256 or 128) rows x 256 output columns (gate_up: 128 gate
// columns and the matching 128 up columns), k-tile 32.  Each k-tile of A
// (gathered rows) and B (weight rows) goes global -> LDS directly (16 B per
// lane) into a ring of NSTAGE stages.  A stage is refilled as soon as the
// barrier in the middle of its k-tile has passed (its last fragments were
// read in the first half), so up to NSTAGE - 1 tiles are in flight while one
// is consumed.  An A row (and a bf16 B row) of a stage is 64 B (32 k
// values); the 16-B chunk c of row r is stored at position c ^ ((r >> 2) & 3),
// which keeps the fragment reads of v_mfma_f32_32x32x16_bf16 free of bank
// conflicts.  WM x WN waves each own a (BM / WM) x (256 / WN) sub-tile.  In a
// fixed issue order, a wave reads the fragments of the next half k-tile and
// issues its share of the next copies between its MFMAs, so that LDS and
// memory latency hide behind the matrix pipe; one barrier per k-tile.
//
// Weights stored below bf16 (WF: int8, E4M3 or MXFP4, the formats of
// wformat.h) stay in their stored form in the ring (32 or 16 B per row and
// k-tile) and widen exactly to bf16 in registers after the fragment read;
// int8 / E4M3 channel scales multiply the k-sums in the epilogue, MXFP4 block
// scales (one per k-tile and row, staged in LDS for the whole tile) the
// widened values.  For these the 16 k values one lane feeds to an MFMA pair
// are a contiguous run of the row (lane group fq of half s takes k = 16 fq +
// 8 s .. + 7, in A and B alike), so that one 16-B (8-B for MXFP4) LDS read
// gives a lane its weights for the whole k-tile.  Every wave copies one A
// chunk per k-tile and the first GN * RB / 1024 waves one B chunk.
constexpr int GN = 256, GK = 32;
// Stored form of the B operand (the WFormat codes).
constexpr int kWfBF16 = 0, kWfInt8 = 1, kWfFP8 = 2, kWfMXFP4 = 3;
// Bytes of one weight row's k-tile (GK weights) as stored.
template <int WF>
constexpr int brow_bytes() { return WF == kWfBF16 ? GK * 2 : WF == kWfMXFP4 ? GK / 2 : GK; }
template <int BM, int WF = kWfBF16>
constexpr int stage_bytes() { return BM * GK * 2 + GN * brow_bytes<WF>(); }
// MXFP4: the tile's E8M0 block-scale rows sit past the ring, one byte per 32
// weights of the contraction, at most this many per row.
constexpr int kMaxScaleCols = 256;
template <int WF>
constexpr int scale_bytes() { return WF == kWfMXFP4 ? GN * kMaxScaleCols : 0; }
template <int BM, int NSTAGE, int WF>
constexpr int loop_bytes() { return NSTAGE * stage_bytes<BM, WF>() + scale_bytes<WF>(); }
// Epilogue staging (the main loop's LDS, free after it): down stages 128
// rows x 256 fp32 per pass, gate_up all BM rows x 128 bf16 at once; rows are
// padded by 16 B.  The down tile's row slots and weights sit past both.
constexpr int kDnStageRows = 128, kDnStride = GN + 4;     // floats
constexpr int kGuStride = GN / 2 + 8;                     // bf16
template <bool GU, int BM, int NSTAGE, int WF>
constexpr int slots_offset() {
  return loop_bytes<BM, NSTAGE, WF>() > kDnStageRows * kDnStride * 4
             ? loop_bytes<BM, NSTAGE, WF>()
             : kDnStageRows * kDnStride * 4;
}
template <bool GU, int BM, int NSTAGE, int WF>
constexpr int gemm_lds_bytes() {
  return GU ? loop_bytes<BM, NSTAGE, WF>() : slots_offset<GU, BM, NSTAGE, WF>() + BM * 8;
}

__device__ __forceinline__ int gswz(int r, int c) { return c ^ ((r >> 2) & 3); }

// 16 stored codes of one weight row (a uint4; MXFP4: the low 8 bytes) ->
// the 8 bf16 values of half s: codes 8 s .. 8 s + 7 (MXFP4 times `scale`).
template <int WF>
__device__ __forceinline__ bf16x8 widen_half(const uint4& c, int s, float scale) {
  union {
    uint32_t u[4];
    bf16x8 v;
  } w;
  if constexpr (WF == kWfInt8) {
    int8x4_to_bf16(s ? c.z : c.x, w.u[0], w.u[1]);
    int8x4_to_bf16(s ? c.w : c.y, w.u[2], w.u[3]);
  } else if constexpr (WF == kWfFP8) {
    fp8x4_to_bf16(s ? c.z : c.x, w.u[0], w.u[1]);
    fp8x4_to_bf16(s ? c.w : c.y, w.u[2], w.u[3]);
  } else {
    fp4x8_to_bf16(s ? c.y : c.x, scale, w.u);
  }
  return w.v;
}

// GU: h[row] = GELU(A[row] . W0[n]) * (A[row] . W1[n]) for the block's 128
// columns n, A row = token of the slot (or the row itself when ident).
// !GU: y[slot] = w[slot] * (h[row] . W0[n]) for the block's 256 columns n.
// W0 / W1 hold the weights in the form WF; S0 / S1 their scales (int8, E4M3:
// fp32 per output channel n at e * s_stride + n; MXFP4: E8M0 rows of Kd / 32
// at e * s_stride + n * Kd / 32), w_stride counts weights between groups.
template <bool GU, int BM, int WM, int WN, int NSTAGE, typename YT, int WF>
__global__ __launch_bounds__(64 * WM * WN, 1) void grouped_gemm_kernel(
    int Kd, int Nout, int E, int K, int rows, int ident, int NT, const bf16* __restrict__ A,
    const void* __restrict__ W0v, const void* __restrict__ W1v, long long w_stride,
    const void* __restrict__ S0v, const void* __restrict__ S1v, long long s_stride,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_slots,
    const float* __restrict__ topk_w, bf16* __restrict__ hout, YT* __restrict__ yout) {
  constexpr bool NARROW = WF != kWfBF16;
  constexpr int SB = stage_bytes<BM, WF>();
  constexpr int NW = WM * WN, ROWS = BM + GN, LPW = ROWS / 16 / NW;
  constexpr int WR = BM / WM, WC = GN / WN, TM = WR / 32, TN = WC / 32;
  constexpr int NF = TM + TN, NMF = TM * TN;
  constexpr int RB = brow_bytes<WF>(), NBC = GN * RB / 1024;  // narrow: B copies per stage
  static_assert(LPW * NW * 16 == ROWS && NF <= NMF && LPW <= NMF, "tile shape");
  static_assert(!NARROW || (BM * GK * 2 == NW * 1024 && NBC <= NW && TN <= TM),
                "narrow weights: one A copy per wave, B copies by the first waves");
  static_assert(!GU || TN % 2 == 0, "gate_up waves need gate/up column pairs");
  static_assert(NSTAGE >= 3 && gemm_lds_bytes<GU, BM, NSTAGE, WF>() <= 160 * 1024, "LDS");
  static_assert(!GU || BM * kGuStride * 2 <= NSTAGE * SB, "gate_up staging fits the ring");
  static_assert(GU || BM % kDnStageRows == 0, "down staging passes");
  static_assert((BM * (GN / 16)) % (64 * NW) == 0 && (kDnStageRows * (GN / 4)) % (64 * NW) == 0,
                "epilogue store loops cover the staged rows exactly");
  extern __shared__ __align__(16) unsigned char smem[];
  const uint8_t* W0 = static_cast<const uint8_t*>(W0v);
  const uint8_t* W1 = static_cast<const uint8_t*>(W1v);

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
    if (ident) {
      nt = item % NT;
      row0 = item / NT * BM;
      row1 = min(row0 + BM, rows);
    } else {
      // down at 8192 skewed tokens 436 -> 414 us against column tiles fastest
      weight_major_item(sc, offsets, BM, item, NT, e, row0, row1, nt);
    }
  }
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int wm = wave / WN, wn = wave % WN;
  const int nbase = GU ? nt * (GN / 2) : nt * GN;
  // B row br of the tile -> its output column and weight matrix (W0 / W1)
  auto bcol = [&](int br, bool& up) {
    int n;
    if (GU) {
      n = nbase + br % (GN / 2);
      up = br >= GN / 2;
    } else {
      n = nbase + br;
      up = false;
    }
    return n < Nout ? n : 0;  // past the last column: a valid row, output dropped
  };
  // down: output slot and routing weight of each of the tile's rows, fetched
  // now (behind the main loop) into LDS past the loop's, for the epilogue
  int* row_slot = reinterpret_cast<int*>(smem + slots_offset<GU, BM, NSTAGE, WF>());
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
  // MXFP4: the tile's block-scale rows into LDS past the ring
  const int nsb = Kd / 32;
  uint8_t* sS = smem + NSTAGE * SB;
  if constexpr (WF == kWfMXFP4) {
    const uint8_t* S0 = static_cast<const uint8_t*>(S0v);
    const uint8_t* S1 = static_cast<const uint8_t*>(S1v);
    for (int i = threadIdx.x; i < GN * nsb; i += 64 * NW) {
      const int br = i / nsb, c = i % nsb;
      bool up;
      const int n = bcol(br, up);
      sS[i] = (up ? S1 : S0)[(size_t)e * s_stride + (size_t)n * nsb + c];
    }
  }
  const int nk = Kd / GK;

  // bf16 copies: copy q of a stage fills LDS rows 16 q .. 16 q + 15; lane ->
  // row 16 q + lane / 4, position lane % 4.  This lane's LPW copies per k-tile:
  const bf16* src[LPW];
  // narrow copies: A rows 16 wave .. (as above), B rows of copy `wave`
  const uint8_t* srcA = nullptr;
  const uint8_t* srcB = nullptr;
  auto a_row = [&](int r) {
    int gr = row0 + r;
    if (gr >= row1) gr = row0;  // past the tile: re-read a valid row, output dropped
    const int arow = GU && !ident ? sorted_slots[gr] / K : gr;
    return A + (size_t)arow * Kd;
  };
  if constexpr (!NARROW) {
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int q = wave * LPW + j;
      const int r = 16 * q + lane / 4;
      const int c = gswz(r, lane % 4);
      const bf16* p;
      if (r < BM) {
        p = a_row(r);
      } else {
        bool up;
        const int n = bcol(r - BM, up);
        p = reinterpret_cast<const bf16*>(up ? W1 : W0) + (size_t)e * w_stride + (size_t)n * Kd;
      }
      src[j] = p + c * 8;
    }
  } else {
    const int r = 16 * wave + lane / 4;
    srcA = reinterpret_cast<const uint8_t*>(a_row(r)) + gswz(r, lane % 4) * 16;
    if (wave < NBC) {
      constexpr int LPR = RB / 16;  // lanes per B row: 2 (8-bit), 1 (MXFP4)
      const int br = (1024 / RB) * wave + lane / LPR;
      bool up;
      const int n = bcol(br, up);
      constexpr int UNIT = WF == kWfMXFP4 ? 2 : 1;  // weights per byte
      const uint8_t* row = (up ? W1 : W0) + ((long long)e * w_stride + (long long)n * Kd) / UNIT;
      // 8-bit rows: the two 16-B chunks swap places on every other 8-row band
      srcB = row + (LPR == 2 ? ((lane % 2) ^ ((br >> 3) & 1)) * 16 : 0);
    }
  }
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
  auto copy_q = [&](int kt) {
    const int ktc = kt < nk ? kt : nk - 1;
    unsigned char* st = smem + (kt % NSTAGE) * SB;
#if defined(__HIP_DEVICE_COMPILE__)
    lds_copy16(srcA + ktc * (GK * 2), st + wave * 1024);
    if (wave < NBC) lds_copy16(srcB + ktc * RB, st + BM * GK * 2 + wave * 1024);
#endif
  };
  // narrow: the copies in flight past the last `tiles` k-tiles' (per wave)
  auto wait_ring = [&](auto tiles_tag) {
    constexpr int TL = decltype(tiles_tag)::value;
    if (wave < NBC)
      wait_vmem<2 * TL>();
    else
      wait_vmem<TL>();
  };

  // Fragment byte offsets within a stage, per k16 half s: A sub-tiles 0..TM-1,
  // then B sub-tiles (gate_up: gate halves first, then up).  Narrow weights:
  // B holds one offset per sub-tile (all 32 k values of the lane's run).
  const int fr = lane % 32, fq = lane / 32;
  int off[2][NF];
  int brow[TN];  // B row of each sub-tile (MXFP4 scale rows)
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = wm * WR + i * 32 + fr;
      off[s][i] = r * 64 + gswz(r, NARROW ? 2 * fq + s : 2 * s + fq) * 16;
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      int r;
      if (GU) {
        constexpr int half = TN / 2;
        r = (j < half ? 0 : GN / 2) + wn * (WC / 2) + (j % half) * 32 + fr;
      } else {
        r = wn * WC + j * 32 + fr;
      }
      brow[j] = r;
      if constexpr (!NARROW)
        off[s][TM + j] = (BM + r) * 64 + gswz(BM + r, 2 * s + fq) * 16;
      else if constexpr (WF == kWfMXFP4)
        off[s][TM + j] = BM * 64 + r * RB + 8 * fq;
      else
        off[s][TM + j] = BM * 64 + r * RB + 16 * (fq ^ ((r >> 3) & 1));
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
    if constexpr (!NARROW) {
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
    } else {
      // B codes of the current tile for every sub-tile (and MXFP4 scales)
      uint4 bc[TN];
      float bs[TN];
      auto rd_b = [&](const unsigned char* st, int kt, int j) {
        if constexpr (WF == kWfMXFP4) {
          const uint2 v = *reinterpret_cast<const uint2*>(st + off[0][TM + j]);
          bc[j] = make_uint4(v.x, v.y, 0u, 0u);
          bs[j] = e8m0_to_f32(sS[brow[j] * nsb + min(kt, nk - 1)]);
        } else {
          bc[j] = *reinterpret_cast<const uint4*>(st + off[0][TM + j]);
          bs[j] = 1.0f;
        }
      };
#pragma unroll
      for (int s = 0; s < NSTAGE; ++s) copy_q(s);
      wait_ring(std::integral_constant<int, NSTAGE - 1>{});
      wait_lds();  // the MXFP4 scale rows
      block_barrier();
#pragma unroll
      for (int i = 0; i < TM; ++i) rd(smem, 0, i, f0);
#pragma unroll
      for (int j = 0; j < TN; ++j) rd_b(smem, 0, j);
      wait_lds();
#pragma unroll
      for (int j = 0; j < TN; ++j) f0[TM + j] = widen_half<WF>(bc[j], 0, bs[j]);
      __builtin_amdgcn_sched_barrier(0);
      for (int kt = 0; kt < nk; ++kt) {
        const unsigned char* st = smem + (kt % NSTAGE) * SB;
        const unsigned char* sn = smem + ((kt + 1) % NSTAGE) * SB;
        // first half: MFMAs on f0; this tile's second-half A fragments; the
        // second half of the B codes widened
#pragma unroll
        for (int m = 0; m < NMF; ++m) {
          if (m < TM) rd(st, 1, m, f1);
          mf(m, f0);
          if (m < TN) f1[TM + m] = widen_half<WF>(bc[m], 1, bs[m]);
          __builtin_amdgcn_sched_barrier(0);
        }
        wait_lds();
        wait_ring(std::integral_constant<int, NSTAGE - 2>{});
        block_barrier();
        __builtin_amdgcn_sched_barrier(0);
        // second half: MFMAs on f1; tile kt+1's first-half A fragments and B
        // codes; the copies of tile kt+NSTAGE
#pragma unroll
        for (int m = 0; m < NMF; ++m) {
          if (m < TM) rd(sn, 0, m, f0);
          if (m < TN) rd_b(sn, kt + 1, m);
          mf(m, f1);
          if (m == NMF - 1) copy_q(kt + NSTAGE);
          __builtin_amdgcn_sched_barrier(0);
        }
        wait_lds();
#pragma unroll
        for (int j = 0; j < TN; ++j) f0[TM + j] = widen_half<WF>(bc[j], 0, bs[j]);
      }
      wait_vmem<0>();
    }
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
  constexpr bool CHS = WF == kWfInt8 || WF == kWfFP8;  // channel scales
  if constexpr (GU) {
    constexpr int half = TN / 2;
    float sg[half], su[half];
#pragma unroll
    for (int j = 0; j < half; ++j) {
      sg[j] = su[j] = 1.0f;
      if constexpr (CHS) {
        const int n = min(nbase + wn * (WC / 2) + j * 32 + fr, Nout - 1);
        sg[j] = static_cast<const float*>(S0v)[(size_t)e * s_stride + n];
        su[j] = static_cast<const float*>(S1v)[(size_t)e * s_stride + n];
      }
    }
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
          float g = acc[i][j][q], u = acc[i][j + half][q];
          if constexpr (CHS) {
            g *= sg[j];
            u *= su[j];
          }
          stg[r * kGuStride + c] = (bf16)(gelu_tanh(g) * u);
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
    float sd[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      sd[j] = 1.0f;
      if constexpr (CHS) {
        const int n = min(nbase + wn * WC + j * 32 + fr, Nout - 1);
        sd[j] = static_cast<const float*>(S0v)[(size_t)e * s_stride + n];
      }
    }
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
              float v = acc[i][j][q];
              if constexpr (CHS) v *= sd[j];
              stg[r * kDnStride + wn * WC + j * 32 + fr] = v;
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
            // streaming stores: the slot rows (369 MB at 4096 tokens) are read
            // once, by the combine, long after; 4096 / 8192 skewed tokens
            // 260 -> 248 / 417 -> 400 us
            const f32x4 o = {sc * v.x, sc * v.y, sc * v.z, sc * v.w};
            __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(dst));
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

}  // namespace

namespace {

template <bool GU, int BM, int WM, int WN, int NSTAGE, typename YT, int WF>
hipError_t launch_grouped(int Kd, int Nout, int E, int K, int rows, bool ident, int RT, int NT,
                          const bf16* A, const void* W0, const void* W1, long long w_stride,
                          const void* S0, const void* S1, long long s_stride,
                          const int32_t* offsets, const int32_t* sorted_slots,
                          const float* topk_w, bf16* hout, YT* yout, hipStream_t s,
                          hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr) {
  auto kf = grouped_gemm_kernel<GU, BM, WM, WN, NSTAGE, YT, WF>;
  // ring (+ MXFP4 scale rows) or staging (+ row slots, weights)
  const int lds = gemm_lds_bytes<GU, BM, NSTAGE, WF>();
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kf), hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  launch_maybe_timed(kf, dim3(RT * NT), dim3(64 * WM * WN), lds, s, ev_start, ev_stop, Kd, Nout, E,
                     K, rows, (int)ident, NT, A, W0, W1, w_stride, S0, S1, s_stride, offsets,
                     sorted_slots, topk_w, hout, yout);
  return hipSuccess;
}

// Ring depth of the tiled gate_up: bf16 takes 5 stages of 32 KB, the whole
// 160 KB of LDS (2048 tokens 302 -> 280 us, 4096 skewed 428 -> 420 against
// 4 stages); int8 and E4M3 (24 KB stages) take 6 (int8 at 2048 tokens 353 ->
// 306 us); MXFP4 keeps 4, its scale rows sitting past the ring.  down stays
// at 4 stages in every format (6 were 2-5% slower for int8 and E4M3).
template <int WF>
constexpr int gate_up_stages() { return WF == kWfBF16 ? 5 : WF == kWfMXFP4 ? 4 : 6; }

template <int WF>
hipError_t launch_gate_up_tiled(const GateUpArgs& a, hipStream_t s) {
  const int NT = (a.N + GN / 2 - 1) / (GN / 2);
  // bf16 expert groups of 256 rows or more on average: 8 waves of 128 x 64
  // (a quarter fewer fragment reads per MFMA), bit-identical; over three A/B
  // runs 4096 skewed tokens 487 -> 478 us, 8192 skewed 761 -> 750, one full
  // group of 32768 rows 298 -> 289.  Groups of ~128 rows leave half of such a
  // tile's waves idle, one wave per SIMD, and there the 16 waves of 64 x 64
  // win (2048 tokens 306 against 318 us); the dense branch keeps them too.
  if constexpr (WF == kWfBF16) {
    if (!a.ident && (long long)a.rows >= 256LL * a.E)
      return launch_grouped<true, 256, 2, 4, gate_up_stages<WF>(), float, WF>(
          a.H, a.N, a.E, a.K, a.rows, a.ident, tile_count_bound(a.ident, a.rows, a.T, a.E, 256),
          NT, static_cast<const bf16*>(a.x), a.w_gate, a.w_up, a.w_stride, a.s_gate, a.s_up,
          a.s_stride, a.offsets, a.sorted_slots, nullptr, static_cast<bf16*>(a.h),
          static_cast<float*>(nullptr), s, a.ev_start, a.ev_stop);
  }
  return launch_grouped<true, 256, 4, 4, gate_up_stages<WF>(), float, WF>(
      a.H, a.N, a.E, a.K, a.rows, a.ident, tile_count_bound(a.ident, a.rows, a.T, a.E, 256), NT,
      static_cast<const bf16*>(a.x), a.w_gate, a.w_up, a.w_stride, a.s_gate, a.s_up, a.s_stride,
      a.offsets, a.sorted_slots, nullptr, static_cast<bf16*>(a.h), static_cast<float*>(nullptr),
      s, a.ev_start, a.ev_stop);
}

template <typename YT, int WF>
hipError_t launch_down_tiled(const DownArgs& a, hipStream_t s) {
  const int NT = (a.H + GN - 1) / GN;
  return launch_grouped<false, 256, 4, 4, 4, YT, WF>(
      a.N, a.H, a.E, a.K, a.rows, a.ident, tile_count_bound(a.ident, a.rows, a.T, a.E, 256), NT,
      static_cast<const bf16*>(a.h), a.w_down, a.w_down, a.w_stride, a.s_down, a.s_down,
      a.s_stride, a.offsets, a.sorted_slots, a.topk_w, nullptr, static_cast<YT*>(a.y), s);
}

template <typename YT>
hipError_t launch_down_tiled_fmt(const DownArgs& a, hipStream_t s) {
  switch (a.w_fmt) {
    case WFormat::kBF16: return launch_down_tiled<YT, kWfBF16>(a, s);
    case WFormat::kInt8: return launch_down_tiled<YT, kWfInt8>(a, s);
    case WFormat::kFP8: return launch_down_tiled<YT, kWfFP8>(a, s);
    case WFormat::kMXFP4: return launch_down_tiled<YT, kWfMXFP4>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool quant_uses_stream_kernels(int T) { return T <= kMaxQuantStreamTokens; }

hipError_t launch_gate_up(const GateUpArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  if (a.w_fmt != WFormat::kBF16) {
    if (!a.bf16) return hipErrorInvalidValue;
    if (quant_uses_stream_kernels(a.T)) return launch_gate_up_stream(a, s);
    switch (a.w_fmt) {
      case WFormat::kInt8: return launch_gate_up_tiled<kWfInt8>(a, s);
      case WFormat::kFP8: return launch_gate_up_tiled<kWfFP8>(a, s);
      case WFormat::kMXFP4: return launch_gate_up_tiled<kWfMXFP4>(a, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (a.bf16 && use_stream_kernels(a.T, a.rows, a.E, a.ident)) return launch_gate_up_stream(a, s);
  if (a.bf16) {
    const hipError_t e = launch_gate_up_tiled<kWfBF16>(a, s);
    if (e != hipSuccess) return e;
  } else {
    dim3 grid(tile_count_bound(a.ident, a.rows, a.T, a.E, kFT), (a.N + kFT - 1) / kFT);
    launch_maybe_timed(gate_up_f32_kernel, grid, dim3(256), 0, s, a.ev_start, a.ev_stop, a.H, a.N,
                       a.E, a.K, a.rows, (int)a.ident, static_cast<const float*>(a.x),
                       static_cast<const float*>(a.w_gate), static_cast<const float*>(a.w_up),
                       a.w_stride, a.offsets, a.sorted_slots, static_cast<float*>(a.h));
  }
  return hipGetLastError();
}

hipError_t launch_down(const DownArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  if (a.w_fmt != WFormat::kBF16) {
    if (!a.bf16) return hipErrorInvalidValue;
    if (quant_uses_stream_kernels(a.T)) return launch_down_stream(a, s);
  } else if (a.bf16 && use_stream_kernels(a.T, a.rows, a.E, a.ident)) {
    return launch_down_stream(a, s);
  }
  if (a.bf16) {
    const hipError_t e =
        a.y_bf16 ? launch_down_tiled_fmt<bf16>(a, s) : launch_down_tiled_fmt<float>(a, s);
    if (e != hipSuccess) return e;
  } else {
    dim3 grid(tile_count_bound(a.ident, a.rows, a.T, a.E, kFT), (a.H + 2 * kFT - 1) / (2 * kFT));
    hipLaunchKernelGGL(down_f32_kernel, grid, dim3(256), 0, s, a.H, a.N, a.E, a.rows,
                       (int)a.ident, static_cast<const float*>(a.h),
                       static_cast<const float*>(a.w_down), a.w_stride, a.offsets,
                       a.sorted_slots, a.topk_w, static_cast<float*>(a.y));
  }
  return hipGetLastError();
}

}  // namespace moe
