// Decode-sized grouped expert GEMMs (few rows per expert): weight streaming.
//
// At decode batch sizes an expert sees a handful of rows, so the two expert
// GEMMs are bound by reading each touched expert's weights from HBM once
// (gate_up [2I, H] and down [H, I] of the page "Porting a 128-expert MoE
// (Gemma-4 26B-A4B) to AWS Inferentia2", section "The architecture: a
// dual-path FFN nobody warned me about").  These kernels keep the weight
// operand out of LDS: per k-block every lane loads 32 contiguous bytes of
// one weight row straight into registers (four lanes cover a 128-byte line,
// which is then used whole) and feeds them to v_mfma_f32_16x16x32_bf16 in
// 8-element operands; the activation rows (at most 16 * MB per tile,
// resident in L2) are loaded the same way.  Loads run NS - 1 k-blocks ahead
// of the MFMAs (a register ring).  A block's waves split the contraction;
// their partial sums meet in LDS and are added in wave order
// (deterministic), then the epilogue applies GELU-tanh(gate) * up (gate_up)
// or the routing weight and the slot scatter (down).
//
// k mapping: a lane's span is L = 32 bytes of weights (L = 16 bf16, 32 int8
// or E4M3, 64 MXFP4 weights); a k-block is 4 L.  In k-block kb, lane l (row
// or column l % 16, group g = l / 16) holds k = 4 L kb + L g + [0, L); MFMA j
// of the block uses its elements [8 j, 8 j + 8).  A and B use the same
// mapping, so the 2 L / 16 MFMAs of a block sum over all of its k.
// Contraction lengths are multiples of 32, so each 16-element sub-group of a
// span is either wholly inside or wholly past the end.
//
// Weights below bf16 (int8, E4M3, MXFP4; wformat.h) are loaded as stored
// and widened to bf16 in registers right before their MFMAs.  With
// 16-element spans for every format, a line of an int8 or MXFP4 row was
// used by 2 or 4 successive k-blocks, microseconds apart, and the L2 dropped
// it in between: 17% and 45% more HBM reads than the weights.
//
// The loads carry no conditions in the steady state of the k-loop (clamped
// addresses instead, see the kernels).  A load under a condition leaves the
// compiler unsure how many loads are outstanding on each path, and it then
// waits for all of them before every MFMA: the ring was being drained at
// every k-block.
#include "common.h"
#include "launch.h"
#include "wformat.h"

#include <type_traits>

namespace moe {
namespace {

typedef W16 Frag;  // 16 bf16 activations of one row

// Block scales (MXFP4) of the weight rows a block streams, staged in LDS at
// block start: one E8M0 byte per 32 weights of a row, contraction up to
// 32 * kMaxScaleRow.  Read from HBM once per block instead of once per
// k-block and row (their cache lines would not survive the weight stream).
constexpr int kMaxScaleRow = 256;

// Copies n_rows scale rows of row_bytes each, consecutive in memory from
// src (rows past valid_rows are left unset and never read: the kernels clamp
// their row index), into dst; ends with a barrier.
__device__ __forceinline__ void stage_scales(uint8_t* dst, const uint8_t* src, int n_rows,
                                             int valid_rows, int row_bytes) {
  const int n = min(n_rows, max(valid_rows, 0)) * row_bytes;
  for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = src[i];
  __syncthreads();
}

__device__ __forceinline__ void ld_frag(Frag& f, const bf16* p) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int i = 0; i < 2; ++i) f.u[i] = q[i];
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// gate_up: one block = one row tile (<= 16 * MB rows) x NC groups of 16 gate
// + 16 up columns; its WK waves split H.  A wave's activation fragments serve
// all NC groups, so narrow weight formats stream more bytes per wave.
template <typename WQ, int WK, int MB, int NS, int NC>
__global__ __launch_bounds__(64 * WK) void gate_up_stream_kernel(
    int H, int N, int E, int K, int rows, int ident, const bf16* __restrict__ x,
    const WQ* __restrict__ wg, const WQ* __restrict__ wu, long long w_stride,
    const void* __restrict__ sg, const void* __restrict__ su, long long s_stride,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_slots,
    bf16* __restrict__ h) {
  typedef WFmt<WQ> F;
  static_assert(NS >= 2, "the load ring needs two slots or more");
  __shared__ f32x4 red[WK][MB][NC][2][kWave];
  // gate and up block scales of the block's 16 * NC rows (MXFP4 only)
  __shared__ uint8_t ssc[F::kBlockScale ? 2 * 16 * NC * kMaxScaleRow : 1];
  int e, row0, row1, cg;
  const int CG = (N + 16 * NC - 1) / (16 * NC);
  if (!stream_item(ident, rows, offsets, E, 16 * MB, CG, e, row0, row1, cg)) return;
  if constexpr (F::kBlockScale) {
    const long long first = (long long)e * s_stride + (long long)cg * 16 * NC * (H / 32);
    const int valid = N - cg * 16 * NC;
    stage_scales(ssc, static_cast<const uint8_t*>(sg) + first, 16 * NC, valid, H / 32);
    stage_scales(ssc + 16 * NC * (H / 32), static_cast<const uint8_t*>(su) + first, 16 * NC,
                 valid, H / 32);
  }
  constexpr int LK = F::kLaneK, U = LK / 16, KBK = 4 * LK;
  const int lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int fr = lane % 16, fg = lane / 16;
  const int n0 = cg * 16 * NC + fr;  // column of group c: n0 + 16 c
  // Every load below is unconditional and in bounds.  A column past N (a
  // ragged last group) reads row N - 1 and a row past row1 reads row row0:
  // their MFMA outputs are never stored.  A weight span past the end of the
  // contraction (only in a ragged last k-block) re-reads the row's last span
  // that starts inside, part of the lines this k-block reads anyway, and is
  // zeroed where it is used.  (Re-reading k = 0 instead fetched the row's
  // first line a second time, long after the first: the int8 / E4M3 down
  // projection, 704 long, read 1.15x its bytes.)
  const int klast = (H - 1) / LK * LK;  // start of the row's last span
  long long wel[NC];  // first element of the weight row of column n0 + 16 c
  const uint8_t* gsr[NC];
  const uint8_t* usr[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    wel[c] = (long long)e * w_stride + (long long)min(n0 + 16 * c, N - 1) * H;
    gsr[c] = usr[c] = nullptr;
    if constexpr (F::kBlockScale) {
      const int sr = min(16 * c + fr, N - 1 - cg * 16 * NC);  // staged rows only
      gsr[c] = ssc + sr * (H / 32);
      usr[c] = ssc + (16 * NC + sr) * (H / 32);
    }
  }
  const int nmb = (row1 - row0 + 15) / 16;  // active 16-row blocks (uniform)
  const bf16* ap[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int r = row0 + 16 * mb + fr, rr = r < row1 ? r : row0;
    const int tok = ident ? rr : sorted_slots[rr] / K;
    ap[mb] = x + (size_t)tok * H;
  }
  const int KB = (H + KBK - 1) / KBK;
  const int kb0 = wave * KB / WK, kb1 = (wave + 1) * KB / WK;

  f32x4 accg[MB][NC], accu[MB][NC];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      accg[mb][c] = f32x4{0, 0, 0, 0};
      accu[mb][c] = f32x4{0, 0, 0, 0};
    }
  WRaw<WQ> bg[NS][NC], bu[NS][NC];
  Frag ba[NS][MB][U];
  auto load = [&](int kb, int slot) {
    const int ks = kb * KBK + LK * fg;  // first weight of this lane's span
    const bool kv = ks < H;
    const int kc = kv ? ks : klast;          // in-bounds start
    const bool kfull = kc + LK <= H;       // else only its first half lies inside
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      bg[slot][c].load(wrow(wg, wel[c]), kc, gsr[c], kfull);
      bu[slot][c].load(wrow(wu, wel[c]), kc, usr[c], kfull);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      if (mb == 0 || mb < nmb)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int ku = kc + 16 * u;
          ld_frag(ba[slot][mb][u], ap[mb] + (ku < H ? ku : 0));
        }
  };
  // NS steps: step s loads k-block kb + s + NS - 1 into its ring slot, then
  // runs the MFMAs of k-block kb + s.  In the steady state (kTail false)
  // every load is in range and unconditional, so the compiler's waits count
  // exactly the loads still outstanding and the ring stays in flight; the
  // tail (the last 2 NS - 2 k-blocks at most) checks the ends and masks the
  // ragged last k-block.
  auto steps = [&](int kb, auto tail) {
    constexpr bool kTail = decltype(tail)::value;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (kTail && kb + s >= kb1) break;
      const int kl = kb + s + NS - 1;
      if (!kTail || kl < kb1) load(kl, (s + NS - 1) % NS);
      if constexpr (!kTail) __builtin_amdgcn_sched_barrier(0);  // slots issued in order
      if (kTail && (kb + s + 1) * KBK > H) {  // uniform
        const int ks = (kb + s) * KBK + LK * fg;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          bg[s][c].mask(ks < H, ks + LK <= H);
          bu[s][c].mask(ks < H, ks + LK <= H);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const Frag fgt = bg[s][c].widen(u), fup = bu[s][c].widen(u);
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
              if (mb == 0 || mb < nmb) {
                accg[mb][c] = mfma16(ba[s][mb][u].v[j], fgt.v[j], accg[mb][c]);
                accu[mb][c] = mfma16(ba[s][mb][u].v[j], fup.v[j], accu[mb][c]);
              }
        }
      if constexpr (!kTail) __builtin_amdgcn_sched_barrier(0);
    }
  };
  // The ring's first slots, unconditionally and in order: a wave with fewer
  // k-blocks loads a valid one again and never uses it.  (After a load under
  // a condition the compiler's waits count as if it had not been issued, and
  // the steady state drained the ring at the top of every round.)
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) {
    load(max(min(kb0 + s, kb1 - 1), 0), s);
    __builtin_amdgcn_sched_barrier(0);
  }
  int kb = kb0;
  for (; kb + 2 * NS - 2 < kb1; kb += NS) steps(kb, std::false_type{});
  for (; kb < kb1; kb += NS) steps(kb, std::true_type{});
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      red[wave][mb][c][0][lane] = accg[mb][c];
      red[wave][mb][c][1][lane] = accu[mb][c];
    }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    if (mb >= nmb) break;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int n = n0 + 16 * c;
      const bool nvalid = n < N;
      f32x4 g = red[0][mb][c][0][lane], u = red[0][mb][c][1][lane];
#pragma unroll
      for (int w = 1; w < WK; ++w) {
        g += red[w][mb][c][0][lane];
        u += red[w][mb][c][1][lane];
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
}

// down: one block = one row tile x WN waves of NC groups of 16 output
// columns; WK waves split the contraction (the intermediate width N).  With
// AL the tile's activation rows (at most 16 * MB rows of h) are staged once
// in LDS (dynamic, rows padded by 16 B) and every wave reads its fragments
// there: the WN waves of a block share the same rows and k range, and a
// lane's activation loads were as large as its weight loads.
template <typename WQ, int WN, int WK, int MB, int NS, int NC, typename YT, bool AL>
__global__ __launch_bounds__(64 * WN * WK) void down_stream_kernel(
    int H, int N, int E, int rows, int ident, const bf16* __restrict__ hbuf,
    const WQ* __restrict__ wd, long long w_stride, const void* __restrict__ sd,
    long long s_stride, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_slots, const float* __restrict__ topk_w,
    YT* __restrict__ y) {
  typedef WFmt<WQ> F;
  static_assert(NS >= 2, "the load ring needs two slots or more");
  __shared__ f32x4 red[WK > 1 ? WN * WK : 1][MB][NC][kWave];
  // block scales of the block's 16 * WN * NC output rows (MXFP4 only)
  __shared__ uint8_t ssc[F::kBlockScale ? 16 * WN * NC * kMaxScaleRow : 1];
  int e, row0, row1, cg;
  const int CG = (H + 16 * WN * NC - 1) / (16 * WN * NC);
  if (!stream_item(ident, rows, offsets, E, 16 * MB, CG, e, row0, row1, cg)) return;
  if constexpr (F::kBlockScale)
    stage_scales(ssc,
                 static_cast<const uint8_t*>(sd) + (long long)e * s_stride +
                     (long long)cg * 16 * WN * NC * (N / 32),
                 16 * WN * NC, H - cg * 16 * WN * NC, N / 32);
  constexpr int LK = F::kLaneK, U = LK / 16, KBK = 4 * LK;
  const int lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wn = wave % WN, wk = wave / WN;
  const int fr = lane % 16, fg = lane / 16;
  const int n0 = (cg * WN + wn) * 16 * NC + fr;  // column of group c: n0 + 16 c
  // Unconditional in-bounds loads, as in gate_up: a column past H reads row
  // H - 1, a row past row1 reads row row0, a weight span past N re-reads the
  // row's last span that starts inside, zeroed where it is used.
  const int klast = (N - 1) / LK * LK;
  long long wel[NC];
  const uint8_t* bsr[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    wel[c] = (long long)e * w_stride + (long long)min(n0 + 16 * c, H - 1) * N;
    bsr[c] = nullptr;
    if constexpr (F::kBlockScale)
      bsr[c] = ssc + min(16 * (wn * NC + c) + fr, H - 1 - cg * 16 * WN * NC) * (N / 32);
  }
  const int nmb = (row1 - row0 + 15) / 16;
  // Output slot and routing weight of this lane's rows (rows past the tile
  // clamp to its last row), fetched behind the weight stream: the slots
  // before the ring's first loads, the weights after them.  In the epilogue
  // they were two dependent loads per row after the stream had ended.  The
  // loads carry no condition (the dense branch, which has neither array,
  // reads the first element of h instead and ignores it), so the ring's
  // waits stay exact.
  int oslot[MB][4];
  float ow[MB][4];
  {
    const int32_t* sp = ident ? reinterpret_cast<const int32_t*>(hbuf) : sorted_slots;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = min(row0 + 16 * mb + 4 * fg + r, row1 - 1);
        const int v = sp[ident ? 0 : row];
        oslot[mb][r] = ident ? row : v;
      }
  }
  extern __shared__ __align__(16) unsigned char dyn_lds[];
  const int ALS = N + 8;  // staged row pitch (bf16)
  const bf16* ap[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int r = row0 + 16 * mb + fr;
    if constexpr (AL)
      ap[mb] = reinterpret_cast<const bf16*>(dyn_lds) + (r < row1 ? r - row0 : 0) * ALS;
    else
      ap[mb] = hbuf + (size_t)(r < row1 ? r : row0) * N;
  }
  const int KB = (N + KBK - 1) / KBK;
  const int kb0 = wk * KB / WK, kb1 = (wk + 1) * KB / WK;

  f32x4 acc[MB][NC];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[mb][c] = f32x4{0, 0, 0, 0};
  WRaw<WQ> bb[NS][NC];
  Frag ba[NS][MB][U];
  auto load_w = [&](int kb, int slot) {
    const int ks = kb * KBK + LK * fg;  // first weight of this lane's span
    const bool kv = ks < N;
    const int kc = kv ? ks : klast;          // in-bounds start
    const bool kfull = kc + LK <= N;       // else only its first half lies inside
#pragma unroll
    for (int c = 0; c < NC; ++c) bb[slot][c].load(wrow(wd, wel[c]), kc, bsr[c], kfull);
  };
  auto load_a = [&](int kb, int slot) {
    const int ks = kb * KBK + LK * fg;
    const int kc = ks < N ? ks : 0;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      if (mb == 0 || mb < nmb)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int ku = kc + 16 * u;
          ld_frag(ba[slot][mb][u], ap[mb] + (ku < N ? ku : 0));
        }
  };
  auto load = [&](int kb, int slot) {
    load_w(kb, slot);
    load_a(kb, slot);
  };
  // The same steady state and tail as gate_up.
  auto steps = [&](int kb, auto tail) {
    constexpr bool kTail = decltype(tail)::value;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (kTail && kb + s >= kb1) break;
      const int kl = kb + s + NS - 1;
      if (!kTail || kl < kb1) load(kl, (s + NS - 1) % NS);
      if constexpr (!kTail) __builtin_amdgcn_sched_barrier(0);  // slots issued in order
      if (kTail && (kb + s + 1) * KBK > N) {  // uniform
        const int ks = (kb + s) * KBK + LK * fg;
#pragma unroll
        for (int c = 0; c < NC; ++c) bb[s][c].mask(ks < N, ks + LK <= N);
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const Frag fb = bb[s][c].widen(u);
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
              if (mb == 0 || mb < nmb) acc[mb][c] = mfma16(ba[s][mb][u].v[j], fb.v[j], acc[mb][c]);
        }
      if constexpr (!kTail) __builtin_amdgcn_sched_barrier(0);
    }
  };
  // the first k-blocks' weight loads go out before the activation staging,
  // unconditionally and in order (as in gate_up)
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) {
    load_w(max(min(kb0 + s, kb1 - 1), 0), s);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (AL) {
    // Loads in batches of four chunks, then their stores: one copy a chunk
    // at a time waited for each load before its store (a round trip per
    // chunk, ~6 per block at 704 columns).  A chunk index past the tile
    // stands for the last chunk, which it re-reads and stores again with the
    // same value: no condition, so the loads are not sunk to their stores.
    const int nrows = row1 - row0, cpr = N / 8;  // 16-B chunks per row
    const int n = nrows * cpr;
    constexpr int NT = 64 * WN * WK, kBatch = 4;
    bf16* al = reinterpret_cast<bf16*>(dyn_lds);
    for (int i0 = 0; i0 < n; i0 += kBatch * NT) {
      uint4 c[kBatch];
      int dst[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int i = min(i0 + (int)threadIdx.x + j * NT, n - 1);
        const int r = i / cpr, ch = i - r * cpr;
        c[j] = *reinterpret_cast<const uint4*>(hbuf + (size_t)(row0 + r) * N + ch * 8);
        dst[j] = r * ALS + ch * 8;
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) *reinterpret_cast<uint4*>(al + dst[j]) = c[j];
    }
    __syncthreads();
  }
  {
    const float* wp = ident ? reinterpret_cast<const float*>(hbuf) : topk_w;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = wp[ident ? 0 : oslot[mb][r]];
        ow[mb][r] = ident ? 1.0f : v;
      }
  }
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) load_a(max(min(kb0 + s, kb1 - 1), 0), s);
  int kb = kb0;
  for (; kb + 2 * NS - 2 < kb1; kb += NS) steps(kb, std::false_type{});
  for (; kb < kb1; kb += NS) steps(kb, std::true_type{});
  if constexpr (WK > 1) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int c = 0; c < NC; ++c) red[wave][mb][c][lane] = acc[mb][c];
    __syncthreads();
    if (wk != 0) return;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        acc[mb][c] = red[wn][mb][c][lane];
#pragma unroll
        for (int w = 1; w < WK; ++w) acc[mb][c] += red[wn + w * WN][mb][c][lane];
      }
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int n = n0 + 16 * c;
    const bool nvalid = n < H;
    float chs = 1.0f;
    if constexpr (F::kChannelScale)
      if (nvalid) chs = static_cast<const float*>(sd)[(size_t)e * s_stride + n];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (mb >= nmb) break;
      f32x4 v = acc[mb][c];
      if constexpr (F::kChannelScale) v *= chs;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + 16 * mb + 4 * fg + r;
        if (row >= row1 || !nvalid) continue;
        y[(size_t)oslot[mb][r] * H + n] = from_f32<YT>(ow[mb][r] * v[r]);
      }
    }
  }
}

template <typename WQ, int WK, int MB, int NS, int NC>
void launch_gu(const GateUpArgs& a, hipStream_t s) {
  const long long cgs = (a.N + 16 * NC - 1) / (16 * NC);
  dim3 grid((unsigned)(tile_count_bound(a.ident, a.rows, a.T, a.E, 16 * MB) * cgs));
  launch_maybe_timed(gate_up_stream_kernel<WQ, WK, MB, NS, NC>, grid, dim3(64 * WK), 0, s,
                     a.ev_start, a.ev_stop, a.H, a.N, a.E, a.K, a.rows, (int)a.ident,
                     static_cast<const bf16*>(a.x), static_cast<const WQ*>(a.w_gate),
                     static_cast<const WQ*>(a.w_up), a.w_stride, a.s_gate, a.s_up, a.s_stride,
                     a.offsets, a.sorted_slots, static_cast<bf16*>(a.h));
}

// Activation rows of a down tile staged in LDS while they and the block's
// staged MXFP4 scales take at most this many bytes (the 26B-A4B experts: 16
// rows x 712 bf16 = 22.8 KB; MXFP4's 32 KB of scales leave it out, since
// fewer blocks per CU made it slower), above 8 tokens: at 64 tokens bf16
// down went 102 -> 97 us; at 8 tokens the staging's fixed cost made it
// slower (40 -> 44 us).
constexpr int kDnActLdsMax = 32 * 1024;
constexpr int kDnActLdsMinTokens = 9;

template <typename WQ, int WN, int WK, int MB, int NS, int NC, typename YT>
void launch_dn(const DownArgs& a, hipStream_t s) {
  const long long cgs = (a.H + 16 * WN * NC - 1) / (16 * WN * NC);
  dim3 grid((unsigned)(tile_count_bound(a.ident, a.rows, a.T, a.E, 16 * MB) * cgs));
  const int al = 16 * MB * (a.N + 8) * 2;
  const int scales = WFmt<WQ>::kBlockScale ? 16 * WN * NC * kMaxScaleRow : 0;
  if (al + scales <= kDnActLdsMax && a.T >= kDnActLdsMinTokens)
    hipLaunchKernelGGL((down_stream_kernel<WQ, WN, WK, MB, NS, NC, YT, true>), grid,
                       dim3(64 * WN * WK), al, s, a.H, a.N, a.E, a.rows, (int)a.ident,
                       static_cast<const bf16*>(a.h), static_cast<const WQ*>(a.w_down),
                       a.w_stride, a.s_down, a.s_stride, a.offsets, a.sorted_slots, a.topk_w,
                       static_cast<YT*>(a.y));
  else
    hipLaunchKernelGGL((down_stream_kernel<WQ, WN, WK, MB, NS, NC, YT, false>), grid,
                       dim3(64 * WN * WK), 0, s, a.H, a.N, a.E, a.rows, (int)a.ident,
                       static_cast<const bf16*>(a.h), static_cast<const WQ*>(a.w_down),
                       a.w_stride, a.s_down, a.s_stride, a.offsets, a.sorted_slots, a.topk_w,
                       static_cast<YT*>(a.y));
}

template <typename YT>
void launch_dn_t(const DownArgs& a, hipStream_t s) {
  switch (a.w_fmt) {
    // the dense branch (ident): 64-row tiles and the contraction split over 4
    // waves, as for its bf16 form (the int8 layer at 64 tokens: 211 -> 207 us)
    case WFormat::kInt8:
      if (a.ident) launch_dn<int8_t, 2, 4, 4, 2, 1, YT>(a, s);
      else launch_dn<int8_t, 4, 1, 1, 2, 1, YT>(a, s);
      return;
    case WFormat::kFP8:
      if (a.ident) launch_dn<fp8e4m3, 2, 4, 4, 2, 1, YT>(a, s);
      else launch_dn<fp8e4m3, 4, 1, 1, 2, 1, YT>(a, s);
      return;
    case WFormat::kMXFP4: launch_dn<fp4x2, 4, 1, 1, 2, 2, YT>(a, s); return;
    case WFormat::kBF16: break;
  }
  // up to 8 tokens: two 16-column groups per wave (1 token: 11.7 -> 9.1 us)
  if (a.T <= 8) launch_dn<bf16, 4, 1, 1, 2, 2, YT>(a, s);
  else launch_dn<bf16, 4, 1, 1, 2, 1, YT>(a, s);
}

}  // namespace

// Weight streaming pays while every expert's row group is a few 16-row
// tiles: for the expert groups at most 256 tokens and at most 16 rows per
// expert on average (top-8 of 128 experts: 256 tokens; the all-experts
// layout has T rows per expert, and takes the tiled GEMMs past 16 tokens).
// On the 26B-A4B experts the streaming pair beats the tiled GEMMs at every
// size up to that limit (256 tokens: 203 + 124 us against 218 + 131) and
// loses past it (512 tokens: 261 + 173 against 225 + 141).  The dense
// branch (one 2112-wide MLP) streams its weights once per 32-row tile, and
// the tiled GEMMs win there past 64 tokens.
bool use_stream_kernels(int T, int rows, int E, bool ident) {
  return ident ? T <= 64 : (T <= 256 && rows <= 16 * E);
}

// The dense branch (ident) at <= 64 tokens takes 32-row tiles (its weights
// are streamed once per tile, the second time mostly from L2); its down
// projection splits the contraction over 4 waves to keep enough loads in
// flight.
hipError_t launch_gate_up_stream(const GateUpArgs& a, hipStream_t s) {
  switch (a.w_fmt) {
    // past 128 tokens (8 rows per expert on average) 32-row tiles: at 256
    // tokens int8 / E4M3 / MXFP4 experts 238 / 234 / 279 -> 222 / 218 / 262 us
    case WFormat::kInt8:
      if (a.T <= 128) launch_gu<int8_t, 2, 1, 3, 1>(a, s);
      else launch_gu<int8_t, 2, 2, 3, 1>(a, s);
      break;
    case WFormat::kFP8:
      if (a.T <= 128) launch_gu<fp8e4m3, 2, 1, 3, 1>(a, s);
      else launch_gu<fp8e4m3, 2, 2, 3, 1>(a, s);
      break;
    case WFormat::kMXFP4:
      if (a.T <= 128) launch_gu<fp4x2, 1, 1, 2, 1>(a, s);
      else launch_gu<fp4x2, 1, 2, 2, 1>(a, s);
      break;
    case WFormat::kBF16:
      if (a.ident) launch_gu<bf16, 8, 2, 2, 1>(a, s);
      else if (a.T <= 64) launch_gu<bf16, 4, 1, 4, 1>(a, s);
      else launch_gu<bf16, 4, 2, 3, 1>(a, s);  // 16 rows per expert at 128 tokens
      break;
  }
  return hipGetLastError();
}

hipError_t launch_down_stream(const DownArgs& a, hipStream_t s) {
  if (a.ident && a.w_fmt == WFormat::kBF16) {
    if (a.y_bf16) launch_dn<bf16, 2, 4, 2, 2, 1, bf16>(a, s);
    else launch_dn<bf16, 2, 4, 2, 2, 1, float>(a, s);
  } else if (a.y_bf16) {
    launch_dn_t<bf16>(a, s);
  } else {
    launch_dn_t<float>(a, s);
  }
  return hipGetLastError();
}

}  // namespace moe
