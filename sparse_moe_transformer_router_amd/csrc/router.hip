// Router of the Gemma-4 26B-A4B mixture-of-experts block (Gemma4TextRouter on
// the page "Porting a 128-expert MoE (Gemma-4 26B-A4B) to AWS Inferentia2",
// section "The architecture: a dual-path FFN nobody warned me about"): an
// RMSNorm of its own, a scale, the H -> E projection, softmax in fp32, top-K,
// renormalisation over the K, times per_expert_scale.
//
// Routing must come out bit-identical on any IEEE fp32 machine, so every
// reduction over H follows one fixed order: 64-element chunks, each a fused
// multiply-add chain in ascending index from +0, the chunk results added in
// ascending chunk order from +0.  Division and square root are the correctly
// rounded ones (HIP's default for sqrtf and '/'), and contraction is off in
// this file so that products written separately stay separate.
//
// Small batches (T <= 448, H <= 3072) take two kernels:
//   router_logits_small  a block takes up to 4 tokens and 4 * EW experts.  Each
//                 wave first issues the loads of its EW experts' weights (lane
//                 c holds chunk c in registers), then one wave per token
//                 computes the norms (lane c runs chunk c's chain, lane 0 adds
//                 the chunk results in order) and writes the normalised,
//                 scaled input to LDS in a padded [chunk][65] layout; every
//                 lane then runs its chunk's chains against LDS, and one lane
//                 per (token, expert) adds the chunk results in order;
//   route_topk_dispatch  one wave per token over several blocks; when asked
//                 and T*K <= 1024, the last block to finish groups the slots
//                 (else the dispatch kernels of dispatch.hip follow).
// Large batches take three:
//   router_prep   one wave per token: the inverse RMS of x (and, with a
//                 pre-norm gain, of v = x * r0 * gain), in the fixed order;
//   router_logits_split  (E % 4 == 0) a block takes 32 tokens x 64 experts;
//                 each chunk's weights are read from [E, H] and transposed
//                 in registers on their way into LDS; a thread 4
//                 tokens x 4 experts (16 chains, one 16-B weight and one 16-B
//                 input LDS read per 16 fmas); the block's G wave groups take
//                 the chunks in turn (chunk c to group c % G), and the
//                 groups' chunk results meet in LDS, where group 0 adds them
//                 in chunk order;
//   router_logits_tiled  (E % 4 != 0) a block takes 64 tokens x 32 experts,
//                 lane = token, the expert weights read as LDS broadcasts;
//   router_topk   one wave per token.
// Top-K (route_dev.h): experts in descending logit order, ties to the lower
// index, found with wave-wide DPP maxima of order-preserving keys; weights
// z_k / sum z with z = exp(l - max l), times per_expert_scale.
#include "launch.h"
#include "route_dev.h"

#pragma clang fp contract(off)

namespace moe {
namespace {

constexpr int kChunk = 64;

__device__ __forceinline__ void load8(const float* p, float v[8]) {
  const float4* q = reinterpret_cast<const float4*>(p);
  float4 a = q[0], b = q[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ void load8(const bf16* p, float v[8]) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  v[0] = __uint_as_float(u.x << 16); v[1] = __uint_as_float(u.x & 0xffff0000u);
  v[2] = __uint_as_float(u.y << 16); v[3] = __uint_as_float(u.y & 0xffff0000u);
  v[4] = __uint_as_float(u.z << 16); v[5] = __uint_as_float(u.z & 0xffff0000u);
  v[6] = __uint_as_float(u.w << 16); v[7] = __uint_as_float(u.w & 0xffff0000u);
}

// One 64-element chunk of an input row, loaded raw (16-B loads) and widened
// to fp32 only when used.
template <typename XT>
struct RawChunk;
template <>
struct RawChunk<bf16> {
  uint4 u[kChunk / 8];
  __device__ __forceinline__ void load(const bf16* p) {
#pragma unroll
    for (int i = 0; i < kChunk / 8; ++i) u[i] = reinterpret_cast<const uint4*>(p)[i];
  }
  __device__ __forceinline__ void get(float* v) const {
#pragma unroll
    for (int i = 0; i < kChunk / 8; ++i) {
      v[8 * i + 0] = __uint_as_float(u[i].x << 16); v[8 * i + 1] = __uint_as_float(u[i].x & 0xffff0000u);
      v[8 * i + 2] = __uint_as_float(u[i].y << 16); v[8 * i + 3] = __uint_as_float(u[i].y & 0xffff0000u);
      v[8 * i + 4] = __uint_as_float(u[i].z << 16); v[8 * i + 5] = __uint_as_float(u[i].z & 0xffff0000u);
      v[8 * i + 6] = __uint_as_float(u[i].w << 16); v[8 * i + 7] = __uint_as_float(u[i].w & 0xffff0000u);
    }
  }
};
template <>
struct RawChunk<float> {
  float4 u[kChunk / 4];
  __device__ __forceinline__ void load(const float* p) {
#pragma unroll
    for (int i = 0; i < kChunk / 4; ++i) u[i] = reinterpret_cast<const float4*>(p)[i];
  }
  __device__ __forceinline__ void get(float* v) const {
#pragma unroll
    for (int i = 0; i < kChunk / 4; ++i) {
      v[4 * i + 0] = u[i].x; v[4 * i + 1] = u[i].y; v[4 * i + 2] = u[i].z; v[4 * i + 3] = u[i].w;
    }
  }
};

// Sum of squares of one 64-element chunk, as one fma chain from +0.
template <typename XT>
__device__ __forceinline__ float chunk_sumsq(const XT* p) {
  float part = 0.0f;
#pragma unroll
  for (int i = 0; i < kChunk; i += 8) {
    float v[8];
    load8(p + i, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) part = __builtin_fmaf(v[j], v[j], part);
  }
  return part;
}

// Inverse RMS from the chunk partial sums held in LDS: sum in chunk order,
// then 1 / sqrt(sum / H + eps), each operation rounded once.
__device__ __forceinline__ float inv_rms_from_parts(const float* sp, int nc, int H, float eps) {
  float total = 0.0f;
  for (int c = 0; c < nc; ++c) total = total + sp[c];
  float mean = total / (float)H;
  return 1.0f / sqrtf(mean + eps);
}

template <typename XT>
__global__ __launch_bounds__(256) void router_prep_kernel(int T, int H, float eps,
                                                          const XT* __restrict__ x,
                                                          const float* __restrict__ pre_gain,
                                                          float* __restrict__ r0_out,
                                                          float* __restrict__ r_out) {
  __shared__ float parts[4][256];
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int t = blockIdx.x * 4 + wave;
  const bool active = t < T;
  const int nc = H / kChunk;
  const XT* xr = x + (size_t)(active ? t : 0) * H;
  float* sp = parts[wave];
  // The lane's first chunk stays in registers for the second norm, which
  // read it from memory again (H <= 4096: the whole row; 2048 / 4096 / 8192
  // tokens at 26B-A4B shapes 11.6 / 15.4 / 26.7 us for this kernel before).
  RawChunk<XT> xc;
  if (active && lane < nc) xc.load(xr + lane * kChunk);

  if (active)
    for (int c = lane; c < nc; c += kWave) {
      if (c == lane) {
        float v[kChunk];
        xc.get(v);
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < kChunk; ++i) part = __builtin_fmaf(v[i], v[i], part);
        sp[c] = part;
      } else {
        sp[c] = chunk_sumsq(xr + c * kChunk);
      }
    }
  __syncthreads();
  float r0 = 0.0f;
  if (active && lane == 0) r0 = inv_rms_from_parts(sp, nc, H, eps);
  r0 = __shfl(r0, 0, kWave);
  if (pre_gain == nullptr) {
    if (active && lane == 0) r_out[t] = r0;
    return;
  }
  __syncthreads();
  // second norm on v = (x * r0) * gain
  if (active) {
    for (int c = lane; c < nc; c += kWave) {
      float part = 0.0f;
      if (c == lane) {
        float v[kChunk];
        xc.get(v);
#pragma unroll
        for (int i = 0; i < kChunk; i += 8) {
          float g[8];
          load8(pre_gain + c * kChunk + i, g);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            float vv = (v[i + j] * r0) * g[j];
            part = __builtin_fmaf(vv, vv, part);
          }
        }
      } else {
        for (int i = 0; i < kChunk; i += 8) {
          float v[8], g[8];
          load8(xr + c * kChunk + i, v);
          load8(pre_gain + c * kChunk + i, g);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            float vv = (v[j] * r0) * g[j];
            part = __builtin_fmaf(vv, vv, part);
          }
        }
      }
      sp[c] = part;
    }
  }
  __syncthreads();
  if (active && lane == 0) {
    r0_out[t] = r0;
    r_out[t] = inv_rms_from_parts(sp, nc, H, eps);
  }
}

// Router input element after both norms: vhat = (v * r) * scale with
// v = x, or v = (x * r0) * gain under a pre-norm.
__device__ __forceinline__ float router_vhat(float x, bool pre, float r0, float g, float r,
                                             float s) {
  float v = pre ? (x * r0) * g : x;
  return (v * r) * s;
}

constexpr int kSmallMaxChunks = 48;  // H <= 3072

// Small batches: block = TB (<= 4) tokens x 4 * EW experts; lane c owns
// chunk c (H / 64 <= 64).  Dynamic LDS: vhat [TB][nc][65] + parts
// [4][TB * EW][65] + norm partials [4][64] + (four tokens a block) the
// router scale and the pre-norm gain [2][nc][65], staged at the start so that
// their loads overlap the weights' and the input's instead of following the
// norms.
template <typename XT, int TB, int EW>
__global__ __launch_bounds__(256) void router_logits_small_kernel(
    int T, int H, int E, float eps, const XT* __restrict__ x, const float* __restrict__ pre_gain,
    const float* __restrict__ scale, const float* __restrict__ W, float* __restrict__ logits,
    unsigned* __restrict__ done_counter) {
  extern __shared__ float lds[];
  constexpr int P = TB * EW;
  // Four tokens a block: the router scale and the pre-norm gain are staged in
  // LDS with the first loads (128 tokens 24 -> 18 us, 256 tokens 45 -> 30);
  // with one or two tokens a block the staging costs more than it saves
  // (1 token 8 -> 11 us), and wave 0 loads them after the norms.
  constexpr bool kStage = TB >= 4;
  // the completion counter of the top-K kernel that follows on the stream
  if (done_counter != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0)
    *done_counter = 0u;
  const int nc = H / kChunk;
  float* vh = lds;                              // [TB][nc][65]
  float* parts = vh + TB * nc * (kChunk + 1);   // [4][P][65]
  float* normp = parts + 4 * P * (kChunk + 1);  // [4][64]
  float* scl = normp + 4 * kWave;               // [nc][65]
  float* gnl = scl + nc * (kChunk + 1);         // [nc][65]
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int t0 = blockIdx.x * TB;
  const int e0 = blockIdx.y * 4 * EW + wave * EW;
  const bool pre = pre_gain != nullptr;
  const bool lc = lane < nc;

  // 1. this wave's experts: chunk `lane` of each, straight into registers
  float wr[EW][kChunk];
#pragma unroll
  for (int b = 0; b < EW; ++b) {
    const float* src = W + (size_t)min(e0 + b, E - 1) * H + lane * kChunk;
#pragma unroll
    for (int i = 0; i < kChunk; i += 8) {
      if (lc) load8(src + i, &wr[b][i]);
      else {
#pragma unroll
        for (int j = 0; j < 8; ++j) wr[b][i + j] = 0.0f;
      }
    }
  }

  // 2. norms and the normalised input: wave w takes token t0 + w
  const int tw = t0 + wave;
  const bool tok = wave < TB && tw < T;
  // The input chunk (kept raw), the router scale and the pre-norm gain: every
  // load goes out before any result is used, so that all of them (and the
  // weights above) come back in one round trip.
  RawChunk<XT> xraw;
  if (tok && lc) xraw.load(x + (size_t)tw * H + lane * kChunk);
  if constexpr (kStage) {
    constexpr int kPer = kSmallMaxChunks * kChunk / 256;
    float sv[kPer], gv[kPer];
    auto put = [&](float* dst, const float (&v)[kPer]) {
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int i = threadIdx.x + 256 * k;
        if (i < H) dst[(i / kChunk) * (kChunk + 1) + i % kChunk] = v[k];
      }
    };
    if (pre) {  // uniform
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int i = min((int)threadIdx.x + 256 * k, H - 1);
        sv[k] = scale[i];
        gv[k] = pre_gain[i];
      }
      put(scl, sv);
      put(gnl, gv);
    } else {
#pragma unroll
      for (int k = 0; k < kPer; ++k) sv[k] = scale[min((int)threadIdx.x + 256 * k, H - 1)];
      put(scl, sv);
    }
  }
  float xv[kChunk];
  float part = 0.0f;
  if (tok && lc) {
    xraw.get(xv);
#pragma unroll
    for (int i = 0; i < kChunk; ++i) part = __builtin_fmaf(xv[i], xv[i], part);
  }
  normp[wave * kWave + lane] = part;
  __syncthreads();
  float r = 0.0f;
  if (tok && lane == 0) r = inv_rms_from_parts(normp + wave * kWave, nc, H, eps);
  r = __shfl(r, 0, kWave);
  if (pre) {
    part = 0.0f;
    if (tok && lc) {
      auto apply = [&](const float* g) {
#pragma unroll
        for (int i = 0; i < kChunk; ++i) {
          xv[i] = (xv[i] * r) * g[i];
          part = __builtin_fmaf(xv[i], xv[i], part);
        }
      };
      if constexpr (kStage) {
        apply(gnl + lane * (kChunk + 1));
      } else {
        float g[kChunk];
#pragma unroll
        for (int i = 0; i < kChunk; i += 8) load8(pre_gain + lane * kChunk + i, &g[i]);
        apply(g);
      }
    }
    __syncthreads();
    normp[wave * kWave + lane] = part;
    __syncthreads();
    if (tok && lane == 0) r = inv_rms_from_parts(normp + wave * kWave, nc, H, eps);
    r = __shfl(r, 0, kWave);
  }
  if (wave < TB && lc) {
    float* dst = vh + (wave * nc + lane) * (kChunk + 1);
    auto put = [&](const float* sc) {
#pragma unroll
      for (int i = 0; i < kChunk; ++i) dst[i] = tok ? (xv[i] * r) * sc[i] : 0.0f;
    };
    if constexpr (kStage) {
      put(scl + lane * (kChunk + 1));
    } else {
      float sc[kChunk];
#pragma unroll
      for (int i = 0; i < kChunk; i += 8) load8(scale + lane * kChunk + i, &sc[i]);
      put(sc);
    }
  }
  __syncthreads();

  // 3. chunk chains: acc[t][b] over chunk `lane`, ascending index from +0
  float acc[TB][EW];
#pragma unroll
  for (int t = 0; t < TB; ++t)
#pragma unroll
    for (int b = 0; b < EW; ++b) acc[t][b] = 0.0f;
  if (lc) {
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
#pragma unroll
      for (int t = 0; t < TB; ++t) {
        const float v = vh[(t * nc + lane) * (kChunk + 1) + i];
#pragma unroll
        for (int b = 0; b < EW; ++b) acc[t][b] = __builtin_fmaf(v, wr[b][i], acc[t][b]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TB; ++t)
#pragma unroll
    for (int b = 0; b < EW; ++b) parts[(wave * P + t * EW + b) * (kChunk + 1) + lane] = acc[t][b];
  __syncthreads();

  // 4. one lane per (token, expert) adds the chunk results in chunk order
  if (lane < P) {
    const int t = t0 + lane / EW, e = e0 + lane % EW;
    if (t < T && e < E) {
      const float* pp = parts + (wave * P + lane) * (kChunk + 1);
      float total = 0.0f;
      for (int c = 0; c < nc; ++c) total = total + pp[c];
      logits[(size_t)t * E + e] = total;
    }
  }
}

// Large batches: 64 tokens (lane = token) x 32 experts (8 per wave) per block.
template <typename XT>
__global__ __launch_bounds__(256) void router_logits_tiled_kernel(
    int T, int H, int E, const XT* __restrict__ x, const float* __restrict__ pre_gain,
    const float* __restrict__ r0v, const float* __restrict__ rv,
    const float* __restrict__ scale, const float* __restrict__ W, float* __restrict__ logits) {
  __shared__ float wl[kChunk][32];
  __shared__ float sl[kChunk], gl[kChunk];
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 32;
  const int t = t0 + lane;
  const bool tv = t < T;
  const int tc = tv ? t : T - 1;
  const bool pre = pre_gain != nullptr;
  const float r = rv[tc];
  const float r0 = pre ? r0v[tc] : 0.0f;
  const XT* xr = x + (size_t)tc * H;
  const int nc = H / kChunk;

  float total[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) total[j] = 0.0f;

  for (int c = 0; c < nc; ++c) {
    float xv[kChunk];
#pragma unroll
    for (int i = 0; i < kChunk; i += 8) load8(xr + c * kChunk + i, xv + i);
    __syncthreads();  // the previous chunk's LDS reads are done
    {
      const int ei = threadIdx.x / 8, ks = (threadIdx.x % 8) * 8;
      const int e = e0 + ei;
      float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (e < E) load8(W + (size_t)e * H + c * kChunk + ks, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) wl[ks + j][ei] = v[j];
      if (threadIdx.x < kChunk) sl[threadIdx.x] = scale[c * kChunk + threadIdx.x];
      else if (threadIdx.x < 2 * kChunk)
        gl[threadIdx.x - kChunk] = pre ? pre_gain[c * kChunk + threadIdx.x - kChunk] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kChunk; ++k) xv[k] = router_vhat(xv[k], pre, r0, gl[k], r, sl[k]);
    float part[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) part[j] = 0.0f;
#pragma unroll
    for (int k = 0; k < kChunk; ++k) {
      const float4* wp = reinterpret_cast<const float4*>(&wl[k][wave * 8]);
      float4 wa = wp[0], wb = wp[1];
      part[0] = __builtin_fmaf(xv[k], wa.x, part[0]);
      part[1] = __builtin_fmaf(xv[k], wa.y, part[1]);
      part[2] = __builtin_fmaf(xv[k], wa.z, part[2]);
      part[3] = __builtin_fmaf(xv[k], wa.w, part[3]);
      part[4] = __builtin_fmaf(xv[k], wb.x, part[4]);
      part[5] = __builtin_fmaf(xv[k], wb.y, part[5]);
      part[6] = __builtin_fmaf(xv[k], wb.z, part[6]);
      part[7] = __builtin_fmaf(xv[k], wb.w, part[7]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) total[j] = total[j] + part[j];
  }
  if (tv) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = e0 + wave * 8 + j;
      if (e < E) logits[(size_t)t * E + e] = total[j];
    }
  }
}

// Large batches, E % 4 == 0, chunks split over wave groups: block = 8 TQ
// tokens x 64 experts (TQ = 4 or 2), G groups of 128 threads; group g takes
// chunks g, g + G, ...  Thread (tq, eq) of a group runs 4 TQ chains: tokens
// TQ tq .. TQ tq + TQ - 1 x experts 4 eq .. 4 eq + 3, with one 16-B weight
// read and one 4 TQ-B input read per 4 TQ fmas.  Per round every group
// stages its chunk (weights transposed to [64 k][64 e], router input [64][8
// TQ + 4]) in its own LDS region, runs its chains, and groups 1 .. G-1 leave
// their chunk results in LDS, which group 0 adds to its totals in chunk
// order.  TQ = 2 halves a block's work where 32-token blocks would leave
// CUs idle (up to 2048 tokens at 26B-A4B shapes): a block then also waits
// less for a CU that another kernel holds (the layer's dense branch runs
// beside the router).
constexpr int kSplitE = 64;
// Column swizzle of the staged weight tile: k quad kq's expert quads are
// permuted by an XOR with 2 (kq mod 8), a bijection on 0 .. 15.
__device__ __forceinline__ int wswz(int kq) { return 2 * (kq & 7); }
template <typename XT, int G, int TQ>
__global__ __launch_bounds__(128 * G) void router_logits_split_kernel(
    int T, int H, int E, const XT* __restrict__ x, const float* __restrict__ pre_gain,
    const float* __restrict__ r0v, const float* __restrict__ rv,
    const float* __restrict__ scale, const float* __restrict__ W, float* __restrict__ logits) {
  static_assert(TQ == 4 || TQ == 2, "tokens per thread");
  constexpr int kSplitT = 8 * TQ, kSplitVP = kSplitT + 4;
  constexpr int SK = kChunk * kSplitT / 128;  // input values a thread stages per chunk
  __shared__ __align__(16) float wl[G][kChunk][kSplitE];
  __shared__ __align__(16) float vl[G][kChunk][kSplitVP];
  __shared__ float ex[G > 1 ? G - 1 : 1][4 * TQ][128];
  const int g = threadIdx.x / 128, tig = threadIdx.x % 128;
  const int tq = tig / 16, eq = tig % 16;
  const int t0 = blockIdx.x * kSplitT, e0 = blockIdx.y * kSplitE;
  const bool pre = pre_gain != nullptr;
  const int nc = H / kChunk;
  const int R = (nc + G - 1) / G;
  // staging of the input: token st, k values sk .. sk + SK - 1 of the chunk
  const int st = tig % kSplitT, sk = (tig / kSplitT) * SK;
  const int tcl = min(t0 + st, T - 1);
  const float r0 = pre ? r0v[tcl] : 0.0f, r = rv[tcl];
  const XT* xr = x + (size_t)tcl * H + sk;

  // The chunk's weights come straight from W [E, H].  Pair j (< 2) of this
  // thread is expert quad eq = tig / 8 and k quad kq = tig % 8 + 8 j, so the 8
  // lanes of an expert row read 128 contiguous bytes and one load instruction
  // covers 8 whole lines.  Its 4 x 4 block (4 rows of 16 B) is transposed in
  // registers and stored as 4 float4 along the experts: the LDS tile is
  // W^T [k][e] as the chains read it, with expert quad column eq ^ wswz(kq),
  // so that the 16 lanes of a store phase fill 16 distinct bank quads.
  // The input stays as loaded (bf16 bits or fp32) until lstore, so nothing
  // waits on these loads before the round's chains run.
  constexpr bool kBf16In = std::is_same<XT, bf16>::value;
  float4 wreg[8];
  uint4 xu[SK / 8];
  float xv[SK], sv[SK], gv[SK];
  auto gload = [&](int c) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int eqj = tig / 8, kq = tig % 8 + 8 * j;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // Rows past E (a partial last expert tile) load row E - 1: only the
        // chains of experts past E read them, and those results are dropped.
        // No condition around the load, so the loads of a chunk all go out
        // before the first wait.
        const int e = min(e0 + 4 * eqj + i, E - 1);
        wreg[4 * j + i] =
            *reinterpret_cast<const float4*>(W + (size_t)e * H + c * kChunk + 4 * kq);
      }
    }
#pragma unroll
    for (int h = 0; h < SK / 8; ++h) {
      if constexpr (kBf16In)
        xu[h] = *reinterpret_cast<const uint4*>(xr + c * kChunk + 8 * h);
      else
        load8(reinterpret_cast<const float*>(xr) + c * kChunk + 8 * h, xv + 8 * h);
    }
#pragma unroll
    for (int h = 0; h < SK / 8; ++h) load8(scale + c * kChunk + sk + 8 * h, sv + 8 * h);
    if (pre) {
#pragma unroll
      for (int h = 0; h < SK / 8; ++h) load8(pre_gain + c * kChunk + sk + 8 * h, gv + 8 * h);
    } else {
#pragma unroll
      for (int i = 0; i < SK; ++i) gv[i] = 0.0f;
    }
  };
  auto lstore = [&]() {
    if constexpr (kBf16In) {
#pragma unroll
      for (int h = 0; h < SK / 8; ++h) {
        const unsigned u[4] = {xu[h].x, xu[h].y, xu[h].z, xu[h].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xv[8 * h + 2 * i] = __uint_as_float(u[i] << 16);
          xv[8 * h + 2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int eqj = tig / 8, kq = tig % 8 + 8 * j;
      const int col = 4 * (eqj ^ wswz(kq));
      const float4* b = wreg + 4 * j;  // b[i] = expert 4 eqj + i, k 4 kq .. 4 kq + 3
      *reinterpret_cast<float4*>(&wl[g][4 * kq + 0][col]) = make_float4(b[0].x, b[1].x, b[2].x, b[3].x);
      *reinterpret_cast<float4*>(&wl[g][4 * kq + 1][col]) = make_float4(b[0].y, b[1].y, b[2].y, b[3].y);
      *reinterpret_cast<float4*>(&wl[g][4 * kq + 2][col]) = make_float4(b[0].z, b[1].z, b[2].z, b[3].z);
      *reinterpret_cast<float4*>(&wl[g][4 * kq + 3][col]) = make_float4(b[0].w, b[1].w, b[2].w, b[3].w);
    }
#pragma unroll
    for (int i = 0; i < SK; ++i) vl[g][sk + i][st] = router_vhat(xv[i], pre, r0, gv[i], r, sv[i]);
  };

  float total[TQ][4];
#pragma unroll
  for (int i = 0; i < TQ; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) total[i][j] = 0.0f;
  if (g < nc) gload(g);
  for (int rr = 0; rr < R; ++rr) {
    const int c = rr * G + g;
    const bool have = c < nc;
    if (have) lstore();
    __syncthreads();
    if (c + G < nc) gload(c + G);
    float p[TQ][4];
#pragma unroll
    for (int i = 0; i < TQ; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) p[i][j] = 0.0f;
    if (have) {
#pragma unroll 8
      for (int k = 0; k < kChunk; ++k) {
        const float4 w = *reinterpret_cast<const float4*>(&wl[g][k][4 * (eq ^ wswz(k / 4))]);
        float vv[TQ];
        if constexpr (TQ == 4) {
          const float4 v = *reinterpret_cast<const float4*>(&vl[g][k][4 * tq]);
          vv[0] = v.x; vv[1] = v.y; vv[2] = v.z; vv[3] = v.w;
        } else {
          const float2 v = *reinterpret_cast<const float2*>(&vl[g][k][2 * tq]);
          vv[0] = v.x; vv[1] = v.y;
        }
#pragma unroll
        for (int i = 0; i < TQ; ++i) {
          p[i][0] = __builtin_fmaf(vv[i], w.x, p[i][0]);
          p[i][1] = __builtin_fmaf(vv[i], w.y, p[i][1]);
          p[i][2] = __builtin_fmaf(vv[i], w.z, p[i][2]);
          p[i][3] = __builtin_fmaf(vv[i], w.w, p[i][3]);
        }
      }
      if (g > 0) {
#pragma unroll
        for (int i = 0; i < TQ; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) ex[g - 1][4 * i + j][tig] = p[i][j];
      }
    }
    __syncthreads();
    if (g == 0) {
#pragma unroll
      for (int i = 0; i < TQ; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) total[i][j] = total[i][j] + p[i][j];
#pragma unroll
      for (int h = 1; h < G; ++h) {
        if (rr * G + h >= nc) break;  // uniform
#pragma unroll
        for (int i = 0; i < TQ; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) total[i][j] = total[i][j] + ex[h - 1][4 * i + j][tig];
      }
    }
  }
  if (g != 0) return;
  const int e = e0 + 4 * eq;
  if (e >= E) return;
#pragma unroll
  for (int i = 0; i < TQ; ++i) {
    const int t = t0 + TQ * tq + i;
    if (t < T)
      *reinterpret_cast<float4*>(logits + (size_t)t * E + e) =
          make_float4(total[i][0], total[i][1], total[i][2], total[i][3]);
  }
}

// One wave per token.
__global__ __launch_bounds__(256) void router_topk_kernel(int T, int E, int K,
                                                          const float* __restrict__ logits,
                                                          const float* __restrict__ pes,
                                                          int32_t* __restrict__ idx,
                                                          float* __restrict__ w) {
  const int t = blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= T) return;  // whole wave; no block barrier below
  wave_topk(logits + (size_t)t * E, E, K, pes, idx + (size_t)t * K, w + (size_t)t * K, nullptr);
}

// Small batches: one wave per token, kTopkTok tokens per 1024-thread block,
// so the top-K of the batch is spread over many CUs.  With counts != null
// the last block to finish (a completion counter, zeroed by the logits kernel
// of the same call) groups all T*K <= 1024 slots by expert.  The counter only
// orders the blocks; every result is computed in one fixed order.  Up to
// kTopkOneBlockTokens tokens one block does it all: its 16 waves take a token
// each, the slots' experts stay in LDS, and the dispatch follows a block
// barrier; no completion counter, so none of the device-scope release /
// acquire fences around it (an L2 write-back and invalidate).  The route at
// 1 token went 22 -> 18 us; from 32 tokens, where a wave would take two or
// more tokens in turn, the spread-out form is faster (64 tokens: 24 against
// 35 us).
constexpr int kTopkTok = 4;
constexpr int kTopkOneBlockTokens = kChunkWaves;
__global__ __launch_bounds__(kChunkSlots) void route_topk_dispatch_kernel(
    int T, int E, int K, const float* __restrict__ logits, const float* __restrict__ pes,
    int32_t* __restrict__ idx, float* __restrict__ w, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slots,
    unsigned* __restrict__ done_counter) {
  __shared__ int wave_base[kChunkWaves][kMaxE];
  __shared__ int totals[kMaxE];
  __shared__ int offs[kMaxE + 1];
  __shared__ int last;
  __shared__ int slot_e[kChunkSlots];
  const int wave = threadIdx.x / kWave;
  if (gridDim.x == 1) {  // uniform: the one-block form
    for (int t = wave; t < T; t += kChunkWaves)
      wave_topk(logits + (size_t)t * E, E, K, pes, idx + (size_t)t * K, w + (size_t)t * K,
                counts != nullptr ? slot_e + t * K : nullptr);
    if (counts == nullptr) return;
    __syncthreads();
    const bool valid = (int)threadIdx.x < T * K;
    const int e = valid ? slot_e[threadIdx.x] : 0;
    dispatch_lone_chunk(e, valid, E, counts, offsets, sorted_slots, wave_base, totals, offs);
    return;
  }
  const int t = blockIdx.x * kTopkTok + wave;
  if (wave < kTopkTok && t < T)
    wave_topk(logits + (size_t)t * E, E, K, pes, idx + (size_t)t * K, w + (size_t)t * K, nullptr);
  if (counts == nullptr) return;  // uniform
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();  // release: the block's idx stores (ordered by the barrier) go device-wide
    last = atomicAdd(done_counter, 1u) == gridDim.x - 1;
    if (last) __threadfence();  // acquire: the other blocks' idx stores
  }
  __syncthreads();
  if (!last) return;  // uniform
  const bool valid = (int)threadIdx.x < T * K;
  const int e = valid ? __builtin_nontemporal_load(idx + threadIdx.x) : 0;
  dispatch_lone_chunk(e, valid, E, counts, offsets, sorted_slots, wave_base, totals, offs);
}

template <typename XT, int TB, int EW>
void launch_small(const RouterArgs& a, bool count, hipStream_t s) {
  const int nc = a.H / kChunk;
  constexpr int kStaged = TB >= 4 ? 2 : 0;  // scale and gain rows staged in LDS
  const size_t lds = sizeof(float) * ((size_t)TB * nc * (kChunk + 1) +
                                      4 * TB * EW * (kChunk + 1) + 4 * kWave +
                                      kStaged * nc * (kChunk + 1));
  // past 64 KB at 4 tokens per block (26B-A4B: 78 KB, two blocks per CU)
  constexpr size_t kMaxLds = sizeof(float) * ((size_t)TB * kSmallMaxChunks * (kChunk + 1) +
                                              4 * TB * EW * (kChunk + 1) + 4 * kWave +
                                              kStaged * kSmallMaxChunks * (kChunk + 1));
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(router_logits_small_kernel<XT, TB, EW>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds);
  (void)attr;  // a failure shows in the launch's error
  dim3 grid((a.T + TB - 1) / TB, (a.E + 4 * EW - 1) / (4 * EW));
  hipLaunchKernelGGL((router_logits_small_kernel<XT, TB, EW>), grid, dim3(256), lds, s, a.T, a.H,
                     a.E, a.eps, static_cast<const XT*>(a.x), a.pre_gain, a.router_scale,
                     a.router_w, a.ws_logits, count ? a.ws_counter : nullptr);
}

}  // namespace

// Small-batch logits: up to 448 tokens, H <= 3072 (LDS within 96 KB).  The
// chunk-parallel kernel spreads a token's 44 chunk chains (26B-A4B) over a
// wave; the large-batch kernels run them one after another in a thread and
// pay a fixed ~80 us for the chunk rounds (the whole route at 128 tokens:
// 30 us here against 105 us with the earlier 16-token-block kernel; 384
// tokens: 73 us; at 512 tokens this kernel's 92 us loses to the split
// kernel's ~80).  The dispatch joins the top-K kernel while the batch has at
// most 1024 slots.
constexpr int kSmallLogitsMaxT = 448;
static bool router_small_logits(int T, int H) {
  return H / kChunk <= kSmallMaxChunks && T <= kSmallLogitsMaxT;
}
// Four wave groups (one 8-wave block per CU, 124 KB of LDS) while the grid
// of 32-token blocks fits the 256 CUs at one block each; past that two
// groups (58 KB, two 4-wave blocks per CU).  The whole route at 4096 tokens:
// 146 us with the earlier kernel (one token per thread, 5 B of LDS per fma),
// 91 us with four groups; at 8192 tokens with the pre-norm 191 -> 157 us
// with two groups (four: 179 us).  Below 256 such blocks the blocks take 16
// tokens while twice as many still fit one round (at 26B-A4B shapes up to
// 2048 tokens; the route at 512 / 1024 / 2048 tokens with the pre-norm 85 /
// 87 / 95 -> 69 / 71 / 79 us with four groups, routing bit-identical; at 3000
// tokens, two rounds of them, 100 -> 124 us); their smaller input tile
// leaves room for six wave groups (146 KB), so a block runs 8 chunk rounds
// instead of 11.
constexpr long long kSplitOneBlockPerCu = 256;
constexpr int kSplitG16 = 6;

bool router_fuses_dispatch(int T, int H, int E, int K) {
  return router_small_logits(T, H) && T * K <= kChunkSlots;
}

namespace {

DispatchArgs dispatch_args(const RouterArgs& a) {
  DispatchArgs d{};
  d.T = a.T; d.E = a.E; d.K = a.K; d.topk_idx = a.topk_idx; d.counts = a.counts;
  d.offsets = a.offsets; d.sorted_slots = a.sorted_slots; d.ws_blk_counts = a.ws_blk_counts;
  d.ws_local_rank = a.ws_local_rank;
  return d;
}

template <typename XT>
hipError_t launch_router_t(const RouterArgs& a, hipStream_t s) {
  const XT* x = static_cast<const XT*>(a.x);
  const int nc = a.H / kChunk;
  const bool want_dispatch = a.counts != nullptr;
  if (router_small_logits(a.T, a.H)) {
    const bool fuse = want_dispatch && router_fuses_dispatch(a.T, a.H, a.E, a.K);
    if (a.T == 1) launch_small<XT, 1, 1>(a, fuse, s);
    else if (a.T <= 8) launch_small<XT, 2, 1>(a, fuse, s);
    // 4 experts per block up to 32 tokens (twice the blocks): the route at
    // 12 tokens 21 -> 14 us, at 32 tokens 21 -> 19 us; from 40 tokens 8 win
    else if (a.T <= 32) launch_small<XT, 4, 1>(a, fuse, s);
    else launch_small<XT, 4, 2>(a, fuse, s);
    const int tb = a.T <= kTopkOneBlockTokens ? 1 : (a.T + kTopkTok - 1) / kTopkTok;
    hipLaunchKernelGGL(route_topk_dispatch_kernel, dim3(tb),
                       dim3(kChunkSlots), 0, s, a.T, a.E, a.K, a.ws_logits, a.per_expert_scale,
                       a.topk_idx, a.topk_w, fuse ? a.counts : nullptr, a.offsets,
                       a.sorted_slots, a.ws_counter);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || fuse || !want_dispatch) return e;
    return launch_dispatch(dispatch_args(a), s);
  }
  hipLaunchKernelGGL(router_prep_kernel<XT>, dim3((a.T + 3) / 4), dim3(256), 0, s, a.T, a.H,
                     a.eps, x, a.pre_gain, a.ws_r0, a.ws_r);
  if (a.E % 4 == 0) {
    const int ne = (a.E + kSplitE - 1) / kSplitE;
    const dim3 sg((a.T + 31) / 32, ne), sg16((a.T + 15) / 16, ne);
    if ((long long)sg16.x * sg16.y <= kSplitOneBlockPerCu)
      hipLaunchKernelGGL((router_logits_split_kernel<XT, kSplitG16, 2>), sg16,
                         dim3(128 * kSplitG16), 0, s, a.T, a.H, a.E, x, a.pre_gain, a.ws_r0,
                         a.ws_r, a.router_scale, a.router_w, a.ws_logits);
    else if ((long long)sg.x * sg.y <= kSplitOneBlockPerCu)
      hipLaunchKernelGGL((router_logits_split_kernel<XT, 4, 4>), sg, dim3(512), 0, s, a.T, a.H,
                         a.E, x, a.pre_gain, a.ws_r0, a.ws_r, a.router_scale, a.router_w,
                         a.ws_logits);
    else
      hipLaunchKernelGGL((router_logits_split_kernel<XT, 2, 4>), sg, dim3(256), 0, s, a.T, a.H,
                         a.E, x, a.pre_gain, a.ws_r0, a.ws_r, a.router_scale, a.router_w,
                         a.ws_logits);
  } else {
    hipLaunchKernelGGL(router_logits_tiled_kernel<XT>, dim3((a.T + 63) / 64, (a.E + 31) / 32),
                       dim3(256), 0, s, a.T, a.H, a.E, x, a.pre_gain, a.ws_r0, a.ws_r,
                       a.router_scale, a.router_w, a.ws_logits);
  }
  hipLaunchKernelGGL(router_topk_kernel, dim3((a.T + 3) / 4), dim3(256), 0, s, a.T, a.E, a.K,
                     a.ws_logits, a.per_expert_scale, a.topk_idx, a.topk_w);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !want_dispatch) return e;
  return launch_dispatch(dispatch_args(a), s);
}

}  // namespace


hipError_t launch_router(const RouterArgs& a, hipStream_t s) {
  return a.x_bf16 ? launch_router_t<bf16>(a, s) : launch_router_t<float>(a, s);
}

}  // namespace moe
