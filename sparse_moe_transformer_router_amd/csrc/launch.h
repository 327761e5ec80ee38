// Host-side launchers of the libmoe kernels.  Each returns the HIP error of
// its launches (hipSuccess when all were enqueued).  Arguments are validated
// by the C ABI layer before any launcher is called.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

struct RouterArgs {
  int T, H, E, K;
  float eps;
  bool x_bf16;
  const void* x;                 // [T,H]
  const float* pre_gain;         // [H] or nullptr
  const float* router_w;         // [E,H]
  const float* router_scale;     // [H]
  const float* per_expert_scale; // [E]
  int32_t* topk_idx;             // [T,K]
  float* topk_w;                 // [T,K]
  float* ws_r0;                  // [T]   inverse RMS of x (pre-norm), if pre_gain
  float* ws_r;                   // [T]   inverse RMS of the router input
  float* ws_logits;              // [T,E]
  unsigned* ws_counter;          // completion counter of the small-batch top-K kernel
  // Optional dispatch right after the top-K (all null = router only).
  int32_t* counts;               // [E]
  int32_t* offsets;              // [E+1]
  int32_t* sorted_slots;         // [T*K]
  int32_t* ws_blk_counts;        // dispatch scratch (multi-chunk path)
  int32_t* ws_local_rank;
};
hipError_t launch_router(const RouterArgs& a, hipStream_t s);
bool router_fuses_dispatch(int T, int H, int E, int K);

struct DispatchArgs {
  int T, E, K;
  const int32_t* topk_idx;   // [T*K]
  int32_t* counts;           // [E]
  int32_t* offsets;          // [E+1]
  int32_t* sorted_slots;     // [T*K]
  int32_t* ws_blk_counts;    // [nblk*E]
  int32_t* ws_local_rank;    // [T*K]
};
int dispatch_num_blocks(int S);
hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s);
// All-experts slot layout: offsets[e] = e * T, sorted_slots[e * T + t] =
// t * E + e, w_dense[t * E + e] = the token's weight for e or 0.
hipError_t launch_dense_mask(int T, int E, int K, const int32_t* topk_idx, const float* topk_w,
                             int32_t* offsets, int32_t* sorted_slots, float* w_dense,
                             hipStream_t s);

// Storage format of the expert weights: see wformat.h.  The values equal the
// moe_wformat codes of include/moe.h.
enum class WFormat : int { kBF16 = 0, kInt8 = 1, kFP8 = 2, kMXFP4 = 3, kMXFP8 = 4 };

// Grouped gated-MLP over row groups.  Group e owns rows [offsets[e],
// offsets[e+1]) of the sorted order; row r reads input row
// sorted_slots[r] / K (or r itself when ident).  w_gate / w_up point at the
// first group's [N,H] gate and up rows; group e's are at + e * w_stride.
struct GateUpArgs {
  int T, H, N, E, K;   // N = intermediate width (I or D)
  int rows;            // total rows S (or T when ident)
  bool ident;          // rows are the tokens themselves (dense branch)
  bool bf16;
  const void* x;               // [T,H]
  const void* w_gate;
  const void* w_up;
  long long w_stride;          // elements between consecutive groups' weights
  const int32_t* offsets;      // [E+1] (unused when ident)
  const int32_t* sorted_slots; // [rows] (unused when ident)
  void* h;                     // [rows, N] act dtype, sorted order
  // Weights below bf16: w_gate / w_up hold codes; int8 and E4M3 rows n of
  // group e are scaled by the fp32 s_gate / s_up[e * s_stride + n]; MXFP4
  // rows carry E8M0 block scales at s_gate / s_up + e * s_stride + n * (H /
  // 32).  w_stride counts weights (not stored units).
  WFormat w_fmt;
  const void* s_gate;
  const void* s_up;
  long long s_stride;
  // Optional events recorded by the kernel's own dispatch packet (extended
  // launch) at its start and end; null: none.
  hipEvent_t ev_start, ev_stop;
};
hipError_t launch_gate_up(const GateUpArgs& a, hipStream_t s);

// Launches kernel f like hipLaunchKernelGGL, or with the extended launch
// when either event is set, so that the events time exactly that kernel
// without packets of their own between launches.
template <typename F, typename... Args>
inline void launch_maybe_timed(F f, dim3 grid, dim3 block, unsigned shmem, hipStream_t s,
                               hipEvent_t ev_start, hipEvent_t ev_stop, Args... args) {
  if (ev_start != nullptr || ev_stop != nullptr)
    hipExtLaunchKernelGGL(f, grid, block, shmem, s, ev_start, ev_stop, 0, args...);
  else
    hipLaunchKernelGGL(f, grid, block, shmem, s, args...);
}

// Down projection of the gated rows; row r of group e goes to output row
// sorted_slots[r] (or r when ident), scaled by topk_w of that slot (1 when
// ident).
struct DownArgs {
  int T, H, N, E, K;   // N = intermediate width (contraction length)
  int rows;
  bool ident;
  bool bf16;           // act dtype (h and w_down)
  bool y_bf16;         // output dtype
  const void* h;               // [rows, N]
  const void* w_down;          // group 0's [H, N]
  long long w_stride;
  const int32_t* offsets;
  const int32_t* sorted_slots;
  const float* topk_w;         // [T*K] (unused when ident)
  void* y;                     // [T*K, H] slot-major (or [T,H] when ident)
  WFormat w_fmt;               // as GateUpArgs (block scales per N / 32 of a row)
  const void* s_down;
  long long s_stride;
};
hipError_t launch_down(const DownArgs& a, hipStream_t s);

// Decode-sized variants (few rows per group): weight-streaming kernels.
// launch_gate_up / launch_down pick them for bf16 weights where
// use_stream_kernels holds, and for weights below bf16 (which need bf16
// activations) up to kMaxQuantStreamTokens tokens; past that, the tiled
// kernels widen those weights after their LDS reads.
constexpr int kMaxQuantStreamTokens = 256;
bool use_stream_kernels(int T, int rows, int E, bool ident);
bool quant_uses_stream_kernels(int T);
hipError_t launch_gate_up_stream(const GateUpArgs& a, hipStream_t s);
hipError_t launch_down_stream(const DownArgs& a, hipStream_t s);

// int8 per-channel symmetric quantization of rows x cols bf16 weights
// (cols % 8 == 0): codes q [rows, cols], scales [rows].
hipError_t launch_quantize_rows(long long rows, int cols, const void* w, int8_t* q, float* scale,
                                hipStream_t s);
// E4M3 per row: codes [rows, cols], fp32 scales [rows].
hipError_t launch_quantize_fp8(long long rows, int cols, const void* w, uint8_t* q, float* scale,
                               hipStream_t s);
// MXFP4 along each row (cols % 32 == 0): codes [rows, cols / 2], E8M0 [rows, cols / 32].
hipError_t launch_quantize_mxfp4(long long rows, int cols, const void* w, uint8_t* q,
                                 uint8_t* scale, hipStream_t s);
// Codes back to fp32 values (times their scales), with the experts' widening.
hipError_t launch_dequantize(WFormat f, long long rows, int cols, const void* q,
                             const void* scale, float* out, hipStream_t s);

// Experts on the 8-bit / 4-bit matrix cores (expert_mx.hip): MXFP8
// activations times E4M3 (fp32 scale per output row) or MXFP4 weights.
struct MxArgs {
  int T, H, I, E, K;
  int rows;                    // T * K
  WFormat fmt;                 // kFP8 or kMXFP4
  bool y_bf16;
  const void* x;               // [T,H] bf16 expert input
  uint8_t* xq;                 // [T,H] MXFP8 codes of x (workspace)
  uint8_t* xs;                 // [T,H/32] their E8M0 scales (workspace)
  uint8_t* hq;                 // [rows,I] MXFP8 codes of the gated product h, sorted
                               // order (workspace)
  uint8_t* hs;                 // [rows,I/32] (workspace)
  const void* gate_up_q;       // [E,2I,H] codes (MXFP4: two per byte)
  const void* gate_up_s;       // fp32 [E,2I] (E4M3) or E8M0 [E,2I,H/32] (MXFP4)
  const void* down_q;          // [E,H,I]
  const void* down_s;          // fp32 [E,H] or E8M0 [E,H,I/32]
  const int32_t* offsets;
  const int32_t* sorted_slots;
  const float* topk_w;
  void* y;                     // [T*K,H] slot dtype
};
hipError_t launch_expert_ffn_mx(const MxArgs& a, hipStream_t s);
bool mx_uses_stream_kernels(int T, int rows, int E);
// The tiled (prefill) form needs H and I multiples of 64 and the tile's scale
// rows in LDS beside the copy ring.
bool mx_tiled_supported(int H, int I);
// MXFP8 codes and E8M0 block scales of rows x cols bf16 (cols % 32 == 0).
hipError_t launch_mx8_quantize(long long rows, int cols, const void* in, uint8_t* q,
                               uint8_t* e8, hipStream_t s);
hipError_t launch_mx8_dequantize(long long rows, int cols, const uint8_t* q, const uint8_t* e8,
                                 float* out, hipStream_t s);

struct CombineArgs {
  int T, H, K;
  bool y_bf16, act_bf16;
  const void* y;       // [T,K,H]
  const void* addend;  // [T,H] act or nullptr
  void* out;           // [T,H] act
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);

struct PreNormArgs {
  int T, H;
  float eps;
  bool bf16;
  const void* x;
  const float* g_pre;
  const float* g_pre2;
  void* xd;
  void* xm;
};
hipError_t launch_prenorm(const PreNormArgs& a, hipStream_t s);

struct EpilogueArgs {
  int T, H, K;
  float eps;
  float layer_scalar;
  bool y_bf16, act_bf16;
  const void* y;       // [T,K,H] slot dtype
  const void* dn;      // [T,H] slot dtype (dense branch output)
  const void* x;       // [T,H] act (residual)
  const float* g_post1;
  const float* g_post2;
  const float* g_post;
  void* out;           // [T,H] act
  float* ffn_out;      // [T,H] fp32 or nullptr
};
hipError_t launch_block_epilogue(const EpilogueArgs& a, hipStream_t s);

}  // namespace moe
