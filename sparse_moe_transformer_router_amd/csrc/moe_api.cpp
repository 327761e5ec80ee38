// C ABI of libmoe (declared in include/moe.h): host-side argument checks,
// workspace layout, and the kernel sequence of each call on the caller's
// stream.  No call synchronises or allocates.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/moe.h"
#include "launch.h"

namespace {

// Quantized experts run on the weight-streaming kernels only, which pay up to
// about 16 rows per expert (256 tokens at top-8 of 128 experts).

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(MOE_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

size_t dtype_size(int32_t dt) { return dt == MOE_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// any_k: calls that only see token-slots (experts, combine) take any top_k up
// to num_experts, e.g. every expert per token; routing needs top_k <= 32.
int check_dims(const moe_dims* d, bool any_k = false) {
  if (!d) return fail(MOE_ERR_ARG, "dims is NULL");
  if (d->hidden < 64 || d->hidden > 8192 || d->hidden % 64)
    return fail(MOE_ERR_UNSUPPORTED, "hidden=%d: need a multiple of 64 in [64, 8192]", d->hidden);
  if (d->num_experts < 1 || d->num_experts > 256)
    return fail(MOE_ERR_UNSUPPORTED, "num_experts=%d: need 1..256", d->num_experts);
  if (d->top_k < 1 || d->top_k > d->num_experts || (!any_k && d->top_k > 32))
    return fail(MOE_ERR_UNSUPPORTED, "top_k=%d: need 1..min(num_experts, %d)", d->top_k,
                any_k ? d->num_experts : 32);
  if (d->expert_inter < 32 || d->expert_inter > 8192 || d->expert_inter % 32)
    return fail(MOE_ERR_UNSUPPORTED, "expert_inter=%d: need a multiple of 32 in [32, 8192]",
                d->expert_inter);
  if (d->dense_inter < 0 || d->dense_inter > 16384 || d->dense_inter % 32)
    return fail(MOE_ERR_UNSUPPORTED, "dense_inter=%d: need 0 or a multiple of 32 up to 16384",
                d->dense_inter);
  if (!(d->eps > 0.0f)) return fail(MOE_ERR_ARG, "eps must be > 0");
  if (d->act_dtype != MOE_F32 && d->act_dtype != MOE_BF16)
    return fail(MOE_ERR_ARG, "act_dtype=%d unknown", d->act_dtype);
  if (d->slot_dtype != MOE_F32 && d->slot_dtype != MOE_BF16)
    return fail(MOE_ERR_ARG, "slot_dtype=%d unknown", d->slot_dtype);
  if (d->act_dtype == MOE_F32 && d->slot_dtype != MOE_F32)
    return fail(MOE_ERR_UNSUPPORTED, "act_dtype F32 requires slot_dtype F32");
  return MOE_OK;
}

int check_tokens(const moe_dims* d, int32_t T) {
  if (T < 0 || T > 65536) return fail(MOE_ERR_ARG, "T=%d: need 0..65536", T);
  if ((long long)T * d->top_k > (1 << 20))
    return fail(MOE_ERR_UNSUPPORTED, "T*top_k=%lld exceeds 2^20", (long long)T * d->top_k);
  return MOE_OK;
}

#define REQUIRE_PTR(p)                                                                   \
  do {                                                                                   \
    if (!(p)) return fail(MOE_ERR_ARG, "%s is NULL", #p);                                \
    if (!aligned16(p)) return fail(MOE_ERR_ARG, "%s is not 16-byte aligned", #p);        \
  } while (0)
#define OPTIONAL_PTR(p)                                                                  \
  do {                                                                                   \
    if ((p) && !aligned16(p)) return fail(MOE_ERR_ARG, "%s is not 16-byte aligned", #p); \
  } while (0)

// Workspace regions (byte offsets), all 256-byte aligned, monotone in T so
// that a workspace sized for max_tokens serves every T <= max_tokens.
struct Layout {
  size_t r0, r, logits;             // router
  size_t blk_counts, local_rank;    // dispatch
  size_t h;                         // expert gate_up output
  size_t idx, w, counts, offsets, sorted, y;  // experts-only path / layer
  size_t xd, xm, hd, dn;            // layer only
  size_t counter;                   // small-batch top-K completion counter
  size_t base_end;                  // end of the regions above (all but the MXFP8 ones)
  size_t xq, xs, hq, hs;            // MXFP8 activations of the 8-bit / 4-bit experts
  size_t total;
};

Layout layout(const moe_dims* d, long long T) {
  Layout L{};
  const long long S = T * d->top_k;
  const long long nblk = (S + 1023) / 1024;
  const size_t act = dtype_size(d->act_dtype), slot = dtype_size(d->slot_dtype);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o += align256(bytes);
    return at;
  };
  L.r0 = take(4 * T);
  L.r = take(4 * T);
  L.logits = take(4 * T * d->num_experts);
  L.blk_counts = take(4 * nblk * d->num_experts);
  L.local_rank = take(4 * S);
  L.h = take(act * S * d->expert_inter);
  L.idx = take(4 * S);
  L.w = take(4 * S);
  L.counts = take(4 * (size_t)d->num_experts);
  L.offsets = take(4 * (size_t)(d->num_experts + 1));
  L.sorted = take(4 * S);
  L.y = take(slot * S * d->hidden);
  L.xd = take(act * T * d->hidden);
  L.xm = take(act * T * d->hidden);
  L.hd = take(act * T * d->dense_inter);
  L.dn = take(slot * T * d->hidden);
  L.counter = take(4);
  L.base_end = o;
  L.xq = take((size_t)T * d->hidden);
  L.xs = take((size_t)T * (d->hidden / 32));
  L.hq = take((size_t)S * d->expert_inter);
  L.hs = take((size_t)S * (d->expert_inter / 32));
  L.total = o;
  return L;
}

// The block's dense branch runs on a library-owned side stream (one per
// device, default priority, created on first use and kept), forked from and
// joined back into the caller's stream with two events.  A mutex keeps one
// call's record / wait sequence from interleaving with another thread's.
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mu;
SideStream g_side[64];

hipError_t side_stream(SideStream*& out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  SideStream& ss = g_side[dev];
  if (ss.stream == nullptr) {
    if ((e = hipStreamCreateWithFlags(&ss.stream, hipStreamNonBlocking)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&ss.join, hipEventDisableTiming)) != hipSuccess) return e;
  }
  out = &ss;
  return hipSuccess;
}

template <typename P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

int check_ws(const moe_dims* d, int32_t T, const void* ws, size_t ws_bytes) {
  const size_t need = layout(d, T).total;
  if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) & 255u)
    return fail(MOE_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed for T=%d", ws_bytes, need,
                T);
  return MOE_OK;
}

// ---- scratch of the entry point that allocates nothing --------------------
// moe_forward_noalloc takes its workspace from this file-scope device array
// instead of a caller's buffer.  Each GPU the library runs on holds its own
// copy until the process ends.  In host code the array's name is only a
// host-side stand-in: the device address of a GPU's copy comes from
// hipGetSymbolAddress, taken once per device (with that device current) and
// kept; only that address is ever handed to kernels.  Every call on a GPU
// shares the array and finds the last call's contents; the path clears what
// it needs cleared itself (the router's completion counter is zeroed by its
// logits kernel), and calls that overlap on one GPU race.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];

hipError_t noalloc_scratch(void*& out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  out = g_scratch_ptr[dev];
  return hipSuccess;
}

int run_forward(const moe_dims* dims, int32_t T, const void* x, const float* router_w,
                const float* router_scale, const float* per_expert_scale,
                const void* w_gate_up, const void* w_down, void* out, int32_t* topk_idx,
                float* topk_w, void* ws, hipStream_t s);

// ---- launch sequences (arguments already checked) -------------------------

// Router, and when counts is not null the dispatch as well (fused into the
// router's top-K kernel for small batches).
int run_router(const moe_dims* d, int32_t T, const void* x, const float* router_w,
               const float* router_scale, const float* pes, const float* pre_gain,
               int32_t* idx, float* w, int32_t* counts, int32_t* offsets, int32_t* sorted,
               void* ws, hipStream_t s) {
  const Layout L = layout(d, T);
  moe::RouterArgs a{};
  a.T = T; a.H = d->hidden; a.E = d->num_experts; a.K = d->top_k; a.eps = d->eps;
  a.x_bf16 = d->act_dtype == MOE_BF16;
  a.x = x; a.pre_gain = pre_gain; a.router_w = router_w; a.router_scale = router_scale;
  a.per_expert_scale = pes; a.topk_idx = idx; a.topk_w = w;
  a.ws_r0 = at<float>(ws, L.r0); a.ws_r = at<float>(ws, L.r);
  a.ws_logits = at<float>(ws, L.logits);
  a.ws_counter = at<unsigned>(ws, L.counter);
  a.counts = counts; a.offsets = offsets; a.sorted_slots = sorted;
  a.ws_blk_counts = at<int32_t>(ws, L.blk_counts);
  a.ws_local_rank = at<int32_t>(ws, L.local_rank);
  hipError_t e = moe::launch_router(a, s);
  return e == hipSuccess ? MOE_OK : hip_fail(e, counts ? "moe_route" : "moe_router");
}

int run_dispatch(const moe_dims* d, int32_t T, const int32_t* idx, int32_t* counts,
                 int32_t* offsets, int32_t* sorted, void* ws, hipStream_t s) {
  const Layout L = layout(d, T);
  moe::DispatchArgs a{};
  a.T = T; a.E = d->num_experts; a.K = d->top_k;
  a.topk_idx = idx; a.counts = counts; a.offsets = offsets; a.sorted_slots = sorted;
  a.ws_blk_counts = at<int32_t>(ws, L.blk_counts);
  a.ws_local_rank = at<int32_t>(ws, L.local_rank);
  hipError_t e = moe::launch_dispatch(a, s);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_dispatch");
}

int run_gate_up(const moe_dims* d, int32_t T, const void* x, const void* w_gate_up,
                const int32_t* offsets, const int32_t* sorted, void* h, hipStream_t s,
                hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr) {
  const size_t act = dtype_size(d->act_dtype);
  const long long H = d->hidden, I = d->expert_inter;
  moe::GateUpArgs g{};
  g.T = T; g.H = d->hidden; g.N = d->expert_inter; g.E = d->num_experts; g.K = d->top_k;
  g.rows = T * d->top_k; g.ident = false; g.bf16 = d->act_dtype == MOE_BF16;
  g.x = x;
  g.w_gate = w_gate_up;
  g.w_up = static_cast<const char*>(w_gate_up) + act * I * H;
  g.w_stride = 2 * I * H;
  g.offsets = offsets; g.sorted_slots = sorted; g.h = h;
  g.ev_start = ev_start; g.ev_stop = ev_stop;
  hipError_t e = moe::launch_gate_up(g, s);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "expert gate_up");
}

int run_down(const moe_dims* d, int32_t T, const void* h, const void* w_down,
             const float* topk_w, const int32_t* offsets, const int32_t* sorted, void* y,
             hipStream_t s) {
  moe::DownArgs dn{};
  dn.T = T; dn.H = d->hidden; dn.N = d->expert_inter; dn.E = d->num_experts; dn.K = d->top_k;
  dn.rows = T * d->top_k; dn.ident = false; dn.bf16 = d->act_dtype == MOE_BF16;
  dn.y_bf16 = d->slot_dtype == MOE_BF16;
  dn.h = h; dn.w_down = w_down; dn.w_stride = (long long)d->hidden * d->expert_inter;
  dn.offsets = offsets; dn.sorted_slots = sorted; dn.topk_w = topk_w; dn.y = y;
  hipError_t e = moe::launch_down(dn, s);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "expert down");
}

int run_expert_ffn(const moe_dims* d, int32_t T, const void* x, const void* w_gate_up,
                   const void* w_down, const float* topk_w, const int32_t* offsets,
                   const int32_t* sorted, void* y, void* ws, hipStream_t s) {
  void* h = at<void>(ws, layout(d, T).h);
  int rc = run_gate_up(d, T, x, w_gate_up, offsets, sorted, h, s);
  if (rc) return rc;
  return run_down(d, T, h, w_down, topk_w, offsets, sorted, y, s);
}

// Experts on weights stored below bf16 (fmt: int8, E4M3 or MXFP4).  Codes
// of gate_up are [E, 2I, H] and of down [E, H, I] (MXFP4: two per byte);
// scales are fp32 [E, 2I] / [E, H] (int8, E4M3) or E8M0 [E, 2I, H/32] /
// [E, H, I/32] (MXFP4).  Weight-streaming kernels up to 256 tokens, the
// tiled grouped GEMMs past that.
int run_expert_ffn_q(const moe_dims* d, moe::WFormat fmt, int32_t T, const void* x,
                     const void* guq, const void* gus, const void* dnq, const void* dns,
                     const float* topk_w, const int32_t* offsets, const int32_t* sorted,
                     void* y, void* ws, hipStream_t s) {
  void* h = at<void>(ws, layout(d, T).h);
  const long long H = d->hidden, I = d->expert_inter;
  const bool mx = fmt == moe::WFormat::kMXFP4;
  const long long unit = mx ? 2 : 1;  // weights per stored byte
  const unsigned char* gq = static_cast<const unsigned char*>(guq);
  moe::GateUpArgs g{};
  g.T = T; g.H = d->hidden; g.N = d->expert_inter; g.E = d->num_experts; g.K = d->top_k;
  g.rows = T * d->top_k; g.ident = false; g.bf16 = true;
  g.x = x; g.w_gate = gq; g.w_up = gq + I * H / unit; g.w_stride = 2 * I * H;
  g.offsets = offsets; g.sorted_slots = sorted; g.h = h;
  g.w_fmt = fmt;
  if (mx) {
    g.s_gate = gus;
    g.s_up = static_cast<const unsigned char*>(gus) + I * (H / 32);
    g.s_stride = 2 * I * (H / 32);
  } else {
    g.s_gate = gus;
    g.s_up = static_cast<const float*>(gus) + I;
    g.s_stride = 2 * I;
  }
  hipError_t e = moe::launch_gate_up(g, s);
  if (e != hipSuccess) return hip_fail(e, "expert gate_up (quantized weights)");
  moe::DownArgs dn{};
  dn.T = T; dn.H = d->hidden; dn.N = d->expert_inter; dn.E = d->num_experts; dn.K = d->top_k;
  dn.rows = T * d->top_k; dn.ident = false; dn.bf16 = true;
  dn.y_bf16 = d->slot_dtype == MOE_BF16;
  dn.h = h; dn.w_down = dnq; dn.w_stride = H * I;
  dn.offsets = offsets; dn.sorted_slots = sorted; dn.topk_w = topk_w; dn.y = y;
  dn.w_fmt = fmt; dn.s_down = dns; dn.s_stride = mx ? H * (I / 32) : H;
  e = moe::launch_down(dn, s);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "expert down (quantized weights)");
}

// MXFP4 kernels stage a block's E8M0 scale rows in LDS, one byte per 32
// weights of a contraction of at most this length.
constexpr int kMaxMxContraction = 8192;

// Format code of the ABI -> the kernels' format, or -1 if unknown.
int wformat_of(int32_t fmt, moe::WFormat& f) {
  switch (fmt) {
    case MOE_W_INT8: f = moe::WFormat::kInt8; return 0;
    case MOE_W_FP8: f = moe::WFormat::kFP8; return 0;
    case MOE_W_MXFP4: f = moe::WFormat::kMXFP4; return 0;
    case MOE_W_MXFP8: f = moe::WFormat::kMXFP8; return 0;
    default: return fail(MOE_ERR_ARG, "weight format %d unknown", fmt);
  }
}

int run_combine(const moe_dims* d, int32_t T, const void* y, const void* addend, void* out,
                hipStream_t s) {
  moe::CombineArgs a{};
  a.T = T; a.H = d->hidden; a.K = d->top_k;
  a.y_bf16 = d->slot_dtype == MOE_BF16; a.act_bf16 = d->act_dtype == MOE_BF16;
  a.y = y; a.addend = addend; a.out = out;
  hipError_t e = moe::launch_combine(a, s);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_combine");
}

// The matrices of one layer: in the activation dtype (quant == false), or
// codes and scales in format fmt.  Gains, router and layer_scalar are fp32.
struct LayerW {
  const float *g_pre, *g_pre2, *g_post1, *g_post2, *g_post;
  const float *router_w, *router_scale, *per_expert_scale;
  float layer_scalar;
  bool quant;
  moe::WFormat fmt;
  const void *dg, *dgs, *du, *dus, *dd, *dds;  // dense gate, up, down (and scales)
  const void *gu, *gus, *dn, *dns;             // experts' gate_up, down (and scales)
};

// One dual-path layer: pre-norms; the dense branch on the side stream; router,
// dispatch and experts on the caller's stream; the epilogue after the join.
int run_layer(const moe_dims* dims, int32_t T, const void* residual, const LayerW& lw,
              void* out, float* ffn_out, int32_t* topk_idx, float* topk_w, void* ws,
              hipStream_t s) {
  int rc;
  const Layout L = layout(dims, T);
  const bool bf = dims->act_dtype == MOE_BF16;
  int32_t* idx = topk_idx ? topk_idx : at<int32_t>(ws, L.idx);
  float* w = topk_w ? topk_w : at<float>(ws, L.w);
  int32_t* counts = at<int32_t>(ws, L.counts);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* sorted = at<int32_t>(ws, L.sorted);
  void* y = at<void>(ws, L.y);
  void* xd = at<void>(ws, L.xd);
  void* xm = at<void>(ws, L.xm);
  void* hd = at<void>(ws, L.hd);
  void* dnb = at<void>(ws, L.dn);

  moe::PreNormArgs pn{};
  pn.T = T; pn.H = dims->hidden; pn.eps = dims->eps; pn.bf16 = bf;
  pn.x = residual; pn.g_pre = lw.g_pre; pn.g_pre2 = lw.g_pre2; pn.xd = xd; pn.xm = xm;
  hipError_t e = moe::launch_prenorm(pn, s);
  if (e != hipSuccess) return hip_fail(e, "ffn layer (prenorm)");

  // dense branch on the side stream, after the pre-norms
  std::lock_guard<std::mutex> lock(g_side_mu);
  SideStream* side = nullptr;
  if ((e = side_stream(side)) != hipSuccess) return hip_fail(e, "ffn layer (side stream)");
  hipStream_t s2 = side->stream;
  if ((e = hipEventRecord(side->fork, s)) != hipSuccess ||
      (e = hipStreamWaitEvent(s2, side->fork, 0)) != hipSuccess)
    return hip_fail(e, "ffn layer (fork)");

  moe::GateUpArgs g{};
  g.T = T; g.H = dims->hidden; g.N = dims->dense_inter; g.E = 1; g.K = 1; g.rows = T;
  g.ident = true; g.bf16 = bf; g.x = xd; g.w_gate = lw.dg; g.w_up = lw.du;
  g.w_stride = 0; g.offsets = nullptr; g.sorted_slots = nullptr; g.h = hd;
  moe::DownArgs dd{};
  dd.T = T; dd.H = dims->hidden; dd.N = dims->dense_inter; dd.E = 1; dd.K = 1; dd.rows = T;
  dd.ident = true; dd.bf16 = bf; dd.y_bf16 = dims->slot_dtype == MOE_BF16; dd.h = hd;
  dd.w_down = lw.dd; dd.w_stride = 0; dd.offsets = nullptr; dd.sorted_slots = nullptr;
  dd.topk_w = nullptr; dd.y = dnb;
  if (lw.quant) {
    // one group: the per-expert strides are never applied
    g.w_fmt = lw.fmt; g.s_gate = lw.dgs; g.s_up = lw.dus; g.s_stride = 0;
    dd.w_fmt = lw.fmt; dd.s_down = lw.dds; dd.s_stride = 0;
    if ((e = moe::launch_gate_up(g, s2)) != hipSuccess)
      return hip_fail(e, "ffn layer (dense gate_up, quantized weights)");
    if ((e = moe::launch_down(dd, s2)) != hipSuccess)
      return hip_fail(e, "ffn layer (dense down, quantized weights)");
  } else {
    if ((e = moe::launch_gate_up(g, s2)) != hipSuccess)
      return hip_fail(e, "ffn layer (dense gate_up)");
    if ((e = moe::launch_down(dd, s2)) != hipSuccess)
      return hip_fail(e, "ffn layer (dense down)");
  }
  if ((e = hipEventRecord(side->join, s2)) != hipSuccess)
    return hip_fail(e, "ffn layer (join)");

  // router and experts on the caller's stream, meanwhile
  if ((rc = run_router(dims, T, residual, lw.router_w, lw.router_scale, lw.per_expert_scale,
                       lw.g_pre2, idx, w, counts, offsets, sorted, ws, s)))
    return rc;
  rc = lw.quant ? run_expert_ffn_q(dims, lw.fmt, T, xm, lw.gu, lw.gus, lw.dn, lw.dns, w,
                                   offsets, sorted, y, ws, s)
                : run_expert_ffn(dims, T, xm, lw.gu, lw.dn, w, offsets, sorted, y, ws, s);
  if (rc) return rc;
  if ((e = hipStreamWaitEvent(s, side->join, 0)) != hipSuccess)
    return hip_fail(e, "ffn layer (join)");

  moe::EpilogueArgs ep{};
  ep.T = T; ep.H = dims->hidden; ep.K = dims->top_k; ep.eps = dims->eps;
  ep.layer_scalar = lw.layer_scalar; ep.y_bf16 = dims->slot_dtype == MOE_BF16; ep.act_bf16 = bf;
  ep.y = y; ep.dn = dnb; ep.x = residual; ep.g_post1 = lw.g_post1; ep.g_post2 = lw.g_post2;
  ep.g_post = lw.g_post; ep.out = out; ep.ffn_out = ffn_out;
  if ((e = moe::launch_block_epilogue(ep, s)) != hipSuccess)
    return hip_fail(e, "ffn layer (epilogue)");
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_workspace_size(const moe_dims* dims, int32_t max_tokens) {
  if (check_dims(dims, true) != MOE_OK) return 0;
  if (check_tokens(dims, max_tokens) != MOE_OK) return 0;
  return layout(dims, max_tokens).total;
}

const char* moe_last_error(void) { return g_err.c_str(); }

int moe_router(const moe_dims* dims, int32_t T, const void* x, const float* router_w,
               const float* router_scale, const float* per_expert_scale,
               const float* pre_norm_gain, int32_t* topk_idx, float* topk_w, void* ws,
               size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_dims(dims)) || (rc = check_tokens(dims, T))) return rc;
  g_err.clear();
  if (T == 0) return MOE_OK;
  REQUIRE_PTR(x); REQUIRE_PTR(router_w); REQUIRE_PTR(router_scale);
  REQUIRE_PTR(per_expert_scale); OPTIONAL_PTR(pre_norm_gain);
  REQUIRE_PTR(topk_idx); REQUIRE_PTR(topk_w);
  if ((rc = check_ws(dims, T, ws, ws_bytes))) return rc;
  return run_router(dims, T, x, router_w, router_scale, per_expert_scale, pre_norm_gain,
                    topk_idx, topk_w, nullptr, nullptr, nullptr, ws,
                    static_cast<hipStream_t>(stream));
}

int moe_route(const moe_dims* dims, int32_t T, const void* x, const float* router_w,
              const float* router_scale, const float* per_expert_scale,
              const float* pre_norm_gain, int32_t* topk_idx, float* topk_w,
              int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_slots, void* ws,
              size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_dims(dims)) || (rc = check_tokens(dims, T))) return rc;
  g_err.clear();
  if (T == 0) return MOE_OK;
  REQUIRE_PTR(x); REQUIRE_PTR(router_w); REQUIRE_PTR(router_scale);
  REQUIRE_PTR(per_expert_scale); OPTIONAL_PTR(pre_norm_gain);
  REQUIRE_PTR(topk_idx); REQUIRE_PTR(topk_w); REQUIRE_PTR(expert_counts);
  REQUIRE_PTR(expert_offsets); REQUIRE_PTR(sorted_slots);
  if ((rc = check_ws(dims, T, ws, ws_bytes))) return rc;
  return run_router(dims, T, x, router_w, router_scale, per_expert_scale, pre_norm_gain,
                    topk_idx, topk_w, expert_counts, expert_offsets, sorted_slots, ws,
                    static_cast<hipStream_t>(stream));
}

int moe_dispatch(const moe_dims* dims, int32_t T, const int32_t* topk_idx,
                 int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_slots,
                 void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_dims(dims)) || (rc = check_tokens(dims, T))) return rc;
  g_err.clear();
  if (T == 0) return MOE_OK;
  REQUIRE_PTR(topk_idx); REQUIRE_PTR(expert_counts); REQUIRE_PTR(expert_offsets);
  REQUIRE_PTR(sorted_slots);
  if ((rc = check_ws(dims, T, ws, ws_bytes))) return rc;
  return run_dispatch(dims, T, topk_idx, expert_counts, expert_offsets, sorted_slots, ws,
                      static_cast<hipStream_t>(stream));
}

int moe_dense_mask_dispatch(const moe_dims* dims, int32_t T, const int32_t* topk_idx,
                            const float* topk_w, int32_t* expert_offsets, int32_t* sorted_slots,
                            float* w_dense, void* stream) {
  int rc;
  if ((rc = check_dims(dims)) || (rc = check_tokens(dims, T))) return rc;
  g_err.clear();
  if ((long long)T * dims->num_experts > (1 << 20))
    return fail(MOE_ERR_UNSUPPORTED, "T*num_experts=%lld exceeds 2^20",
                (long long)T * dims->num_experts);
  if (T == 0) return MOE_OK;
  REQUIRE_PTR(topk_idx); REQUIRE_PTR(topk_w); REQUIRE_PTR(expert_offsets);
  REQUIRE_PTR(sorted_slots); REQUIRE_PTR(w_dense);
  hipError_t e = moe::launch_dense_mask(T, dims->num_experts, dims->top_k, topk_idx, topk_w,
                                        expert_offsets, sorted_slots, w_dense,
                                        static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_dense_mask_dispatch");
}

int moe_expert_ffn(const moe_dims* dims, int32_t T, const void* x, const void* w_gate_up,
                   const void* w_down, const float* topk_w, const int32_t* expert_offsets,
                   const int32_t* sorted_slots, void* y_slots, void* ws, size_t ws_bytes,
                   void* stream) {
  int rc;
  if ((rc = check_dims(dims, true)) || (rc = check_tokens(dims, T))) return rc;
  g_err.clear();
  if (T == 0) return MOE_OK;
  REQUIRE_PTR(x); REQUIRE_PTR(w_gate_up); REQUIRE_PTR(w_down); REQUIRE_PTR(topk_w);
  REQUIRE_PTR(expert_offsets); REQUIRE_PTR(sorted_slots); REQUIRE_PTR(y_slots);
  if ((rc = check_ws(dims, T, ws, ws_bytes))) return rc;
  return run_expert_ffn(dims, T, x, w_gate_up, w_down, topk_w, expert_offsets, sorted_slots,
                        y_slots, ws, static_cast<hipStream_t>(stream));
}

int moe_quantize(int32_t fmt, int64_t rows, int32_t cols, const void* w, void* q, void* scale,
                 void* stream) {
  g_err.clear();
  moe::WFormat f;
  if (wformat_of(fmt, f)) return MOE_ERR_ARG;
  if (rows < 0 || rows > (int64_t)1 << 36) return fail(MOE_ERR_ARG, "rows out of range");
  const int align = f == moe::WFormat::kMXFP4 || f == moe::WFormat::kMXFP8 ? 32 : 8;
  if (cols <= 0 || cols % align != 0)
    return fail(MOE_ERR_ARG, "cols must be a positive multiple of %d", align);
  if (rows == 0) return MOE_OK;
  REQUIRE_PTR(w); REQUIRE_PTR(q); REQUIRE_PTR(scale);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (f) {
    case moe::WFormat::kMXFP8:
      e = moe::launch_mx8_quantize(rows, cols, w, static_cast<uint8_t*>(q),
                                   static_cast<uint8_t*>(scale), s);
      break;
    case moe::WFormat::kInt8:
      e = moe::launch_quantize_rows(rows, cols, w, static_cast<int8_t*>(q),
                                    static_cast<float*>(scale), s);
      break;
    case moe::WFormat::kFP8:
      e = moe::launch_quantize_fp8(rows, cols, w, static_cast<uint8_t*>(q),
                                   static_cast<float*>(scale), s);
      break;
    default:
      e = moe::launch_quantize_mxfp4(rows, cols, w, static_cast<uint8_t*>(q),
                                     static_cast<uint8_t*>(scale), s);
      break;
  }
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_quantize");
}

int moe_dequantize(int32_t fmt, int64_t rows, int32_t cols, const void* q, const void* scale,
                   float* out, void* stream) {
  g_err.clear();
  moe::WFormat f;
  if (wformat_of(fmt, f)) return MOE_ERR_ARG;
  if (rows < 0 || rows > (int64_t)1 << 36) return fail(MOE_ERR_ARG, "rows out of range");
  const int align = f == moe::WFormat::kMXFP4 || f == moe::WFormat::kMXFP8 ? 32 : 16;
  if (cols <= 0 || cols % align != 0)
    return fail(MOE_ERR_ARG, "cols must be a positive multiple of %d", align);
  if (rows == 0) return MOE_OK;
  REQUIRE_PTR(q); REQUIRE_PTR(scale); REQUIRE_PTR(out);
  hipError_t e =
      f == moe::WFormat::kMXFP8
          ? moe::launch_mx8_dequantize(rows, cols, static_cast<const uint8_t*>(q),
                                       static_cast<const uint8_t*>(scale), out,
                                       static_cast<hipStream_t>(stream))
          : moe::launch_dequantize(f, rows, cols, q, scale, out,
                                   static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_dequantize");
}

int moe_expert_ffn_q(const moe_dims* dims, int32_t fmt, int32_t T, const void* x,
                     const void* w_gate_up_q, const void* w_gate_up_scale, const void* w_down_q,
                     const void* w_down_scale, const float* topk_w,
                     const int32_t* expert_offsets, const int32_t* sorted_slots, void* y_slots,
                     void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_dims(dims, true)) || (rc = check_tokens(dims, T))) return rc;
  g_err.clear();
  moe::WFormat f;
  if (wformat_of(fmt, f)) return MOE_ERR_ARG;
  if (f == moe::WFormat::kMXFP8)
    return fail(MOE_ERR_ARG, "MXFP8 is an activation format, not an expert weight format here");
  if (dims->act_dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "quantized experts take bf16 activations");
  if (T == 0) return MOE_OK;
  REQUIRE_PTR(x); REQUIRE_PTR(w_gate_up_q); REQUIRE_PTR(w_gate_up_scale); REQUIRE_PTR(w_down_q);
  REQUIRE_PTR(w_down_scale); REQUIRE_PTR(topk_w); REQUIRE_PTR(expert_offsets);
  REQUIRE_PTR(sorted_slots); REQUIRE_PTR(y_slots);
  if ((rc = check_ws(dims, T, ws, ws_bytes))) return rc;
  return run_expert_ffn_q(dims, f, T, x, w_gate_up_q, w_gate_up_scale, w_down_q, w_down_scale,
                          topk_w, expert_offsets, sorted_slots, y_slots, ws,
                          static_cast<hipStream_t>(stream));
}

int moe_expert_ffn_mx(const moe_dims* dims, int32_t fmt, int32_t T, const void* x,
                      const void* w_gate_up_q, const void* w_gate_up_scale, const void* w_down_q,
                      const void* w_down_scale, const float* topk_w,
                      const int32_t* expert_offsets, const int32_t* sorted_slots, void* y_slots,
                      void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_dims(dims, true)) || (rc = check_tokens(dims, T))) return rc;
  g_err.clear();
  moe::WFormat f;
  if (wformat_of(fmt, f)) return MOE_ERR_ARG;
  if (f != moe::WFormat::kFP8 && f != moe::WFormat::kMXFP4)
    return fail(MOE_ERR_ARG, "moe_expert_ffn_mx takes E4M3 or MXFP4 expert weights");
  if (dims->act_dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "8-bit / 4-bit experts take bf16 activations");
  if (!moe::mx_uses_stream_kernels(T, T * dims->top_k, dims->num_experts) &&
      !moe::mx_tiled_supported(dims->hidden, dims->expert_inter))
    return fail(MOE_ERR_UNSUPPORTED, "8-bit / 4-bit experts past 256 tokens: hidden and "
                                     "expert_inter must be multiples of 64, at most 4096");
  if (T == 0) return MOE_OK;
  REQUIRE_PTR(x); REQUIRE_PTR(w_gate_up_q); REQUIRE_PTR(w_gate_up_scale); REQUIRE_PTR(w_down_q);
  REQUIRE_PTR(w_down_scale); REQUIRE_PTR(topk_w); REQUIRE_PTR(expert_offsets);
  REQUIRE_PTR(sorted_slots); REQUIRE_PTR(y_slots);
  if ((rc = check_ws(dims, T, ws, ws_bytes))) return rc;
  const Layout L = layout(dims, T);
  moe::MxArgs a{};
  a.T = T; a.H = dims->hidden; a.I = dims->expert_inter; a.E = dims->num_experts;
  a.K = dims->top_k; a.rows = T * dims->top_k; a.fmt = f;
  a.y_bf16 = dims->slot_dtype == MOE_BF16;
  a.x = x; a.xq = at<uint8_t>(ws, L.xq); a.xs = at<uint8_t>(ws, L.xs);
  a.hq = at<uint8_t>(ws, L.hq); a.hs = at<uint8_t>(ws, L.hs);
  a.gate_up_q = w_gate_up_q; a.gate_up_s = w_gate_up_scale;
  a.down_q = w_down_q; a.down_s = w_down_scale;
  a.offsets = expert_offsets; a.sorted_slots = sorted_slots; a.topk_w = topk_w; a.y = y_slots;
  hipError_t e = moe::launch_expert_ffn_mx(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_expert_ffn_mx");
}

int moe_quantize_int8(int64_t rows, int32_t cols, const void* w, int8_t* q, float* scale,
                      void* stream) {
  return moe_quantize(MOE_W_INT8, rows, cols, w, q, scale, stream);
}

int moe_expert_ffn_int8(const moe_dims* dims, int32_t T, const void* x, const int8_t* w_gate_up_q,
                        const float* w_gate_up_scale, const int8_t* w_down_q,
                        const float* w_down_scale, const float* topk_w,
                        const int32_t* expert_offsets, const int32_t* sorted_slots, void* y_slots,
                        void* ws, size_t ws_bytes, void* stream) {
  return moe_expert_ffn_q(dims, MOE_W_INT8, T, x, w_gate_up_q, w_gate_up_scale, w_down_q,
                          w_down_scale, topk_w, expert_offsets, sorted_slots, y_slots, ws,
                          ws_bytes, stream);
}

int moe_expert_gate_up(const moe_dims* dims, int32_t T, const void* x, const void* w_gate_up,
                       const int32_t* expert_offsets, const int32_t* sorted_slots, void* h,
                       void* stream) {
  int rc;
  if ((rc = check_dims(dims, true)) || (rc = check_tokens(dims, T))) return rc;
  g_err.clear();
  if (T == 0) return MOE_OK;
  REQUIRE_PTR(x); REQUIRE_PTR(w_gate_up); REQUIRE_PTR(expert_offsets);
  REQUIRE_PTR(sorted_slots); REQUIRE_PTR(h);
  return run_gate_up(dims, T, x, w_gate_up, expert_offsets, sorted_slots, h,
                     static_cast<hipStream_t>(stream));
}

int moe_expert_gate_up_timed(const moe_dims* dims, int32_t T, const void* x,
                             const void* w_gate_up, const int32_t* expert_offsets,
                             const int32_t* sorted_slots, void* h, void* stream,
                             void* start_event, void* stop_event) {
  int rc;
  if ((rc = check_dims(dims, true)) || (rc = check_tokens(dims, T))) return rc;
  g_err.clear();
  if (!start_event || !stop_event) return fail(MOE_ERR_ARG, "start_event and stop_event are required");
  if (T == 0) return MOE_OK;
  REQUIRE_PTR(x); REQUIRE_PTR(w_gate_up); REQUIRE_PTR(expert_offsets);
  REQUIRE_PTR(sorted_slots); REQUIRE_PTR(h);
  return run_gate_up(dims, T, x, w_gate_up, expert_offsets, sorted_slots, h,
                     static_cast<hipStream_t>(stream), static_cast<hipEvent_t>(start_event),
                     static_cast<hipEvent_t>(stop_event));
}

int moe_expert_down(const moe_dims* dims, int32_t T, const void* h, const void* w_down,
                    const float* topk_w, const int32_t* expert_offsets,
                    const int32_t* sorted_slots, void* y_slots, void* stream) {
  int rc;
  if ((rc = check_dims(dims, true)) || (rc = check_tokens(dims, T))) return rc;
  g_err.clear();
  if (T == 0) return MOE_OK;
  REQUIRE_PTR(h); REQUIRE_PTR(w_down); REQUIRE_PTR(topk_w); REQUIRE_PTR(expert_offsets);
  REQUIRE_PTR(sorted_slots); REQUIRE_PTR(y_slots);
  return run_down(dims, T, h, w_down, topk_w, expert_offsets, sorted_slots, y_slots,
                  static_cast<hipStream_t>(stream));
}

int moe_combine(const moe_dims* dims, int32_t T, const void* y_slots, const void* addend,
                void* out, void* stream) {
  int rc;
  if ((rc = check_dims(dims, true)) || (rc = check_tokens(dims, T))) return rc;
  g_err.clear();
  if (T == 0) return MOE_OK;
  REQUIRE_PTR(y_slots); OPTIONAL_PTR(addend); REQUIRE_PTR(out);
  return run_combine(dims, T, y_slots, addend, out, static_cast<hipStream_t>(stream));
}

int moe_forward(const moe_dims* dims, int32_t T, const void* x, const float* router_w,
                const float* router_scale, const float* per_expert_scale,
                const void* w_gate_up, const void* w_down, void* out, int32_t* topk_idx,
                float* topk_w, void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_dims(dims)) || (rc = check_tokens(dims, T))) return rc;
  g_err.clear();
  if (T == 0) return MOE_OK;
  REQUIRE_PTR(x); REQUIRE_PTR(router_w); REQUIRE_PTR(router_scale);
  REQUIRE_PTR(per_expert_scale); REQUIRE_PTR(w_gate_up); REQUIRE_PTR(w_down); REQUIRE_PTR(out);
  OPTIONAL_PTR(topk_idx); OPTIONAL_PTR(topk_w);
  if ((rc = check_ws(dims, T, ws, ws_bytes))) return rc;
  return run_forward(dims, T, x, router_w, router_scale, per_expert_scale, w_gate_up, w_down,
                     out, topk_idx, topk_w, ws, static_cast<hipStream_t>(stream));
}

int moe_forward_noalloc(const moe_dims* dims, int32_t T, const void* x, const float* router_w,
                        const float* router_scale, const float* per_expert_scale,
                        const void* w_gate_up, const void* w_down, void* out, int32_t* topk_idx,
                        float* topk_w, void* stream) {
  int rc;
  if ((rc = check_dims(dims)) || (rc = check_tokens(dims, T))) return rc;
  g_err.clear();
  if (T == 0) return MOE_OK;
  REQUIRE_PTR(x); REQUIRE_PTR(router_w); REQUIRE_PTR(router_scale);
  REQUIRE_PTR(per_expert_scale); REQUIRE_PTR(w_gate_up); REQUIRE_PTR(w_down); REQUIRE_PTR(out);
  OPTIONAL_PTR(topk_idx); OPTIONAL_PTR(topk_w);
  const size_t need = layout(dims, T).base_end;  // moe_forward uses no MXFP8 region
  if (need > kNoAllocScratchBytes)
    return fail(MOE_ERR_WORKSPACE,
                "moe_forward_noalloc: T=%d needs %zu bytes of scratch, the library's array "
                "holds %zu",
                T, need, kNoAllocScratchBytes);
  void* ws = nullptr;
  hipError_t e = noalloc_scratch(ws);
  if (e != hipSuccess) return hip_fail(e, "moe_forward_noalloc (scratch address)");
  return run_forward(dims, T, x, router_w, router_scale, per_expert_scale, w_gate_up, w_down,
                     out, topk_idx, topk_w, ws, static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

int run_forward(const moe_dims* dims, int32_t T, const void* x, const float* router_w,
                const float* router_scale, const float* per_expert_scale,
                const void* w_gate_up, const void* w_down, void* out, int32_t* topk_idx,
                float* topk_w, void* ws, hipStream_t s) {
  int rc;
  const Layout L = layout(dims, T);
  int32_t* idx = topk_idx ? topk_idx : at<int32_t>(ws, L.idx);
  float* w = topk_w ? topk_w : at<float>(ws, L.w);
  int32_t* counts = at<int32_t>(ws, L.counts);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* sorted = at<int32_t>(ws, L.sorted);
  void* y = at<void>(ws, L.y);
  if ((rc = run_router(dims, T, x, router_w, router_scale, per_expert_scale, nullptr, idx, w,
                       counts, offsets, sorted, ws, s)))
    return rc;
  if ((rc = run_expert_ffn(dims, T, x, w_gate_up, w_down, w, offsets, sorted, y, ws, s)))
    return rc;
  return run_combine(dims, T, y, nullptr, out, s);
}

}  // namespace

extern "C" {

int gemma4_ffn_block(const moe_dims* dims, int32_t T, const void* residual,
                     const gemma4_ffn_weights* wt, void* out, float* ffn_out,
                     int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                     void* stream) {
  int rc;
  if ((rc = check_dims(dims)) || (rc = check_tokens(dims, T))) return rc;
  if (dims->dense_inter <= 0)
    return fail(MOE_ERR_UNSUPPORTED, "gemma4_ffn_block needs dense_inter > 0");
  g_err.clear();
  if (T == 0) return MOE_OK;
  if (!wt) return fail(MOE_ERR_ARG, "weights is NULL");
  REQUIRE_PTR(residual); REQUIRE_PTR(out); OPTIONAL_PTR(ffn_out);
  OPTIONAL_PTR(topk_idx); OPTIONAL_PTR(topk_w);
  REQUIRE_PTR(wt->g_pre); REQUIRE_PTR(wt->g_pre2); REQUIRE_PTR(wt->g_post1);
  REQUIRE_PTR(wt->g_post2); REQUIRE_PTR(wt->g_post);
  REQUIRE_PTR(wt->dense_gate); REQUIRE_PTR(wt->dense_up); REQUIRE_PTR(wt->dense_down);
  REQUIRE_PTR(wt->router_w); REQUIRE_PTR(wt->router_scale); REQUIRE_PTR(wt->per_expert_scale);
  REQUIRE_PTR(wt->w_gate_up); REQUIRE_PTR(wt->w_down);
  if ((rc = check_ws(dims, T, ws, ws_bytes))) return rc;
  LayerW lw{};
  lw.g_pre = wt->g_pre; lw.g_pre2 = wt->g_pre2; lw.g_post1 = wt->g_post1;
  lw.g_post2 = wt->g_post2; lw.g_post = wt->g_post;
  lw.router_w = wt->router_w; lw.router_scale = wt->router_scale;
  lw.per_expert_scale = wt->per_expert_scale; lw.layer_scalar = wt->layer_scalar;
  lw.quant = false;
  lw.dg = wt->dense_gate; lw.du = wt->dense_up; lw.dd = wt->dense_down;
  lw.gu = wt->w_gate_up; lw.dn = wt->w_down;
  return run_layer(dims, T, residual, lw, out, ffn_out, topk_idx, topk_w, ws,
                   static_cast<hipStream_t>(stream));
}

int gemma4_ffn_block_q(const moe_dims* dims, int32_t T, const void* residual,
                       const gemma4_ffn_weights_q* wt, void* out, float* ffn_out,
                       int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                       void* stream) {
  int rc;
  if ((rc = check_dims(dims)) || (rc = check_tokens(dims, T))) return rc;
  if (dims->dense_inter <= 0)
    return fail(MOE_ERR_UNSUPPORTED, "gemma4_ffn_block_q needs dense_inter > 0");
  if (dims->act_dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "quantized layer takes bf16 activations");
  g_err.clear();
  if (T == 0) return MOE_OK;
  if (!wt) return fail(MOE_ERR_ARG, "weights is NULL");
  moe::WFormat f;
  if (wformat_of(wt->fmt, f)) return MOE_ERR_ARG;
  if (f == moe::WFormat::kMXFP8)
    return fail(MOE_ERR_ARG, "MXFP8 is an activation format, not a weight format here");
  if (f == moe::WFormat::kMXFP4 && dims->dense_inter > kMaxMxContraction)
    return fail(MOE_ERR_UNSUPPORTED, "MXFP4 weights: dense_inter=%d exceeds %d",
                dims->dense_inter, kMaxMxContraction);
  REQUIRE_PTR(residual); REQUIRE_PTR(out); OPTIONAL_PTR(ffn_out);
  OPTIONAL_PTR(topk_idx); OPTIONAL_PTR(topk_w);
  REQUIRE_PTR(wt->g_pre); REQUIRE_PTR(wt->g_pre2); REQUIRE_PTR(wt->g_post1);
  REQUIRE_PTR(wt->g_post2); REQUIRE_PTR(wt->g_post);
  REQUIRE_PTR(wt->dense_gate_q); REQUIRE_PTR(wt->dense_gate_scale);
  REQUIRE_PTR(wt->dense_up_q); REQUIRE_PTR(wt->dense_up_scale);
  REQUIRE_PTR(wt->dense_down_q); REQUIRE_PTR(wt->dense_down_scale);
  REQUIRE_PTR(wt->router_w); REQUIRE_PTR(wt->router_scale); REQUIRE_PTR(wt->per_expert_scale);
  REQUIRE_PTR(wt->gate_up_q); REQUIRE_PTR(wt->gate_up_scale);
  REQUIRE_PTR(wt->down_q); REQUIRE_PTR(wt->down_scale);
  if ((rc = check_ws(dims, T, ws, ws_bytes))) return rc;
  LayerW lw{};
  lw.g_pre = wt->g_pre; lw.g_pre2 = wt->g_pre2; lw.g_post1 = wt->g_post1;
  lw.g_post2 = wt->g_post2; lw.g_post = wt->g_post;
  lw.router_w = wt->router_w; lw.router_scale = wt->router_scale;
  lw.per_expert_scale = wt->per_expert_scale; lw.layer_scalar = wt->layer_scalar;
  lw.quant = true; lw.fmt = f;
  lw.dg = wt->dense_gate_q; lw.dgs = wt->dense_gate_scale;
  lw.du = wt->dense_up_q; lw.dus = wt->dense_up_scale;
  lw.dd = wt->dense_down_q; lw.dds = wt->dense_down_scale;
  lw.gu = wt->gate_up_q; lw.gus = wt->gate_up_scale;
  lw.dn = wt->down_q; lw.dns = wt->down_scale;
  return run_layer(dims, T, residual, lw, out, ffn_out, topk_idx, topk_w, ws,
                   static_cast<hipStream_t>(stream));
}

}  // extern "C"
