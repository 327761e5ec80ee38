/*
 * libmoe: the Gemma-4 26B-A4B mixture-of-experts feed-forward block on one
 * AMD Instinct MI355X (gfx950), as a C ABI.
 *
 * The layer these calls implement is described on the page "Porting a
 * 128-expert MoE (Gemma-4 26B-A4B) to AWS Inferentia2", section "The
 * architecture: a dual-path FFN nobody warned me about": a router (its own
 * RMSNorm, a scale, an H -> E projection, softmax in fp32, top-K,
 * renormalisation, x per_expert_scale), E gated experts stored as a fused
 * gate_up_proj [E, 2I, H] and a down_proj [E, H, I] evaluated as a sparse
 * gather / compute / weighted scatter-add, and beside them a dense gated MLP,
 * with pre- and post-norms on each branch, a final norm, the residual and a
 * layer_scalar.  The experts' activation is the tanh form of GELU ("Porting
 * Gemma-4 (2B / 4B / 12B) to AWS Inferentia2", section 4.5).
 *
 * The calls split along the page's seams: moe_router is Gemma4TextRouter
 * (whose output weights already carry the renormalisation and the
 * per-expert scale); moe_dispatch + moe_expert_ffn + moe_combine are
 * Gemma4TextExperts' gather, compute and scatter-add; gemma4_ffn_block is the
 * whole dual-path layer; moe_forward chains the four experts-only calls.
 *
 * Conventions (all calls):
 *   - Every array argument is a DEVICE pointer owned by the caller; nothing is
 *     retained after the call returns.  Inputs must stay alive and unmodified
 *     until the stream has executed the enqueued work.
 *   - Each call validates its arguments on the host first.  On a validation
 *     failure it returns a negative moe_status, launches nothing and makes no
 *     HIP call; moe_last_error() then names the problem.  Otherwise it enqueues
 *     kernels on `stream` (a hipStream_t; NULL is the default stream) and
 *     returns MOE_OK without synchronising.  A launch failure returns
 *     MOE_ERR_HIP.
 *   - T = 0 is a valid no-op.
 *   - No call allocates device memory.  Calls that need scratch take a
 *     workspace `ws` of at least moe_workspace_size() bytes, 256-byte aligned.
 *     Two calls in flight must not share a workspace.
 *   - Pointers must be 16-byte aligned.
 *   - Preconditions that are not checked: inputs are finite; topk_idx given to
 *     moe_dispatch lies in [0, E) with K distinct experts per token (a slot
 *     whose id is outside [0, E) is dropped: it is counted for no expert,
 *     is missing from sorted_slots, expert_offsets[E] falls short of T*K,
 *     and its y_slots row is left unwritten); the
 *     offsets / sorted_slots given to moe_expert_ffn are moe_dispatch's output
 *     for the same topk_idx.
 *   - Results are deterministic: no floating-point atomics; the same inputs
 *     give the same bits on every run.
 *
 * Layouts (row-major, innermost index last):
 *   x, residual, out          [T, H]        act dtype
 *   router_w                  [E, H]        fp32
 *   router_scale, gains       [H]           fp32
 *   per_expert_scale          [E]           fp32
 *   w_gate_up                 [E, 2I, H]    act dtype; rows [0,I) gate, [I,2I) up
 *   w_down                    [E, H, I]     act dtype
 *   dense_gate, dense_up      [D, H]        act dtype
 *   dense_down                [H, D]        act dtype
 *   topk_idx                  [T, K]        int32; slot k is the k-th largest logit
 *   topk_w                    [T, K]        fp32
 *   y_slots                   [T, K, H]     slot dtype; y_slots[t,k] = w[t,k] * expert(x_t)
 *   expert_counts             [E]           int32
 *   expert_offsets            [E + 1]       int32 exclusive prefix sum of counts
 *   sorted_slots              [T * K]       int32 slot ids t*K+k grouped by expert,
 *                                           ascending within each expert
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_ARG = -1,          /* NULL pointer, bad size, misaligned pointer */
  MOE_ERR_UNSUPPORTED = -2,  /* dimensions outside the supported range */
  MOE_ERR_WORKSPACE = -3,    /* workspace missing or smaller than required */
  MOE_ERR_HIP = -4           /* a HIP launch reported an error */
} moe_status;

/* Storage formats of expert weights below bf16 (batches of up to 256 tokens):
 *   MOE_W_INT8   int8 codes, one fp32 scale per output channel;
 *   MOE_W_FP8    E4M3 codes (OCP 8-bit floating point: bias 7, no
 *                infinities, largest finite 448), one fp32 scale per output
 *                channel;
 *   MOE_W_MXFP4  E2M1 codes, two per byte with the even element in the low
 *                nibble, and one E8M0 scale code per 32 consecutive weights of
 *                a row (OCP Microscaling), value = code * 2^(scale - 127). */
typedef enum moe_wformat {
  MOE_W_INT8 = 1,
  MOE_W_FP8 = 2,
  MOE_W_MXFP4 = 3,
  MOE_W_MXFP8 = 4   /* E4M3 codes with one E8M0 scale per 32 consecutive values
                     * of a row (OCP Microscaling MXFP8): the activation format
                     * of moe_expert_ffn_mx; moe_quantize / moe_dequantize only */
} moe_wformat;

typedef enum moe_dtype {
  MOE_F32 = 0,   /* fp32 storage and fp32 arithmetic (debug path) */
  MOE_BF16 = 1   /* bf16 storage, fp32 accumulation (fast path) */
} moe_dtype;

/* Layer dimensions.  Supported: hidden % 64 == 0 and 64 <= hidden <= 8192;
 * 1 <= num_experts <= 256; 1 <= top_k <= min(num_experts, 32);
 * expert_inter % 32 == 0, 32 <= expert_inter <= 8192; dense_inter == 0 or
 * dense_inter % 32 == 0, <= 16384; eps > 0.  act_dtype MOE_F32 requires
 * slot_dtype MOE_F32.  Token counts up to 65536 with T * top_k <= 2^20. */
typedef struct moe_dims {
  int32_t hidden;        /* H (2816 for 26B-A4B) */
  int32_t num_experts;   /* E (128) */
  int32_t top_k;         /* K (8) */
  int32_t expert_inter;  /* I (704) */
  int32_t dense_inter;   /* D (2112); 0 = no dense branch */
  float eps;             /* RMSNorm epsilon (1e-6), inside the square root */
  int32_t act_dtype;     /* moe_dtype of activations and expert / dense weights */
  int32_t slot_dtype;    /* moe_dtype of y_slots and of the dense branch output.
                          * MOE_F32 is the default and the one held to the
                          * accuracy bar (max |err| <= 2e-2 x RMS of an exact
                          * evaluation).  MOE_BF16 halves the slot traffic but
                          * rounds every slot once more and is OUTSIDE that
                          * bar (0.026 x RMS on one 64-token 26B-A4B batch);
                          * each bf16 slot is the fp32 slot rounded to
                          * nearest-even, so its extra error is at most 2^-8
                          * of each slot's magnitude. */
} moe_dims;

/* Weights of one dual-path layer (all device pointers). */
typedef struct gemma4_ffn_weights {
  const float* g_pre;      /* [H] pre_feedforward_layernorm gain (effective multiplier) */
  const float* g_pre2;     /* [H] pre_feedforward_layernorm_2 */
  const float* g_post1;    /* [H] post_feedforward_layernorm_1 (dense branch) */
  const float* g_post2;    /* [H] post_feedforward_layernorm_2 (MoE branch) */
  const float* g_post;     /* [H] post_feedforward_layernorm */
  const void* dense_gate;  /* [D, H] act dtype */
  const void* dense_up;    /* [D, H] act dtype */
  const void* dense_down;  /* [H, D] act dtype */
  const float* router_w;   /* [E, H] */
  const float* router_scale;      /* [H] */
  const float* per_expert_scale;  /* [E] */
  const void* w_gate_up;   /* [E, 2I, H] act dtype */
  const void* w_down;      /* [E, H, I] act dtype */
  float layer_scalar;      /* multiplies (FFN + residual) */
} gemma4_ffn_weights;

/* Bytes of workspace sufficient for every call below with T <= max_tokens.
 * Returns 0 if the dimensions are unsupported (moe_last_error() says why). */
size_t moe_workspace_size(const moe_dims* dims, int32_t max_tokens);

/* Message of the last failure on the calling thread ("" if none). */
const char* moe_last_error(void);

/* Router (Gemma4TextRouter): for each token, v = x (or, when pre_norm_gain is
 * not NULL, v = RMSNorm(x) * pre_norm_gain, i.e. pre_feedforward_layernorm_2);
 * vhat = v / sqrt(mean(v^2) + eps) * router_scale; logits = router_w . vhat
 * (fp32); p = softmax(logits) in fp32; the K experts with the largest logits
 * (ties to the lower index) in descending order; w_k = p_k / sum_j p_j *
 * per_expert_scale[e_k].  All router arithmetic is fp32; every reduction over
 * H runs in 64-element chunks, each a fused multiply-add chain in ascending
 * index from +0, the chunk results added in ascending chunk order, and the
 * square root and divisions are correctly rounded, so that the logits are
 * reproducible bit for bit on any IEEE fp32 machine.
 * x: [T,H] act dtype.  Outputs topk_idx [T,K], topk_w [T,K]. */
int moe_router(const moe_dims* dims, int32_t T, const void* x, const float* router_w,
               const float* router_scale, const float* per_expert_scale,
               const float* pre_norm_gain, int32_t* topk_idx, float* topk_w,
               void* ws, size_t ws_bytes, void* stream);

/* moe_router followed by moe_dispatch of its result, in one call (for small
 * batches the dispatch runs inside the router's top-K kernel).  Outputs are
 * those of the two calls. */
int moe_route(const moe_dims* dims, int32_t T, const void* x, const float* router_w,
              const float* router_scale, const float* per_expert_scale,
              const float* pre_norm_gain, int32_t* topk_idx, float* topk_w,
              int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_slots, void* ws,
              size_t ws_bytes, void* stream);

/* Groups the T*K token-slots by expert (the gather side of the experts'
 * sparse loop): expert_counts[e] = #slots with topk_idx == e, expert_offsets
 * their exclusive prefix sum (expert_offsets[E] = T*K), sorted_slots the slot
 * ids of expert 0, then expert 1, ..., ascending within each expert.
 * Integer-only and exact. */
int moe_dispatch(const moe_dims* dims, int32_t T, const int32_t* topk_idx,
                 int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_slots,
                 void* ws, size_t ws_bytes, void* stream);

/* Slot layout of the all-experts form of the experts (the page "Porting a
 * 128-expert MoE (Gemma-4 26B-A4B) to AWS Inferentia2", section "The
 * traceable trick: compute all experts, mask to top-8"): every expert takes
 * every token, weighted by the token's routing weight for it, which is 0 for
 * an expert outside its top-K; the sum over experts equals the sparse form's
 * sum over its K slots.  From the routing (topk_idx, topk_w [T,K], K =
 * dims->top_k) it writes, for E = dims->num_experts: expert_offsets[e] = e*T
 * (e = 0..E), sorted_slots[e*T + t] = t*E + e, w_dense[t*E + e] = topk_w[t,k]
 * when topk_idx[t,k] == e, else 0.  Pass these to moe_expert_ffn and
 * moe_combine with top_k = E (those calls take any top_k up to num_experts)
 * and a workspace sized for that top_k.  Integer and copy work only, exact.
 * Device pointers, 16-byte aligned; T*E must not exceed 2^20
 * (MOE_ERR_UNSUPPORTED). */
int moe_dense_mask_dispatch(const moe_dims* dims, int32_t T, const int32_t* topk_idx,
                            const float* topk_w, int32_t* expert_offsets, int32_t* sorted_slots,
                            float* w_dense, void* stream);

/* The experts (Gemma4TextExperts' compute): for every slot s = t*K+k routed
 * to expert e, y_slots[t,k,:] = topk_w[t,k] * down[e] (gelu_tanh(gate[e] x_t)
 * * (up[e] x_t)).  x: [T,H] expert input (act dtype).  bf16 path: bf16 MFMA
 * with fp32 accumulation, the GELU product rounded to bf16 before the down
 * projection.  fp32 path: fp32 arithmetic throughout. */
int moe_expert_ffn(const moe_dims* dims, int32_t T, const void* x, const void* w_gate_up,
                   const void* w_down, const float* topk_w, const int32_t* expert_offsets,
                   const int32_t* sorted_slots, void* y_slots, void* ws, size_t ws_bytes,
                   void* stream);

/* The two halves of moe_expert_ffn, for callers that schedule or time them
 * separately.  moe_expert_gate_up: for every expert-sorted row r of expert e
 * (slot s = sorted_slots[r], token t = s / K),
 * h[r,:] = gelu_tanh(gate[e] x_t) * (up[e] x_t); h: [T*K, I] act dtype (bf16 path:
 * rounded to bf16).  moe_expert_down: y_slots[s,:] = topk_w[s] * down[e] h[r,:]. */
int moe_expert_gate_up(const moe_dims* dims, int32_t T, const void* x, const void* w_gate_up,
                       const int32_t* expert_offsets, const int32_t* sorted_slots, void* h,
                       void* stream);
int moe_expert_down(const moe_dims* dims, int32_t T, const void* h, const void* w_down,
                    const float* topk_w, const int32_t* expert_offsets,
                    const int32_t* sorted_slots, void* y_slots, void* stream);

/* moe_expert_gate_up with its kernel timed: start_event and stop_event
 * (hipEvent_t, created by the caller with timing enabled, not NULL) are
 * recorded by the gate_up kernel's own dispatch (HIP's extended launch) when
 * it starts and ends, so hipEventElapsedTime(start, stop) is that kernel's
 * duration and no event packets sit between the stream's launches (a
 * hipEventRecord pair around a launch holds back the next dispatch until the
 * previous kernel has finished, ~5 us per record on MI355X).  Same result as
 * moe_expert_gate_up, bit for bit.  T == 0 launches nothing and leaves the
 * events untouched. */
int moe_expert_gate_up_timed(const moe_dims* dims, int32_t T, const void* x,
                             const void* w_gate_up, const int32_t* expert_offsets,
                             const int32_t* sorted_slots, void* h, void* stream,
                             void* start_event, void* stop_event);

/* int8 per-channel symmetric weights, the int8-expert variant on the page
 * "Porting a 128-expert MoE (Gemma-4 26B-A4B) to AWS Inferentia2", section
 * "Can it run on a smaller box? Yes, no, and "deeper than it looks"".
 * moe_quantize_int8: w is rows x cols bf16 (row-major; a row is one output
 * channel, cols % 8 == 0); writes scale[r] = max_c |w[r,c]| / 127 and
 * q[r,c] = round-half-to-even(w[r,c] / scale[r]) clamped to [-127, 127]
 * (fp32 divisions; a zero row gives scale 0 and codes 0).  For the experts:
 * quantize gate_up as E*2I rows of H and down as E*H rows of I.  Deterministic
 * and exact: codes and scales are the same on any IEEE machine.  Device
 * pointers, 16-byte aligned; returns MOE_ERR_ARG on bad sizes or pointers.
 *
 * moe_expert_ffn_int8: moe_expert_ffn with the experts' weights as int8 codes
 * and per-row scales (gate_up: codes [E,2I,H], scales [E,2I]; down: codes
 * [E,H,I], scales [E,H]).  The code rows enter bf16 MFMAs exactly and each
 * output channel is multiplied by its scale after the k-sum.  Act dtype bf16,
 * else MOE_ERR_UNSUPPORTED; any T that moe_expert_ffn takes (as
 * moe_expert_ffn_q with MOE_W_INT8). */
int moe_quantize_int8(int64_t rows, int32_t cols, const void* w, int8_t* q, float* scale,
                      void* stream);
int moe_expert_ffn_int8(const moe_dims* dims, int32_t T, const void* x,
                        const int8_t* w_gate_up_q, const float* w_gate_up_scale,
                        const int8_t* w_down_q, const float* w_down_scale, const float* topk_w,
                        const int32_t* expert_offsets, const int32_t* sorted_slots,
                        void* y_slots, void* ws, size_t ws_bytes, void* stream);

/* Expert weights below bf16: the int8 variant above and the 8-bit and 4-bit
 * floating-point options of the same page (section "The fp4 rabbit hole (two
 * of them, both dead ends)": FP8, and fp4 in a 32-element microscaling
 * block), in the formats of moe_wformat.
 *
 * moe_quantize: w is rows x cols bf16, a row one output channel (for the
 * experts: gate_up as E*2I rows of H, down as E*H rows of I).
 *   MOE_W_INT8   q int8 [rows, cols], scale fp32 [rows]: as moe_quantize_int8.
 *   MOE_W_FP8    q uint8 [rows, cols], scale fp32 [rows]: scale = max |w| /
 *                448, code = E4M3 nearest to w / scale (fp32 divisions; ties
 *                to the even mantissa; 448 at most), sign bit = w < 0; a zero
 *                row gives scale 0 and codes 0.  cols % 8 == 0.
 *   MOE_W_MXFP4  q uint8 [rows, cols / 2], scale uint8 [rows, cols / 32]: per
 *                32-weight block, shared = floor(log2 max |w|) - 2 clamped to
 *                [-127, 127], scale code = shared + 127, element = E2M1
 *                nearest to |w| / 2^shared (ties to the even mantissa, 6 at
 *                most) with sign bit w < 0; a zero block gives scale code 0
 *                and codes 0.  cols % 32 == 0.
 * Deterministic and exact (the same codes on any IEEE machine).
 *
 * moe_dequantize: codes (and scales) back to fp32 values, out [rows, cols];
 * int8 / E4M3: value * scale rounded once; MXFP4: value * 2^(scale - 127),
 * exact.  It widens codes exactly as moe_expert_ffn_q does.  cols % 16 == 0
 * (MXFP4: % 32).
 *
 * moe_expert_ffn_q: moe_expert_ffn with the experts' weights in format fmt
 * (gate_up codes of [E, 2I, H] weights and down codes of [E, H, I], scales
 * as moe_quantize lays them out).  Codes widen to bf16 exactly in registers
 * (MXFP4 with its block scale; block scales must exceed 2^-125 to stay in
 * bf16's normal range), enter bf16 MFMAs, and int8 / E4M3 output channels
 * are multiplied by their scale after the k-sum.  Up to 256 tokens the
 * weights are streamed from HBM (decode kernels); past that the tiled grouped
 * GEMMs stage the codes in LDS as stored and widen them after the LDS reads.
 * Act dtype bf16, else MOE_ERR_UNSUPPORTED; T as for moe_expert_ffn.
 *
 *   MOE_W_MXFP8  q uint8 [rows, cols], scale uint8 [rows, cols / 32]: per
 *                32-value block, shared = floor(log2 max |w|) - 8 clamped to
 *                [-127, 127], scale code = shared + 127, element = E4M3
 *                nearest to w / 2^shared (ties to the even mantissa, 448 at
 *                most); a zero block gives scale code 0 and codes 0.  cols %
 *                32 == 0.  Dequantized: value * 2^(scale - 127), exact.  Not
 *                a weight format of moe_expert_ffn_q / gemma4_ffn_block_q.
 * All three: device pointers, 16-byte aligned; MOE_ERR_ARG for an unknown
 * format, bad sizes or pointers. */
int moe_quantize(int32_t fmt, int64_t rows, int32_t cols, const void* w, void* q, void* scale,
                 void* stream);
int moe_dequantize(int32_t fmt, int64_t rows, int32_t cols, const void* q, const void* scale,
                   float* out, void* stream);
int moe_expert_ffn_q(const moe_dims* dims, int32_t fmt, int32_t T, const void* x,
                     const void* w_gate_up_q, const void* w_gate_up_scale, const void* w_down_q,
                     const void* w_down_scale, const float* topk_w,
                     const int32_t* expert_offsets, const int32_t* sorted_slots, void* y_slots,
                     void* ws, size_t ws_bytes, void* stream);

/* The E4M3 and MXFP4 experts on gfx950's 8-bit / 4-bit matrix instructions
 * (the FP8 and microscaling fp4 options of the page "Porting a 128-expert MoE
 * (Gemma-4 26B-A4B) to AWS Inferentia2", section "The fp4 rabbit hole (two
 * of them, both dead ends)"): the weights are multiplied in their own format,
 * never widened.  The activations enter those products in 8 bits too, as
 * MXFP8 (MOE_W_MXFP8 above: per block of 32 consecutive values along the
 * contraction, shared = floor(log2 max |v|) - 8 clamped to [-127, 127],
 * element = the E4M3 value nearest to v / 2^shared, ties to the even
 * mantissa, saturating at 448; a zero block gets scale code 0): the expert
 * input x before gate_up, and the gated product h = gelu_tanh(gate) * up
 * (from its fp32 value) before down.  Products accumulate in fp32; E4M3
 * weights' row scales multiply the k-sums.  So y_slots[t,k,:] = topk_w[t,k]
 * * down[e] MX(gelu_tanh(gate[e] MX(x_t)) * (up[e] MX(x_t))), MX() being the
 * MXFP8 value.  fmt: MOE_W_FP8 or MOE_W_MXFP4, weights and scales as
 * moe_quantize lays them out.  act dtype bf16.  Up to 256 tokens with at
 * most 16 rows per expert on average (T * top_k <= 16 * num_experts) the
 * weights are streamed per row tile; larger batches take tiled grouped GEMMs,
 * which need hidden and expert_inter to be multiples of 64 and at most 4096
 * (else MOE_ERR_UNSUPPORTED).  The workspace as for moe_expert_ffn. */
int moe_expert_ffn_mx(const moe_dims* dims, int32_t fmt, int32_t T, const void* x,
                      const void* w_gate_up_q, const void* w_gate_up_scale, const void* w_down_q,
                      const void* w_down_scale, const float* topk_w,
                      const int32_t* expert_offsets, const int32_t* sorted_slots, void* y_slots,
                      void* ws, size_t ws_bytes, void* stream);

/* The experts' scatter-add: out[t] = sum_{k=0..K-1} y_slots[t,k] (fp32, k
 * ascending, no atomics) + addend[t] (if addend is not NULL).
 * y_slots slot dtype; addend and out act dtype. */
int moe_combine(const moe_dims* dims, int32_t T, const void* y_slots, const void* addend,
                void* out, void* stream);

/* Experts-only path in one call: moe_route (no pre-norm), moe_expert_ffn,
 * moe_combine (no addend).  If topk_idx / topk_w are not NULL
 * the routing is also written there. */
int moe_forward(const moe_dims* dims, int32_t T, const void* x, const float* router_w,
                const float* router_scale, const float* per_expert_scale,
                const void* w_gate_up, const void* w_down, void* out, int32_t* topk_idx,
                float* topk_w, void* ws, size_t ws_bytes, void* stream);

/* moe_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments and result as moe_forward (bit for bit: the same kernels),
 * but the workspace is a library-owned device array of
 * MOE_NOALLOC_SCRATCH_BYTES per GPU (allocated with the code object when
 * the library loads on a device, held until the process ends) instead of a
 * caller buffer; the call makes no allocation of its own.  Sizes whose
 * workspace exceeds that array are refused with MOE_ERR_WORKSPACE (at
 * 26B-A4B shapes: up to 538 tokens; moe_forward needs less workspace than
 * moe_workspace_size, which also covers the MXFP8 buffers of
 * moe_expert_ffn_mx).  Every call on a
 * GPU shares that GPU's array: calls that may overlap on one GPU (two
 * streams, or threads) race and must be serialised by the caller. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_forward_noalloc(const moe_dims* dims, int32_t T, const void* x, const float* router_w,
                        const float* router_scale, const float* per_expert_scale,
                        const void* w_gate_up, const void* w_down, void* out,
                        int32_t* topk_idx, float* topk_w, void* stream);

/* One dual-path feed-forward layer (the page's diagram):
 *   xd = RMSNorm_pre(x); xm = RMSNorm_pre2(x)
 *   moe = experts(xm) routed on pre_feedforward_layernorm_2(x) (moe_router)
 *   dn  = dense_down (gelu_tanh(dense_gate xd) * (dense_up xd))
 *   o   = RMSNorm_post(RMSNorm_post1(dn) + RMSNorm_post2(moe))
 *   out = (o + x) * layer_scalar
 * residual x and out: [T,H] act dtype.  ffn_out (optional, [T,H] fp32) receives
 * o, the layer's output before the residual; topk_idx / topk_w (optional)
 * receive the routing.  Requires dims->dense_inter > 0.
 * The dense branch runs on a stream owned by the library (one per device,
 * created on the first call and kept until the process ends), forked from
 * `stream` after the pre-norms and joined back before the epilogue, so it
 * overlaps the router and the experts; all work is still ordered after the
 * earlier work on `stream`, and later work on `stream` waits for all of it. */
int gemma4_ffn_block(const moe_dims* dims, int32_t T, const void* residual,
                     const gemma4_ffn_weights* weights, void* out, float* ffn_out,
                     int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                     void* stream);

/* The same layer with the experts' and the dense MLP's weights stored in a
 * format below bf16 (moe_wformat), the int8 option of the page "Porting a
 * 128-expert MoE (Gemma-4 26B-A4B) to AWS Inferentia2", section "Can it run
 * on a smaller box? Yes, no, and "deeper than it looks"" (there for the
 * expert and dense MLP weights), and the 8-bit / 4-bit formats of section
 * "The fp4 rabbit hole (two of them, both dead ends)".  Every matrix is
 * quantized per output row as moe_quantize lays it out: the dense gate and
 * up [D, H] and down [H, D] each with their own scales, the experts' gate_up
 * [E, 2I, H] and down [E, H, I].  Norm gains, router weights and
 * layer_scalar stay fp32; activations are bf16 (act_dtype MOE_BF16).  The
 * codes widen to bf16 exactly in registers, as in moe_expert_ffn_q, so the
 * result is the bf16 layer on the dequantized weights.  Every matrix goes
 * through the weight-streaming kernels up to 256 tokens and through the tiled
 * grouped GEMMs past that, as in moe_expert_ffn_q.  Otherwise as
 * gemma4_ffn_block, including the side stream of the dense branch.
 * MOE_ERR_UNSUPPORTED for act_dtype MOE_F32, dense_inter == 0, or MXFP4 with
 * dense_inter > 8192 (its kernels stage the block scales of a contraction of
 * at most 8192 weights);
 * MOE_ERR_ARG for an unknown format or a missing pointer. */
typedef struct gemma4_ffn_weights_q {
  int32_t fmt;                   /* moe_wformat of every quantized matrix */
  const float* g_pre;            /* [H] the five RMSNorm gains, as in gemma4_ffn_weights */
  const float* g_pre2;
  const float* g_post1;
  const float* g_post2;
  const float* g_post;
  const void* dense_gate_q;      /* [D, H] codes */
  const void* dense_gate_scale;  /* its scales (fp32 [D], or E8M0 [D, H/32] for MXFP4) */
  const void* dense_up_q;        /* [D, H] */
  const void* dense_up_scale;
  const void* dense_down_q;      /* [H, D] */
  const void* dense_down_scale;
  const float* router_w;         /* [E, H] fp32 */
  const float* router_scale;     /* [H] */
  const float* per_expert_scale; /* [E] */
  const void* gate_up_q;         /* [E, 2I, H] codes */
  const void* gate_up_scale;
  const void* down_q;            /* [E, H, I] codes */
  const void* down_scale;
  float layer_scalar;
} gemma4_ffn_weights_q;

int gemma4_ffn_block_q(const moe_dims* dims, int32_t T, const void* residual,
                       const gemma4_ffn_weights_q* weights, void* out, float* ffn_out,
                       int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
