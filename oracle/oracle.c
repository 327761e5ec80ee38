/*
 * CPU oracle for the Gemma-4 26B-A4B mixture-of-experts feed-forward block.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP library and its Python binding) never calls it; the two share no code,
 * no headers and no constant tables.
 *
 * What it computes follows the page "Porting a 128-expert MoE (Gemma-4
 * 26B-A4B) to AWS Inferentia2", section "The architecture: a dual-path FFN
 * nobody warned me about":
 *   - the router (Gemma4TextRouter): an RMSNorm of its own, a scale, a
 *     2816 -> 128 projection, softmax over the 128 logits in fp32, top-8,
 *     renormalisation over the 8, then a multiply by per_expert_scale;
 *   - the experts (Gemma4TextExperts): fused gate_up_proj [E, 2I, H] and
 *     down_proj [E, H, I], evaluated as a sparse gather / compute / weighted
 *     scatter-add over each token's selected experts;
 *   - the layer: a dense MLP (intermediate 2112) beside the experts, with a
 *     pre-norm and a post-norm on each branch, the two branches summed, a final
 *     post-feed-forward norm, the residual added and the result multiplied by
 *     layer_scalar (the diagram in the same section).
 * The activation is the tanh form of GELU written out on "Porting Gemma-4
 * (2B / 4B / 12B) to AWS Inferentia2", section 4.5; layer_scalar multiplies
 * the layer's output as described in section 4.6 of that page.
 *
 * Precision.  The router takes its decisions in fp32, the precision the page
 * fixes for its softmax; its reductions follow one stated order (see
 * spec_dot) so that a GPU can reproduce the logits bit for bit.  Everything
 * after routing (expert FFNs, dense MLP, norms of the layer, combine) runs in
 * fp64 as plain loops.
 *
 * Readings where the pages leave a step open:
 *   - the router's RMSNorm carries no gain of its own; "a scale" is a vector
 *     router_scale[H] applied after it;
 *   - experts are chosen by sorting the fp32 logits in descending order, ties
 *     going to the lower expert index (softmax is monotone, so this is the
 *     same set as sorting probabilities); slot k holds the k-th choice;
 *   - rows [0, I) of gate_up[e] are the gate, rows [I, 2I) the up projection;
 *   - every RMSNorm is v / sqrt(mean(v^2) + eps) * gain with eps = 1e-6 and
 *     gain the effective multiplier;
 *   - in the layer, both the router and the experts read
 *     pre_feedforward_layernorm_2(x).
 *
 * Parity pins: see the tests that exercise each function (toy closed forms,
 * invariants, library special cases, brute-force dense-masked evaluation).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define CHUNK 64

/* ---------------------------------------------------------------------------
 * fp32 reductions in the stated order: the length n is cut into 64-element
 * chunks (the last one shorter when n is not a multiple of 64); each chunk is a
 * chain of fused multiply-adds from +0.0 in ascending index; the chunk results
 * are then added left to right, starting from +0.0.  Compiled with
 * -ffp-contract=off so that the separate additions stay separate.
 * ------------------------------------------------------------------------- */
static float spec_dot(const float* a, const float* b, int n) {
  float total = 0.0f;
  for (int c = 0; c < n; c += CHUNK) {
    float part = 0.0f;
    int end = c + CHUNK < n ? c + CHUNK : n;
    for (int i = c; i < end; ++i) part = fmaf(a[i], b[i], part);
    total = total + part;
  }
  return total;
}

/* Router RMSNorm step in fp32: 1 / sqrt(sum(v^2) / n + eps), each operation
 * rounded once (IEEE division and square root). */
static float spec_inv_rms(const float* v, int n, float eps) {
  float s = spec_dot(v, v, n);
  float mean = s / (float)n;
  return 1.0f / sqrtf(mean + eps);
}

/* Returns 1 when expert a ranks before expert b: larger logit first, equal
 * logits broken towards the lower index. */
static int ranks_before(const float* logit, int a, int b) {
  if (logit[a] > logit[b]) return 1;
  if (logit[a] < logit[b]) return 0;
  return a < b;
}

/* One token of the router.  v is the router input row (H values, fp32);
 * scratch has room for H + 2E floats. */
static void router_token(int H, int E, int K, float eps, const float* v,
                         const float* router_w, const float* router_scale,
                         const float* per_expert_scale, int32_t* idx, float* w,
                         float* logits_out, float* scratch) {
  float* vhat = scratch;          /* [H] */
  float* logit = scratch + H;     /* [E] */
  float* prob = logit + E;        /* [E] */

  /* RMSNorm without gain, then the router's scale (two separate products). */
  float r = spec_inv_rms(v, H, eps);
  for (int h = 0; h < H; ++h) vhat[h] = (v[h] * r) * router_scale[h];

  /* 2816 -> 128 projection. */
  for (int e = 0; e < E; ++e) logit[e] = spec_dot(vhat, router_w + (size_t)e * H, H);
  if (logits_out) memcpy(logits_out, logit, sizeof(float) * E);

  /* Softmax over all E logits in fp32. */
  float m = logit[0];
  for (int e = 1; e < E; ++e) if (logit[e] > m) m = logit[e];
  float z = 0.0f;
  for (int e = 0; e < E; ++e) { prob[e] = expf(logit[e] - m); z = z + prob[e]; }
  for (int e = 0; e < E; ++e) prob[e] = prob[e] / z;

  /* Top-K by selection: each pass takes the best expert not yet chosen. */
  unsigned char taken[1024];
  memset(taken, 0, (size_t)E);
  for (int k = 0; k < K; ++k) {
    int best = -1;
    for (int e = 0; e < E; ++e) {
      if (taken[e]) continue;
      if (best < 0 || ranks_before(logit, e, best)) best = e;
    }
    taken[best] = 1;
    idx[k] = best;
  }

  /* Renormalise over the K chosen probabilities, then apply per_expert_scale. */
  float q = 0.0f;
  for (int k = 0; k < K; ++k) q = q + prob[idx[k]];
  for (int k = 0; k < K; ++k) w[k] = (prob[idx[k]] / q) * per_expert_scale[idx[k]];
}

/* Router over T tokens.  x [T,H] is the layer input (fp32 values).  When
 * pre_gain is not NULL the router input is pre_feedforward_layernorm_2(x),
 * evaluated here in fp32 with the stated reduction order:
 * v = (x * (1/sqrt(mean(x^2)+eps))) * pre_gain.  Outputs idx [T,K] int32,
 * w [T,K] fp32 and, if logits is not NULL, the fp32 logits [T,E]. */
void oracle_router(int T, int H, int E, int K, float eps, const float* x,
                   const float* pre_gain, const float* router_w, const float* router_scale,
                   const float* per_expert_scale, int32_t* idx, float* w, float* logits) {
#pragma omp parallel
  {
    float* scratch = (float*)malloc(sizeof(float) * (size_t)(2 * H + 2 * E));
    float* v = scratch + H + 2 * E;
#pragma omp for schedule(static)
    for (int t = 0; t < T; ++t) {
      const float* xt = x + (size_t)t * H;
      const float* in = xt;
      if (pre_gain) {
        float r = spec_inv_rms(xt, H, eps);
        for (int h = 0; h < H; ++h) v[h] = (xt[h] * r) * pre_gain[h];
        in = v;
      }
      router_token(H, E, K, eps, in, router_w, router_scale, per_expert_scale,
                   idx + (size_t)t * K, w + (size_t)t * K,
                   logits ? logits + (size_t)t * E : NULL, scratch);
    }
    free(scratch);
  }
}

/* Grouping of token-slots by expert.  Slot s = t*K + k carries expert idx[s].
 * counts[e] = number of slots routed to e; offsets[e] = exclusive prefix sum
 * (offsets[E] = T*K); sorted_slots lists the slot ids of expert 0, then of
 * expert 1, ..., each group in ascending slot order. */
void oracle_dispatch(int T, int E, int K, const int32_t* idx, int32_t* counts,
                     int32_t* offsets, int32_t* sorted_slots) {
  int S = T * K;
  if (E <= 0) return;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int s = 0; s < S; ++s) counts[idx[s]] += 1;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* fill = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  for (int s = 0; s < S; ++s) {
    int e = idx[s];
    sorted_slots[offsets[e] + fill[e]] = s;
    fill[e] += 1;
  }
  free(fill);
}

/* tanh form of GELU: 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))). */
double oracle_gelu_tanh(double z) {
  const double c = sqrt(2.0 / 3.14159265358979323846);
  return 0.5 * z * (1.0 + tanh(c * (z + 0.044715 * z * z * z)));
}

static double dot_f64(const double* a, const float* b, int n) {
  double acc = 0.0;
  for (int i = 0; i < n; ++i) acc += a[i] * (double)b[i];
  return acc;
}

/* RMSNorm in fp64 over T rows of length H: out = x / sqrt(mean(x^2) + eps) * gain
 * (gain NULL means 1). */
void oracle_rmsnorm(int T, int H, double eps, const double* x, const float* gain,
                    double* out) {
  for (int t = 0; t < T; ++t) {
    const double* r = x + (size_t)t * H;
    double s = 0.0;
    for (int h = 0; h < H; ++h) s += r[h] * r[h];
    double inv = 1.0 / sqrt(s / H + eps);
    for (int h = 0; h < H; ++h)
      out[(size_t)t * H + h] = r[h] * inv * (gain ? (double)gain[h] : 1.0);
  }
}

/* One gated GELU-tanh MLP applied to one row: y = Wd (gelu(Wg x) * (Wu x)).
 * wg, wu: [N, H] rows; wd: [H, N] rows; a: scratch [N]. */
static void gated_mlp_row(int H, int N, const double* x, const float* wg, const float* wu,
                          const float* wd, double* y, double* a) {
  for (int i = 0; i < N; ++i) {
    double g = dot_f64(x, wg + (size_t)i * H, H);
    double u = dot_f64(x, wu + (size_t)i * H, H);
    a[i] = oracle_gelu_tanh(g) * u;
  }
  for (int j = 0; j < H; ++j) y[j] = dot_f64(a, wd + (size_t)j * N, N);
}

/* Sparse expert evaluation: for each token t and each of its K slots
 * (k ascending) with expert e = idx[t,k] and weight w[t,k],
 *   out[t] += w[t,k] * down[e] (gelu(gate[e] x_t) * (up[e] x_t)),
 * out starting from zero.  xin [T,H] fp64; gate_up [E,2I,H]; down [E,H,I]. */
void oracle_experts(int T, int H, int E, int K, int I, const double* xin,
                    const float* gate_up, const float* down, const int32_t* idx,
                    const float* w, double* out) {
  (void)E;
#pragma omp parallel
  {
    double* y = (double*)malloc(sizeof(double) * (size_t)(H + I));
    double* a = y + H;
#pragma omp for schedule(dynamic, 1)
    for (int t = 0; t < T; ++t) {
      double* o = out + (size_t)t * H;
      for (int h = 0; h < H; ++h) o[h] = 0.0;
      for (int k = 0; k < K; ++k) {
        int e = idx[(size_t)t * K + k];
        const float* wg = gate_up + (size_t)e * 2 * I * H;
        const float* wu = wg + (size_t)I * H;
        const float* wd = down + (size_t)e * H * I;
        gated_mlp_row(H, I, xin + (size_t)t * H, wg, wu, wd, y, a);
        double wk = (double)w[(size_t)t * K + k];
        for (int h = 0; h < H; ++h) o[h] += wk * y[h];
      }
    }
    free(y);
  }
}

/* Dense gated MLP over T rows: out[t] = Wd (gelu(Wg x_t) * (Wu x_t));
 * wg, wu [D,H]; wd [H,D]. */
void oracle_dense_mlp(int T, int H, int D, const double* xin, const float* wg,
                      const float* wu, const float* wd, double* out) {
#pragma omp parallel
  {
    double* a = (double*)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 1)
    for (int t = 0; t < T; ++t)
      gated_mlp_row(H, D, xin + (size_t)t * H, wg, wu, wd, out + (size_t)t * H, a);
    free(a);
  }
}

/* One dual-path feed-forward layer over T rows of the residual x [T,H]:
 *   xd = RMSNorm_pre(x), xm = RMSNorm_pre2(x)                      (fp64)
 *   routing from pre_feedforward_layernorm_2(x) in fp32            (oracle_router)
 *   moe = sparse experts on xm with the routing weights
 *   dn  = dense MLP on xd
 *   o   = RMSNorm_post( RMSNorm_post1(dn) + RMSNorm_post2(moe) )
 *   out = (o + x) * layer_scalar
 * Outputs out, o, moe [T,H] fp64, and idx/w [T,K].  x is given both as fp32
 * (for the router) and fp64 (same values). */
void oracle_block(int T, int H, int E, int K, int I, int D, float eps,
                  const float* x32, const double* x,
                  const float* g_pre, const float* g_pre2, const float* g_post1,
                  const float* g_post2, const float* g_post,
                  const float* dense_gate, const float* dense_up, const float* dense_down,
                  const float* router_w, const float* router_scale,
                  const float* per_expert_scale, const float* gate_up, const float* down,
                  double layer_scalar, int32_t* idx, float* w,
                  double* out, double* o, double* moe) {
  size_t n = (size_t)T * H;
  double* xd = (double*)malloc(sizeof(double) * n);
  double* xm = (double*)malloc(sizeof(double) * n);
  double* dn = (double*)malloc(sizeof(double) * n);
  double* t1 = (double*)malloc(sizeof(double) * n);
  double* t2 = (double*)malloc(sizeof(double) * n);

  oracle_rmsnorm(T, H, eps, x, g_pre, xd);
  oracle_rmsnorm(T, H, eps, x, g_pre2, xm);
  oracle_router(T, H, E, K, eps, x32, g_pre2, router_w, router_scale, per_expert_scale,
                idx, w, NULL);
  oracle_experts(T, H, E, K, I, xm, gate_up, down, idx, w, moe);
  oracle_dense_mlp(T, H, D, xd, dense_gate, dense_up, dense_down, dn);
  oracle_rmsnorm(T, H, eps, dn, g_post1, t1);
  oracle_rmsnorm(T, H, eps, moe, g_post2, t2);
  for (size_t i = 0; i < n; ++i) t1[i] += t2[i];
  oracle_rmsnorm(T, H, eps, t1, g_post, o);
  for (size_t i = 0; i < n; ++i) out[i] = (o[i] + x[i]) * layer_scalar;

  free(xd); free(xm); free(dn); free(t1); free(t2);
}

/* ---------------------------------------------------------------------------
 * int8 per-channel symmetric weights (the int8-expert variant on the page
 * "Porting a 128-expert MoE (Gemma-4 26B-A4B) to AWS Inferentia2", section
 * "Can it run on a smaller box? Yes, no, and "deeper than it looks"").
 * Reading: a channel is one output row of an [out, in] weight; its scale is
 * s = max |w| / 127 (fp32 division), its codes q = round-half-to-even(w / s)
 * (fp32 division) clamped to [-127, 127]; a row of zeros gets s = 0, q = 0.
 * The dequantized weight is q * s.
 * ------------------------------------------------------------------------- */
void oracle_quantize_rows(long long rows, int cols, const float* w, int8_t* q, float* s) {
#pragma omp parallel for schedule(static)
  for (long long r = 0; r < rows; ++r) {
    const float* wr = w + r * cols;
    float amax = 0.0f;
    for (int c = 0; c < cols; ++c) {
      const float a = fabsf(wr[c]);
      if (a > amax) amax = a;
    }
    const float sc = amax / 127.0f;
    s[r] = sc;
    for (int c = 0; c < cols; ++c) {
      float v = 0.0f;
      if (sc > 0.0f) v = rintf(wr[c] / sc);
      if (v > 127.0f) v = 127.0f;
      if (v < -127.0f) v = -127.0f;
      q[r * cols + c] = (int8_t)v;
    }
  }
}

/* Dequantized weights as fp32: out = q * s rounded once to fp32. */
void oracle_dequantize_rows(long long rows, int cols, const int8_t* q, const float* s,
                            float* out) {
#pragma omp parallel for schedule(static)
  for (long long r = 0; r < rows; ++r)
    for (int c = 0; c < cols; ++c)
      out[r * cols + c] = (float)((double)q[r * cols + c] * (double)s[r]);
}

/* -------------------------------------------------------------------------
 * 8-bit and 4-bit floating-point expert weights, the low-precision options
 * the page "Porting a 128-expert MoE (Gemma-4 26B-A4B) to AWS Inferentia2"
 * weighs for the experts (section "The fp4 rabbit hole (two of them, both
 * dead ends)": FP8, and the microscaling fp4 format of 32 E2M1 values per
 * block).  The formats themselves are those of the published OCP standards:
 *
 * E4M3 (OCP 8-bit floating point): sign, 4 exponent bits with bias 7, 3
 * mantissa bits; exponent field 0 holds the subnormals m/8 * 2^-6; there are
 * no infinities, S.1111.111 is NaN, and the largest finite magnitude is
 * 1.75 * 2^8 = 448.
 *
 * MXFP4 (OCP Microscaling, MX): blocks of 32 consecutive values share one
 * E8M0 scale 2^(e - 127); the elements are E2M1 (sign, 2 exponent bits with
 * bias 1, 1 mantissa bit): magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.  The
 * shared exponent is floor(log2(max |v|)) minus 2 (the largest E2M1
 * exponent), and each element is v / 2^shared rounded to the nearest E2M1
 * value, saturating at 6.
 *
 * Rounding here works on the table of representable values: the nearer of
 * the two values around v wins, and a value exactly halfway between them
 * takes the code whose lowest mantissa bit is 0 (round half to even).
 * ------------------------------------------------------------------------- */

/* Value of an E4M3 code (NaN for S.1111.111). */
double oracle_e4m3_value(int code) {
  const int sign = (code >> 7) & 1, ex = (code >> 3) & 15, m = code & 7;
  double v;
  if (ex == 15 && m == 7) return NAN;
  if (ex == 0) v = (double)m / 8.0 * ldexp(1.0, -6);
  else v = (1.0 + (double)m / 8.0) * ldexp(1.0, ex - 7);
  return sign ? -v : v;
}

/* Value of an E2M1 code (4 bits). */
double oracle_e2m1_value(int code) {
  static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  const double v = mag[code & 7];
  return (code & 8) ? -v : v;
}

/* Nearest code among the non-negative codes 0..n-1, whose values f(c)
 * ascend with c: the two codes around a (found by bisection) are compared,
 * and a value exactly half-way takes the code with even lowest bit. */
static int nearest_code(double a, int n, double (*f)(int)) {
  if (a <= f(0)) return 0;
  if (a >= f(n - 1)) return n - 1;
  int lo = 0, hi = n - 1;  /* f(lo) < a < f(hi) or on one of them */
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (f(mid) <= a) lo = mid;
    else hi = mid;
  }
  const double dl = a - f(lo), dh = f(hi) - a;
  if (dl < dh) return lo;
  if (dh < dl) return hi;
  return (lo & 1) == 0 ? lo : hi;
}

/* Per-row symmetric E4M3: s = max |w| / 448 (fp32 division), code = nearest
 * E4M3 to w / s (fp32 division; 126 finite non-negative codes 0x00..0x7E,
 * magnitudes past 448 take 448), sign bit = w < 0.  A row of zeros gets
 * s = 0 and codes 0.  The dequantized weight is value(code) * s. */
void oracle_quantize_fp8_rows(long long rows, int cols, const float* w, uint8_t* q, float* s) {
#pragma omp parallel for schedule(static)
  for (long long r = 0; r < rows; ++r) {
    const float* wr = w + r * cols;
    float amax = 0.0f;
    for (int c = 0; c < cols; ++c) {
      const float a = fabsf(wr[c]);
      if (a > amax) amax = a;
    }
    const float sc = amax / 448.0f;
    s[r] = sc;
    for (int c = 0; c < cols; ++c) {
      int code = 0;
      if (sc > 0.0f) {
        const float v = wr[c] / sc;
        code = nearest_code(fabs((double)v), 0x7F, oracle_e4m3_value);
        if (wr[c] < 0.0f) code |= 0x80;
      }
      q[r * cols + c] = (uint8_t)code;
    }
  }
}

/* value(code) * s, rounded once to fp32. */
void oracle_dequantize_fp8_rows(long long rows, int cols, const uint8_t* q, const float* s,
                                float* out) {
#pragma omp parallel for schedule(static)
  for (long long r = 0; r < rows; ++r)
    for (int c = 0; c < cols; ++c)
      out[r * cols + c] = (float)(oracle_e4m3_value(q[r * cols + c]) * (double)s[r]);
}

/* MXFP4 along each row (cols % 32 == 0): block b of row r holds columns
 * 32b .. 32b + 31; e8[r * cols / 32 + b] is its E8M0 scale code, and column
 * c's E2M1 code sits in byte r * cols / 2 + c / 2, low nibble for even c.
 * shared = floor(log2(max |v|)) - 2, clamped to [-127, 127], e8 = shared +
 * 127; a block of zeros gets e8 = 0 and codes 0.  Element code = nearest
 * E2M1 to |v| / 2^shared (magnitudes past 6 take 6), sign bit = v < 0. */
void oracle_quantize_mxfp4_rows(long long rows, int cols, const float* w, uint8_t* q,
                                uint8_t* e8) {
  const int nb = cols / 32;
#pragma omp parallel for schedule(static)
  for (long long r = 0; r < rows; ++r) {
    for (int b = 0; b < nb; ++b) {
      const float* v = w + r * cols + 32 * b;
      double amax = 0.0;
      for (int i = 0; i < 32; ++i)
        if (fabs((double)v[i]) > amax) amax = fabs((double)v[i]);
      int shared = -127;
      if (amax > 0.0) {
        shared = (int)floor(log2(amax)) - 2;
        /* log2 of an exact power of two must not be taken from a rounded log */
        while (ldexp(1.0, shared + 2) > amax) --shared;
        while (ldexp(1.0, shared + 3) <= amax) ++shared;
        if (shared < -127) shared = -127;
        if (shared > 127) shared = 127;
      }
      e8[r * nb + b] = (uint8_t)(amax > 0.0 ? shared + 127 : 0);
      for (int i = 0; i < 32; ++i) {
        int code = 0;
        if (amax > 0.0) {
          code = nearest_code(fabs((double)v[i]) / ldexp(1.0, shared), 8, oracle_e2m1_value);
          if (v[i] < 0.0f) code |= 8;
        }
        const long long c = 32LL * b + i;
        uint8_t* byte = q + r * (cols / 2) + c / 2;
        if (c % 2 == 0) *byte = (uint8_t)code;
        else *byte = (uint8_t)(*byte | (code << 4));
      }
    }
  }
}

/* value(code) * 2^(e8 - 127), exact in fp32. */
void oracle_dequantize_mxfp4_rows(long long rows, int cols, const uint8_t* q, const uint8_t* e8,
                                  float* out) {
  const int nb = cols / 32;
#pragma omp parallel for schedule(static)
  for (long long r = 0; r < rows; ++r)
    for (int c = 0; c < cols; ++c) {
      const uint8_t byte = q[r * (cols / 2) + c / 2];
      const int code = (c % 2 == 0) ? (byte & 15) : (byte >> 4);
      out[r * cols + c] =
          (float)(oracle_e2m1_value(code) * ldexp(1.0, (int)e8[r * nb + c / 32] - 127));
    }
}

/* -------------------------------------------------------------------------
 * Activations for the 8-bit / 4-bit matrix cores.  Running the E4M3 and
 * MXFP4 experts of the page's low-precision options on matrix units that
 * multiply 8-bit or 4-bit operands natively means the activations enter the
 * product in 8 bits as well (the page gives no rule for them; its int8
 * variant kept the activations wide).  Reading taken: MXFP8 in the OCP
 * Microscaling sense, the same block structure as the MXFP4 weights: blocks
 * of 32 consecutive values along the contraction share one E8M0 scale
 * 2^shared with shared = floor(log2(max |v|)) - 8 (8 is E4M3's largest
 * exponent), clamped to [-127, 127]; each element is the E4M3 value nearest
 * to v / 2^shared (ties to the even mantissa, magnitudes past 448 take 448)
 * with the sign of v; a block of zeros gets scale code 0 and zero codes.
 * Both the expert input x (blocks along H) and the gated product h = GELU(g)
 * * u (blocks along I) are quantized so before their projections; the
 * products and sums themselves are exact (fp64 here).
 * ------------------------------------------------------------------------- */
static void mx8_block(const double* v, int n, uint8_t* q, uint8_t* e8) {
  double amax = 0.0;
  for (int i = 0; i < n; ++i)
    if (fabs(v[i]) > amax) amax = fabs(v[i]);
  int shared = -127;
  if (amax > 0.0) {
    shared = (int)floor(log2(amax)) - 8;
    while (ldexp(1.0, shared + 8) > amax) --shared;
    while (ldexp(1.0, shared + 9) <= amax) ++shared;
    if (shared < -127) shared = -127;
    if (shared > 127) shared = 127;
  }
  *e8 = (uint8_t)(amax > 0.0 ? shared + 127 : 0);
  for (int i = 0; i < n; ++i) {
    int code = 0;
    if (amax > 0.0) {
      code = nearest_code(fabs(v[i]) / ldexp(1.0, shared), 0x7F, oracle_e4m3_value);
      if (v[i] < 0.0) code |= 0x80;
    }
    q[i] = (uint8_t)code;
  }
}

static double mx8_value(uint8_t code, uint8_t e8) {
  return oracle_e4m3_value(code) * ldexp(1.0, (int)e8 - 127);
}

/* MXFP8 along each row (cols % 32 == 0): codes q [rows, cols], E8M0 scale
 * codes e8 [rows, cols / 32]. */
void oracle_quantize_mx8_rows(long long rows, int cols, const double* v, uint8_t* q,
                              uint8_t* e8) {
  const int nb = cols / 32;
#pragma omp parallel for schedule(static)
  for (long long r = 0; r < rows; ++r)
    for (int b = 0; b < nb; ++b)
      mx8_block(v + r * cols + 32 * b, 32, q + r * cols + 32 * b, e8 + r * nb + b);
}

/* value(code) * 2^(e8 - 127), exact in fp64. */
void oracle_dequantize_mx8_rows(long long rows, int cols, const uint8_t* q, const uint8_t* e8,
                                double* out) {
  const int nb = cols / 32;
#pragma omp parallel for schedule(static)
  for (long long r = 0; r < rows; ++r)
    for (int c = 0; c < cols; ++c)
      out[r * cols + c] = mx8_value(q[r * cols + c], e8[r * nb + c / 32]);
}

/* In place: each row of 32-blocks replaced by its MXFP8 value. */
static void mx8_round_row(double* v, int n) {
  uint8_t q[32], e8;
  for (int b = 0; b < n; b += 32) {
    mx8_block(v + b, 32, q, &e8);
    for (int i = 0; i < 32; ++i) v[b + i] = mx8_value(q[i], e8);
  }
}

/* The sparse expert loop with MXFP8 activations (H % 32 == 0, I % 32 == 0):
 * as oracle_experts, but the token's input row is replaced by its MXFP8
 * value before the gate / up projections, and the gated product a (length
 * I) by its MXFP8 value before the down projection.  gate_up / down are the
 * weights' values (the dequantized codes). */
void oracle_experts_mx8(int T, int H, int E, int K, int I, const double* xin,
                        const float* gate_up, const float* down, const int32_t* idx,
                        const float* w, double* out) {
  (void)E;
#pragma omp parallel
  {
    double* y = (double*)malloc(sizeof(double) * (size_t)(2 * H + I));
    double* a = y + H;
    double* xq = a + I;
#pragma omp for schedule(dynamic, 1)
    for (int t = 0; t < T; ++t) {
      double* o = out + (size_t)t * H;
      memcpy(xq, xin + (size_t)t * H, sizeof(double) * (size_t)H);
      mx8_round_row(xq, H);
      for (int h = 0; h < H; ++h) o[h] = 0.0;
      for (int k = 0; k < K; ++k) {
        int e = idx[(size_t)t * K + k];
        const float* wg = gate_up + (size_t)e * 2 * I * H;
        const float* wu = wg + (size_t)I * H;
        const float* wd = down + (size_t)e * H * I;
        for (int i = 0; i < I; ++i) {
          double g = dot_f64(xq, wg + (size_t)i * H, H);
          double u = dot_f64(xq, wu + (size_t)i * H, H);
          a[i] = oracle_gelu_tanh(g) * u;
        }
        mx8_round_row(a, I);
        for (int j = 0; j < H; ++j) y[j] = dot_f64(a, wd + (size_t)j * I, I);
        double wk = (double)w[(size_t)t * K + k];
        for (int h = 0; h < H; ++h) o[h] += wk * y[h];
      }
    }
    free(y);
  }
}

/* Number of OpenMP threads the parallel loops use. */
int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Sets the number of OpenMP threads later calls use (timing only; results
 * do not depend on it). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
