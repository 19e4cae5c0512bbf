/*
 * CPU oracle for the decode step of a DeepSeek-V4.1-style MoE layer half.
 *
 * TEST INFRASTRUCTURE ONLY (tests, the smoke check and the benchmark's CPU
 * baseline). It shares no code with the GPU library.
 *
 * Sources. The pages name the steps and their rounding points but print no
 * formulas; where a formula is not on the pages it is the plainest reading,
 * marked READING below.
 *  [ds4]   antirez/ds4 PR "v41: fuse the single-box decode glue (HC, MoE,
 *          attention)": "What" section and commit messages (HC fusion,
 *          router/shared fusion, tie-order commit).
 *  [sgl3]  SGLang PR "[DeepSeek-V4] Add mhc_fused_post_pre kernel":
 *          "Motivation" (post + bf16 residual + pre-norm GEMM partials + RMS
 *          square-sum partials) and "Modifications" (bf16 RMSNorm weights).
 *  [sgl1]  SGLang PR "[AMD][V4.1] Mono kernel framework ... DeepSeek-V4.1
 *          decode layers": "DeepSeek-V4.1 layer on mono" figure (K2: FFN
 *          mHC seam, router, shared + routed experts).
 *  [mhc]   the mHC formulation (manifold-constrained hyper-connections):
 *          pre = sigmoid, post = 2 * sigmoid, comb = Sinkhorn-Knopp on exp.
 *          Not on the pages: READING.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp -fPIC -shared -lm
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define NSTREAM 4
#define NMIX 24
#define QBLOCK 32

int or_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void or_set_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ---------------------------------------------------------------------------------------------
 * Number formats (exact decodes; f32 -> bf16 rounds to nearest even). */

double or_bf16_to_f64(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

uint16_t or_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

double or_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1, e = (h >> 10) & 0x1F, m = h & 0x3FF;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(m | 0x400), e - 25);
  return sign ? -v : v;
}

/* e2m1: 1 sign bit, 2 exponent bits, 1 mantissa bit; magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6. */
double or_e2m1_to_f64(unsigned code) {
  static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  double v = mag[code & 7u];
  return (code & 8u) ? -v : v;
}

/* e8m0: a power of two, 2^(e - 127); 0xFF is NaN. */
double or_e8m0_to_f64(uint8_t e) { return e == 0xFF ? NAN : ldexp(1.0, (int)e - 127); }

static double act_get(int act, const void* p, int64_t i) {
  return act == OR_F32 ? (double)((const float*)p)[i] : or_bf16_to_f64(((const uint16_t*)p)[i]);
}

/* Stores f32(v), then bf16 of that when the activation storage is bf16. */
static void act_put(int act, void* p, int64_t i, double v) {
  float f = (float)v;
  if (act == OR_F32)
    ((float*)p)[i] = f;
  else
    ((uint16_t*)p)[i] = or_f32_to_bf16(f);
}

/* Value (row, col) of a [rows][k] matrix, exactly. Quantised formats hold blocks of 32
 * consecutive columns of one row under one scale (READING: blocks run along the contraction
 * dimension). */
double or_mat_elem(const or_mat* m, int64_t k, int64_t row, int64_t col) {
  int64_t i = row * k + col;
  switch (m->fmt) {
    case OR_F32: return (double)((const float*)m->values)[i];
    case OR_BF16: return or_bf16_to_f64(((const uint16_t*)m->values)[i]);
    case OR_Q8_0: {
      double d = or_f16_to_f64(((const uint16_t*)m->scales)[row * (k / QBLOCK) + col / QBLOCK]);
      return d * (double)((const int8_t*)m->values)[i];
    }
    case OR_MXFP4: {
      uint8_t byte = ((const uint8_t*)m->values)[i / 2];
      unsigned code = (i & 1) ? (byte >> 4) : (byte & 0xFu);
      double sc = or_e8m0_to_f64(((const uint8_t*)m->scales)[row * (k / QBLOCK) + col / QBLOCK]);
      return sc * or_e2m1_to_f64(code);
    }
    default: return NAN;
  }
}

/* sum_c M[row][c] * v[c] in f64; each term is the exact weight (as or_mat_elem) times v[c]. */
static double mat_row_dot(const or_mat* m, int64_t k, int64_t row, const double* v) {
  double acc = 0.0;
  const int64_t base = row * k;
  switch (m->fmt) {
    case OR_F32: {
      const float* w = (const float*)m->values + base;
      for (int64_t c = 0; c < k; ++c) acc += (double)w[c] * v[c];
      return acc;
    }
    case OR_BF16: {
      const uint16_t* w = (const uint16_t*)m->values + base;
      for (int64_t c = 0; c < k; ++c) acc += or_bf16_to_f64(w[c]) * v[c];
      return acc;
    }
    case OR_Q8_0: {
      const int8_t* w = (const int8_t*)m->values + base;
      const uint16_t* sc = (const uint16_t*)m->scales + row * (k / QBLOCK);
      for (int64_t b = 0; b < k / QBLOCK; ++b) {
        const double d = or_f16_to_f64(sc[b]);
        for (int64_t c = b * QBLOCK; c < (b + 1) * QBLOCK; ++c) acc += d * (double)w[c] * v[c];
      }
      return acc;
    }
    case OR_MXFP4: {
      const uint8_t* w = (const uint8_t*)m->values + base / 2;
      const uint8_t* sc = (const uint8_t*)m->scales + row * (k / QBLOCK);
      for (int64_t b = 0; b < k / QBLOCK; ++b) {
        const double d = or_e8m0_to_f64(sc[b]);
        for (int64_t c = b * QBLOCK; c < (b + 1) * QBLOCK; ++c) {
          unsigned code = (c & 1) ? (w[c / 2] >> 4) : (w[c / 2] & 0xFu);
          acc += d * or_e2m1_to_f64(code) * v[c];
        }
      }
      return acc;
    }
    default: return NAN;
  }
}

/* ---------------------------------------------------------------------------------------------
 * MXFP8 activations for MXFP4 experts [vLLM "[ROCm][Perf][GLM-5] Fused sparse-layer decode via
 * AITER MonoKernel", Details, Numerics: the activations entering the MXFP4 experts are quantised
 * to MXFP8]. The page names the format only. READING: the conversion is the one of the OCP
 * Microscaling (MX) specification v1.0 with E4M3 elements:
 *   - blocks of 32 consecutive values along the contraction dimension share one e8m0 scale 2^X,
 *     X = floor(log2(max |v|)) - 8 (8 is the exponent of the largest E4M3 power of two),
 *     clamped to [-127, 127]; an all-zero block takes X = -127;
 *   - each value becomes the E4M3 number nearest to v / 2^X, ties to the even mantissa, and a
 *     magnitude above 448 (the largest finite E4M3) becomes 448.
 * The quantised vector replaces the input of each expert matrix stored in MXFP4: the norm row
 * for gate and up, the hidden row for down. The stored tensors (norm, h) are not changed.
 *
 * E4M3 (OFP8): sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the
 * subnormals m / 8 * 2^-6; S.1111.111 is NaN; there are no infinities. */
double or_e4m3_to_f64(uint8_t c) {
  const unsigned e = (c >> 3) & 0xFu, m = c & 7u;
  if (e == 15u && m == 7u) return NAN;
  const double mag = e == 0u ? ldexp((double)m, -9) : ldexp(8.0 + (double)m, (int)e - 10);
  return (c & 0x80u) ? -mag : mag;
}

/* E4M3 code of a value already rounded to E4M3 precision and within +-448. */
static uint8_t e4m3_encode(double r) {
  const uint8_t sign = (r < 0.0 || (r == 0.0 && signbit(r))) ? 0x80u : 0u;
  const double a = fabs(r);
  if (a < ldexp(1.0, -6)) return (uint8_t)(sign | (uint8_t)(a / ldexp(1.0, -9)));
  int e2;
  (void)frexp(a, &e2); /* a = f 2^e2, f in [0.5, 1): floor(log2 a) = e2 - 1 */
  const int e = e2 - 1;
  const unsigned m = (unsigned)(a / ldexp(1.0, e - 3)) - 8u;
  return (uint8_t)(sign | (unsigned)((e + 7) << 3) | m);
}

int or_mxfp8_quant(const double* v, int n, uint8_t* codes, uint8_t* scales) {
  if (!v || !codes || !scales || n < 0 || n % QBLOCK) return -1;
  for (int b = 0; b < n / QBLOCK; ++b) {
    const double* x = v + (int64_t)b * QBLOCK;
    double amax = 0.0;
    for (int i = 0; i < QBLOCK; ++i)
      if (fabs(x[i]) > amax) amax = fabs(x[i]);
    int X = -127;
    if (amax > 0.0) {
      int e2;
      (void)frexp(amax, &e2);
      X = (e2 - 1) - 8;
      if (X < -127) X = -127;
      if (X > 127) X = 127;
    }
    scales[b] = (uint8_t)(X + 127);
    for (int i = 0; i < QBLOCK; ++i) {
      const double t = ldexp(x[i], -X); /* exact */
      const double a = fabs(t);
      double q; /* E4M3 spacing at a */
      if (a < ldexp(1.0, -6)) {
        q = ldexp(1.0, -9);
      } else {
        int e2;
        (void)frexp(a, &e2);
        q = ldexp(1.0, (e2 - 1) - 3);
      }
      double r = nearbyint(t / q) * q; /* default rounding mode: nearest, ties to even */
      if (r > 448.0) r = 448.0;
      if (r < -448.0) r = -448.0;
      if (r == 0.0) r = copysign(0.0, t);
      codes[(int64_t)b * QBLOCK + i] = e4m3_encode(r);
    }
  }
  return 0;
}

/* v[0 .. n) replaced by its MXFP8 round trip: code value times the block's scale. */
static int mxfp8_round_trip(double* v, int n) {
  uint8_t* c = (uint8_t*)malloc((size_t)n + (size_t)n / QBLOCK + 1);
  if (!c) return -2;
  uint8_t* sc = c + n;
  int rc = or_mxfp8_quant(v, n, c, sc);
  if (rc == 0)
    for (int i = 0; i < n; ++i) v[i] = or_e4m3_to_f64(c[i]) * or_e8m0_to_f64(sc[i / QBLOCK]);
  free(c);
  return rc;
}

/* The input a matrix sees: v itself, or its MXFP8 round trip (in vq) when the activations of
 * MXFP4 experts are quantised. */
static const double* matrix_input(const or_shape* s, const or_mat* m, const double* v, double* vq,
                                  int n, int* rc) {
  if (s->act_quant != OR_AQ_MXFP8 || m->fmt != OR_MXFP4) return v;
  memcpy(vq, v, sizeof(double) * (size_t)n);
  *rc = mxfp8_round_trip(vq, n);
  return vq;
}

static int mat_ok(const or_mat* m) {
  if (!m->values) return 0;
  if ((m->fmt == OR_Q8_0 || m->fmt == OR_MXFP4) && !m->scales) return 0;
  return m->fmt >= OR_F32 && m->fmt <= OR_MXFP4;
}

static int shape_ok(const or_shape* s) {
  return s && s->rows >= 0 && s->hidden > 0 && s->n_experts > 0 && s->top_k > 0 &&
         s->top_k <= s->n_experts && s->inter > 0 && s->shared_inter >= 0 &&
         (s->act == OR_F32 || s->act == OR_BF16) && s->sinkhorn_iters >= 0 &&
         s->hidden % QBLOCK == 0 && s->inter % QBLOCK == 0 && s->shared_inter % QBLOCK == 0 &&
         (s->act_quant == OR_AQ_NONE || s->act_quant == OR_AQ_MXFP8);
}

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* ---------------------------------------------------------------------------------------------
 * mHC mix [ds4 HC fusion commit: "rms_norm_mix" over the 4x5120 HC row; sgl3 Motivation:
 * pre-norm GEMM partials + RMS square-sum partials].
 * s = the flattened row (t = stream * H + h), ms = mean(s^2):
 *   mixes[j] = f32( (sum_t W[j][t] s[t]) / sqrt(ms + eps_hc) ).
 * Normalising before the matvec or scaling after it is the same number in exact arithmetic;
 * the f64 form divides once at the end. With a carry (raw sums and sumsq of the row, computed
 * by the previous layer's expand), mixes[j] = f32(raw[j] / sqrt(sumsq / (4H) + eps_hc)). */
int or_mix(const or_shape* s, const void* state, const float* w_mix, const float* carry,
           float* mixes) {
  if (!shape_ok(s) || !mixes || (!carry && (!state || !w_mix))) return -1;
  const int64_t n = (int64_t)NSTREAM * s->hidden;
  for (int r = 0; r < s->rows; ++r) {
    if (carry) {
      const float* c = carry + (int64_t)r * (NMIX + 1);
      double den = sqrt((double)c[NMIX] / (double)n + s->eps_hc);
      for (int j = 0; j < NMIX; ++j) mixes[r * NMIX + j] = (float)((double)c[j] / den);
      continue;
    }
    double* v = (double*)malloc(sizeof(double) * n);
    if (!v) return -2;
    double ss = 0.0;
    for (int64_t t = 0; t < n; ++t) {
      v[t] = act_get(s->act, state, (int64_t)r * n + t);
      ss += v[t] * v[t];
    }
    double den = sqrt(ss / (double)n + s->eps_hc);
    for (int j = 0; j < NMIX; ++j) {
      double acc = 0.0;
      for (int64_t t = 0; t < n; ++t) acc += (double)w_mix[(int64_t)j * n + t] * v[t];
      mixes[r * NMIX + j] = (float)(acc / den);
    }
    free(v);
  }
  return 0;
}

/* ---------------------------------------------------------------------------------------------
 * Split + Sinkhorn [ds4 HC fusion commit: "split/sinkhorn"; 20 iterations from the workload].
 * READING [mhc]: mixes [0:4] -> pre, [4:8] -> post, [8:24] -> comb (row-major i, j);
 *   pre[i]  = f32(sigmoid(a0 * m[i] + b[i]))
 *   post[i] = f32(2 * sigmoid(a1 * m[4 + i] + b[4 + i]))
 *   L[i][j] = a2 * m[8 + 4i + j] + b[8 + 4i + j];  M = exp(L - max L)
 *   repeat iters times: divide each row by its sum, then each column by its sum;
 *   comb = f32(M).  All in f64. */
int or_split(const or_shape* s, const float* mixes, const float* hc_scale, const float* hc_base,
             float* pre, float* post, float* comb) {
  if (!shape_ok(s) || !mixes || !hc_scale || !hc_base || !pre || !post || !comb) return -1;
  const double a0 = hc_scale[0], a1 = hc_scale[1], a2 = hc_scale[2];
  for (int r = 0; r < s->rows; ++r) {
    const float* m = mixes + r * NMIX;
    for (int i = 0; i < NSTREAM; ++i) {
      pre[r * NSTREAM + i] = (float)sigmoid(a0 * m[i] + (double)hc_base[i]);
      post[r * NSTREAM + i] = (float)(2.0 * sigmoid(a1 * m[4 + i] + (double)hc_base[4 + i]));
    }
    double M[NSTREAM][NSTREAM], mx = -INFINITY;
    for (int i = 0; i < NSTREAM; ++i)
      for (int j = 0; j < NSTREAM; ++j) {
        M[i][j] = a2 * m[8 + 4 * i + j] + (double)hc_base[8 + 4 * i + j];
        if (M[i][j] > mx) mx = M[i][j];
      }
    for (int i = 0; i < NSTREAM; ++i)
      for (int j = 0; j < NSTREAM; ++j) M[i][j] = exp(M[i][j] - mx);
    for (int it = 0; it < s->sinkhorn_iters; ++it) {
      for (int i = 0; i < NSTREAM; ++i) {
        double sum = 0.0;
        for (int j = 0; j < NSTREAM; ++j) sum += M[i][j];
        for (int j = 0; j < NSTREAM; ++j) M[i][j] /= sum;
      }
      for (int j = 0; j < NSTREAM; ++j) {
        double sum = 0.0;
        for (int i = 0; i < NSTREAM; ++i) sum += M[i][j];
        for (int i = 0; i < NSTREAM; ++i) M[i][j] /= sum;
      }
    }
    for (int i = 0; i < NSTREAM; ++i)
      for (int j = 0; j < NSTREAM; ++j) comb[r * 16 + i * NSTREAM + j] = (float)M[i][j];
  }
  return 0;
}

/* ---------------------------------------------------------------------------------------------
 * Pre-weighted collapse + weighted RMSNorm [ds4 HC fusion commit: "pre-weighted collapse + BF16
 * + weighted RMSNorm + BF16"; sgl3 Modifications: bf16 RMSNorm weights].
 *   x[h]    = bf16(f32(sum_i pre[i] * state[i][h]))
 *   norm[h] = bf16(f32(x[h] / sqrt(mean(x^2) + eps_norm) * w_norm[h]))   (mean over H) */
int or_collapse_norm(const or_shape* s, const void* state, const float* pre, const void* w_norm,
                     void* x, void* norm) {
  if (!shape_ok(s) || !state || !pre || !w_norm || !x || !norm) return -1;
  const int64_t H = s->hidden;
  for (int r = 0; r < s->rows; ++r) {
    double ss = 0.0;
    for (int64_t h = 0; h < H; ++h) {
      double acc = 0.0;
      for (int i = 0; i < NSTREAM; ++i)
        acc += (double)pre[r * NSTREAM + i] *
               act_get(s->act, state, ((int64_t)r * NSTREAM + i) * H + h);
      act_put(s->act, x, (int64_t)r * H + h, acc);
      double xv = act_get(s->act, x, (int64_t)r * H + h);
      ss += xv * xv;
    }
    double den = sqrt(ss / (double)H + s->eps_norm);
    for (int64_t h = 0; h < H; ++h) {
      double xv = act_get(s->act, x, (int64_t)r * H + h);
      act_put(s->act, norm, (int64_t)r * H + h, xv / den * act_get(s->act, w_norm, h));
    }
  }
  return 0;
}

/* ---------------------------------------------------------------------------------------------
 * Model tail [ds4 single-box commit: the logits' collapse and the output norm reuse the collapse
 * kernel without a split; sgl3 Modifications: the last FFN post deferred to the model tail].
 * READING: the head has its own 4-row mix W_head [4][4H], one scale a and four biases b; its
 * pre weights are the pre half of the split and there is no post, comb or Sinkhorn:
 *   m[i]   = f32( (sum_t W_head[i][t] s[t]) / sqrt(mean(s^2) + eps_hc) )   (as the mix)
 *   pre[i] = f32( sigmoid(a * m[i] + b[i]) )                              (as the split's pre)
 *   x, norm = the pre-weighted collapse and weighted RMSNorm above, with the output norm weight.
 * pre [R][4] (optional), x and norm [R][H] (act). */
int or_head(const or_shape* s, const void* state, const float* w_head, const float* head_scale,
            const float* head_base, const void* w_norm, float* pre, void* x, void* norm) {
  if (!shape_ok(s) || !state || !w_head || !head_scale || !head_base || !w_norm || !x || !norm)
    return -1;
  const int64_t n = (int64_t)NSTREAM * s->hidden;
  float* pw = (float*)malloc(sizeof(float) * (size_t)(s->rows > 0 ? s->rows : 1) * NSTREAM);
  double* v = (double*)malloc(sizeof(double) * (size_t)n);
  if (!pw || !v) {
    free(pw);
    free(v);
    return -2;
  }
  const double a = head_scale[0];
  for (int r = 0; r < s->rows; ++r) {
    double ss = 0.0;
    for (int64_t t = 0; t < n; ++t) {
      v[t] = act_get(s->act, state, (int64_t)r * n + t);
      ss += v[t] * v[t];
    }
    const double rms = sqrt(ss / (double)n + s->eps_hc);
    for (int i = 0; i < NSTREAM; ++i) {
      double acc = 0.0;
      for (int64_t t = 0; t < n; ++t) acc += (double)w_head[(int64_t)i * n + t] * v[t];
      const float m = (float)(acc / rms);
      pw[r * NSTREAM + i] = (float)sigmoid(a * (double)m + (double)head_base[i]);
    }
  }
  free(v);
  const int rc = or_collapse_norm(s, state, pw, w_norm, x, norm);
  if (rc == 0 && pre) memcpy(pre, pw, sizeof(float) * (size_t)s->rows * NSTREAM);
  free(pw);
  return rc;
}

/* ---------------------------------------------------------------------------------------------
 * Router logits [ds4 router commit: "the F32 logits matvec"]: logits[e] = f32(W_r[e] . norm). */
int or_router_logits(const or_shape* s, const void* norm, const float* w_router, float* logits) {
  if (!shape_ok(s) || !norm || !w_router || !logits) return -1;
  const int64_t H = s->hidden;
  const int E = s->n_experts;
  double* v = (double*)malloc(sizeof(double) * H);
  if (!v) return -2;
  for (int r = 0; r < s->rows; ++r) {
    for (int64_t h = 0; h < H; ++h) v[h] = act_get(s->act, norm, (int64_t)r * H + h);
#pragma omp parallel for schedule(static)
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int64_t h = 0; h < H; ++h) acc += (double)w_router[(int64_t)e * H + h] * v[h];
      logits[(int64_t)r * E + e] = (float)acc;
    }
  }
  free(v);
  return 0;
}

/* ---------------------------------------------------------------------------------------------
 * Select [ds4 router commit: sqrt(softplus), the bias, the canonical (score descending, index
 * ascending) top-k, the normalised weights, the clamp, the row division and the scale as
 * separately rounded ops; tie-order commit: equal scores order by ascending index].
 *   sp = f32(softplus(z)), softplus(z) = max(z, 0) + log1p(exp(-|z|));  s = f32(sqrt(sp))
 *   beta = f32(s + bias[e]); idx = first k of (beta desc, e asc)
 *   sum = f32(sum_j s[idx_j]); c = max(sum, 2^-14)   (READING: clamp floor = smallest normal
 *   fp16); w_j = f32(s[idx_j] / c); w_j = f32(w_j * rho)
 * READING: the bias steers the selection only; the weights gather the unbiased s. */
typedef struct {
  float beta;
  int e;
} cand;

static int cand_cmp(const void* pa, const void* pb) {
  const cand* a = (const cand*)pa;
  const cand* b = (const cand*)pb;
  if (a->beta > b->beta) return -1;
  if (a->beta < b->beta) return 1;
  return (a->e > b->e) - (a->e < b->e);
}

int or_select(const or_shape* s, const float* logits, const float* bias, int32_t* idx,
              float* weights, float* beta_sorted) {
  if (!shape_ok(s) || !logits || !bias || !idx || !weights) return -1;
  const int E = s->n_experts, k = s->top_k;
  float* sc = (float*)malloc(sizeof(float) * E);
  cand* c = (cand*)malloc(sizeof(cand) * E);
  if (!sc || !c) {
    free(sc);
    free(c);
    return -2;
  }
  for (int r = 0; r < s->rows; ++r) {
    for (int e = 0; e < E; ++e) {
      double z = logits[(int64_t)r * E + e];
      float sp = (float)(fmax(z, 0.0) + log1p(exp(-fabs(z))));
      sc[e] = (float)sqrt((double)sp);
      c[e].beta = (float)((double)sc[e] + (double)bias[e]);
      c[e].e = e;
    }
    qsort(c, (size_t)E, sizeof(cand), cand_cmp);
    if (beta_sorted)
      for (int e = 0; e < E; ++e) beta_sorted[(int64_t)r * E + e] = c[e].beta;
    double sum = 0.0;
    for (int j = 0; j < k; ++j) sum += (double)sc[c[j].e];
    float sumf = (float)sum;
    double cl = fmax((double)sumf, ldexp(1.0, -14));
    for (int j = 0; j < k; ++j) {
      idx[r * k + j] = c[j].e;
      float w = (float)((double)sc[c[j].e] / cl);
      weights[r * k + j] = (float)((double)w * s->routed_scale);
    }
  }
  free(sc);
  free(c);
  return 0;
}

/* ---------------------------------------------------------------------------------------------
 * Experts [ds4 router/shared commit: gate/up rounded to BF16 before SwiGLU and the product
 * after it; the down projection rounded on its store; the routed + shared sum and its rounding;
 * sgl1 figure: shared + routed experts].
 *   g = bf16(f32(W_g . norm)), u = bf16(f32(W_u . norm)), h = bf16(f32(silu(g) * u)),
 *   silu(g) = g / (1 + exp(-g)).
 * READING: the routed experts use the shared expert's rounding points for g, u and h; their
 * down outputs y_e = f32(W_d[e] . h_e) and the weighted sum stay f32:
 *   routed = f32(sum_j w_j * y_{idx_j})   (selection order)
 *   shared = bf16(f32(W_ds . h_s));  block = bf16(f32(routed + shared)). */
int or_expert_hidden(const or_shape* s, int inter, const or_expert* ex, const void* norm_row,
                     void* h) {
  if (!shape_ok(s) || !ex || !norm_row || !h || !mat_ok(&ex->gate) || !mat_ok(&ex->up)) return -1;
  const int64_t H = s->hidden;
  double* v = (double*)malloc(sizeof(double) * H * 3);
  if (!v) return -2;
  for (int64_t c = 0; c < H; ++c) v[c] = act_get(s->act, norm_row, c);
  int rc = 0;
  const double* vg = matrix_input(s, &ex->gate, v, v + H, (int)H, &rc);
  const double* vu = matrix_input(s, &ex->up, v, v + 2 * H, (int)H, &rc);
  if (rc) {
    free(v);
    return rc;
  }
#pragma omp parallel for schedule(static)
  for (int i = 0; i < inter; ++i) {
    float gf = (float)mat_row_dot(&ex->gate, H, i, vg);
    float uf = (float)mat_row_dot(&ex->up, H, i, vu);
    double g = (s->act == OR_F32) ? (double)gf : or_bf16_to_f64(or_f32_to_bf16(gf));
    double u = (s->act == OR_F32) ? (double)uf : or_bf16_to_f64(or_f32_to_bf16(uf));
    act_put(s->act, h, i, g / (1.0 + exp(-g)) * u);
  }
  free(v);
  return 0;
}

/* y[c] = f32(W_d . h) for c < H. */
static int expert_down(const or_shape* s, int inter, const or_expert* ex, const void* h,
                       float* y) {
  if (!mat_ok(&ex->down)) return -1;
  const int64_t H = s->hidden;
  double* v = (double*)malloc(sizeof(double) * inter * 2);
  if (!v) return -2;
  for (int i = 0; i < inter; ++i) v[i] = act_get(s->act, h, i);
  int rc = 0;
  const double* vd = matrix_input(s, &ex->down, v, v + inter, inter, &rc);
  if (rc) {
    free(v);
    return rc;
  }
#pragma omp parallel for schedule(static)
  for (int64_t c = 0; c < H; ++c) y[c] = (float)mat_row_dot(&ex->down, inter, c, vd);
  free(v);
  return 0;
}

int or_moe(const or_shape* s, const void* norm, const int32_t* idx, const float* weights,
           const or_expert* routed, const or_expert* shared, int force_h, void* h_routed,
           void* h_shared, void* shared_out, float* routed_out, void* block) {
  if (!shape_ok(s) || !idx || !weights || !routed || !h_routed || !routed_out || !block)
    return -1;
  if (!force_h && !norm) return -1;
  if (s->shared_inter > 0 && (!shared || !h_shared || !shared_out)) return -1;
  const int64_t H = s->hidden, I = s->inter, Is = s->shared_inter;
  const int k = s->top_k, E = s->n_experts;
  const int ab = s->act == OR_F32 ? 4 : 2;
  float* y = (float*)malloc(sizeof(float) * H);
  double* acc = (double*)malloc(sizeof(double) * H);
  if (!y || !acc) {
    free(y);
    free(acc);
    return -2;
  }
  int rc = 0;
  for (int r = 0; r < s->rows && rc == 0; ++r) {
    const char* nrow = norm ? (const char*)norm + (int64_t)r * H * ab : NULL;
    for (int64_t c = 0; c < H; ++c) acc[c] = 0.0;
    for (int j = 0; j < k && rc == 0; ++j) {
      int e = idx[r * k + j];
      if (e < 0 || e >= E) {
        rc = -3;
        break;
      }
      char* hrow = (char*)h_routed + ((int64_t)r * k + j) * I * ab;
      if (!force_h) rc = or_expert_hidden(s, (int)I, &routed[e], nrow, hrow);
      if (rc == 0) rc = expert_down(s, (int)I, &routed[e], hrow, y);
      if (rc == 0)
        for (int64_t c = 0; c < H; ++c) acc[c] += (double)weights[r * k + j] * (double)y[c];
    }
    if (rc) break;
    for (int64_t c = 0; c < H; ++c) routed_out[(int64_t)r * H + c] = (float)acc[c];
    if (Is > 0) {
      char* hs = (char*)h_shared + (int64_t)r * Is * ab;
      if (!force_h) rc = or_expert_hidden(s, (int)Is, shared, nrow, hs);
      if (rc == 0) rc = expert_down(s, (int)Is, shared, hs, y);
      if (rc) break;
      for (int64_t c = 0; c < H; ++c) act_put(s->act, shared_out, (int64_t)r * H + c, y[c]);
    }
    for (int64_t c = 0; c < H; ++c) {
      double sh = Is > 0 ? act_get(s->act, shared_out, (int64_t)r * H + c) : 0.0;
      act_put(s->act, block, (int64_t)r * H + c, (double)routed_out[(int64_t)r * H + c] + sh);
    }
  }
  free(y);
  free(acc);
  return rc;
}

/* ---------------------------------------------------------------------------------------------
 * Post/comb expand [ds4 HC fusion commit: "post/comb expand + BF16"] and the carry into the
 * next pre [sgl3 Motivation: previous hc_post + bf16 residual materialisation + pre-norm GEMM
 * partials + RMS square-sum partials in one pass].
 *   new[i][h] = bf16(f32(post[i] * block[h] + sum_j comb[i][j] * state[j][h]))
 * READING [mhc]: comb acts as H_res on the stream axis (row i of comb mixes into stream i).
 * READING: the carry is taken on the bf16-rounded new state:
 *   carry[j] = f32(sum_t W_next[j][t] * new[t]) for j < 24, carry[24] = f32(sum_t new[t]^2). */
int or_expand(const or_shape* s, const void* state, const void* block, const float* post,
              const float* comb, const float* w_mix_next, void* new_state, float* carry) {
  if (!shape_ok(s) || !state || !block || !post || !comb || !new_state) return -1;
  if (w_mix_next && !carry) return -1;
  const int64_t H = s->hidden, n = (int64_t)NSTREAM * H;
  for (int r = 0; r < s->rows; ++r) {
    for (int i = 0; i < NSTREAM; ++i)
      for (int64_t h = 0; h < H; ++h) {
        double acc = (double)post[r * NSTREAM + i] * act_get(s->act, block, (int64_t)r * H + h);
        for (int j = 0; j < NSTREAM; ++j)
          acc += (double)comb[r * 16 + i * NSTREAM + j] *
                 act_get(s->act, state, ((int64_t)r * NSTREAM + j) * H + h);
        act_put(s->act, new_state, ((int64_t)r * NSTREAM + i) * H + h, acc);
      }
    if (w_mix_next) {
      double ss = 0.0;
      for (int64_t t = 0; t < n; ++t) {
        double v = act_get(s->act, new_state, (int64_t)r * n + t);
        ss += v * v;
      }
      for (int j = 0; j < NMIX; ++j) {
        double acc = 0.0;
        for (int64_t t = 0; t < n; ++t)
          acc += (double)w_mix_next[(int64_t)j * n + t] *
                 act_get(s->act, new_state, (int64_t)r * n + t);
        carry[r * (NMIX + 1) + j] = (float)acc;
      }
      carry[r * (NMIX + 1) + NMIX] = (float)ss;
    }
  }
  return 0;
}
