/*
 * fp8q oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU implementation of the W8A8
 * block-scaled FP8 projection.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library; the GPU product path
 * never calls it and shares no code with it.
 *
 * What it computes (sources: the pages "dispatch_proj.rs" and
 * "fp8_act_quant_floor.rs" of spark_model/layers/ops):
 *
 *   quantizer   bf16 activations [M,K] -> OCP FP8 e4m3 codes [M,K] plus one
 *               fp32 scale per (token, 128-wide K group), row-major [M,K/128]
 *               (dispatch_proj.rs, doc of cublas_fp8_proj: one scale per token
 *               and 128 elements of K).  scale = amax/448 in fp32, code =
 *               e4m3(x/scale) with round-to-nearest-even and saturation at
 *               +-448.
 *   relayout    row-major [M,K/128] -> K-major [K/128, ceil16(M)], tokens
 *               contiguous, pad rows M..ceil16(M) zero (dispatch_proj.rs,
 *               doc of cublas_scale_layout_kmajor and fp8_act_scale_to_kmajor;
 *               cublas_fp8_m_pad for ceil16).
 *   GEMM        out[M,N] = act[M,K] . W[N,K]^T with the activation scale of
 *               (m, kb) and the weight scale of the 128x128 block (n/128, kb)
 *               applied to each 128-deep K block (dispatch_proj.rs, doc of
 *               cublas_fp8_proj: both operands 128-block-scaled; weight scale
 *               index (n/128)*(K/128) + k/128 from dequant_fp8_bf16_into).
 *               Computed in fp64 and not rounded.
 *   per-row     the pages' other FP8 weight format: one fp32 scale per
 *               weight row.  Both formats address their scales with one
 *               formula, scale[(n/block_n)*sk + k/block_k], block-scaled
 *               (128, 128, K/128) or per-row (1, K, 1) (dispatch_proj.rs, doc
 *               of dequant_fp8_bf16_into); the GEMM and the FP8 -> bf16
 *               dequantizer below take that geometry.
 *   FFN         the SwiGLU intermediate h = bf16(silu(gate) * up) between
 *               the gate/up projections and the down projection
 *               (dispatch_proj.rs, doc of cublas_fp8_proj_prequant).
 *
 * Readings where the pages are silent (each one is listed in the design
 * notes): amax == 0 gives scale 0 and signed-zero codes; the scale is the
 * IEEE fp32 quotient amax/448 (not amax * (1/448)); q = fl32(x/scale); the
 * e4m3 variant is OCP e4m3fn (bias 7, max 448, no infinities, 0x7F/0xFF NaN);
 * no flush of subnormals anywhere; K must be a multiple of 128.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off (no -ffast-math), x86-64 SSE
 * math, so every float operation below is a single IEEE-754 binary32 or
 * binary64 operation rounded to nearest even.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GROUP 128

/* ---------------------------------------------------------------- codecs */

static float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Value of an OCP e4m3fn code: sign, 4-bit exponent (bias 7), 3-bit
 * mantissa; exponent field 0 is subnormal (m/8 * 2^-6); 0x7F/0xFF is NaN. */
double oracle_e4m3_decode(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

/* Nearest e4m3fn code to q, ties to the even mantissa, saturating to
 * +-448 (code 0x7E | sign).  The sign of q (including -0.0) is kept.  All
 * arithmetic is exact in binary64 so rint() (nearest-even in the default
 * rounding mode) makes the only rounding decision. */
uint8_t oracle_e4m3_encode(float q) {
  uint8_t s = signbit(q) ? 0x80 : 0x00;
  double a = fabs((double)q);
  int e;
  double m;
  if (a >= 448.0) return (uint8_t)(s | 0x7E);
  if (a < ldexp(1.0, -6)) {
    /* subnormal range: multiples of 2^-9; a result of 8 is 2^-6, which is
     * exactly the code 0x08 (exponent field 1, mantissa 0). */
    m = rint(a * 512.0);
    return (uint8_t)(s | (uint8_t)m);
  }
  frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) */
  e -= 1;       /* now a = (1 + t) * 2^e, t in [0, 1) */
  m = rint((ldexp(a, -e) - 1.0) * 8.0);
  if (m == 8.0) {
    e += 1;
    m = 0.0;
  }
  if (e + 7 > 15 || (e + 7 == 15 && m == 7.0)) return (uint8_t)(s | 0x7E);
  return (uint8_t)(s | (uint8_t)((e + 7) << 3) | (uint8_t)m);
}

/* Element-wise encode of n floats (test helper). */
void oracle_e4m3_encode_array(const float *q, uint8_t *out, int64_t n) {
  int64_t i;
#pragma omp parallel for schedule(static)
  for (i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(q[i]);
}

/* Encode of x relative to scale, the quantizer's per-element step. */
static uint8_t quant_elem(float x, float scale) {
  if (scale == 0.0f) return signbit(x) ? 0x80 : 0x00;
  return oracle_e4m3_encode(x / scale);
}

/* ------------------------------------------------------------- quantizer */

/* bf16 x[M,K] -> codes q[M,K], scales[M,K/128] (row-major). */
void oracle_quant_act(const uint16_t *x, uint8_t *q, float *scale, int64_t M,
                      int64_t K) {
  const int64_t G = K / GROUP;
  int64_t r;
#pragma omp parallel for schedule(static)
  for (r = 0; r < M * G; ++r) {
    const int64_t m = r / G, g = r % G;
    const uint16_t *xs = x + m * K + g * GROUP;
    uint8_t *qs = q + m * K + g * GROUP;
    float amax = 0.0f, s;
    int j;
    for (j = 0; j < GROUP; ++j) {
      float v = fabsf(bf16_to_f32(xs[j]));
      if (v > amax) amax = v;
    }
    s = amax / 448.0f;
    scale[m * G + g] = s;
    for (j = 0; j < GROUP; ++j) qs[j] = quant_elem(bf16_to_f32(xs[j]), s);
  }
}

/* -------------------------------------------------------------- relayout */

int64_t oracle_m_pad(int64_t M) { return (M + 15) / 16 * 16; }

/* row-major [M,G] -> K-major [G, Mp], Mp = ceil16(M), pad slots +0.0f. */
void oracle_scale_to_kmajor(const float *rm, float *km, int64_t M, int64_t K) {
  const int64_t G = K / GROUP, Mp = oracle_m_pad(M);
  int64_t g, m;
  for (g = 0; g < G; ++g)
    for (m = 0; m < Mp; ++m) km[g * Mp + m] = (m < M) ? rm[m * G + g] : 0.0f;
}

/* ------------------------------------------------------ weight quantizer */

/* fp32 W[N,K] -> codes [N,K] and one fp32 scale per 128x128 block,
 * [N/128, K/128] row-major; scale = block amax / 448 (same element encoder
 * as the activation quantizer).  Used only to make synthetic FP8 weights. */
void oracle_quant_weight_block(const float *w, uint8_t *q, float *scale,
                               int64_t N, int64_t K) {
  const int64_t NB = N / GROUP, G = K / GROUP;
  int64_t b;
#pragma omp parallel for schedule(static)
  for (b = 0; b < NB * G; ++b) {
    const int64_t nb = b / G, g = b % G;
    float amax = 0.0f, s;
    int i, j;
    for (i = 0; i < GROUP; ++i)
      for (j = 0; j < GROUP; ++j) {
        float v = fabsf(w[(nb * GROUP + i) * K + g * GROUP + j]);
        if (v > amax) amax = v;
      }
    s = amax / 448.0f;
    scale[b] = s;
    for (i = 0; i < GROUP; ++i)
      for (j = 0; j < GROUP; ++j) {
        const int64_t o = (nb * GROUP + i) * K + g * GROUP + j;
        q[o] = quant_elem(w[o], s);
      }
  }
}

/* fp32 W[N,K] -> codes [N,K] and one fp32 scale per row, scale[n] = row
 * amax / 448 (the per-row format; same element encoder).  Synthetic weights
 * only. */
void oracle_quant_weight_row(const float *w, uint8_t *q, float *scale, int64_t N,
                             int64_t K) {
  int64_t n;
#pragma omp parallel for schedule(static)
  for (n = 0; n < N; ++n) {
    float amax = 0.0f, s;
    int64_t k;
    for (k = 0; k < K; ++k) {
      const float v = fabsf(w[n * K + k]);
      if (v > amax) amax = v;
    }
    s = amax / 448.0f;
    scale[n] = s;
    for (k = 0; k < K; ++k) q[n * K + k] = quant_elem(w[n * K + k], s);
  }
}

/* -------------------------------------------------- FP8 -> bf16 weights */

/* fp32 -> bf16 bit pattern, round to nearest even (finite input). */
static uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

/* dst[n,k] = bf16(fl32(dec(w[n,k]) * scale[(n/block_n)*sk + k/block_k]))
 * (dispatch_proj.rs, dequant_fp8_bf16_into: the scale index formula and
 * the two geometries).  The decoded value times the fp32 scale is formed
 * exactly in fp64 (at most 4 + 24 significant bits), rounded once to fp32 and
 * then once to bf16. */
void oracle_dequant_fp8_bf16(const uint8_t *w, const float *scale, uint16_t *dst,
                             int64_t N, int64_t K, int64_t block_n, int64_t block_k,
                             int64_t sk) {
  int64_t n;
#pragma omp parallel for schedule(static)
  for (n = 0; n < N; ++n) {
    int64_t k;
    for (k = 0; k < K; ++k) {
      const double s = (double)scale[(n / block_n) * sk + k / block_k];
      const float prod = (float)(oracle_e4m3_decode(w[n * K + k]) * s);
      dst[n * K + k] = f32_to_bf16_rne(prod);
    }
  }
}

/* ------------------------------------------------------------------ GEMM */

/* One output element in block form:
 *   ref[m,n] = sum_g a_s[m,g] * w_s[(n/block_n)*sk + 128g/block_k] * S(m,n,g),
 *   S(m,n,g) = sum_j dec(a[m,128g+j]) * dec(w[n,128g+j])   (exact in fp64).
 * a_s is the row-major [M, K/128] activation scale; the weight geometry is
 * (128, 128, K/128) for 128x128 block scales and (1, K, 1) per row. */
static double gemm_elem(const uint8_t *a, const float *a_s, const uint8_t *w,
                        const float *w_s, const double *dec, int64_t m,
                        int64_t n, int64_t K, int64_t block_n, int64_t block_k,
                        int64_t sk) {
  const int64_t G = K / GROUP;
  double acc = 0.0;
  int64_t g;
  for (g = 0; g < G; ++g) {
    const uint8_t *ar = a + m * K + g * GROUP;
    const uint8_t *wr = w + n * K + g * GROUP;
    double S = 0.0;
    int j;
    for (j = 0; j < GROUP; ++j) S += dec[ar[j]] * dec[wr[j]];
    acc += (double)a_s[m * G + g] * (double)w_s[(n / block_n) * sk + (g * GROUP) / block_k] * S;
  }
  return acc;
}

static void decode_table(double dec[256]) {
  int c;
  for (c = 0; c < 256; ++c) dec[c] = oracle_e4m3_decode((uint8_t)c);
}

/* Full reference out[M,N] (fp64), weight-scale geometry as for gemm_elem. */
void oracle_gemm_ref_geom(const uint8_t *a, const float *a_s, const uint8_t *w,
                          const float *w_s, double *out, int64_t M, int64_t N,
                          int64_t K, int64_t block_n, int64_t block_k, int64_t sk) {
  double dec[256];
  int64_t r;
  decode_table(dec);
#pragma omp parallel for schedule(dynamic, 16)
  for (r = 0; r < M * N; ++r)
    out[r] = gemm_elem(a, a_s, w, w_s, dec, r / N, r % N, K, block_n, block_k, sk);
}

/* Reference at selected (m, n) pairs only: out[i] = ref[ms[i], ns[i]]. */
void oracle_gemm_ref_at_geom(const uint8_t *a, const float *a_s, const uint8_t *w,
                             const float *w_s, const int64_t *ms, const int64_t *ns,
                             double *out, int64_t count, int64_t K, int64_t block_n,
                             int64_t block_k, int64_t sk) {
  double dec[256];
  int64_t i;
  decode_table(dec);
#pragma omp parallel for schedule(dynamic, 16)
  for (i = 0; i < count; ++i)
    out[i] = gemm_elem(a, a_s, w, w_s, dec, ms[i], ns[i], K, block_n, block_k, sk);
}

/* The 128x128 block-scaled forms. */
void oracle_gemm_ref(const uint8_t *a, const float *a_s, const uint8_t *w,
                     const float *w_s, double *out, int64_t M, int64_t N,
                     int64_t K) {
  oracle_gemm_ref_geom(a, a_s, w, w_s, out, M, N, K, GROUP, GROUP, K / GROUP);
}
void oracle_gemm_ref_at(const uint8_t *a, const float *a_s, const uint8_t *w,
                        const float *w_s, const int64_t *ms, const int64_t *ns,
                        double *out, int64_t count, int64_t K) {
  oracle_gemm_ref_at_geom(a, a_s, w, w_s, ms, ns, out, count, K, GROUP, GROUP, K / GROUP);
}

/* ------------------------------------------------- FFN intermediate */

/* Nearest bf16 value of a double, ties to even, as a bit pattern: the value
 * divided by its bf16 ulp (an exact power-of-two rescaling) is rounded to an
 * integer by nearbyint (the default mode, to nearest even), one rounding in
 * all.  bf16 keeps 8 significant bits and fp32's exponent range: the ulp of
 * a value in [2^e, 2^(e+1)) is 2^(max(e,-126)-7), subnormals included;
 * magnitudes that round to 2^128 or beyond become infinities. */
static uint16_t f64_to_bf16_bits(double v) {
  int e;
  double ulp, r;
  float f;
  uint32_t u;
  if (isnan(v)) return 0x7FC0;
  if (v == 0.0 || isinf(v)) {
    f = (float)v; /* signed zero or infinity, exact */
  } else {
    (void)frexp(v, &e); /* v = f * 2^e with 0.5 <= |f| < 1: binade 2^(e-1) */
    if (e - 1 < -126) e = -125;
    ulp = ldexp(1.0, e - 1 - 7);
    r = nearbyint(v / ulp) * ulp;
    f = (fabs(r) >= ldexp(1.0, 128)) ? (float)copysign(INFINITY, v) : (float)r;
  }
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

void oracle_f64_to_bf16_array(const double *v, uint16_t *out, int64_t n) {
  int64_t i;
  for (i = 0; i < n; ++i) out[i] = f64_to_bf16_bits(v[i]);
}

/* The dense FFN's intermediate (dispatch_proj.rs, doc of
 * cublas_fp8_proj_prequant: gate and up are two projections of the same
 * quantized input; the post-SiLU intermediate is quantized once for down).
 * The pages name SiLU and the product with up but print no formula; the
 * plain reading: h = bf16(silu(g) * u) with silu(g) = g / (1 + e^-g), g and
 * u the bf16 outputs of the gate and up projections.  The value is formed in
 * double (one exp, one add, one divide, one multiply: relative error a few
 * 2^-53) and rounded once to bf16.
 *
 * amb[i] = 1 marks an element whose double value lies within 2^-18 of its
 * own magnitude (or within 2^-146 absolutely) of a bf16 rounding midpoint:
 * there an evaluation in binary32 arithmetic, whose error is a few 2^-24,
 * may round to either neighbour, and both results are correct roundings of
 * a value inside the binary32 evaluation's error. */
void oracle_silu_mul(const uint16_t *g, const uint16_t *u, uint16_t *h, uint8_t *amb,
                     int64_t n) {
  int64_t i;
#pragma omp parallel for schedule(static)
  for (i = 0; i < n; ++i) {
    const double gv = (double)bf16_to_f32(g[i]), uv = (double)bf16_to_f32(u[i]);
    const double v = gv / (1.0 + exp(-gv)) * uv;
    int e;
    double ulp, t, d;
    h[i] = f64_to_bf16_bits(v);
    amb[i] = 0;
    if (v != 0.0 && isfinite(v)) {
      (void)frexp(v, &e);
      if (e - 1 < -126) e = -125;
      ulp = ldexp(1.0, e - 1 - 7);
      t = v / ulp;
      d = fabs(t - (floor(t) + 0.5)) * ulp; /* distance to the nearest midpoint */
      if (d <= ldexp(fabs(v), -18) || d <= ldexp(1.0, -146)) amb[i] = 1;
    }
  }
}

/* Number of OpenMP threads a parallel region here would use. */
int oracle_num_threads(void) {
  int n = 1;
#pragma omp parallel
  {
#pragma omp single
    {
#ifdef _OPENMP
      extern int omp_get_num_threads(void);
      n = omp_get_num_threads();
#endif
    }
  }
  return n;
}
