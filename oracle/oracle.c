/*
 * oracle.c — plain, slow CPU definition of the shared Q8_1 activation-image path.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg may load this library. The product path (the HIP library) never calls it, and the two
 * share no code, header, table or constant generator.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fPIC -shared oracle.c -lm
 * (x86-64 SSE arithmetic: every float operation is a single IEEE binary32 rounding; fmaf is
 * the correctly rounded fused multiply-add of C99.)
 *
 * What it computes. The fused producer must give exactly what "producer, then the separate
 * quantizer, then the readers" gives ("Share temporary Q8_1 activation images", Overview:
 * emission removes a separate quantization launch and reread while reduction trees and
 * quantization rounding stay intact). So this file spells out that plain pipeline:
 *   rms / glu producer (f32, the F32 output the pages keep)  ->  per-32-block Q8_1 quantizer
 *   ->  Q4_0 x Q8_1 readers evaluated in float64 from the quantized operands
 *   ->  routed plan (stable grouping of the live pairs by expert).
 * Where the pages are silent (rounding mode, reduction order, exp/erf, layouts) the reading
 * adopted is stated at the function and listed in the design notes.
 */
#define _DEFAULT_SOURCE /* M_LN2, M_LOG2E, M_SQRT1_2 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------------
 * binary16 conversion. The Q8_1 block stores "half scales/sums" ("Share temporary Q8_1
 * activation images", GLU producer evidence, validation list). f32 -> f16 is IEEE
 * round-to-nearest-even with subnormals kept and overflow to infinity.
 * Written with double arithmetic: the value is scaled to an integer multiple of its f16 ulp
 * (exact in double), rounded with nearbyint (ties to even), and re-encoded.
 * ---------------------------------------------------------------------------------------- */
uint16_t orc_f32_to_f16(float f) {
  uint32_t bits;
  memcpy(&bits, &f, 4);
  uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
  if (isnan(f)) return (uint16_t)(sign | 0x7e00u);
  double a = fabs((double)f);
  if (isinf(f)) return (uint16_t)(sign | 0x7c00u);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);               /* a = m * 2^e, m in [0.5, 1): exponent of a is e-1 */
  int ex = e - 1;             /* a in [2^ex, 2^(ex+1)) */
  if (ex < -14) ex = -14;     /* subnormal range shares the ulp of the smallest normal */
  double ulp = ldexp(1.0, ex - 10);
  double q = nearbyint(a / ulp); /* a/ulp exact (power-of-two scaling); ties to even */
  /* q in [0, 2048]; value = q * ulp */
  uint32_t h;
  if (ex == -14 && q < 1024.0) {
    h = (uint32_t)q; /* subnormal (or the smallest normal when q reaches 1024) */
  } else {
    /* q in [1024, 2048]: q == 2048 carries into the next binade automatically */
    h = (uint32_t)((ex + 15) << 10) + (uint32_t)(q - 1024.0);
    if (h >= 0x7c00u) h = 0x7c00u; /* overflow to infinity */
  }
  return (uint16_t)(sign | h);
}

void orc_f32_to_f16_array(const float* x, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_f16(x[i]);
}

/* Exact binary16 -> double. */
double orc_f16_to_f64(uint16_t h) {
  int s = (h >> 15) & 1, e = (h >> 10) & 0x1f, m = h & 0x3ff;
  double v;
  if (e == 0) v = ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(m + 1024), e - 25);
  return s ? -v : v;
}

/* ------------------------------------------------------------------------------------------
 * exp_q: the exponential the GLU producers use, defined here so that CPU and GPU evaluate the
 * same operation sequence (the pages name the SwiGLU/GeGLU-erf formulas but no exp):
 *   Cody-Waite reduction  n = rint(x * log2(e)), r = (x - n*LN2_HI) - n*LN2_LO (two fmas),
 *   degree-7 Taylor polynomial of e^r (coefficients 1/k! rounded to f32) by Horner with fma,
 *   result = ldexp(p, n).
 * LN2_HI is ln 2 rounded to f32 with its low 12 significand bits cleared (so n*LN2_HI is exact
 * for |n| < 2^12), LN2_LO the f32 nearest ln 2 - LN2_HI. Saturation: NaN passes through;
 * x > 88.8 gives +inf; x < -86 gives +0 (results that would need f32 subnormals are flushed).
 * ---------------------------------------------------------------------------------------- */
static float g_ln2_hi, g_ln2_lo, g_log2e, g_inv_fact[8];
static int g_consts_ready = 0;

static void orc_init_consts(void) {
  if (g_consts_ready) return;
  float ln2f = (float)M_LN2;
  uint32_t b;
  memcpy(&b, &ln2f, 4);
  b &= ~0xfffu;
  memcpy(&g_ln2_hi, &b, 4);
  g_ln2_lo = (float)(M_LN2 - (double)g_ln2_hi);
  g_log2e = (float)M_LOG2E;
  double f = 1.0;
  for (int k = 0; k < 8; ++k) {
    if (k > 0) f *= (double)k;
    g_inv_fact[k] = (float)(1.0 / f);
  }
  g_consts_ready = 1;
}

float orc_exp_q(float x) {
  orc_init_consts();
  if (x != x) return x;
  if (x > 88.8f) return INFINITY;
  if (x < -86.0f) return 0.0f;
  float n = rintf(x * g_log2e);
  float r = fmaf(-n, g_ln2_hi, x);
  r = fmaf(-n, g_ln2_lo, r);
  float p = g_inv_fact[7];
  for (int k = 6; k >= 0; --k) p = fmaf(p, r, g_inv_fact[k]);
  return ldexpf(p, (int)n);
}

void orc_exp_q_array(const float* x, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_exp_q(x[i]);
}

/* ------------------------------------------------------------------------------------------
 * erfc_q(z), z >= 0: the Chebyshev-fitted complementary error function of Numerical Recipes
 * ("erfcc": erfc(z) = t * exp(-z^2 - 1.26551223 + t*P(t)), t = 1/(1 + z/2); published
 * fractional error below 1.2e-7 everywhere), evaluated in f32 by Horner with fma, with exp_q.
 * ---------------------------------------------------------------------------------------- */
float orc_erfc_q(float z) {
  float t = 1.0f / (1.0f + 0.5f * z);
  float p = 0.17087277f;
  p = fmaf(p, t, -0.82215223f);
  p = fmaf(p, t, 1.48851587f);
  p = fmaf(p, t, -1.13520398f);
  p = fmaf(p, t, 0.27886807f);
  p = fmaf(p, t, -0.18628806f);
  p = fmaf(p, t, 0.09678418f);
  p = fmaf(p, t, 0.37409196f);
  p = fmaf(p, t, 1.00002368f);
  p = fmaf(p, t, -1.26551223f);
  float arg = fmaf(-z, z, p);
  return t * orc_exp_q(arg);
}

void orc_erfc_q_array(const float* z, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_erfc_q(z[i]);
}

/* ------------------------------------------------------------------------------------------
 * GLU activations ("Share temporary Q8_1 activation images", Coverage: F32 SwiGLU and
 * GeGLU-erf producers keep their original formulas). Textbook definitions:
 *   SwiGLU    : act(g) = g * sigmoid(g) = g / (1 + exp(-g))
 *   GeGLU-erf : act(g) = g * Phi(g) = 0.5 * g * (1 + erf(g / sqrt 2))
 * with 1 + erf(z) = erfc(-z) for z < 0 and 2 - erfc(z) for z >= 0. y = act(g) * u.
 * ---------------------------------------------------------------------------------------- */
/* g * sigmoid(c g) = g / (1 + exp(-c g)), the shape shared by SwiGLU (c = 1), GeGLU-quick
 * (c = 1.702) and SwiGLU-OAI (c = alpha). */
static float g_sigmoid(float g, float c) {
  float e = orc_exp_q(-(c * g));
  float den = 1.0f + e;
  return g / den;
}

float orc_glu_act(int op, float g) {
  if (op == 0) {
    float e = orc_exp_q(-g);
    float den = 1.0f + e;
    return g / den;
  } else if (op == 1) {
    float z = g * (float)M_SQRT1_2;
    float ope = (z < 0.0f) ? orc_erfc_q(-z) : 2.0f - orc_erfc_q(z);
    return (0.5f * g) * ope;
  } else if (op == 2) {
    /* ReGLU: relu(g) */
    return g > 0.0f ? g : 0.0f;
  } else if (op == 3) {
    /* GeGLU, tanh form: 0.5 g (1 + tanh(z)), z = sqrt(2/pi) (g + 0.044715 g^3). With
     * 0.5 (1 + tanh z) = 1 / (1 + exp(-2z)) it is g / (1 + exp(-c2 (g + 0.044715 g^3))),
     * c2 = 2 sqrt(2/pi) rounded to f32 (no cancellation for either sign of g). */
    float g3 = (g * g) * g;
    float inner = g + 0.044715f * g3;
    float e = orc_exp_q(-((float)(2.0 * sqrt(2.0 / M_PI)) * inner));
    float den = 1.0f + e;
    return g / den;
  } else if (op == 4) {
    /* GeGLU-quick: g sigmoid(1.702 g) */
    return g_sigmoid(g, 1.702f);
  }
  return NAN; /* ops 5 and 6 need their up value and parameters: orc_glu_pair */
}

/* The GLU family with the gate/up clamps of the OpenAI-style SwiGLU:
 *   op 5 SwiGLU-OAI  : g' = min(g, limit), u' = clamp(u, -limit, limit),
 *                      y = g' sigmoid(alpha g') * (u' + 1)
 *   op 6 SwiGLU-clamp: g' = min(g, limit), u' = clamp(u, -limit, limit), y = silu(g') * u'
 * ops 0..4: y = act(g) * u with orc_glu_act. alpha and limit are used by ops 5 and 6 only. */
float orc_glu_pair(int op, float alpha, float limit, float g, float u) {
  if (op < 5) return orc_glu_act(op, g) * u;
  float gg = g < limit ? g : limit;
  float uu = u < -limit ? -limit : (u > limit ? limit : u);
  if (op == 5) return g_sigmoid(gg, alpha) * (uu + 1.0f);
  return orc_glu_act(0, gg) * uu;
}

void orc_glu_pair_array(int op, float alpha, float limit, const float* g, float u, float* out,
                        int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_glu_pair(op, alpha, limit, g[i], u);
}

void orc_glu_act_array(int op, const float* g, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_glu_act(op, g[i]);
}

void orc_glu(int op, const float* gate, int64_t ldg, const float* up, int64_t ldu, int rows, int K,
             float* y, int64_t ldy) {
  for (int i = 0; i < rows; ++i)
    for (int k = 0; k < K; ++k) {
      float act = orc_glu_act(op, gate[(int64_t)i * ldg + k]);
      y[(int64_t)i * ldy + k] = act * up[(int64_t)i * ldu + k];
    }
}

/* Every GLU variant of "Share temporary Q8_1 activation images", Coverage (F32 ReGLU, GeGLU,
 * SwiGLU, GeGLU-erf, GeGLU-quick, SwiGLU-OAI and SwiGLU-clamp producers keep their formulas
 * and alpha/limit parameters; separate, packed and packed-swapped inputs keep independent
 * row strides): y[i][k] = orc_glu_pair(op, alpha, limit, gate[i][k], up[i][k]). */
void orc_glu_ex(int op, float alpha, float limit, const float* gate, int64_t ldg, const float* up,
                int64_t ldu, int rows, int K, float* y, int64_t ldy) {
  for (int i = 0; i < rows; ++i)
    for (int k = 0; k < K; ++k)
      y[(int64_t)i * ldy + k] =
          orc_glu_pair(op, alpha, limit, gate[(int64_t)i * ldg + k], up[(int64_t)i * ldu + k]);
}

/* ------------------------------------------------------------------------------------------
 * RMS producer ("Share temporary Q8_1 activation images", Coverage: RMS-alone and RMS+MUL
 * producers emit the image; original F32 stores remain).
 *   S = sum x^2 in the fixed order below, mean = S / K, r = 1 / sqrt(mean + eps),
 *   y = (x * r) * gamma   (gamma absent: y = x * r), each operation one f32 rounding,
 *   division and square root correctly rounded.
 * Fixed order of S (the pages only require reduction trees to stay intact, Overview):
 *   leaf c (c < K/4) = fma(x3,x3, fma(x2,x2, fma(x1,x1, x0*x0))) over x[4c..4c+3];
 *   lane l in [0,64) owns leaves c = l + 64 j, j < J' (J' = next power of two >= ceil(K/256),
 *   a missing leaf is +0); each lane sums its J' leaves by a balanced pairwise tree over j;
 *   the 64 lane sums are combined by a balanced pairwise tree over l.
 * ---------------------------------------------------------------------------------------- */
static float pairwise_tree(float* v, int n) { /* n a power of two; v is overwritten */
  for (int w = n; w > 1; w >>= 1)
    for (int i = 0; i < w / 2; ++i) v[i] = v[2 * i] + v[2 * i + 1];
  return v[0];
}

float orc_rms_sumsq(const float* x, int K) {
  int C = K / 4;
  int J = (K + 255) / 256;
  int Jp = 1;
  while (Jp < J) Jp <<= 1;
  float lane_sum[64];
  float* v = (float*)malloc(sizeof(float) * (size_t)Jp);
  for (int l = 0; l < 64; ++l) {
    for (int j = 0; j < Jp; ++j) {
      int c = l + 64 * j;
      if (c < C) {
        const float* q = x + 4 * c;
        v[j] = fmaf(q[3], q[3], fmaf(q[2], q[2], fmaf(q[1], q[1], q[0] * q[0])));
      } else {
        v[j] = 0.0f;
      }
    }
    lane_sum[l] = pairwise_tree(v, Jp);
  }
  free(v);
  return pairwise_tree(lane_sum, 64);
}

/* The RMS scale from the regularised mean square v = mean + eps: 1 / sqrt(v), with the
 * correctly rounded sqrt and division of IEEE f32. */
float orc_rms_scale(float v) { return 1.0f / sqrtf(v); }

void orc_rms_scale_array(const float* v, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_rms_scale(v[i]);
}

void orc_rmsnorm(const float* x, int64_t ldx, const float* gamma, float eps, int rows, int K,
                 float* y, int64_t ldy) {
  for (int i = 0; i < rows; ++i) {
    const float* xr = x + (int64_t)i * ldx;
    float S = orc_rms_sumsq(xr, K);
    float mean = S / (float)K;
    float r = orc_rms_scale(mean + eps);
    for (int k = 0; k < K; ++k) {
      float t = xr[k] * r;
      y[(int64_t)i * ldy + k] = gamma ? t * gamma[k] : t;
    }
  }
}

/* The RMS+MUL+ADD and RMS+SCALE producers ("Share temporary Q8_1 activation images",
 * Coverage: RMS-alone, RMS+MUL, RMS+MUL+ADD and RMS+SCALE producers emit images):
 *   t = x * r; if gamma: t = t * gamma; if beta: t = t + beta; y = t * scale,
 * each one f32 rounding, in that order (scale = 1 leaves t unchanged). */
void orc_rmsnorm_ex(const float* x, int64_t ldx, const float* gamma, const float* beta,
                    float scale, float eps, int rows, int K, float* y, int64_t ldy) {
  for (int i = 0; i < rows; ++i) {
    const float* xr = x + (int64_t)i * ldx;
    float S = orc_rms_sumsq(xr, K);
    float mean = S / (float)K;
    float r = orc_rms_scale(mean + eps);
    for (int k = 0; k < K; ++k) {
      float t = xr[k] * r;
      if (gamma) t = t * gamma[k];
      if (beta) t = t + beta[k];
      y[(int64_t)i * ldy + k] = t * scale;
    }
  }
}

/* ------------------------------------------------------------------------------------------
 * Q8_1 quantizer, per 32-element block (the block the pages' image carries: int8 codes with a
 * half scale and a half sum; "Share temporary Q8_1 activation images", GLU producer evidence
 * validation list; the scale is amax/127 and the sum is d times the sum of the codes):
 *   amax = max|y|; if amax == 0: all-zero block.
 *   d = amax / 127, id = 1 / d (if id is not finite: all-zero block),
 *   c = roundf(y * id)  (round half away from zero),
 *   d16 = f16(d), s16 = f16((float)(sum c) * d).
 * Image layout: codes[rows][RB][32] int8, then ds[rows][RB] uint32 (d16 | s16 << 16), with
 * RB = round_up(K/32, 16); blocks K/32 <= b < RB are zero ([P1] Coverage: image row widths are
 * whole blocks; the padding is part of the compared image bytes). Returns the number of
 * non-finite inputs met (the producer's live rows must be finite).
 * ---------------------------------------------------------------------------------------- */
/* The block scale d = amax / 127 and the code multiplier id = 1 / d (both correctly rounded). */
float orc_quant_scale(float amax) { return amax / 127.0f; }

void orc_quant_recip_array(const float* amax, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = 1.0f / orc_quant_scale(amax[i]);
}

void orc_quant_scale_array(const float* amax, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_quant_scale(amax[i]);
}

/* f32 -> binary16 bits, widened to a 32-bit word (high half zero). */
void orc_f32_to_f16_word_array(const float* x, uint32_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_f16(x[i]);
}

int orc_row_blocks(int K) { return ((K / 32 + 15) / 16) * 16; }

int orc_quantize(const float* y, int64_t ldy, int rows, int K, uint8_t* img) {
  int Kb = K / 32, RB = orc_row_blocks(K);
  int8_t* codes = (int8_t*)img;
  uint32_t* ds = (uint32_t*)(img + (size_t)rows * RB * 32);
  int bad = 0;
  for (int i = 0; i < rows; ++i) {
    for (int b = 0; b < RB; ++b) {
      int8_t* cb = codes + ((size_t)i * RB + b) * 32;
      uint32_t* db = ds + (size_t)i * RB + b;
      memset(cb, 0, 32);
      *db = 0;
      if (b >= Kb) continue;
      const float* yb = y + (int64_t)i * ldy + 32 * b;
      float amax = 0.0f;
      for (int j = 0; j < 32; ++j) {
        if (!isfinite(yb[j])) bad++;
        float a = fabsf(yb[j]);
        if (a > amax) amax = a;
      }
      if (amax == 0.0f) continue;
      float d = orc_quant_scale(amax);
      float id = 1.0f / d;
      if (!isfinite(id)) continue;
      int sum = 0;
      for (int j = 0; j < 32; ++j) {
        int c = (int)roundf(yb[j] * id);
        if (c > 127 || c < -127) bad++;
        cb[j] = (int8_t)c;
        sum += c;
      }
      uint16_t d16 = orc_f32_to_f16(d);
      uint16_t s16 = orc_f32_to_f16((float)sum * d);
      *db = (uint32_t)d16 | ((uint32_t)s16 << 16);
    }
  }
  return bad;
}

/* ------------------------------------------------------------------------------------------
 * Readers. Q4_0 weights: qs[N][Kb][16] (byte j: element j low nibble, element j+16 high
 * nibble), d[N][Kb] f16, weight = d * (nibble - 8). The block integer dot
 *   sumi = sum_j (qs[j] & 15) * c[j] + (qs[j] >> 4) * c[j+16]
 * is taken on the raw nibbles; the offset 8 is removed with the image's stored sum s16, which
 * is why a Q8_1 block carries it:
 *   out[t][n] = sum_b dw * (d16 * sumi - 8 * s16)     evaluated in float64, ascending b.
 * ("Share temporary Q8_1 activation images", Coverage: MMVQ readers of the standard Q8_1
 * activation image; GLU producer evidence: Q4_0 component graphs.)
 * ---------------------------------------------------------------------------------------- */
static int32_t block_dot(const uint8_t* qs, const int8_t* c) {
  int32_t s = 0;
  for (int j = 0; j < 16; ++j) s += (int32_t)(qs[j] & 15) * c[j] + (int32_t)(qs[j] >> 4) * c[j + 16];
  return s;
}

void orc_blockdots(const uint8_t* qs, int N, int K, const uint8_t* img, int img_rows, int rows,
                   int32_t* sumi) {
  int Kb = K / 32, RB = orc_row_blocks(K);
  const int8_t* codes = (const int8_t*)img;
  (void)img_rows;
  for (int t = 0; t < rows; ++t)
    for (int n = 0; n < N; ++n)
      for (int b = 0; b < Kb; ++b)
        sumi[((size_t)t * N + n) * Kb + b] =
            block_dot(qs + ((size_t)n * Kb + b) * 16, codes + ((size_t)t * RB + b) * 32);
}

static double reader_row(const uint8_t* qs, const uint16_t* d, int Kb, const int8_t* crow,
                         const uint32_t* dsrow) {
  double acc = 0.0;
  for (int b = 0; b < Kb; ++b) {
    int32_t s = block_dot(qs + (size_t)b * 16, crow + (size_t)b * 32);
    double dw = orc_f16_to_f64(d[b]);
    double da = orc_f16_to_f64((uint16_t)(dsrow[b] & 0xffffu));
    double sa = orc_f16_to_f64((uint16_t)(dsrow[b] >> 16));
    acc += dw * (da * (double)s - 8.0 * sa);
  }
  return acc;
}

/* ------------------------------------------------------------------------------------------
 * Other weight formats of the readers ("Share temporary Q8_1 activation images", Coverage:
 * quantized MUL_MAT readers on MMVQ use the Q8_1 image; the image's half sums s = d * sum(c)
 * are what a format with a per-block minimum needs):
 *   Q8_0: block = 32 int8 codes q and fp16 d, weight = d * q.
 *         term_b = d_w * d_a * sum_j q_j c_j
 *   Q4_1: block = 16 bytes of nibbles (ggml order, as Q4_0), fp16 d and fp16 m,
 *         weight = d * q + m (q in 0..15).
 *         term_b = d_w * d_a * sum_j q_j c_j + m_w * s_a     (s_a = the image's stored sum)
 * out[t][n] = sum_b term_b in float64, ascending b. qs layouts: Q8_0 [N][K/32][32] int8,
 * Q4_1 [N][K/32][16]; d (and m) fp16 [N][K/32].
 * ---------------------------------------------------------------------------------------- */
static int32_t block_dot_q8(const int8_t* q, const int8_t* c) {
  int32_t s = 0;
  for (int j = 0; j < 32; ++j) s += (int32_t)q[j] * c[j];
  return s;
}

void orc_mmvq_fmt(int fmt, const uint8_t* qs, const uint16_t* d, const uint16_t* m, int N, int K,
                  const uint8_t* img, int img_rows, int rows, double* out) {
  int Kb = K / 32, RB = orc_row_blocks(K);
  const int8_t* codes = (const int8_t*)img;
  const uint32_t* ds = (const uint32_t*)(img + (size_t)img_rows * RB * 32);
  for (int t = 0; t < rows; ++t)
    for (int n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int b = 0; b < Kb; ++b) {
        const int8_t* c = codes + ((size_t)t * RB + b) * 32;
        uint32_t w = ds[(size_t)t * RB + b];
        double da = orc_f16_to_f64((uint16_t)(w & 0xffffu));
        double sa = orc_f16_to_f64((uint16_t)(w >> 16));
        double dw = orc_f16_to_f64(d[(size_t)n * Kb + b]);
        if (fmt == 1) { /* Q8_0 */
          int32_t s = block_dot_q8((const int8_t*)qs + ((size_t)n * Kb + b) * 32, c);
          acc += dw * da * (double)s;
        } else { /* Q4_1 */
          int32_t s = block_dot(qs + ((size_t)n * Kb + b) * 16, c);
          double mw = orc_f16_to_f64(m[(size_t)n * Kb + b]);
          acc += dw * da * (double)s + mw * sa;
        }
      }
      out[(size_t)t * N + n] = acc;
    }
}

/* Ordinary reader: out[t][n] for t < rows (the live image rows), image of img_rows rows. */
void orc_mmvq(const uint8_t* qs, const uint16_t* d, int N, int K, const uint8_t* img, int img_rows,
              int rows, double* out) {
  int Kb = K / 32, RB = orc_row_blocks(K);
  const int8_t* codes = (const int8_t*)img;
  const uint32_t* ds = (const uint32_t*)(img + (size_t)img_rows * RB * 32);
  for (int t = 0; t < rows; ++t)
    for (int n = 0; n < N; ++n)
      out[(size_t)t * N + n] = reader_row(qs + (size_t)n * Kb * 16, d + (size_t)n * Kb, Kb,
                                          codes + (size_t)t * RB * 32, ds + (size_t)t * RB);
}

/* ------------------------------------------------------------------------------------------
 * Routed plan ("qwen3_5 CUDA: a captured bucket's padding rows no longer go through the routed
 * experts", What this changes and Receipt): only the first live rows' pairs p = row*top_k+slot
 * (row < live) are planned; the sum of the plan items' counts is live*top_k and the largest
 * member is below that; padding rows get no picks. The plan is a stable counting sort of the
 * live pairs by expert id: counts[E], offsets[E+1] (exclusive prefix), members grouped by
 * ascending expert and ascending p within an expert. Pairs naming an expert outside [0, E)
 * are left out; the function returns how many there were.
 * ---------------------------------------------------------------------------------------- */
int orc_plan(const int32_t* ids, int live, int top_k, int E, int32_t* counts, int32_t* offsets,
             int32_t* members) {
  int P = live * top_k, bad = 0;
  if (E <= 0) return P;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int p = 0; p < P; ++p) {
    int e = ids[p];
    if (e < 0 || e >= E) bad++;
    else counts[e]++;
  }
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* fill = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  for (int p = 0; p < P; ++p) {
    int e = ids[p];
    if (e < 0 || e >= E) continue;
    members[offsets[e] + fill[e]++] = p;
  }
  free(fill);
  return bad;
}

/* Routed reader: out[p][n] for live pairs p < live*top_k whose expert is in range; expert e's
 * weights are qs + e*N*Kb*16, d + e*N*Kb. The image row of pair p = (t, slot) is t for an
 * image of the tokens (one image shared by every slot), or p itself for a per-slot image (one
 * image row per pair, as a GLU producer over the routed gate/up outputs emits it for the down
 * projection: "Share temporary Q8_1 activation images", Overview and Coverage, per-slot
 * routed projections). Pairs with a bad expert are not written. */
static void mmvq_id_rows(const uint8_t* qs, const uint16_t* d, int E, int N, int K,
                         const uint8_t* img, int img_rows, const int32_t* ids, int live,
                         int top_k, int per_slot, double* out) {
  int Kb = K / 32, RB = orc_row_blocks(K);
  const int8_t* codes = (const int8_t*)img;
  const uint32_t* ds = (const uint32_t*)(img + (size_t)img_rows * RB * 32);
  for (int p = 0; p < live * top_k; ++p) {
    int e = ids[p], t = per_slot ? p : p / top_k;
    if (e < 0 || e >= E) continue;
    const uint8_t* qe = qs + (size_t)e * N * Kb * 16;
    const uint16_t* de = d + (size_t)e * N * Kb;
    for (int n = 0; n < N; ++n)
      out[(size_t)p * N + n] = reader_row(qe + (size_t)n * Kb * 16, de + (size_t)n * Kb, Kb,
                                          codes + (size_t)t * RB * 32, ds + (size_t)t * RB);
  }
}

void orc_mmvq_id(const uint8_t* qs, const uint16_t* d, int E, int N, int K, const uint8_t* img,
                 int img_rows, const int32_t* ids, int live, int top_k, double* out) {
  mmvq_id_rows(qs, d, E, N, K, img, img_rows, ids, live, top_k, 0, out);
}

void orc_mmvq_id_per_slot(const uint8_t* qs, const uint16_t* d, int E, int N, int K,
                          const uint8_t* img, int img_rows, const int32_t* ids, int live,
                          int top_k, double* out) {
  mmvq_id_rows(qs, d, E, N, K, img, img_rows, ids, live, top_k, 1, out);
}

/* ------------------------------------------------------------------------------------------
 * Device router and top-k with live-row guards ("qwen3_5 CUDA: a captured bucket's padding rows
 * no longer go through the routed experts", What this changes: the router and the top-k read
 * the live count and skip the padding rows, which get no picks; Receipt: router, top-k, plan,
 * experts, combine as one routed chain).
 *
 * Router: logits[t][e] = sum_k x[t][k] * W[e][k] for live rows t, in a fixed order (the pages
 * give none), the order of the RMS sum of squares with products for squares: leaf c (c < K/4)
 * = fma(x3,w3, fma(x2,w2, fma(x1,w1, x0*w0))) over elements 4c..4c+3; lane l in [0,64) owns
 * leaves c = l + 64 j, j < J' (J' = next power of two >= ceil(K/256); a missing leaf is +0)
 * and sums them by a balanced pairwise tree over j; the 64 lane sums by a balanced pairwise
 * tree over l. (A pairwise tree over j lets a row's K range be split over several waves on
 * subtree boundaries without changing a bit.)
 * ---------------------------------------------------------------------------------------- */
float orc_router_dot(const float* x, const float* w, int K) {
  int C = K / 4;
  int J = (K + 255) / 256;
  int Jp = 1;
  while (Jp < J) Jp <<= 1;
  float lane_sum[64];
  float* v = (float*)malloc(sizeof(float) * (size_t)Jp);
  for (int l = 0; l < 64; ++l) {
    for (int j = 0; j < Jp; ++j) {
      int c = l + 64 * j;
      if (c < C) {
        const float* a = x + 4 * c;
        const float* b = w + 4 * c;
        v[j] = fmaf(a[3], b[3], fmaf(a[2], b[2], fmaf(a[1], b[1], a[0] * b[0])));
      } else {
        v[j] = 0.0f;
      }
    }
    lane_sum[l] = pairwise_tree(v, Jp);
  }
  free(v);
  return pairwise_tree(lane_sum, 64);
}

void orc_moe_router(const float* x, int64_t ldx, const float* w, int E, int live, int K,
                    float* logits, int64_t ldl) {
  for (int t = 0; t < live; ++t)
    for (int e = 0; e < E; ++e)
      logits[(int64_t)t * ldl + e] = orc_router_dot(x + (int64_t)t * ldx, w + (int64_t)e * K, K);
}

/* Top-k: for each live row, the k largest logits in descending order, a tie going to the lower
 * expert id (selection: each round takes the best expert not yet taken). Routing weights are
 * the softmax over the selected logits, in f32 with exp_q:
 *   m = l_0 (the largest), e_r = exp_q(l_r - m), s = e_0 + e_1 + ... (ascending r, from +0),
 *   w_r = e_r / s.
 * Logits of live rows must not be NaN. weights may be NULL. */
void orc_moe_topk(const float* logits, int64_t ldl, int E, int live, int k, int32_t* ids,
                  float* weights) {
  unsigned char* taken = (unsigned char*)malloc((size_t)E);
  float* ev = (float*)malloc(sizeof(float) * (size_t)k);
  for (int t = 0; t < live; ++t) {
    const float* l = logits + (int64_t)t * ldl;
    memset(taken, 0, (size_t)E);
    for (int r = 0; r < k; ++r) {
      int best = -1;
      for (int e = 0; e < E; ++e)
        if (!taken[e] && (best < 0 || l[e] > l[best])) best = e;
      taken[best] = 1;
      ids[(int64_t)t * k + r] = best;
    }
    if (weights) {
      float m = l[ids[(int64_t)t * k]];
      float sum = 0.0f;
      for (int r = 0; r < k; ++r) {
        ev[r] = orc_exp_q(l[ids[(int64_t)t * k + r]] - m);
        sum = sum + ev[r];
      }
      for (int r = 0; r < k; ++r) weights[(int64_t)t * k + r] = ev[r] / sum;
    }
  }
  free(ev);
  free(taken);
}

/* ------------------------------------------------------------------------------------------
 * MoE combine of the routed expert outputs with the routing weights, for live rows only
 * ("qwen3_5 CUDA: a captured bucket's padding rows no longer go through the routed experts",
 * What this changes: padding rows get no combine work and their output rows stay unwritten).
 * out[t][n] = sum over slots s = 0 .. top_k-1 whose expert ids[t][s] is in [0, E) of
 * w[t][s] * x[t][s][n]. The pages fix no arithmetic for the sum; the reading taken here is one
 * f32 fused multiply-add per slot in ascending slot order, from +0:
 *   acc = +0; acc = fmaf(w[t][s], x[t][s][n], acc).
 * x is [rows][top_k][ld_pair] f32, w and ids are [rows][top_k]. Rows t >= live are not touched.
 * ---------------------------------------------------------------------------------------- */
void orc_moe_combine(const float* x, int64_t ld_pair, const float* w, const int32_t* ids, int E,
                     int live, int top_k, int N, float* out, int64_t ldo) {
  for (int t = 0; t < live; ++t)
    for (int n = 0; n < N; ++n) {
      float acc = 0.0f;
      for (int s = 0; s < top_k; ++s) {
        int p = t * top_k + s;
        if (ids[p] < 0 || ids[p] >= E) continue;
        acc = fmaf(w[p], x[(int64_t)p * ld_pair + n], acc);
      }
      out[(int64_t)t * ldo + n] = acc;
    }
}
