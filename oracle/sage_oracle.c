/*
 * sage_oracle.c -- plain, slow CPU oracle for the SageAttention-style quantized
 * attention forward (INT8 per-block Q/K with K smoothing, INT8 QK^T with int32
 * accumulation, fp32 online softmax, FP8 (e4m3) P~ and per-channel-scaled FP8 V,
 * two-level P~V accumulation).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the reference the GPU path is checked
 * against.  Only the test suite, the package smoke check and the benchmark's CPU
 * baseline leg may load it.  It shares no code, header, table or constant
 * generator with the HIP implementation.
 *
 * Sources (web pages, cited by title and section):
 *  [SA]   "SageAttention: Accurate 8-Bit Attention for Plug-and-play Inference
 *         Acceleration", abstract on the dblp author listing (taxoreview.com):
 *         8-bit quantized attention.
 *  [SA2]  The SageAttention2 abstract on the same listing: (P~, V) quantized to
 *         FP8 and a two-level accumulation strategy for P~V.
 *  [BLOG] "Flash Attention vs Sage Attention: Kernel Comparison", sections
 *         "How FlashAttention reduces memory traffic" (tiled online softmax) and
 *         "How SageAttention uses quantization for more throughput" (Q, K to
 *         8-bit before the matmul, then precision-aware scaling); "Attention
 *         kernel benchmarks: speed and memory use" (with a causal mask, the
 *         key blocks wholly after a query block need no work); "FlashAttention
 *         for training and inference: where SageAttention fits" (decode
 *         against a KV cache is bound by reading the cache: the split-KV
 *         form).
 *  [SA3]  The SageAttention3 abstract on the dblp listing: attention on FP4
 *         matrix cores (the 4-bit QK^T variant).
 *  [SA2] also: Q smoothing for the low-bit QK^T (the smoothed 4-bit variant).
 * The concrete arithmetic (K smoothing by the per-channel mean, INT8 per-block
 * Q/K, int32 QK^T, fp32 online softmax, FP8 V with per-channel scales, two-level
 * accumulation) is the method statement followed here; every rounding
 * step that the pages leave open is a stated reading, listed with the design
 * notes.
 *
 * Arithmetic hygiene: build with -ffp-contract=off and without -ffast-math.
 * fp32 operations are IEEE binary32 round-to-nearest-even; the only fused
 * multiply-adds are the explicit fmaf() calls.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Input decoding: IEEE binary16 and bfloat16 to binary32 (both exact).      */
/* ------------------------------------------------------------------------ */
static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

static float half_to_float(uint16_t h) {
  int s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
  float v;
  if (e == 0) v = ldexpf((float)m, -24);                 /* zero / subnormal: m * 2^-24 */
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexpf((float)(1024 + m), e - 25);             /* (1 + m/1024) * 2^(e-15) */
  return s ? -v : v;
}
static float bf16_to_float(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

/* dtype: 0 = float16, 1 = bfloat16 */
static float load_in(const uint16_t* x, size_t idx, int dtype) {
  return dtype == 0 ? half_to_float(x[idx]) : bf16_to_float(x[idx]);
}

/* ------------------------------------------------------------------------ */
/* OCP FP8 E4M3 ("e4m3fn"): sign, 4-bit exponent (bias 7), 3-bit mantissa;   */
/* normals (1 + m/8) 2^(e-7), subnormals (m/8) 2^-6, no infinities, S.1111.111 */
/* is NaN, largest finite 448.  Encoding: round to nearest, ties to even,     */
/* saturating to +-448.  ([SA2] abstract: P~ and V are quantized to FP8.)     */
/* ------------------------------------------------------------------------ */
double oracle_e4m3_decode(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m, -9);
  else v = ldexp(8.0 + m, e - 10);
  return s ? -v : v;
}

uint8_t oracle_e4m3_encode(float x) {
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  double a = fabs((double)x);
  if (isnan(x)) return 0x7F;
  if (a >= 448.0) return sign | 0x7E;                     /* saturate to the largest finite */
  if (a < 0x1p-6) {
    /* subnormal range: grid step 2^-9; r = 8 lands on the smallest normal 0x08 */
    double r = rint(a * 512.0);                            /* exact scaling, ties to even */
    return sign | (uint8_t)r;
  }
  int ex;
  frexp(a, &ex);                                           /* a = fr * 2^ex, fr in [0.5, 1) */
  int k = ex - 1;                                          /* a in [2^k, 2^(k+1)), k >= -6 */
  double r = rint(ldexp(a, 3 - k));                        /* significand in eighths: 8..16 */
  if (r == 16.0) { k += 1; r = 8.0; }                      /* rounded up into the next binade */
  return sign | (uint8_t)(((k + 7) << 3) | ((int)r - 8));
}

/* batch helpers for tests */
void oracle_e4m3_encode_n(const float* x, uint8_t* out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = oracle_e4m3_encode(x[i]);
}
void oracle_e4m3_decode_n(const uint8_t* c, double* out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = oracle_e4m3_decode(c[i]);
}

/* ------------------------------------------------------------------------ */
/* exp2 of the fp32 online softmax ([BLOG] "How FlashAttention reduces       */
/* memory traffic": the softmax is evaluated tile by tile in fp32; folding  */
/* log2 e into the score scale turns exp into exp2).  The argument is an    */
/* fp32 value; 2^t is evaluated in double precision and rounded once to     */
/* fp32 (a result below the fp32 subnormal range rounds to 0, -inf gives    */
/* 0).  The pages fix no cheaper approximation, so none is taken here.      */
/* ------------------------------------------------------------------------ */
float oracle_exp2f(float t) { return (float)exp2((double)t); }

void oracle_exp2f_n(const float* t, float* out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = oracle_exp2f(t[i]);
}

/* ------------------------------------------------------------------------ */
/* Step 1: per-channel mean of K over all N tokens of a head (smoothing K).  */
/* Fixed point, order-free: s = sum_t trunc(clamp(k, +-2^19) * 2^24) in      */
/* int64, mu = float(double(s) * 2^-24 / N).  Exact for float16 inputs;      */
/* each term is at most 2^43 in magnitude, so with N <= 2^19 tokens the sum  */
/* stays within 2^62 (no int64 overflow, even when every token saturates);   */
/* for bfloat16 only bits below 2^-24 of tiny elements are dropped.  Any     */
/* shift vector leaves softmax(QK^T) unchanged; the fixed-point sum makes     */
/* the vector independent of summation order.                                */
/* ------------------------------------------------------------------------ */
/* FP4 (E2M1) and its microscaled blocks, for the 4-bit QK^T variant (the   */
/* SageAttention3 abstract: attention on FP4 tensor cores; here the FP4     */
/* matrix instruction of the target takes E2M1 values with one power-of-two */
/* scale per 32 values along the contraction).                              */
/* E2M1 magnitudes by code 0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6; bit 3 is the    */
/* sign.  Encoding rounds to the nearest magnitude, ties to the code with    */
/* an even last bit, and saturates at 6.                                     */
/* ------------------------------------------------------------------------ */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double oracle_e2m1_decode(uint8_t c) {
  const double m = E2M1_MAG[c & 7];
  return (c & 8) ? -m : m;
}

uint8_t oracle_e2m1_encode(float x) {
  const double a = fabs((double)x);
  int best = 0;
  for (int k = 1; k < 8; k++) {
    const double dk = fabs(a - E2M1_MAG[k]), db = fabs(a - E2M1_MAG[best]);
    if (dk < db || (dk == db && (k & 1) == 0)) best = k;
  }
  return (uint8_t)(best | (signbit(x) ? 8 : 0));
}

/* One block of n values (n <= 32): shared exponent E = floor(log2(max|x|)) - 2
 * (2 = the largest E2M1 exponent), clamped to [-127, 127]; codes =
 * E2M1(x / 2^E); stored scale = E + 127 (an E8M0 byte).  An all-zero block
 * gets scale byte 0 and zero codes. */
static void quant_block_mx4(const float* x, int n, uint8_t* codes, uint8_t* scale) {
  float a = 0.0f;
  for (int k = 0; k < n; k++) a = fmaxf(a, fabsf(x[k]));
  if (a == 0.0f) {
    *scale = 0;
    for (int k = 0; k < n; k++) codes[k] = 0;
    return;
  }
  int e = (int)floor(log2((double)a)) - 2;
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  *scale = (uint8_t)(e + 127);
  for (int k = 0; k < n; k++) codes[k] = oracle_e2m1_encode((float)ldexp((double)x[k], -e));
}

void oracle_e2m1_encode_n(const float* x, uint8_t* out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = oracle_e2m1_encode(x[i]);
}

/* ------------------------------------------------------------------------ */
static const double KMEAN_CLAMP = 524288.0;  /* 2^19 */

static void kmean_head(const uint16_t* K, int dtype, int N, int d, float* mu, int64_t* sums_out) {
  for (int c = 0; c < d; c++) {
    int64_t s = 0;
    for (int t = 0; t < N; t++) {
      double x = (double)load_in(K, (size_t)t * d + c, dtype);
      if (x > KMEAN_CLAMP) x = KMEAN_CLAMP;
      if (x < -KMEAN_CLAMP) x = -KMEAN_CLAMP;
      s += (int64_t)trunc(x * 16777216.0);
    }
    if (sums_out) sums_out[c] = s;
    mu[c] = (float)(((double)s * 0x1p-24) / (double)N);
  }
}

/* ------------------------------------------------------------------------ */
/* Step 2: symmetric INT8 block quantizer ([SA] abstract; [BLOG] "How        */
/* SageAttention uses quantization").  One scale per block of tokens:        */
/*   a = max |x| over the block; if a < 2^-120 the block is zero (d=r=0);     */
/*   delta = RN(a / 127), r = RN(127 / a), code = rint(RN(x * r)) in [-127,127]*/
/* ------------------------------------------------------------------------ */
static void quant_block_i8(const float* x, size_t n, int8_t* codes, float* delta) {
  float a = 0.0f;
  for (size_t k = 0; k < n; k++) { float v = fabsf(x[k]); if (v > a) a = v; }
  if (a < 0x1p-120f) {
    *delta = 0.0f;
    for (size_t k = 0; k < n; k++) codes[k] = 0;
    return;
  }
  float dl = a / 127.0f;
  float r = 127.0f / a;
  *delta = dl;
  for (size_t k = 0; k < n; k++) {
    float y = rintf(x[k] * r);
    if (y > 127.0f) y = 127.0f;
    if (y < -127.0f) y = -127.0f;
    codes[k] = (int8_t)y;
  }
}

/* Q, K: [BH, N, d] (float16/bfloat16 raw bits).  Outputs: q_codes, k_codes
 * [BH, N, d] int8; q_scale [BH, ceil(N/blk_q)]; k_scale [BH, ceil(N/blk_k)];
 * k_mean [BH, d].  Blocks are consecutive runs of blk tokens from token 0;
 * when blk does not divide N the last block holds the N mod blk remaining
 * tokens.  Returns 0, or -1 for a shape the method does not define. */
static int nblocks(int N, int blk) { return (N + blk - 1) / blk; }
static int block_len(int N, int blk, int b) { return (b + 1) * blk <= N ? blk : N - b * blk; }

/* Q: blocks of blk_q tokens of one head, all d channels.  Q tensor [BH, N, d]. */
int oracle_quantize_q(const uint16_t* Q, int dtype, int BH, int N, int d, int blk_q, int8_t* q_codes,
                      float* q_scale) {
  if (BH < 1 || N < 1 || d < 1 || blk_q < 1) return -1;
  int nbq = nblocks(N, blk_q);
#pragma omp parallel for schedule(dynamic)
  for (int bh = 0; bh < BH; bh++) {
    const uint16_t* Qh = Q + (size_t)bh * N * d;
    float* buf = (float*)malloc(sizeof(float) * (size_t)blk_q * d);
    for (int b = 0; b < nbq; b++) {
      const size_t n = (size_t)block_len(N, blk_q, b) * d;
      for (size_t k = 0; k < n; k++) buf[k] = load_in(Qh, (size_t)b * blk_q * d + k, dtype);
      quant_block_i8(buf, n, q_codes + (size_t)bh * N * d + (size_t)b * blk_q * d, q_scale + (size_t)bh * nbq + b);
    }
    free(buf);
  }
  return 0;
}

/* K: per-head channel mean over all N tokens (step 1), then blocks of blk_k
 * tokens of the smoothed K.  K tensor [BH, N, d]. */
int oracle_quantize_k(const uint16_t* K, int dtype, int BH, int N, int d, int blk_k, int8_t* k_codes,
                      float* k_scale, float* k_mean) {
  if (BH < 1 || N < 1 || d < 1 || blk_k < 1) return -1;
  int nbk = nblocks(N, blk_k);
#pragma omp parallel for schedule(dynamic)
  for (int bh = 0; bh < BH; bh++) {
    const uint16_t* Kh = K + (size_t)bh * N * d;
    float* mu = k_mean + (size_t)bh * d;
    kmean_head(Kh, dtype, N, d, mu, NULL);
    float* buf = (float*)malloc(sizeof(float) * (size_t)blk_k * d);
    for (int b = 0; b < nbk; b++) {
      const int len = block_len(N, blk_k, b);
      for (int t = 0; t < len; t++)
        for (int c = 0; c < d; c++) {
          size_t idx = (size_t)(b * blk_k + t) * d + c;
          buf[(size_t)t * d + c] = load_in(Kh, idx, dtype) - mu[c];   /* smoothed K, fp32 */
        }
      quant_block_i8(buf, (size_t)len * d, k_codes + (size_t)bh * N * d + (size_t)b * blk_k * d,
                     k_scale + (size_t)bh * nbk + b);
    }
    free(buf);
  }
  return 0;
}

/* Q and K of the same shape [BH, N, d] */
int oracle_quantize_qk(const uint16_t* Q, const uint16_t* K, int dtype, int BH, int N, int d,
                       int blk_q, int blk_k, int8_t* q_codes, float* q_scale, int8_t* k_codes,
                       float* k_scale, float* k_mean) {
  if (oracle_quantize_q(Q, dtype, BH, N, d, blk_q, q_codes, q_scale)) return -1;
  return oracle_quantize_k(K, dtype, BH, N, d, blk_k, k_codes, k_scale, k_mean);
}

/* exported for tests: the int64 fixed-point channel sums and the mean */
int oracle_kmean(const uint16_t* K, int dtype, int BH, int N, int d, float* mu, int64_t* sums) {
  if (BH < 1 || N < 1 || d < 1) return -1;
  for (int bh = 0; bh < BH; bh++)
    kmean_head(K + (size_t)bh * N * d, dtype, N, d, mu + (size_t)bh * d, sums ? sums + (size_t)bh * d : NULL);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Step 3: V to FP8 with per-channel scales over all tokens of a head        */
/* ([SA2] abstract: V quantized to FP8).                                     */
/*   a_c = max_t |v[t,c]| (a_c < 2^-120: channel is zero),                   */
/*   delta_c = RN(a_c / 448), r_c = RN(448 / a_c), code = E(RN(v * r_c)).    */
/* Output codes in natural layout [BH, N, d].                                */
/* 4-bit Q and K: every token row of d channels in blocks of 32 channels,    */
/* each block its own shared exponent (quant_block_mx4).  K is smoothed     */
/* first, exactly as for the INT8 path (same mean, fp32 subtraction).        */
/* Codes: one E2M1 code per value [BH, N, d]; scales [BH, N, d/32] (E8M0).   */
int oracle_quantize_q4(const uint16_t* Q, int dtype, int BH, int N, int d, uint8_t* q4_codes, uint8_t* q4_scale) {
  if (BH < 1 || N < 1 || d < 32 || d % 32) return -1;
#pragma omp parallel for schedule(dynamic)
  for (int bh = 0; bh < BH; bh++) {
    float buf[32];
    for (int n = 0; n < N; n++)
      for (int b = 0; b < d / 32; b++) {
        const size_t r = ((size_t)bh * N + n);
        for (int k = 0; k < 32; k++) buf[k] = load_in(Q, r * d + 32 * b + k, dtype);
        quant_block_mx4(buf, 32, q4_codes + r * d + 32 * b, q4_scale + r * (d / 32) + b);
      }
  }
  return 0;
}

/* Q smoothing for the 4-bit scores (SageAttention2 abstract: Q is smoothed */
/* to make the low-bit QK^T accurate; no block or precision given).         */
/* Reading: the queries of a head are cut into blocks of 32 consecutive     */
/* rows (the last block holds the N mod 32 remaining rows); the block mean   */
/* qm[c] = fp32(S / n), S the fp64 sum of the block's rows in ascending row  */
/* order; each row is quantized as RN(q - qm) in the E2M1 blocks above.  The */
/* removed part returns in the scores as qm . k (see score4), with qm and  */
/* the smoothed K both in INT8 with one power-of-two scale per block        */
/* (quant_int8_pow2): qm per 32-query block over all d channels, K per      */
/* block of 64 consecutive keys (the last block holds the rest) over all d  */
/* channels (oracle_quantize_k8).  8-bit, since qm can be large and 4-bit K */
/* codes would carry their error into the product; integer, so that the    */
/* term is an exact integer sum times 2^(Em + Ek).                          */
/* Outputs: q4 codes/scales as oracle_quantize_q4; q_mean [BH, nb, d] fp32, */
/* qm_codes [BH, nb, d] int8, qm_scale [BH, nb] exponent bytes; nb =        */
/* ceil(N/32).                                                               */

/* n values with one power-of-two scale 2^E for INT8 codes: E = the smallest */
/* exponent in [-63, 52] with max|x| * 2^-E <= 127 (an all-zero block gets  */
/* -63); codes = RN(x * 2^-E), ties to even, saturated at +-127 (reached    */
/* only at the upper clamp); scale byte E + 127.                             */
static void quant_int8_pow2(const float* x, size_t n, int8_t* codes, uint8_t* scale) {
  float a = 0.0f;
  for (size_t k = 0; k < n; k++) a = fmaxf(a, fabsf(x[k]));
  int e = -63;
  if (a != 0.0f) {
    e = ilogb((double)a) - 6;                       /* a * 2^-e in [64, 128) */
    if (ldexp((double)a, -e) > 127.0) e += 1;       /* then in [32, 64) */
    if (e < -63) e = -63;
    if (e > 52) e = 52;
  }
  *scale = (uint8_t)(e + 127);
  for (size_t k = 0; k < n; k++) {
    double y = nearbyint(ldexp((double)x[k], -e));   /* exact scaling, ties to even */
    if (y > 127.0) y = 127.0;
    if (y < -127.0) y = -127.0;
    codes[k] = (int8_t)y;
  }
}

int oracle_quantize_q4_smooth(const uint16_t* Q, int dtype, int BH, int N, int d, uint8_t* q4_codes,
                              uint8_t* q4_scale, float* q_mean, int8_t* qm_codes, uint8_t* qm_scale) {
  if (BH < 1 || N < 1 || d < 32 || d % 32) return -1;
  const int nb = (N + 31) / 32;
#pragma omp parallel for schedule(dynamic)
  for (int bh = 0; bh < BH; bh++) {
    float buf[32];
    for (int blk = 0; blk < nb; blk++) {
      const int n0 = 32 * blk, n = (N - n0 < 32) ? N - n0 : 32;
      float* qm = q_mean + ((size_t)bh * nb + blk) * d;
      for (int c = 0; c < d; c++) {
        double sum = 0.0;
        for (int i = 0; i < n; i++) sum += (double)load_in(Q, ((size_t)bh * N + n0 + i) * d + c, dtype);
        qm[c] = (float)(sum / n);
      }
      quant_int8_pow2(qm, (size_t)d, qm_codes + ((size_t)bh * nb + blk) * d, qm_scale + (size_t)bh * nb + blk);
      for (int i = 0; i < n; i++)
        for (int b = 0; b < d / 32; b++) {
          const size_t r = (size_t)bh * N + n0 + i;
          for (int k = 0; k < 32; k++) buf[k] = load_in(Q, r * d + 32 * b + k, dtype) - qm[32 * b + k];
          quant_block_mx4(buf, 32, q4_codes + r * d + 32 * b, q4_scale + r * (d / 32) + b);
        }
    }
  }
  return 0;
}

/* The smoothed K (the same mean and fp32 subtraction as oracle_quantize_k4) */
/* in INT8 blocks of 64 keys x d channels, one power-of-two scale each:      */
/* k8_codes [BH, N, d] int8, k8_scale [BH, ceil(N/64)] exponent bytes.       */
int oracle_quantize_k8(const uint16_t* K, int dtype, int BH, int N, int d, int8_t* k8_codes, uint8_t* k8_scale) {
  if (BH < 1 || N < 1 || d < 32 || d % 32) return -1;
  const int nkb = (N + 63) / 64;
#pragma omp parallel for schedule(dynamic)
  for (int bh = 0; bh < BH; bh++) {
    float* mu = (float*)malloc(sizeof(float) * d);
    float* buf = (float*)malloc(sizeof(float) * 64 * d);
    kmean_head(K + (size_t)bh * N * d, dtype, N, d, mu, NULL);
    for (int blk = 0; blk < nkb; blk++) {
      const int n0 = 64 * blk, n = (N - n0 < 64) ? N - n0 : 64;
      for (int i = 0; i < n; i++)
        for (int c = 0; c < d; c++) buf[(size_t)i * d + c] = load_in(K, ((size_t)bh * N + n0 + i) * d + c, dtype) - mu[c];
      quant_int8_pow2(buf, (size_t)n * d, k8_codes + ((size_t)bh * N + n0) * d, k8_scale + (size_t)bh * nkb + blk);
    }
    free(buf);
    free(mu);
  }
  return 0;
}

int oracle_quantize_k4(const uint16_t* K, int dtype, int BH, int N, int d, uint8_t* k4_codes, uint8_t* k4_scale,
                       float* k_mean) {
  if (BH < 1 || N < 1 || d < 32 || d % 32) return -1;
#pragma omp parallel for schedule(dynamic)
  for (int bh = 0; bh < BH; bh++) {
    float* mu = k_mean + (size_t)bh * d;
    kmean_head(K + (size_t)bh * N * d, dtype, N, d, mu, NULL);
    float buf[32];
    for (int n = 0; n < N; n++)
      for (int b = 0; b < d / 32; b++) {
        const size_t r = ((size_t)bh * N + n);
        for (int k = 0; k < 32; k++) buf[k] = load_in(K, r * d + 32 * b + k, dtype) - mu[32 * b + k];
        quant_block_mx4(buf, 32, k4_codes + r * d + 32 * b, k4_scale + r * (d / 32) + b);
      }
  }
  return 0;
}

/* 4-bit V for the FP4 P~V variant (R23), following the OCP Microscaling     */
/* (MX) formats' MXFP4 (E2M1 elements, one E8M0 scale per block of 32): each */
/* channel of a head in blocks of 32 consecutive tokens (the last block holds */
/* the N mod 32 remaining tokens), each block its own shared exponent        */
/* (quant_block_mx4, the rule of the 4-bit Q and K).                          */
/* Codes one per value [BH, N, d] (0..15); scales [BH, ceil(N/32), d].       */
int oracle_quantize_v4(const uint16_t* V, int dtype, int BH, int N, int d, uint8_t* v4_codes, uint8_t* v4_scale) {
  if (BH < 1 || N < 1 || d < 1) return -1;
  const int nb = (N + 31) / 32;
#pragma omp parallel for schedule(dynamic)
  for (int bh = 0; bh < BH; bh++) {
    float buf[32];
    uint8_t cod[32];
    for (int blk = 0; blk < nb; blk++) {
      const int n0 = 32 * blk, n = (N - n0 < 32) ? N - n0 : 32;
      for (int c = 0; c < d; c++) {
        for (int i = 0; i < n; i++) buf[i] = load_in(V, ((size_t)bh * N + n0 + i) * d + c, dtype);
        quant_block_mx4(buf, n, cod, v4_scale + ((size_t)bh * nb + blk) * d + c);
        for (int i = 0; i < n; i++) v4_codes[((size_t)bh * N + n0 + i) * d + c] = cod[i];
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
int oracle_quantize_v(const uint16_t* V, int dtype, int BH, int N, int d, uint8_t* v_codes, float* v_scale) {
  if (BH < 1 || N < 1 || d < 1) return -1;
#pragma omp parallel for schedule(dynamic)
  for (int bh = 0; bh < BH; bh++) {
    const uint16_t* Vh = V + (size_t)bh * N * d;
    for (int c = 0; c < d; c++) {
      float a = 0.0f;
      for (int t = 0; t < N; t++) { float v = fabsf(load_in(Vh, (size_t)t * d + c, dtype)); if (v > a) a = v; }
      float dl = 0.0f, r = 0.0f;
      if (a >= 0x1p-120f) { dl = a / 448.0f; r = 448.0f / a; }
      v_scale[(size_t)bh * d + c] = dl;
      for (int t = 0; t < N; t++) {
        float v = load_in(Vh, (size_t)t * d + c, dtype);
        v_codes[(size_t)bh * N * d + (size_t)t * d + c] = (a >= 0x1p-120f) ? oracle_e4m3_encode(v * r) : 0;
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Head sharing: query head h of batch b reads key/value head h / (Hq/Hkv)   */
/* of the same batch (one head each when Hq = Hkv; grouped-query attention   */
/* otherwise).  The flat index of that head among the B*Hkv K/V heads:       */
/* ------------------------------------------------------------------------ */
static int64_t kv_head(int64_t bh, int Hq, int Hkv) {
  return (bh / Hq) * Hkv + (bh % Hq) / (Hq / Hkv);
}

/* ------------------------------------------------------------------------ */
/* Step 4 (diagnostic): exact int32 S = q_codes . k_codes over d for chosen   */
/* query rows against every key of the K/V head they read.  Q codes          */
/* [B*Hq, Nq, d], K codes [B*Hkv, Nkv, d]; rows[] are flat indices bh*Nq + i */
/* out: [nrows, Nkv].                                                        */
/* ------------------------------------------------------------------------ */
void oracle_qk_int32(const int8_t* q_codes, const int8_t* k_codes, int B, int Hq, int Hkv, int Nq, int Nkv,
                     int d, const int64_t* rows, int nrows, int32_t* out) {
  (void)B;
#pragma omp parallel for schedule(static)
  for (int r = 0; r < nrows; r++) {
    int64_t bh = rows[r] / Nq, i = rows[r] % Nq, bk = kv_head(bh, Hq, Hkv);
    const int8_t* q = q_codes + ((size_t)bh * Nq + i) * d;
    for (int j = 0; j < Nkv; j++) {
      const int8_t* k = k_codes + ((size_t)bk * Nkv + j) * d;
      int32_t s = 0;
      for (int c = 0; c < d; c++) s += (int32_t)q[c] * (int32_t)k[c];
      out[(size_t)r * Nkv + j] = s;
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Steps 4-8: attention for chosen query rows.  For row i of head bh, KV      */
/* tiles of kv_tile keys (the last one shorter when kv_tile does not divide */
/* Nkv) are visited in ascending order, one pass, as in the                  */
/* tiled online softmax ([BLOG] "How FlashAttention reduces memory            */
/* traffic"); tiles with no visible key (causal) are skipped ([BLOG] causal   */
/* masking changes which blocks are skipped).  Causal visibility is aligned */
/* at the end of the sequences: key j is visible to query i iff             */
/* j <= i + (Nkv - Nq) (the usual top-left rule when Nq = Nkv).  Per tile:  */
/*   S_j   = sum_c q_c k_c                       (int32, exact)              */
/*   c2_j  = RN(RN(dQ * dK_j) * s2),  s2 = RN(sm_scale * log2 e)             */
/*   u_j   = RN(float(S_j) * c2_j);  m' = max(m, max_j u_j)                  */
/*   alpha = exp2f(RN(m - m'))   (0 on the first visited tile)               */
/*   INT8 scores, with B = 1.5 * 2^23 (B + S_j is exact in fp32):           */
/*     K_j   = RN(B * c2_j + RN(m' - 8))        (one fused multiply-add)     */
/*     P~_j  = exp2f(RN((B + S_j) * c2_j - K_j)) (one fused multiply-add)    */
/*     i.e. exp2 of RN(S_j c2_j - (m' - 8)) with the offset m' - 8 rounded   */
/*     to fp32 at the magnitude of B c2_j (a shift of the whole tile's       */
/*     exponents by at most one unit of S_j times c2_j)                      */
/*     rowsum = RN(sum_j dec(P^_j))              (the FP8 codes, exact sum)  */
/*   4-bit scores: P~_j = exp2f(fma(S_j, c2_j, -RN(m' - 8)));                */
/*     rowsum = sum_j P~_j                      (fp32, ascending keys)       */
/*   l     = fma(alpha, l, rowsum)               (fp32 state)                */
/*   P^_j  = E(P~_j)                             (FP8 e4m3; P~ scaled by 2^8) */
/*   Oblk_c = sum_j dec(P^_j) dec(v^_jc)             (inner level; exact     */
/*                                                    products, summed in    */
/*                                                    fp64, rounded to fp32) */
/*   Oacc_c = fma(alpha, Oacc_c, Oblk_c)             (outer fp32 level)      */
/*   m = m'                                                                  */
/* O_c = Oacc_c * deltaV_c / l.  ([SA2] abstract: two-level accumulation of  */
/* FP8 P~V.)  Q codes/scales of B*Hq heads of Nq tokens, K and V codes and  */
/* scales of B*Hkv heads of Nkv tokens (kv_head above); rows[] are flat     */
/* indices bh*Nq + i; out: [nrows, d] fp32; p_codes (optional):             */
/* [nrows, Nkv], 0 where a key is not visible.                               */
/* ------------------------------------------------------------------------ */
static const float LOG2E_F = 0x1.715476p+0f;   /* RN(log2 e) */
/* Offset of the INT8 scores in the exponent argument: 1.5 * 2^23, so that   */
/* B + S is an integer in [2^23, 2^24) for every |S| < 2^21, exact in fp32.  */
static const float SCORE_BIAS = 12582912.0f;

/* One query row against the keys of one K/V head (shared by the two entry  */
/* points below).                                                            */
typedef struct {
  const int8_t* q;        /* the row's d codes */
  float dq;               /* the row's Q scale */
  /* 4-bit QK^T instead (q4 != NULL): the row's E2M1 codes and block scales,
   * the head's K codes [Nkv, d] and scales [Nkv, d/32] */
  const uint8_t* q4;
  const uint8_t* q4s;
  const uint8_t* k4;
  const uint8_t* k4s;
  /* with Q smoothing (qm != NULL): the INT8 codes and the exponent byte of
   * the mean of the row's 32-query block, and the head's INT8 K codes
   * [Nkv, d] and exponent bytes [ceil(Nkv/64)] */
  const int8_t* qm;
  int qms;
  const int8_t* k8;
  const uint8_t* k8s;
  /* FP4 P~V instead of FP8 (v4 != NULL, R23): the head's V codes [Nkv, d]
   * (0..15) and block scales [ceil(Nkv/32), d] */
  const uint8_t* v4;
  const uint8_t* v4s;
  const int8_t* k;        /* the head's K codes [Nkv, d] */
  const float* ks;        /* the head's K scales [ceil(Nkv/blk_k)] */
  const uint8_t* v;       /* the head's V codes [Nkv, d] */
  int Nkv, d, blk_k, kv_tile;
  int64_t last;           /* last visible key (Nkv - 1 without the mask) */
  float s2;
  const double* vdec;     /* e4m3 decode table */
} row_ctx;

/* 4-bit score of the row against key j: the exact sum over the 32-channel   */
/* blocks of 2^(Eq + Ek) times the block's E2M1 dot product, plus with Q     */
/* smoothing the integer dot product of the block mean's INT8 codes with    */
/* the key's INT8 codes times 2^(Em + Ek8) (Ek8 of the key's 64-key block);  */
/* fp64, exact for the exponent spreads that occur, rounded once to fp32.   */
static float score4(const row_ctx* x, int j) {
  const int d = x->d;
  const uint8_t* k = x->k4 + (size_t)j * d;
  const uint8_t* ks = x->k4s + (size_t)j * (d / 32);
  double s = 0.0;
  for (int b = 0; b < d / 32; b++) {
    double blk = 0.0;
    for (int c = 32 * b; c < 32 * b + 32; c++) blk += oracle_e2m1_decode(x->q4[c]) * oracle_e2m1_decode(k[c]);
    s += ldexp(blk, (int)x->q4s[b] + (int)ks[b] - 254);
  }
  if (x->qm) {
    const int8_t* k8 = x->k8 + (size_t)j * d;
    int64_t dot = 0;
    for (int c = 0; c < d; c++) dot += (int64_t)x->qm[c] * (int64_t)k8[c];
    s += ldexp((double)dot, x->qms + (int)x->k8s[j / 64] - 254);
  }
  return (float)s;
}

/* The online softmax over the tiles j0 = j_begin, j_begin + kv_tile, ...    */
/* below j_end (j_begin a multiple of kv_tile), from a fresh state: returns  */
/* the number of visited tiles and leaves m, l and Oacc[d] (Oacc without the */
/* V scale).  prow (optional): FP8 codes of P~ of the visited keys, indexed  */
/* by key.                                                                   */
static int attend_range(const row_ctx* x, int j_begin, int j_end, float* m_out, float* l_out, float* oacc,
                        uint8_t* prow) {
  const int kv_tile = x->kv_tile, d = x->d;
  float* S = (float*)malloc(sizeof(float) * kv_tile);
  float* c2 = (float*)malloc(sizeof(float) * kv_tile);
  float* pt = (float*)malloc(sizeof(float) * kv_tile);
  uint8_t* ph = (uint8_t*)malloc(kv_tile);
  float* ag = (float*)malloc(sizeof(float) * kv_tile);
  double* pd = (double*)malloc(sizeof(double) * kv_tile);
  double* oblk = (double*)malloc(sizeof(double) * d);
  for (int c = 0; c < d; c++) oacc[c] = 0.0f;
  float m = 0.0f, l = 0.0f;
  int visited = 0;
  for (int j0 = j_begin; j0 < j_end; j0 += kv_tile) {
    if (j0 > x->last) break;   /* no visible key from here on */
    int nvis = j0 + kv_tile <= j_end ? kv_tile : j_end - j0;
    if (x->last - j0 + 1 < nvis) nvis = (int)(x->last - j0 + 1);
    /* scores of the visible keys j0 .. j0+nvis-1, as fp32 S and its factor c2 */
    float mt = -INFINITY;
    for (int jj = 0; jj < nvis; jj++) {
      int j = j0 + jj;
      if (x->q4) {
        S[jj] = score4(x, j);
        c2[jj] = x->s2;
      } else {
        const int8_t* k = x->k + (size_t)j * d;
        int32_t s = 0;
        for (int c = 0; c < d; c++) s += (int32_t)x->q[c] * (int32_t)k[c];
        S[jj] = (float)s;   /* exact: |s| < 2^24 */
        c2[jj] = (x->dq * x->ks[j / x->blk_k]) * x->s2;
      }
      float u = S[jj] * c2[jj];
      if (u > mt) mt = u;
    }
    const int first = visited == 0;
    float mnew = first ? mt : (mt > m ? mt : m);
    float alpha = first ? 0.0f : oracle_exp2f(m - mnew);
    float mm = mnew - 8.0f;
    float rowsum = 0.0f;
    double code_sum = 0.0;
    if (x->v4) {
      /* FP4 P~ (R23): the tile's keys in blocks of 32 (keys j0 .. j0+31 and  */
      /* j0+32 .. j0+63, visible ones only), each with the MX shared exponent */
      /* of its largest value taken on the exponent argument, E = floor(max   */
      /* arg) - 2 clamped to [-126, 127] (no visible key: -126); P^ = E2M1 of */
      /* P~ / 2^E, P~ below 2^-126 counted as 0; l_tile = sum of the decoded   */
      /* values P^ 2^E; the block product uses the same values.              */
      for (int b0 = 0; b0 < nvis; b0 += 32) {
        const int b1 = b0 + 32 < nvis ? b0 + 32 : nvis;
        float amax = -INFINITY;
        for (int jj = b0; jj < b1; jj++) {
          ag[jj] = fmaf(S[jj], c2[jj], -mm);
          if (ag[jj] > amax) amax = ag[jj];
        }
        float fe = floorf(amax) - 2.0f;
        if (!(fe >= -126.0f)) fe = -126.0f;
        if (fe > 127.0f) fe = 127.0f;
        const int e = (int)fe;
        for (int jj = b0; jj < b1; jj++) {
          float p = oracle_exp2f(ag[jj]);
          if (p < 0x1p-126f) p = 0.0f;
          pt[jj] = p;
          ph[jj] = oracle_e2m1_encode(ldexpf(p, -e));
          pd[jj] = ldexp(oracle_e2m1_decode(ph[jj]), e);
          code_sum += pd[jj];
          if (prow) prow[j0 + jj] = ph[jj];
        }
      }
      rowsum = (float)code_sum;   /* exact: 64 values of at most 4 significant bits */
      for (int c = 0; c < d; c++) {
        double acc = 0.0;
        for (int jj = 0; jj < nvis; jj++) {
          const int j = j0 + jj;
          acc += pd[jj] * ldexp(oracle_e2m1_decode(x->v4[(size_t)j * d + c]), (int)x->v4s[(size_t)(j / 32) * d + c] - 127);
        }
        oblk[c] = acc;
      }
    } else {
      for (int jj = 0; jj < nvis; jj++) {
        if (x->q4) {
          pt[jj] = oracle_exp2f(fmaf(S[jj], c2[jj], -mm));
          rowsum += pt[jj];
        } else {
          const float K = fmaf(SCORE_BIAS, c2[jj], mm);
          pt[jj] = oracle_exp2f(fmaf(SCORE_BIAS + S[jj], c2[jj], -K));
        }
        ph[jj] = oracle_e4m3_encode(pt[jj]);
        code_sum += x->vdec[ph[jj]];
        if (prow) prow[j0 + jj] = ph[jj];
      }
      if (!x->q4) rowsum = (float)code_sum;   /* exact: at most 2^10 codes per tile */
      for (int c = 0; c < d; c++) {
        double acc = 0.0;
        for (int jj = 0; jj < nvis; jj++) acc += x->vdec[ph[jj]] * x->vdec[x->v[(size_t)(j0 + jj) * d + c]];
        oblk[c] = acc;
      }
    }
    for (int c = 0; c < d; c++) oacc[c] = fmaf(alpha, oacc[c], (float)oblk[c]);
    l = fmaf(alpha, l, rowsum);
    m = mnew;
    visited++;
  }
  free(S); free(c2); free(pt); free(ph); free(ag); free(pd); free(oblk);
  *m_out = m;
  *l_out = l;
  return visited;
}

static int attn_args_ok(int B, int Hq, int Hkv, int Nq, int Nkv, int d, int blk_q, int blk_k, int kv_tile,
                        int causal, float sm_scale) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || Nq < 1 || Nkv < 1 || d < 1) return 0;
  if (blk_q < 1 || blk_k < 1 || kv_tile < 1) return 0;
  if (causal && Nkv < Nq) return 0;   /* the first queries would see no key */
  if (!(sm_scale > 0.0f) || isinf(sm_scale)) return 0;
  return 1;
}

static void row_setup(row_ctx* x, const int8_t* q_codes, const float* q_scale, const int8_t* k_codes,
                      const float* k_scale, const uint8_t* v_codes, int Hq, int Hkv, int Nq, int Nkv, int d,
                      int blk_q, int blk_k, int kv_tile, int causal, float sm_scale, int64_t row,
                      const double* vdec, int64_t* bk_out) {
  const int nbq = nblocks(Nq, blk_q), nbk = nblocks(Nkv, blk_k);
  int64_t bh = row / Nq, i = row % Nq, bk = kv_head(bh, Hq, Hkv);
  memset(x, 0, sizeof *x);   /* every optional pointer (4-bit, smoothing, FP4 V) NULL */
  x->q = q_codes + ((size_t)bh * Nq + i) * d;
  x->dq = q_scale[(size_t)bh * nbq + i / blk_q];
  x->k = k_codes + (size_t)bk * Nkv * d;
  x->ks = k_scale + (size_t)bk * nbk;
  x->v = v_codes + (size_t)bk * Nkv * d;
  x->Nkv = Nkv; x->d = d; x->blk_k = blk_k; x->kv_tile = kv_tile;
  x->last = causal ? i + ((int64_t)Nkv - Nq) : (int64_t)Nkv - 1;
  x->s2 = sm_scale * LOG2E_F;
  x->vdec = vdec;
  *bk_out = bk;
}

int oracle_attn_rows(const int8_t* q_codes, const float* q_scale, const int8_t* k_codes,
                     const float* k_scale, const uint8_t* v_codes, const float* v_scale, int B, int Hq,
                     int Hkv, int Nq, int Nkv, int d, int blk_q, int blk_k, int kv_tile, int causal,
                     float sm_scale, const int64_t* rows, int nrows, float* out, uint8_t* p_codes) {
  if (!attn_args_ok(B, Hq, Hkv, Nq, Nkv, d, blk_q, blk_k, kv_tile, causal, sm_scale)) return -1;
  double vdec[256];
  for (int c = 0; c < 256; c++) vdec[c] = oracle_e4m3_decode((uint8_t)c);
  for (int r = 0; r < nrows; r++)
    if (rows[r] < 0 || rows[r] >= (int64_t)B * Hq * Nq) return -1;
#pragma omp parallel for schedule(dynamic)
  for (int r = 0; r < nrows; r++) {
    row_ctx x;
    int64_t bk;
    row_setup(&x, q_codes, q_scale, k_codes, k_scale, v_codes, Hq, Hkv, Nq, Nkv, d, blk_q, blk_k, kv_tile, causal,
              sm_scale, rows[r], vdec, &bk);
    float* oacc = (float*)malloc(sizeof(float) * d);
    float m, l;
    uint8_t* prow = p_codes ? p_codes + (size_t)r * Nkv : NULL;
    if (prow) memset(prow, 0, Nkv);
    attend_range(&x, 0, Nkv, &m, &l, oacc, prow);
    for (int c = 0; c < d; c++)
      out[(size_t)r * d + c] = (float)(((double)oacc[c] * (double)v_scale[(size_t)bk * d + c]) / (double)l);
    free(oacc);
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* The same attention with 4-bit QK^T: scores from the E2M1 codes and block  */
/* scales of oracle_quantize_q4 / _k4 (score4), dequantization factor        */
/* c2 = s2 for every key (the block scales are inside the score); softmax,   */
/* FP8 P~ and the two-level P~V exactly as above.  Codes [B*H, N, d], scales */
/* [B*H, N, d/32]; out [nrows, d]; p_codes (optional) as above.              */
/* ------------------------------------------------------------------------ */
static int attn_rows_4bit(const uint8_t* q4_codes, const uint8_t* q4_scale, const uint8_t* k4_codes,
                          const uint8_t* k4_scale, const int8_t* qm_codes, const uint8_t* qm_scale,
                          const int8_t* k8_codes, const uint8_t* k8_scale, const uint8_t* v_codes,
                          const float* v_scale, const uint8_t* v4_codes, const uint8_t* v4_scale, int B, int Hq,
                          int Hkv, int Nq, int Nkv, int d, int kv_tile, int causal, float sm_scale,
                          const int64_t* rows, int nrows, float* out, uint8_t* p_codes) {
  if (!attn_args_ok(B, Hq, Hkv, Nq, Nkv, d, 1, 1, kv_tile, causal, sm_scale) || d % 32) return -1;
  double vdec[256];
  for (int c = 0; c < 256; c++) vdec[c] = oracle_e4m3_decode((uint8_t)c);
  for (int r = 0; r < nrows; r++)
    if (rows[r] < 0 || rows[r] >= (int64_t)B * Hq * Nq) return -1;
#pragma omp parallel for schedule(dynamic)
  for (int r = 0; r < nrows; r++) {
    const int64_t bh = rows[r] / Nq, i = rows[r] % Nq, bk = kv_head(bh, Hq, Hkv);
    row_ctx x;
    memset(&x, 0, sizeof x);
    x.q4 = q4_codes + ((size_t)bh * Nq + i) * d;
    x.q4s = q4_scale + ((size_t)bh * Nq + i) * (d / 32);
    x.k4 = k4_codes + (size_t)bk * Nkv * d;
    x.k4s = k4_scale + (size_t)bk * Nkv * (d / 32);
    if (qm_codes) {
      const int64_t blk = (bh * ((Nq + 31) / 32) + i / 32);
      x.qm = qm_codes + (size_t)blk * d;
      x.qms = qm_scale[blk];
      x.k8 = k8_codes + (size_t)bk * Nkv * d;
      x.k8s = k8_scale + (size_t)bk * ((Nkv + 63) / 64);
    }
    if (v4_codes) {
      x.v4 = v4_codes + (size_t)bk * Nkv * d;
      x.v4s = v4_scale + (size_t)bk * ((Nkv + 31) / 32) * d;
    } else {
      x.v = v_codes + (size_t)bk * Nkv * d;
    }
    x.Nkv = Nkv; x.d = d; x.blk_k = 1; x.kv_tile = kv_tile;
    x.last = causal ? i + ((int64_t)Nkv - Nq) : (int64_t)Nkv - 1;
    x.s2 = sm_scale * LOG2E_F;
    x.vdec = vdec;
    float* oacc = (float*)malloc(sizeof(float) * d);
    float m, l;
    uint8_t* prow = p_codes ? p_codes + (size_t)r * Nkv : NULL;
    if (prow) memset(prow, 0, Nkv);
    attend_range(&x, 0, Nkv, &m, &l, oacc, prow);
    for (int c = 0; c < d; c++)
      out[(size_t)r * d + c] = v4_codes ? (float)((double)oacc[c] / (double)l)
                                        : (float)(((double)oacc[c] * (double)v_scale[(size_t)bk * d + c]) / (double)l);
    free(oacc);
  }
  return 0;
}

int oracle_attn_rows_qk4(const uint8_t* q4_codes, const uint8_t* q4_scale, const uint8_t* k4_codes,
                         const uint8_t* k4_scale, const int8_t* qm_codes, const uint8_t* qm_scale,
                         const int8_t* k8_codes, const uint8_t* k8_scale, const uint8_t* v_codes,
                         const float* v_scale, int B, int Hq,
                         int Hkv, int Nq, int Nkv, int d, int kv_tile, int causal, float sm_scale,
                         const int64_t* rows, int nrows, float* out, uint8_t* p_codes) {
  return attn_rows_4bit(q4_codes, q4_scale, k4_codes, k4_scale, qm_codes, qm_scale, k8_codes, k8_scale, v_codes,
                        v_scale, NULL, NULL, B, Hq, Hkv, Nq, Nkv, d, kv_tile, causal, sm_scale, rows, nrows, out,
                        p_codes);
}

/* FP4 attention (R21 scores, R23 P~V): the 4-bit scores of oracle_attn_rows_qk4, */
/* P~ and V in E2M1 blocks of 32 with E8M0 scales (V from oracle_quantize_v4),   */
/* O = O_acc / l (the V scales are inside the products).  p_codes (optional):   */
/* the E2M1 code (0..15) of every visited key.                                   */
int oracle_attn_rows_fp4(const uint8_t* q4_codes, const uint8_t* q4_scale, const uint8_t* k4_codes,
                         const uint8_t* k4_scale, const uint8_t* v4_codes, const uint8_t* v4_scale, int B, int Hq,
                         int Hkv, int Nq, int Nkv, int d, int kv_tile, int causal, float sm_scale,
                         const int64_t* rows, int nrows, float* out, uint8_t* p_codes) {
  if (!v4_codes || !v4_scale || kv_tile % 32) return -1;
  return attn_rows_4bit(q4_codes, q4_scale, k4_codes, k4_scale, NULL, NULL, NULL, NULL, NULL, NULL, v4_codes,
                        v4_scale, B, Hq, Hkv, Nq, Nkv, d, kv_tile, causal, sm_scale, rows, nrows, out, p_codes);
}

/* fp32 4-bit scores (score4) of flat query rows bh*Nq + i against every key: [nrows, Nkv] */
int oracle_qk4_scores(const uint8_t* q4_codes, const uint8_t* q4_scale, const uint8_t* k4_codes,
                      const uint8_t* k4_scale, const int8_t* qm_codes, const uint8_t* qm_scale,
                      const int8_t* k8_codes, const uint8_t* k8_scale, int B, int Hq,
                      int Hkv, int Nq, int Nkv, int d, const int64_t* rows,
                      int nrows, float* out) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || d % 32) return -1;
#pragma omp parallel for schedule(dynamic)
  for (int r = 0; r < nrows; r++) {
    const int64_t bh = rows[r] / Nq, i = rows[r] % Nq, bk = kv_head(bh, Hq, Hkv);
    row_ctx x;
    memset(&x, 0, sizeof x);
    x.q4 = q4_codes + ((size_t)bh * Nq + i) * d;
    x.q4s = q4_scale + ((size_t)bh * Nq + i) * (d / 32);
    x.k4 = k4_codes + (size_t)bk * Nkv * d;
    x.k4s = k4_scale + (size_t)bk * Nkv * (d / 32);
    if (qm_codes) {
      const int64_t blk = (bh * ((Nq + 31) / 32) + i / 32);
      x.qm = qm_codes + (size_t)blk * d;
      x.qms = qm_scale[blk];
      x.k8 = k8_codes + (size_t)bk * Nkv * d;
      x.k8s = k8_scale + (size_t)bk * ((Nkv + 63) / 64);
    }
    x.d = d;
    for (int j = 0; j < Nkv; j++) out[(size_t)r * Nkv + j] = score4(&x, j);
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Split-KV form of the same attention (decode: few queries, a long KV      */
/* cache; the pages note that decode is bound by reading the KV cache).     */
/* The keys are cut into chunks of kv_chunk keys (a multiple of kv_tile);   */
/* each chunk runs the online softmax above from a fresh state, giving      */
/* (m_c, l_c, Oacc_c) (a chunk with no visible key is left out), and the    */
/* chunks are merged in ascending order with the log-sum-exp rule:          */
/*   m* = max_c m_c,  w_c = exp2f(RN(m_c - m*)),                            */
/*   L = fma(w_c, l_c, L),  O'_c = fma(w_c, Oacc_c, O'_c)   (fp32, from 0)  */
/*   O = O' * deltaV / L   (as above).                                      */
/* With kv_chunk >= Nkv this is oracle_attn_rows exactly.                   */
/* ------------------------------------------------------------------------ */
int oracle_attn_rows_split(const int8_t* q_codes, const float* q_scale, const int8_t* k_codes,
                           const float* k_scale, const uint8_t* v_codes, const float* v_scale, int B, int Hq,
                           int Hkv, int Nq, int Nkv, int d, int blk_q, int blk_k, int kv_tile, int kv_chunk,
                           int causal, float sm_scale, const int64_t* rows, int nrows, float* out) {
  if (!attn_args_ok(B, Hq, Hkv, Nq, Nkv, d, blk_q, blk_k, kv_tile, causal, sm_scale)) return -1;
  if (kv_chunk < kv_tile || kv_chunk % kv_tile) return -1;
  double vdec[256];
  for (int c = 0; c < 256; c++) vdec[c] = oracle_e4m3_decode((uint8_t)c);
  for (int r = 0; r < nrows; r++)
    if (rows[r] < 0 || rows[r] >= (int64_t)B * Hq * Nq) return -1;
  const int nc = (Nkv + kv_chunk - 1) / kv_chunk;
#pragma omp parallel for schedule(dynamic)
  for (int r = 0; r < nrows; r++) {
    row_ctx x;
    int64_t bk;
    row_setup(&x, q_codes, q_scale, k_codes, k_scale, v_codes, Hq, Hkv, Nq, Nkv, d, blk_q, blk_k, kv_tile, causal,
              sm_scale, rows[r], vdec, &bk);
    float* mc = (float*)malloc(sizeof(float) * nc);
    float* lc = (float*)malloc(sizeof(float) * nc);
    int* vis = (int*)malloc(sizeof(int) * nc);
    float* oc = (float*)malloc(sizeof(float) * (size_t)nc * d);
    float* o = (float*)calloc(d, sizeof(float));
    float mstar = -INFINITY;
    for (int c = 0; c < nc; c++) {
      const int j1 = (c + 1) * kv_chunk < Nkv ? (c + 1) * kv_chunk : Nkv;
      vis[c] = attend_range(&x, c * kv_chunk, j1, &mc[c], &lc[c], oc + (size_t)c * d, NULL) > 0;
      if (vis[c] && mc[c] > mstar) mstar = mc[c];
    }
    float L = 0.0f;
    for (int c = 0; c < nc; c++) {
      if (!vis[c]) continue;
      const float w = oracle_exp2f(mc[c] - mstar);
      L = fmaf(w, lc[c], L);
      for (int ch = 0; ch < d; ch++) o[ch] = fmaf(w, oc[(size_t)c * d + ch], o[ch]);
    }
    for (int ch = 0; ch < d; ch++)
      out[(size_t)r * d + ch] = (float)(((double)o[ch] * (double)v_scale[(size_t)bk * d + ch]) / (double)L);
    free(mc); free(lc); free(vis); free(oc); free(o);
  }
  return 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
