/*
 * Plain fp64 CPU oracle for the batch-1 fused dequantise + GEMV
 *     y[r] = sum_i x[i] * w[r][i]      (alpha = 1, beta = 0)
 * over three block formats.  TEST INFRASTRUCTURE ONLY: the test suite, the
 * smoke check and the CPU baseline leg of the bench are the only callers.  It
 * shares no code, header, table or constant with the HIP library.
 *
 * Every function is a scalar "dequantise then dot" written from the pages'
 * definitions; nothing is blocked, fused or factored.  All arithmetic is fp64;
 * each dequantised weight is an exact fp64 value (the products involved have
 * fewer than 53 significant bits), so float(w) is the correctly rounded fp32
 * weight.  The GEMV sums x_i*w_i and |x_i*w_i| sequentially in i.
 *
 * Sources (titles of the pages):
 *  [Q4K]  "Writing a high performant GEMV + dequant for Metal": sections
 *         "What is a GEMV" (the operation), "What is a weight block?" (256
 *         weights in 144 bytes, 8 groups of 32), "Compute" (w_i = d s_g q_i -
 *         dmin m_g) and "Kernel code" (byte offsets of d, dmin, scales, qs and
 *         the nibble-to-element and scale-to-group assignment its index
 *         arithmetic implies).
 *  [FP4]  Mojo module "fp4_gemv": E2M1 nibbles, one FP8 E4M3 scale per 16
 *         weights, weight = e2m1 * |scale|.
 *  [TQ1]  "metal: TQ1_0 kernel performance": sections 1 (qs[48] then qh[4],
 *         five digits per qs byte, four per qh byte), 2 (which elements each
 *         digit feeds) and "Not applicable" (digits from floor(3^k b / 256)).
 *  [DENSE] The Mojo "fp4_gemv" page compares against a dense bf16 GEMV of the
 *         same shape: w_i is the fp16 / bf16 value itself.
 *  [PREFILL] Many activation rows at once (the Mojo page's M > 1 matmul path,
 *         the TQ1_0 page's prefill): Y[t][r] = sum_i X[t][i] w[r][i].
 *  [ROWS] Materialising rows (the TQ1_0 page's dequantize template, the Mojo
 *         page's fp32 dequant): out = the fp32 weight, optionally cast to
 *         fp16 / bf16 with round-to-nearest-even.
 *
 * Readings where the pages leave a choice (all recorded in the design notes):
 *  - fp16 d at byte 0, dmin at byte 2, little-endian (Q4_K).
 *  - NVFP4 buffer = [N][K/2] nibble bytes then [N][K/16] scale bytes; the even
 *    element sits in the low nibble; E4M3 is the OCP "fn" flavour (bias 7,
 *    subnormals, S.1111.111 = NaN, no infinities); the scale's sign is ignored.
 *  - TQ1_0 block = qs[48] | qh[4] | fp16 d; trit t maps to weight d*(t-1);
 *    qh digit k of byte m feeds element 240 + 4k + m.
 *  - A 16-bit materialisation rounds the fp32 weight (not the exact one):
 *    fp16(fp32(w)).  Only Q4_K weights can differ between the two readings.
 *  - A row index outside [0, n) materialises as a row of the output type's
 *    quiet NaN with a clear sign bit.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- scalar number formats ------------------------------------------------ */

/* IEEE binary16 -> fp64, from the bit fields. */
double oracle_f16(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
  return s ? -v : v;
}

/* bfloat16 -> fp64: the top 16 bits of an IEEE binary32. */
double oracle_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* OCP FP8 E4M3 ("fn") -> fp64. */
double oracle_e4m3(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7)
    return NAN;
  if (e == 0)
    v = ldexp((double)m, -9); /* (m/8) * 2^-6 */
  else
    v = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
  return s ? -v : v;
}

/* FP4 E2M1 -> fp64: sign, 2-bit exponent (bias 1), 1-bit mantissa. */
double oracle_e2m1(uint8_t n) {
  int s = (n >> 3) & 1, e = (n >> 1) & 3, m = n & 1;
  double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -v : v;
}

/* TQ1_0 base-3 digit k (0..4) of byte b: floor(3 * ((3^k * b) mod 256) / 256). */
int oracle_tq1_digit(uint8_t b, int k) {
  int p = 1;
  for (int j = 0; j < k; ++j)
    p *= 3;
  int r = (p * (int)b) % 256;
  return (3 * r) / 256;
}

/* Nearest value of a binary floating-point format with P significand bits
 * (implicit bit included), exponent bias BIAS and EBITS exponent bits, ties to
 * even; returns its bit pattern (sign in bit EBITS + P - 1).  Overflow gives
 * infinity, NaN a quiet NaN of the same sign. */
static uint32_t round_bits(double v, int p, int bias, int ebits) {
  const uint32_t sign = signbit(v) ? 1u << (ebits + p - 1) : 0u;
  const uint32_t emask = (1u << ebits) - 1u;
  const uint32_t inf = sign | (emask << (p - 1));
  if (isnan(v))
    return inf | (1u << (p - 2));
  double a = fabs(v);
  if (isinf(a))
    return inf;
  if (a == 0.0)
    return sign;
  int x;
  frexp(a, &x);              /* a = f * 2^x, 0.5 <= f < 1 */
  int e = x - 1;             /* 2^e <= a < 2^(e+1) */
  const int emin = 1 - bias; /* smallest normal exponent */
  if (e < emin)
    e = emin; /* subnormal range: same quantum as the smallest normals */
  int qe = e - (p - 1);      /* value of one unit in the last place */
  double scaled = ldexp(a, -qe); /* exact: a power-of-two scaling */
  double n = floor(scaled);
  double frac = scaled - n;
  if (frac > 0.5 || (frac == 0.5 && fmod(n, 2.0) != 0.0))
    n += 1.0;
  if (n == ldexp(1.0, p)) { /* rounded up to the next binade */
    n = ldexp(1.0, p - 1);
    qe += 1;
  }
  const double half = ldexp(1.0, p - 1);
  if (n < half) /* subnormal (or zero): exponent field 0 */
    return sign | (uint32_t)n;
  const int field = qe + (p - 1) + bias;
  if (field >= (int)emask)
    return inf;
  return sign | ((uint32_t)field << (p - 1)) | (uint32_t)(n - half);
}

uint16_t oracle_round_f16(double v) { return (uint16_t)round_bits(v, 11, 15, 5); }
uint16_t oracle_round_bf16(double v) { return (uint16_t)round_bits(v, 8, 127, 8); }

/* ---- per-block dequantisation (fp64, 256 weights) ------------------------- */

static uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* Q4_K: d@0, dmin@2, scales[12]@4, qs[128]@16; w_i = d*s_g*q_i - dmin*m_g. */
static void q4k_block(const uint8_t* b, double* w) {
  double d = oracle_f16(rd16(b + 0));
  double dmin = oracle_f16(rd16(b + 2));
  const uint8_t* sc = b + 4;
  const uint8_t* qs = b + 16;
  int s[8], m[8];
  for (int g = 0; g < 8; ++g) {
    if (g < 4) {
      s[g] = sc[g] & 63;
      m[g] = sc[g + 4] & 63;
    } else {
      s[g] = (sc[g + 4] & 15) | ((sc[g - 4] >> 6) << 4);
      m[g] = (sc[g + 4] >> 4) | ((sc[g] >> 6) << 4);
    }
  }
  for (int i = 0; i < 256; ++i) {
    int c = i / 64, l = i % 64;
    uint8_t byte = qs[32 * c + (l % 32)];
    int q = (l < 32) ? (byte & 15) : (byte >> 4);
    int g = i / 32;
    w[i] = d * s[g] * q - dmin * m[g];
  }
}

/* TQ1_0: qs[48]@0, qh[4]@48, d@52. */
static void tq1_block(const uint8_t* b, double* w) {
  const uint8_t* qs = b;
  const uint8_t* qh = b + 48;
  double d = oracle_f16(rd16(b + 52));
  for (int j = 0; j < 32; ++j)
    for (int k = 0; k < 5; ++k)
      w[32 * k + j] = d * (oracle_tq1_digit(qs[j], k) - 1);
  for (int j = 0; j < 16; ++j)
    for (int k = 0; k < 5; ++k)
      w[160 + 16 * k + j] = d * (oracle_tq1_digit(qs[32 + j], k) - 1);
  for (int m = 0; m < 4; ++m)
    for (int k = 0; k < 4; ++k)
      w[240 + 4 * k + m] = d * (oracle_tq1_digit(qh[m], k) - 1);
}

/* NVFP4 single weight (row r, column i) of the one-buffer layout. */
static double nvfp4_weight(const uint8_t* buf, int64_t n, int64_t k, int64_t r, int64_t i) {
  uint8_t byte = buf[r * (k / 2) + i / 2];
  uint8_t nib = (i % 2 == 0) ? (byte & 15) : (byte >> 4);
  uint8_t sc = buf[n * (k / 2) + r * (k / 16) + i / 16];
  return oracle_e2m1(nib) * fabs(oracle_e4m3(sc));
}

/* Dense 16-bit weight (row r, column i): fmt 3 = fp16, 4 = bf16. */
static double dense_weight(int fmt, const uint8_t* buf, int64_t k, int64_t r, int64_t i) {
  uint16_t h = rd16(buf + 2 * (r * k + i));
  return fmt == 3 ? oracle_f16(h) : oracle_bf16(h);
}

/* fp64 weights of row r, all K of them. */
static void dequant_row(int fmt, const uint8_t* w, int64_t n, int64_t k, int64_t r, double* out) {
  int64_t nb = k / 256;
  if (fmt == 1) {
    for (int64_t i = 0; i < k; ++i)
      out[i] = nvfp4_weight(w, n, k, r, i);
  } else if (fmt == 3 || fmt == 4) {
    for (int64_t i = 0; i < k; ++i)
      out[i] = dense_weight(fmt, w, k, r, i);
  } else {
    for (int64_t b = 0; b < nb; ++b) {
      if (fmt == 0)
        q4k_block(w + (r * nb + b) * 144, out + b * 256);
      else
        tq1_block(w + (r * nb + b) * 54, out + b * 256);
    }
  }
}

/* ---- public entry points --------------------------------------------------- */

int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_threads(int t) {
#ifdef _OPENMP
  if (t > 0)
    omp_set_num_threads(t);
#else
  (void)t;
#endif
}

/* Dequantise rows [0, n) into out[n][k] (fp64).  fmt: 0 = Q4_K, 1 = NVFP4,
 * 2 = TQ1_0, 3 = dense fp16, 4 = dense bf16. */
void oracle_dequant(int fmt, const uint8_t* w, int64_t n, int64_t k, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r)
    dequant_row(fmt, w, n, k, r, out + r * k);
}

/* Rows rows[0..nrows) of the weights, each weight rounded to fp32 and then to
 * the output type (0 = fp32, 1 = fp16, 2 = bf16), into out[nrows][k] (4- or
 * 2-byte elements).  An index outside [0, n) gives a row of quiet NaNs. */
void oracle_get_rows(int fmt, const uint8_t* w, int64_t n, int64_t k, const int64_t* rows,
                     int64_t nrows, int out_dtype, void* out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < nrows; ++j) {
    int64_t r = rows[j];
    double* row = (double*)malloc((size_t)k * sizeof(double));
    int valid = r >= 0 && r < n;
    if (valid)
      dequant_row(fmt, w, n, k, r, row);
    for (int64_t i = 0; i < k; ++i) {
      const int64_t o = j * k + i;
      if (!valid) {
        if (out_dtype == 0)
          ((uint32_t*)out)[o] = 0x7FC00000u;
        else
          ((uint16_t*)out)[o] = out_dtype == 1 ? 0x7E00 : 0x7FC0;
        continue;
      }
      const float f = (float)row[i]; /* round to nearest even (C default mode) */
      if (out_dtype == 0)
        memcpy((uint32_t*)out + o, &f, sizeof f);
      else if (out_dtype == 1)
        ((uint16_t*)out)[o] = oracle_round_f16((double)f);
      else
        ((uint16_t*)out)[o] = oracle_round_bf16((double)f);
    }
    free(row);
  }
}

/* Decode n 16-bit values (dtype 1 = fp16, 2 = bf16) to fp64. */
void oracle_decode16(int dtype, const uint16_t* h, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i)
    out[i] = dtype == 1 ? oracle_f16(h[i]) : oracle_bf16(h[i]);
}

/* y[r] = sum_i x_i w_ri and a[r] = sum_i |x_i w_ri| over rows listed in
 * rows[0..nrows) (rows == NULL means all n rows, in order).  x holds fp16 bits
 * (Q4_K, TQ1_0, dense fp16) or bf16 bits (NVFP4, dense bf16). */
void oracle_gemv(int fmt, const uint8_t* w, const uint16_t* x, int64_t n, int64_t k,
                 const int64_t* rows, int64_t nrows, double* y, double* a) {
  if (rows == NULL)
    nrows = n;
  const int x_bf16 = fmt == 1 || fmt == 4;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < nrows; ++t) {
    int64_t r = rows ? rows[t] : t;
    double acc = 0.0, aacc = 0.0;
    double* wr = (double*)malloc((size_t)k * sizeof(double));
    dequant_row(fmt, w, n, k, r, wr);
    for (int64_t i = 0; i < k; ++i) {
      double p = (x_bf16 ? oracle_bf16(x[i]) : oracle_f16(x[i])) * wr[i];
      acc += p;
      aacc += fabs(p);
    }
    free(wr);
    y[t] = acc;
    a[t] = aacc;
  }
}

/* Y[a][b] = sum_i X[tok[a]][i] w[row[b]][i] and A[a][b] = sum_i |X[tok[a]][i] w[row[b]][i]|
 * for the listed activation rows (tokens) and weight rows: the prefill form,
 * one plain GEMV per token.  X is [T][k] 16-bit codes (fp16, or bf16 for NVFP4
 * and dense bf16). */
void oracle_gemm(int fmt, const uint8_t* w, const uint16_t* x, int64_t t_count, int64_t n, int64_t k,
                 const int64_t* tok, int64_t ntok, const int64_t* rows, int64_t nrows, double* y,
                 double* a) {
  const int x_bf16 = fmt == 1 || fmt == 4;
  (void)t_count;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t b = 0; b < nrows; ++b) {
    double* wr = (double*)malloc((size_t)k * sizeof(double));
    dequant_row(fmt, w, n, k, rows[b], wr);
    for (int64_t q = 0; q < ntok; ++q) {
      const uint16_t* xt = x + tok[q] * k;
      double acc = 0.0, aacc = 0.0;
      for (int64_t i = 0; i < k; ++i) {
        double p = (x_bf16 ? oracle_bf16(xt[i]) : oracle_f16(xt[i])) * wr[i];
        acc += p;
        aacc += fabs(p);
      }
      y[q * nrows + b] = acc;
      a[q * nrows + b] = aacc;
    }
    free(wr);
  }
}
