/* Drives every entry point of oracle/oracle.c on small random inputs of each
 * format under host AddressSanitizer / UndefinedBehaviorSanitizer (built
 * without OpenMP, so every loop runs on one thread): every decoder over all
 * of its codes, the rounding encoders over landmark and random values,
 * dequantisation, row gathers with indices out of range, the GEMV over all
 * rows and a row subset, and the many-row form (random bytes: NaN and
 * infinite scales occur and propagate).  Exits non-zero if a decoder returns
 * a value outside its range. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_f16(uint16_t h);
double oracle_bf16(uint16_t h);
double oracle_e4m3(uint8_t c);
double oracle_e2m1(uint8_t n);
int oracle_tq1_digit(uint8_t b, int k);
uint16_t oracle_round_f16(double v);
uint16_t oracle_round_bf16(double v);
void oracle_dequant(int fmt, const uint8_t* w, int64_t n, int64_t k, double* out);
void oracle_get_rows(int fmt, const uint8_t* w, int64_t n, int64_t k, const int64_t* rows, int64_t nrows,
                     int out_dtype, void* out);
void oracle_decode16(int dtype, const uint16_t* h, int64_t n, double* out);
void oracle_gemv(int fmt, const uint8_t* w, const uint16_t* x, int64_t n, int64_t k, const int64_t* rows,
                 int64_t nrows, double* y, double* a);
void oracle_gemm(int fmt, const uint8_t* w, const uint16_t* x, int64_t t_count, int64_t n, int64_t k,
                 const int64_t* tok, int64_t ntok, const int64_t* rows, int64_t nrows, double* y, double* a);
int oracle_threads(void);
void oracle_set_threads(int t);

static uint32_t g_state = 12345u;
static uint32_t rnd(void) {
  g_state = g_state * 1664525u + 1013904223u;
  return g_state >> 8;
}

static int64_t weight_bytes(int fmt, int64_t n, int64_t k) {
  switch (fmt) {
    case 0: return n * (k / 256) * 144;
    case 1: return n * k / 2 + n * k / 16;
    case 2: return n * (k / 256) * 54;
    default: return 2 * n * k;
  }
}

int main(void) {
  int bad = 0;
  for (uint32_t c = 0; c < 65536; ++c) {
    volatile double a = oracle_f16((uint16_t)c), b = oracle_bf16((uint16_t)c);
    (void)a;
    (void)b;
  }
  for (uint32_t c = 0; c < 256; ++c) {
    volatile double a = oracle_e4m3((uint8_t)c);
    (void)a;
    for (int k = 0; k < 5; ++k) bad |= oracle_tq1_digit((uint8_t)c, k) > 2;
  }
  for (uint32_t c = 0; c < 16; ++c) bad |= !isfinite(oracle_e2m1((uint8_t)c));
  const double land[] = {0.0, -0.0, 1.0, 65504.0, 65520.0, 1e30, -1e30, 5.96e-8, 1e-40, INFINITY, -INFINITY, NAN,
                         3.3895313892515355e38, 1.0000000001};
  for (size_t i = 0; i < sizeof land / sizeof land[0]; ++i) {
    volatile uint16_t a = oracle_round_f16(land[i]), b = oracle_round_bf16(land[i]);
    (void)a;
    (void)b;
  }
  for (int i = 0; i < 100000; ++i) {
    const double v = ldexp((double)rnd() - 8388608.0, (int)(rnd() % 80) - 60);
    volatile uint16_t a = oracle_round_f16(v), b = oracle_round_bf16(v);
    (void)a;
    (void)b;
  }

  const int64_t n = 7, k = 768, t = 3;
  for (int fmt = 0; fmt < 5; ++fmt) {
    const int64_t kk = fmt >= 3 ? 40 : k;
    const int64_t wb = weight_bytes(fmt, n, kk);
    uint8_t* w = (uint8_t*)malloc((size_t)wb);
    for (int64_t i = 0; i < wb; ++i) w[i] = (uint8_t)rnd();
    uint16_t* x = (uint16_t*)malloc((size_t)(t * kk) * 2);
    for (int64_t i = 0; i < t * kk; ++i) x[i] = (uint16_t)(rnd() & 0x3FFF);  /* finite, |x| < 2 */
    double* deq = (double*)malloc((size_t)(n * kk) * sizeof(double));
    oracle_dequant(fmt, w, n, kk, deq);
    const int64_t rows[] = {6, -1, 0, 7, 3, INT64_MAX};
    void* out = malloc((size_t)(6 * kk) * 4);
    for (int dt = 0; dt < 3; ++dt) oracle_get_rows(fmt, w, n, kk, rows, 6, dt, out);
    double* xd = (double*)malloc((size_t)kk * sizeof(double));
    oracle_decode16(fmt == 1 || fmt == 4 ? 2 : 1, x, kk, xd);
    double y[7], a[7];
    oracle_gemv(fmt, w, x, n, kk, NULL, 0, y, a);
    const int64_t sub[] = {5, 0};
    oracle_gemv(fmt, w, x, n, kk, sub, 2, y, a);
    const int64_t tok[] = {2, 0};
    double yy[2 * 3], aa[2 * 3];
    const int64_t wr[] = {1, 6, 2};
    oracle_gemm(fmt, w, x, t, n, kk, tok, 2, wr, 3, yy, aa);
    free(w);
    free(x);
    free(deq);
    free(out);
    free(xd);
  }
  oracle_set_threads(1);
  bad |= oracle_threads() < 1;
  if (bad) {
    fprintf(stderr, "oracle driver: unexpected value\n");
    return 1;
  }
  printf("oracle: ok\n");
  return 0;
}
