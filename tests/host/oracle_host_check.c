/* oracle_host_check.c -- runs every entry point of oracle/attn_oracle.c on
 * small inputs (both element types, GQA, a key prefix, row lists, one thread
 * and several) and its argument rejections, so that AddressSanitizer and
 * UBSan see all of its indexing. Built by tests/test_host_sanitized.py. The
 * numerical pins are the Python tests; here only cheap closed forms are
 * checked: row 0 equals V[0], rows of P sum to one, a row list equals the full
 * result. Prints one line per failed check, exits non-zero if any failed. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_decode_bf16(uint16_t h);
double oracle_decode_e4m3fn(uint8_t c);
int oracle_attn_f64(const void* q, const void* k, const void* v, int dtype, int B, int Hq, int Hkv, int S, int Dqk,
                    int Dv, double scale, double dq, double dk, double dv, const int64_t* rows, int64_t nrows,
                    double* out, int nthreads);
int oracle_attn_lse_f64(const void* q, const void* k, const void* v, int dtype, int B, int Hq, int Hkv, int S,
                        int Dqk, int Dv, double scale, double dq, double dk, double dv, const int64_t* rows,
                        int64_t nrows, double* out, double* lse, int nthreads);
int oracle_attn_prefix_f64(const void* q, const void* k, const void* v, int dtype, int B, int Hq, int Hkv, int Sq,
                           int Sk, int Dqk, int Dv, double scale, double dq, double dk, double dv,
                           const int64_t* rows, int64_t nrows, double* out, double* lse, int nthreads);
int oracle_attn_probs_f64(const void* q, const void* k, int dtype, int B, int Hq, int Hkv, int S, int Dqk,
                          double scale, double dq, double dk, int b, int h, double* P);

static int g_fail = 0;
#define CHECK(cond)                                              \
  do {                                                           \
    if (!(cond)) {                                               \
      printf("FAILED line %d: %s\n", __LINE__, #cond);           \
      ++g_fail;                                                  \
    }                                                            \
  } while (0)

static uint32_t g_state = 12345u;
static uint32_t next_u32(void) {
  g_state = g_state * 1664525u + 1013904223u;
  return g_state >> 8;
}
/* a finite code of each element type: bf16 values in about [-2, 2], e4m3 codes
 * of magnitude below 64 (no NaN codes) */
static void fill(void* x, int dtype, size_t n) {
  for (size_t i = 0; i < n; ++i) {
    if (dtype == 0) {
      float f = ((float)(next_u32() % 4001) - 2000.0f) / 1000.0f;
      uint32_t u;
      memcpy(&u, &f, 4);
      ((uint16_t*)x)[i] = (uint16_t)(u >> 16);
    } else {
      ((uint8_t*)x)[i] = (uint8_t)((next_u32() % 0x50) | ((next_u32() & 1) << 7));
    }
  }
}

static void run_case(int dtype, int B, int Hq, int Hkv, int Sq, int Sk, int Dqk, int Dv, int nthreads) {
  const size_t es = dtype == 0 ? 2 : 1;
  void* q = malloc(es * B * Sq * Hq * Dqk);
  void* k = malloc(es * B * Sk * Hkv * Dqk);
  void* v = malloc(es * B * Sk * Hkv * Dv);
  double* out = malloc(sizeof(double) * B * Sq * Hq * Dv);
  double* lse = malloc(sizeof(double) * B * Hq * Sq);
  fill(q, dtype, (size_t)B * Sq * Hq * Dqk);
  fill(k, dtype, (size_t)B * Sk * Hkv * Dqk);
  fill(v, dtype, (size_t)B * Sk * Hkv * Dv);
  const double scale = 0.3, dq = dtype ? 0.02 : 1.0, dk = dtype ? 0.03 : 1.0, dv = dtype ? 0.5 : 1.0;
  CHECK(oracle_attn_prefix_f64(q, k, v, dtype, B, Hq, Hkv, Sq, Sk, Dqk, Dv, scale, dq, dk, dv, NULL, 0, out, lse,
                               nthreads) == 0);
  if (Sq == Sk) {
    /* row 0 sees only key 0: O = dv * V[0] */
    for (int b = 0; b < B; ++b)
      for (int h = 0; h < Hq; ++h)
        for (int d = 0; d < Dv; ++d) {
          const size_t vo = (((size_t)b * Sk) * Hkv + h / (Hq / Hkv)) * Dv + d;
          const double v0 = dtype ? oracle_decode_e4m3fn(((uint8_t*)v)[vo]) : oracle_decode_bf16(((uint16_t*)v)[vo]);
          CHECK(out[(((size_t)b * Sq) * Hq + h) * Dv + d] == dv * v0);
        }
    double* out2 = malloc(sizeof(double) * B * Sq * Hq * Dv);
    CHECK(oracle_attn_f64(q, k, v, dtype, B, Hq, Hkv, Sq, Dqk, Dv, scale, dq, dk, dv, NULL, 0, out2, 1) == 0);
    CHECK(memcmp(out, out2, sizeof(double) * B * Sq * Hq * Dv) == 0);
    double* P = malloc(sizeof(double) * Sq * Sq);
    CHECK(oracle_attn_probs_f64(q, k, dtype, B, Hq, Hkv, Sq, Dqk, scale, dq, dk, B - 1, Hq - 1, P) == 0);
    for (int i = 0; i < Sq; ++i) {
      double s = 0.0;
      for (int j = 0; j < Sq; ++j) s += P[(size_t)i * Sq + j];
      CHECK(fabs(s - 1.0) <= 1e-12);
    }
    free(P);
    free(out2);
  }
  /* a row list, including repeats, equals the full result */
  int64_t rows[3 * 5] = {0, 0, 0, B - 1, Hq - 1, Sq - 1, 0, Hq / 2, Sq / 2, B - 1, 0, Sq - 1, 0, 0, 0};
  double ro[5 * 256], rl[5];
  CHECK(oracle_attn_prefix_f64(q, k, v, dtype, B, Hq, Hkv, Sq, Sk, Dqk, Dv, scale, dq, dk, dv, rows, 5, ro, rl,
                               nthreads) == 0);
  for (int r = 0; r < 5; ++r) {
    const int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
    CHECK(memcmp(ro + (size_t)r * Dv, out + (((size_t)b * Sq + i) * Hq + h) * Dv, sizeof(double) * Dv) == 0);
    CHECK(rl[r] == lse[((size_t)b * Hq + h) * Sq + i]);
  }
  free(q); free(k); free(v); free(out); free(lse);
}

int main(void) {
  for (int c = 0; c < 256; ++c) (void)oracle_decode_e4m3fn((uint8_t)c);
  for (int c = 0; c < 65536; c += 7) (void)oracle_decode_bf16((uint16_t)c);
  run_case(0, 1, 2, 2, 17, 17, 128, 128, 1);
  run_case(1, 2, 4, 2, 33, 33, 128, 128, 3);
  run_case(1, 1, 3, 1, 9, 9, 192, 128, 8);
  run_case(0, 2, 4, 1, 5, 40, 64, 32, 2);
  run_case(1, 1, 2, 2, 1, 1, 16, 8, 4);
  /* rejections */
  uint8_t x[64] = {0};
  double o[64];
  int64_t bad[3] = {0, 5, 0};
  CHECK(oracle_attn_f64(NULL, x, x, 1, 1, 1, 1, 4, 4, 4, 1.0, 1, 1, 1, NULL, 0, o, 1) == -1);
  CHECK(oracle_attn_f64(x, x, x, 2, 1, 1, 1, 4, 4, 4, 1.0, 1, 1, 1, NULL, 0, o, 1) == -1);
  CHECK(oracle_attn_f64(x, x, x, 1, 1, 3, 2, 4, 4, 4, 1.0, 1, 1, 1, NULL, 0, o, 1) == -1);
  CHECK(oracle_attn_f64(x, x, x, 1, 1, 1, 1, 4, 4, 4, 1.0, 1, 1, 1, bad, 1, o, 1) == -1);
  CHECK(oracle_attn_prefix_f64(x, x, x, 1, 1, 1, 1, 5, 4, 4, 4, 1.0, 1, 1, 1, NULL, 0, o, NULL, 1) == -1);
  CHECK(oracle_attn_probs_f64(x, x, 1, 1, 1, 1, 4, 4, 1.0, 1, 1, 0, 1, o) == -1);
  printf("oracle: %d failed\n", g_fail);
  return g_fail ? 1 : 0;
}
