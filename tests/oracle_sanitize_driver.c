/* Test driver for the CPU oracle under AddressSanitizer and
 * UndefinedBehaviorSanitizer (host code only): calls every entry point of
 * oracle/attn_oracle.c on small seeded inputs, including row subsets, S = 1,
 * non-causal problems, both element types and every byte of the e4m3 codec.
 * Built and run by tests/test_oracle_sanitize.py; exits 0 when every call
 * returns its documented status. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

double oracle_bf16_decode(uint16_t bits);
double oracle_e4m3_decode(uint8_t code);
uint8_t oracle_e4m3_encode(float xf);
float oracle_descale_amax(const float* x, int64_t n);
void oracle_quantize_e4m3(const float* x, int64_t n, float descale, uint8_t* out);
int oracle_attn_stats(const void* q, const void* k, const void* v, int dtype, float q_descale,
                      float k_descale, float v_descale, int64_t B, int64_t S, int64_t H,
                      int64_t d_qk, int64_t d_v, double tau, int causal, const int64_t* rows,
                      int64_t nrows, double* o, double* lse, double* kappa, double* wmax,
                      double* sabs);
int oracle_attn(const void* q, const void* k, const void* v, int dtype, float q_descale,
                float k_descale, float v_descale, int64_t B, int64_t S, int64_t H, int64_t d_qk,
                int64_t d_v, double tau, int causal, const int64_t* rows, int64_t nrows, double* o,
                double* lse);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) { /* splitmix64 */
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return (uint32_t)((z ^ (z >> 31)) >> 32);
}

static int run_case(int dtype, int64_t B, int64_t S, int64_t H, int64_t dqk, int64_t dv,
                    int causal, int subset) {
  const int64_t esz = dtype == 0 ? 2 : 1;
  const int64_t nq = B * S * H * dqk, nv = B * S * H * dv;
  void* q = malloc((size_t)(nq * esz));
  void* k = malloc((size_t)(nq * esz));
  void* v = malloc((size_t)(nv * esz));
  for (int64_t i = 0; i < nq; ++i) {
    if (dtype == 0) {
      ((uint16_t*)q)[i] = (uint16_t)(0x3C00 + (next_u32() & 0x3FF) - 0x200 + ((next_u32() & 1) << 15));
      ((uint16_t*)k)[i] = (uint16_t)(0x3C00 + (next_u32() & 0x3FF) - 0x200 + ((next_u32() & 1) << 15));
    } else {
      ((uint8_t*)q)[i] = (uint8_t)(next_u32() % 0x7E) | (uint8_t)((next_u32() & 1) << 7);
      ((uint8_t*)k)[i] = (uint8_t)(next_u32() % 0x7E) | (uint8_t)((next_u32() & 1) << 7);
    }
  }
  for (int64_t i = 0; i < nv; ++i) {
    if (dtype == 0) ((uint16_t*)v)[i] = (uint16_t)(0x3C00 + (next_u32() & 0x3FF) - 0x200);
    else ((uint8_t*)v)[i] = (uint8_t)(next_u32() % 0x7E);
  }
  const int64_t nrows = subset ? (S + 1) / 2 : S;
  int64_t* rows = malloc(sizeof(int64_t) * (size_t)nrows);
  for (int64_t r = 0; r < nrows; ++r) rows[r] = subset ? (S - 1 - 2 * r) : r;
  double* o = malloc(sizeof(double) * (size_t)(B * nrows * H * dv));
  double* lse = malloc(sizeof(double) * (size_t)(B * H * nrows));
  double* st[3];
  for (int i = 0; i < 3; ++i) st[i] = malloc(sizeof(double) * (size_t)(B * H * nrows));
  int rc = oracle_attn_stats(q, k, v, dtype, 0.5f, 0.25f, 2.0f, B, S, H, dqk, dv, 0.3, causal,
                             rows, nrows, o, lse, st[0], st[1], st[2]);
  int rc2 = oracle_attn(q, k, v, dtype, 0.5f, 0.25f, 2.0f, B, S, H, dqk, dv, 0.3, causal, rows,
                        nrows, o, lse);
  int bad = rc != 0 || rc2 != 0;
  for (int64_t i = 0; i < B * H * nrows; ++i)
    bad |= !isfinite(lse[i]) || !(st[0][i] >= 0) || !(st[1][i] > 0) || !(st[2][i] >= 0);
  /* invalid arguments are rejected */
  rows[0] = S;
  bad |= oracle_attn(q, k, v, dtype, 1.0f, 1.0f, 1.0f, B, S, H, dqk, dv, 0.3, causal, rows,
                     nrows, o, lse) != -1;
  bad |= oracle_attn(q, k, v, 7, 1.0f, 1.0f, 1.0f, B, S, H, dqk, dv, 0.3, causal, rows, nrows,
                     o, lse) != -1;
  free(q); free(k); free(v); free(rows); free(o); free(lse);
  for (int i = 0; i < 3; ++i) free(st[i]);
  return bad;
}

int main(void) {
  int bad = 0;
  for (int c = 0; c < 256; ++c) {
    const double x = oracle_e4m3_decode((uint8_t)c);
    if (!isnan(x)) bad |= oracle_e4m3_encode((float)x) != (uint8_t)c && !(x == 0.0);
  }
  for (uint32_t b = 0; b < 65536; b += 97) (void)oracle_bf16_decode((uint16_t)b);
  float xs[1000];
  uint8_t codes[1000];
  for (int i = 0; i < 1000; ++i) xs[i] = (float)((int)(next_u32() % 20001) - 10000) * 0.137f;
  xs[17] = NAN;
  const float ds = oracle_descale_amax(xs, 1000);
  oracle_quantize_e4m3(xs, 1000, ds, codes);
  bad |= codes[17] != 0x7F;
  bad |= run_case(0, 2, 9, 3, 16, 8, 1, 0);
  bad |= run_case(0, 1, 1, 2, 128, 128, 1, 0);
  bad |= run_case(1, 2, 17, 2, 192, 128, 1, 1);
  bad |= run_case(1, 1, 33, 1, 128, 128, 0, 1);
  bad |= run_case(0, 1, 5, 4, 8, 16, 0, 0);
  printf("%s\n", bad ? "FAILED" : "ok");
  return bad;
}
