/*
 * Reference oracle for causal prefill attention (forward) -- TEST
 * INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load this library.  The GPU product path never links, loads
 * or calls it, and it shares no code, header or constant table with the GPU
 * kernels.
 *
 * What it computes (plain definition, IEEE binary64, no blocking, no online
 * softmax, fixed summation order j = 0, 1, 2, ...):
 *
 *   s_ij  = tau * sum_c qhat[b,i,h,c] * khat[b,j,h,c]
 *   key j visible from query i  iff  (causal ? j <= i : true)
 *   m_i   = max over visible j of s_ij
 *   l_i   = sum over visible j of exp(s_ij - m_i)
 *   o_i   = sum over visible j of exp(s_ij - m_i) * vhat[b,j,h,:] / l_i
 *   lse_i = m_i + ln(l_i)
 *
 * This is attention as the ZYFA pages describe it: a product Q.K^T, a softmax
 * between the two matrix products, and a product with V ("Por que a atencao
 * FP8 tem desempenho inferior no MI355X?" on the acheiumaia.com.br page; "Como
 * o motor de atencao FP8 da Zyphra funciona" on the miraibroadcast.com page),
 * restricted to causal forward prefill ("Ce que couvrent les noyaux" on the
 * ai-daily-news.org page), with the fp64 result as the error yardstick
 * ("ZYFA acelera atencao em ate 1,76x com menos erro" and "Precisao,
 * estabilidade e efeito na pratica" on the miraibroadcast.com page).  The
 * pages print no formula; the one above is the textbook definition.
 *
 * qhat/khat/vhat are the exact real values the caller's element encodings
 * denote: bf16 widened exactly, or OCP E4M3FN decoded exactly and multiplied
 * by the per-tensor fp32 descale (FP8 e4m3 as named in the TL;DR of the
 * acheiumaia.com.br page; the descale = amax/448 reading is documented with
 * the quantizer below).
 *
 * Layouts: q,k [B,S,H,d_qk]; v [B,S,H,d_v] (row-major, contiguous).
 * Outputs for a list of query rows: o [B,nrows,H,d_v], lse [B,H,nrows].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- codecs */

/* bf16: the upper 16 bits of an IEEE binary32. Exact widening. */
double oracle_bf16_decode(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* OCP 8-bit floating point E4M3 ("FN" variant): 1 sign, 4 exponent bits
 * (bias 7), 3 mantissa bits, no infinities, S.1111.111 is NaN, largest
 * finite 448, smallest subnormal 2^-9.  Decoding straight from the bit
 * fields. */
double oracle_e4m3_decode(uint8_t code) {
  int sign = code >> 7;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double v;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9); /* subnormal: m/8 * 2^(1-7) */
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return sign ? -v : v;
}

/* Round-to-nearest-even into E4M3FN, saturating magnitudes above 448 to
 * +-448 (never producing NaN from a finite input).  NaN input gives the NaN
 * code 0x7F.  The input is an fp32 value; all arithmetic below is exact in
 * binary64. */
uint8_t oracle_e4m3_encode(float xf) {
  double x = (double)xf;
  if (isnan(x)) return 0x7F;
  uint8_t sign = (x < 0 || (x == 0 && signbit(x))) ? 0x80 : 0x00;
  double a = fabs(x);
  if (a >= 448.0) return sign | 0x7E;
  /* Quantum of the binade containing a: subnormals and the first normal
   * binade [2^-6, 2^-5) share quantum 2^-9. */
  int ex;
  frexp(a, &ex); /* a = f * 2^ex with f in [0.5,1): binade [2^(ex-1), 2^ex) */
  int unb = ex - 1;
  if (unb < -6) unb = -6;
  double q = ldexp(1.0, unb - 3);
  double n = a / q; /* exact: power-of-two division */
  double r = floor(n);
  double frac = n - r;
  if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
  double v = r * q; /* representable (possibly the next binade's first value) */
  if (v > 448.0) v = 448.0;
  if (v < ldexp(1.0, -6)) /* subnormal or zero: exponent field 0, m = v / 2^-9 */
    return sign | (uint8_t)(v / ldexp(1.0, -9));
  int ev;
  double f = frexp(v, &ev); /* v = f * 2^ev, f in [0.5, 1) */
  int E = ev - 1;            /* v = (2f) * 2^E, 2f in [1, 2) */
  int mant = (int)((2.0 * f - 1.0) * 8.0);
  return sign | (uint8_t)(((E + 7) << 3) | mant);
}

/* Per-tensor scaling before FP8 rounding: descale = amax / 448 in fp32
 * (1 when the tensor is all zero), so the largest magnitude lands on the
 * largest finite E4M3 value.  The pages attribute most of the FP8 error to
 * this quantization of Q, K and V ("Precisao, estabilidade e efeito na
 * pratica", miraibroadcast.com page); the amax/448 rule itself is the plain
 * reading of "per-tensor descale" for the e4m3 format. */
float oracle_descale_amax(const float* x, int64_t n) {
  float amax = 0.0f;
  for (int64_t i = 0; i < n; ++i) {
    float a = fabsf(x[i]);
    if (a > amax) amax = a;
  }
  if (amax == 0.0f) return 1.0f;
  return amax / 448.0f;
}

/* code_i = encode(fp32(x_i / descale)): the quotient is rounded once to fp32
 * (IEEE division), then once to E4M3. */
void oracle_quantize_e4m3(const float* x, int64_t n, float descale, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    float t = x[i] / descale;
    out[i] = oracle_e4m3_encode(t);
  }
}

/* ------------------------------------------------------------- attention */

enum { ORACLE_BF16 = 0, ORACLE_FP8 = 1 };

static double g_e4m3_table[256];
static int g_table_ready = 0;

static void build_table(void) {
  if (g_table_ready) return;
  for (int c = 0; c < 256; ++c) g_e4m3_table[c] = oracle_e4m3_decode((uint8_t)c);
  g_table_ready = 1;
}

/* value of element idx of a tensor in the given encoding, times descale */
static inline double elem(const void* base, int64_t idx, int dtype, double descale) {
  if (dtype == ORACLE_BF16) return oracle_bf16_decode(((const uint16_t*)base)[idx]);
  return g_e4m3_table[((const uint8_t*)base)[idx]] * descale;
}

/*
 * Attention for the query rows listed in `rows` (each in [0,S)), all batches
 * and heads.  Returns 0 on success, -1 on bad arguments.
 *
 * Optional per-row statistics of the same softmax (each array [B,H,nrows],
 * skipped when NULL), for judging how a row's result reacts to rounding of
 * its probabilities, which is where a reduced-precision evaluation of the
 * method loses accuracy (the pages round P to e4m3, "Como o motor de atencao
 * FP8 da Zyphra funciona" on the miraibroadcast.com page, and measure the
 * error against fp64, "Precisao, estabilidade e efeito na pratica" on the
 * same page).  With w_ij = exp(s_ij - m_i) / l_i the softmax weights:
 *
 *   kappa_i = sqrt(sum_j w_ij^2 |vhat_j - o_i|^2) / |o_i|
 *       If every weight is perturbed as w_ij (1 + e_j), with e_j independent,
 *       zero-mean and of RMS e, and the row renormalised, then to first
 *       order o_i moves by sum_j w_ij e_j (vhat_j - o_i), whose RMS norm is
 *       e * kappa_i * |o_i|: kappa_i is the factor by which relative errors
 *       of the probabilities become a relative error of the row.  0 / 0 is
 *       taken as 0 (a single visible key, or equal value rows), x / 0 as inf.
 *   wmax_i  = sum of w_ij over the keys whose score equals m_i (the softmax
 *       mass at the row maximum).
 *   sabs_i  = sum_j w_ij * |tau| * sum_c |qhat_ic * khat_jc|: the
 *       softmax-weighted magnitude of the terms of the row's scores.  An
 *       evaluation of a score that loses precision relative to its terms
 *       rather than to its (possibly cancelled) value errs by a multiple of
 *       that score's term magnitude; weighted by w_ij this bounds the
 *       resulting first-order change of the row's log-sum-exp and scales
 *       the resulting relative errors of its weights.
 */
int oracle_attn_stats(const void* q, const void* k, const void* v, int dtype, float q_descale,
                      float k_descale, float v_descale, int64_t B, int64_t S, int64_t H,
                      int64_t d_qk, int64_t d_v, double tau, int causal, const int64_t* rows,
                      int64_t nrows, double* o, double* lse, double* kappa, double* wmax,
                      double* sabs) {
  if (!q || !k || !v || !o || !lse || !rows) return -1;
  if (B < 1 || S < 1 || H < 1 || d_qk < 1 || d_v < 1 || nrows < 1) return -1;
  if (dtype != ORACLE_BF16 && dtype != ORACLE_FP8) return -1;
  for (int64_t r = 0; r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= S) return -1;
  build_table();
  const double dq = (dtype == ORACLE_FP8) ? (double)q_descale : 1.0;
  const double dk = (dtype == ORACLE_FP8) ? (double)k_descale : 1.0;
  const double dv = (dtype == ORACLE_FP8) ? (double)v_descale : 1.0;
  const int64_t total = B * H * nrows;

#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)S);
    double* qi = (double*)malloc(sizeof(double) * (size_t)d_qk);
    double* acc = (double*)malloc(sizeof(double) * (size_t)d_v);
#pragma omp for schedule(dynamic, 1)
    for (int64_t t = 0; t < total; ++t) {
      const int64_t r = t % nrows;
      const int64_t h = (t / nrows) % H;
      const int64_t b = t / (nrows * H);
      const int64_t i = rows[r];
      const int64_t nvis = causal ? i + 1 : S; /* keys 0..nvis-1 are visible */
      for (int64_t c = 0; c < d_qk; ++c)
        qi[c] = elem(q, ((b * S + i) * H + h) * d_qk + c, dtype, dq);
      double m = -INFINITY;
      for (int64_t j = 0; j < nvis; ++j) {
        double dot = 0.0;
        const int64_t kb = ((b * S + j) * H + h) * d_qk;
        for (int64_t c = 0; c < d_qk; ++c) dot += qi[c] * elem(k, kb + c, dtype, dk);
        s[j] = tau * dot;
        if (s[j] > m) m = s[j];
      }
      double l = 0.0;
      for (int64_t c = 0; c < d_v; ++c) acc[c] = 0.0;
      for (int64_t j = 0; j < nvis; ++j) {
        const double p = exp(s[j] - m);
        l += p;
        const int64_t vb = ((b * S + j) * H + h) * d_v;
        for (int64_t c = 0; c < d_v; ++c) acc[c] += p * elem(v, vb + c, dtype, dv);
      }
      double* orow = o + ((b * nrows + r) * H + h) * d_v;
      for (int64_t c = 0; c < d_v; ++c) orow[c] = acc[c] / l;
      const int64_t srow = (b * H + h) * nrows + r;
      lse[srow] = m + log(l);
      if (kappa) {
        double num = 0.0, den = 0.0;
        for (int64_t c = 0; c < d_v; ++c) den += orow[c] * orow[c];
        for (int64_t j = 0; j < nvis; ++j) {
          const double w = exp(s[j] - m) / l;
          const int64_t vb = ((b * S + j) * H + h) * d_v;
          double dist = 0.0;
          for (int64_t c = 0; c < d_v; ++c) {
            const double e = elem(v, vb + c, dtype, dv) - orow[c];
            dist += e * e;
          }
          num += w * w * dist;
        }
        kappa[srow] = num == 0.0 ? 0.0 : (den == 0.0 ? INFINITY : sqrt(num) / sqrt(den));
      }
      if (wmax) {
        int64_t at_max = 0;
        for (int64_t j = 0; j < nvis; ++j) at_max += s[j] == m;
        wmax[srow] = (double)at_max / l;
      }
      if (sabs) {
        double acc_w = 0.0;
        for (int64_t j = 0; j < nvis; ++j) {
          const int64_t kb = ((b * S + j) * H + h) * d_qk;
          double a = 0.0;
          for (int64_t c = 0; c < d_qk; ++c) a += fabs(qi[c] * elem(k, kb + c, dtype, dk));
          acc_w += exp(s[j] - m) / l * fabs(tau) * a;
        }
        sabs[srow] = acc_w;
      }
    }
    free(s);
    free(qi);
    free(acc);
  }
  return 0;
}

int oracle_attn(const void* q, const void* k, const void* v, int dtype, float q_descale,
                float k_descale, float v_descale, int64_t B, int64_t S, int64_t H, int64_t d_qk,
                int64_t d_v, double tau, int causal, const int64_t* rows, int64_t nrows, double* o,
                double* lse) {
  return oracle_attn_stats(q, k, v, dtype, q_descale, k_descale, v_descale, B, S, H, d_qk, d_v,
                           tau, causal, rows, nrows, o, lse, NULL, NULL, NULL);
}

/* Number of threads the parallel regions above use (for reporting). */
#ifdef _OPENMP
#include <omp.h>
int oracle_num_threads(void) { return omp_get_max_threads(); }
#else
int oracle_num_threads(void) { return 1; }
#endif
