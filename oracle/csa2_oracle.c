/*
 * csa2_oracle.c -- plain CPU oracle (double precision) for the CSA2 path.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the GPU library.  Each function is
 * the plain definition of its step; OpenMP only spreads independent rows
 * over threads and changes no arithmetic.  Citations are in csa2_oracle.h.
 */
#include "csa2_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* E2M1: sign | e1 e0 | m.  Exponent bias 1; exponent 0 is subnormal
 * (value m * 2^-1 * ... = m/2); otherwise 2^(e-1) * (1 + m/2). */
double csa2o_e2m1_value(int code) {
  int sign = (code >> 3) & 1;
  int e = (code >> 1) & 3;
  int m = code & 1;
  double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return sign ? -mag : mag;
}

/* E4M3FN: sign | 4 exponent bits (bias 7) | 3 mantissa bits.  Exponent 0
 * is subnormal (m/8 * 2^-6); 0x7F and 0xFF are NaN; no infinities. */
double csa2o_e4m3_value(int byte) {
  int sign = (byte >> 7) & 1;
  int e = (byte >> 3) & 15;
  int m = byte & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp(m / 8.0, -6);
  else
    mag = ldexp(1.0 + m / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* Nearest E4M3 value to amax/6.  Distances are compared as |amax - 6 v|:
 * amax is an fp32 value below 2688 and 6 v has at most 7 significant bits,
 * so every difference is exact in double and the search is exact. */
int csa2o_scale_byte(double amax) {
  /* Every candidate is <= 448, so from 6*448 up the nearest is 448 (and
   * the distance below would no longer be exact for huge amax). */
  if (amax >= 6.0 * 448.0) return 0x7E;
  int best = 0;
  double best_d = INFINITY;
  for (int b = 0; b <= 126; ++b) { /* 127 non-negative finite values */
    double d = fabs(amax - 6.0 * csa2o_e4m3_value(b));
    if (d < best_d || (d == best_d && (b & 1) == 0 && (best & 1) != 0)) {
      best_d = d;
      best = b;
    }
  }
  return best;
}

/* Nearest E2M1 magnitude g*s to |x|, ties to the even code; the distance
 * |x| - g s is exact in double (x fp32, g s at most 6 significant bits). */
int csa2o_e2m1_code(double x, double s) {
  int sign = signbit(x) ? 8 : 0;
  if (s == 0.0) return sign;
  double a = fabs(x);
  int best = 0;
  double best_d = INFINITY;
  for (int c = 0; c < 8; ++c) {
    double d = fabs(a - csa2o_e2m1_value(c) * s);
    if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) != 0)) {
      best_d = d;
      best = c;
    }
  }
  return sign | best;
}

void csa2o_quantize_rows(const float* x, int64_t rows, int32_t dim,
                         uint8_t* codes, uint8_t* scales) {
  const int32_t nb = dim / 16;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const float* xr = x + r * (int64_t)dim;
    uint8_t* cr = codes + r * (int64_t)(dim / 2);
    uint8_t* sr = scales + r * (int64_t)nb;
    for (int32_t b = 0; b < nb; ++b) {
      double amax = 0.0;
      for (int c = 0; c < 16; ++c) {
        double a = fabs((double)xr[b * 16 + c]);
        if (a > amax) amax = a;
      }
      int sb = csa2o_scale_byte(amax);
      double s = csa2o_e4m3_value(sb);
      sr[b] = (uint8_t)sb;
      for (int c = 0; c < 16; c += 2) {
        int lo = csa2o_e2m1_code((double)xr[b * 16 + c], s);
        int hi = csa2o_e2m1_code((double)xr[b * 16 + c + 1], s);
        cr[(b * 16 + c) / 2] = (uint8_t)(lo | (hi << 4));
      }
    }
  }
}

static void dequant_row(const uint8_t* cr, const uint8_t* sr, int32_t dim,
                        double* out) {
  for (int32_t c = 0; c < dim; ++c) {
    int byte = cr[c / 2];
    int code = (c & 1) ? (byte >> 4) : (byte & 15);
    out[c] = csa2o_e2m1_value(code) * csa2o_e4m3_value(sr[c / 16]);
  }
}

void csa2o_dequant_rows(const uint8_t* codes, const uint8_t* scales,
                        int64_t rows, int32_t dim, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    dequant_row(codes + r * (int64_t)(dim / 2), scales + r * (int64_t)(dim / 16),
                dim, out + r * (int64_t)dim);
}

void csa2o_index_score(const uint8_t* codes, const uint8_t* scales,
                       int32_t dim, const float* q, const float* w,
                       int32_t H, const int64_t* rows, int64_t n,
                       double* out) {
#pragma omp parallel
  {
    double* k = (double*)malloc(sizeof(double) * (size_t)dim);
#pragma omp for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
      int64_t r = rows[i];
      dequant_row(codes + r * (int64_t)(dim / 2), scales + r * (int64_t)(dim / 16),
                  dim, k);
      double score = 0.0;
      for (int32_t h = 0; h < H; ++h) {
        double dot = 0.0;
        for (int32_t c = 0; c < dim; ++c) dot += (double)q[h * dim + c] * k[c];
        score += (double)w[h] * (dot > 0.0 ? dot : 0.0);
      }
      out[i] = score;
    }
    free(k);
  }
}

typedef struct {
  double score;
  int64_t slot;
} ranked;

/* Descending score; equal scores (including -0 == +0) by ascending slot. */
static int by_rank(const void* a, const void* b) {
  const ranked* x = (const ranked*)a;
  const ranked* y = (const ranked*)b;
  if (x->score > y->score) return -1;
  if (x->score < y->score) return 1;
  return (x->slot < y->slot) ? -1 : (x->slot > y->slot);
}

static int by_value(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

int32_t csa2o_topk(const double* score, int64_t n_valid, int32_t k,
                   const int32_t* slot_pos, int32_t* out) {
  int64_t take = n_valid < k ? n_valid : k;
  if (take < 0) take = 0;
  ranked* all = (ranked*)malloc(sizeof(ranked) * (size_t)(n_valid > 0 ? n_valid : 1));
  for (int64_t i = 0; i < n_valid; ++i) {
    all[i].score = score[i];
    all[i].slot = i;
  }
  qsort(all, (size_t)n_valid, sizeof(ranked), by_rank);
  for (int64_t i = 0; i < take; ++i)
    out[i] = slot_pos ? slot_pos[all[i].slot] : (int32_t)all[i].slot;
  qsort(out, (size_t)take, sizeof(int32_t), by_value);
  for (int64_t i = take; i < k; ++i) out[i] = -1;
  free(all);
  return (int32_t)take;
}

void csa2o_sparse_attn(const float* q, int32_t H, int32_t D, int32_t dv,
                       const uint8_t* codes, const uint8_t* scales,
                       const int32_t* idx, int32_t K,
                       const uint8_t* swa, double swa_scale, int32_t S,
                       double sm_scale, double* out, double* lse) {
  int32_t n = 0;
  for (int32_t j = 0; j < K; ++j) n += idx[j] >= 0;
  n += S;
  /* Rows of the union, dequantized: first the selected cache rows, then
   * the window rows.  No de-duplication between the two sets. */
  double* rows = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * (size_t)D);
  int32_t e = 0;
  for (int32_t j = 0; j < K; ++j) {
    if (idx[j] < 0) continue;
    dequant_row(codes + (int64_t)idx[j] * (D / 2), scales + (int64_t)idx[j] * (D / 16),
                D, rows + (int64_t)e * D);
    ++e;
  }
  for (int32_t j = 0; j < S; ++j, ++e)
    for (int32_t c = 0; c < D; ++c)
      rows[(int64_t)e * D + c] = csa2o_e4m3_value(swa[(int64_t)j * D + c]) * swa_scale;
  double* logit = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  for (int32_t h = 0; h < H; ++h) {
    double* o = out + (int64_t)h * dv;
    for (int32_t c = 0; c < dv; ++c) o[c] = 0.0;
    if (n == 0) {
      lse[h] = -INFINITY;
      continue;
    }
    double m = -INFINITY;
    for (int32_t j = 0; j < n; ++j) {
      double dot = 0.0;
      for (int32_t c = 0; c < D; ++c) dot += (double)q[h * D + c] * rows[(int64_t)j * D + c];
      logit[j] = sm_scale * dot;
      if (logit[j] > m) m = logit[j];
    }
    double l = 0.0;
    for (int32_t j = 0; j < n; ++j) {
      double p = exp(logit[j] - m);
      l += p;
      for (int32_t c = 0; c < dv; ++c) o[c] += p * rows[(int64_t)j * D + c];
    }
    for (int32_t c = 0; c < dv; ++c) o[c] /= l;
    lse[h] = m + log(l);
  }
  free(logit);
  free(rows);
}

int32_t csa2o_num_threads(void) {
#ifdef _OPENMP
  return (int32_t)omp_get_max_threads();
#else
  return 1;
#endif
}

void csa2o_set_num_threads(int32_t n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads((int)n);
#else
  (void)n;
#endif
}
