/*
 * CPU oracle for C = A*B on CSR matrices.  TEST INFRASTRUCTURE ONLY: see
 * oracle.h for the contract and for who may call it.
 *
 * Method: Gustavson's row-wise formulation (gMAGNUS page, §II-B, Eq. 1 and
 * Algorithm 1; Ocean page, §2): row i of C is the sum of the rows B[k,:]
 * scaled by A[i,k].  Each thread owns a dense accumulator over all columns of
 * C, a row stamp per column telling whether the column was touched by the
 * current row, and a list of touched columns, which is sorted before the row
 * is written (SortAndWrite).  Nothing here is blocked, fused or reordered
 * beyond that: products are visited in the stored order of A[i,:] and then of
 * B[k,:].
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC oracle.c
 */
#include "oracle.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>
#include <string.h>

int64_t oracle_row_products(int64_t r0, int64_t r1, const int32_t *a_rp,
                                 const int32_t *a_col, const int32_t *b_rp,
                                 int64_t *P) {
  int64_t total = 0;
  for (int64_t i = r0; i < r1; ++i) {
    int64_t p = 0;
    for (int64_t j = a_rp[i]; j < a_rp[i + 1]; ++j) {
      int32_t k = a_col[j];
      p += (int64_t)b_rp[k + 1] - (int64_t)b_rp[k];
    }
    P[i - r0] = p;
    total += p;
  }
  return total;
}

int oracle_symbolic(int64_t r0, int64_t r1, int64_t n, const int32_t *a_rp,
                    const int32_t *a_col, const int32_t *b_rp,
                    const int32_t *b_col, int64_t *cnt, int nthreads) {
  int failed = 0;
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
  {
    int64_t *mark = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
    if (!mark) {
#pragma omp atomic write
      failed = 1;
    } else {
      for (int64_t c = 0; c < n; ++c) mark[c] = -1;
    }
    /* Every thread takes part in the work-sharing loop, also one whose
     * allocation failed, so that the loop's implicit barrier is reached. */
#pragma omp for schedule(dynamic, 64)
    for (int64_t i = r0; i < r1; ++i) {
      if (!mark) continue;
      {
        int64_t count = 0;
        for (int64_t j = a_rp[i]; j < a_rp[i + 1]; ++j) {
          int32_t k = a_col[j];
          for (int64_t b = b_rp[k]; b < b_rp[k + 1]; ++b) {
            int32_t c = b_col[b];
            if (mark[c] != i) {
              mark[c] = i;
              ++count;
            }
          }
        }
        cnt[i - r0] = count;
      }
    }
    free(mark);
  }
  return failed ? -1 : 0;
}

static int cmp_i32(const void *x, const void *y) {
  int32_t a = *(const int32_t *)x, b = *(const int32_t *)y;
  return (a > b) - (a < b);
}

/* Per-thread scratch of the row accumulation: a dense accumulator over all
 * columns, its Neumaier compensation, the sum of |terms|, the number of
 * terms, a row stamp and the list of touched columns. */
typedef struct {
  double *acc, *cmp, *mag;
  int32_t *terms;
  int64_t *mark;
  int32_t *touched;
} row_scratch;

static int scratch_init(row_scratch *w, int64_t n) {
  size_t nn = (size_t)(n > 0 ? n : 1);
  w->acc = (double *)malloc(sizeof(double) * nn);
  w->cmp = (double *)malloc(sizeof(double) * nn);
  w->mag = (double *)malloc(sizeof(double) * nn);
  w->terms = (int32_t *)malloc(sizeof(int32_t) * nn);
  w->mark = (int64_t *)malloc(sizeof(int64_t) * nn);
  w->touched = (int32_t *)malloc(sizeof(int32_t) * nn);
  if (!(w->acc && w->cmp && w->mag && w->terms && w->mark && w->touched)) return 0;
  for (int64_t c = 0; c < n; ++c) w->mark[c] = -1;
  return 1;
}

static void scratch_free(row_scratch *w) {
  free(w->acc);
  free(w->cmp);
  free(w->mag);
  free(w->terms);
  free(w->mark);
  free(w->touched);
}

/* Row i of C = A*B into the scratch: every product A[i,k]*B[k,j] in the
 * stored order of A[i,:] and then of B[k,:], added into column j; the
 * touched columns are sorted at the end (SortAndWrite).  The value of
 * column touched[e] is acc + cmp.  Returns the number of columns. */
static int64_t accumulate_row(int64_t i, const int32_t *a_rp, const int32_t *a_col,
                              const void *a_val, const int32_t *b_rp,
                              const int32_t *b_col, const void *b_val, int val_is_f32,
                              row_scratch *w) {
  const double *ad = (const double *)a_val, *bd = (const double *)b_val;
  const float *af = (const float *)a_val, *bf = (const float *)b_val;
  double *acc = w->acc, *cmp = w->cmp, *mag = w->mag;
  int32_t *terms = w->terms, *touched = w->touched;
  int64_t *mark = w->mark;
  int64_t nt = 0;
  for (int64_t j = a_rp[i]; j < a_rp[i + 1]; ++j) {
    int32_t k = a_col[j];
    double a = val_is_f32 ? (double)af[j] : ad[j];
    for (int64_t b = b_rp[k]; b < b_rp[k + 1]; ++b) {
      int32_t c = b_col[b];
      double p = a * (val_is_f32 ? (double)bf[b] : bd[b]);
      if (mark[c] != i) {
        mark[c] = i;
        acc[c] = 0.0;
        cmp[c] = 0.0;
        mag[c] = 0.0;
        terms[c] = 0;
        touched[nt++] = c;
      }
      /* Neumaier's compensated addition of p into (acc, cmp). */
      double s = acc[c];
      double t = s + p;
      if (fabs(s) >= fabs(p))
        cmp[c] += (s - t) + p;
      else
        cmp[c] += (p - t) + s;
      acc[c] = t;
      mag[c] += fabs(p);
      terms[c] += 1;
    }
  }
  qsort(touched, (size_t)nt, sizeof(int32_t), cmp_i32);
  return nt;
}

int oracle_numeric(int64_t r0, int64_t r1, int64_t n, const int32_t *a_rp,
                   const int32_t *a_col, const void *a_val, const int32_t *b_rp,
                   const int32_t *b_col, const void *b_val, int val_is_f32,
                   const int64_t *c_rp, int32_t *c_col, double *c_val,
                   double *c_mag, int32_t *c_terms, int nthreads) {
  int status = 0;
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
  {
    row_scratch w;
    int ok = scratch_init(&w, n);
    if (!ok) {
#pragma omp critical
      status = -1;
    }
#pragma omp for schedule(dynamic, 64)
    for (int64_t i = r0; i < r1; ++i) {
      if (!ok) continue;
      {
        const int64_t nt = accumulate_row(i, a_rp, a_col, a_val, b_rp, b_col, b_val,
                                          val_is_f32, &w);
        int64_t base = c_rp[i - r0];
        if (c_rp[i - r0 + 1] - base != nt) {
#pragma omp critical
          status = -2;
          continue;
        }
        for (int64_t e = 0; e < nt; ++e) {
          int32_t c = w.touched[e];
          c_col[base + e] = c;
          c_val[base + e] = w.acc[c] + w.cmp[c];
          if (c_mag) c_mag[base + e] = w.mag[c];
          if (c_terms) c_terms[base + e] = w.terms[c];
        }
      }
    }
    scratch_free(&w);
  }
  return status;
}

int64_t oracle_check_rows(int64_t r0, int64_t r1, int64_t n, const int32_t *a_rp,
                          const int32_t *a_col, const void *a_val, const int32_t *b_rp,
                          const int32_t *b_col, const void *b_val, int val_is_f32,
                          const int64_t *g_rp, int64_t g_base, const int32_t *g_col,
                          const void *g_val, int g_val_is_f32, double rtol, int exact,
                          int64_t *report, double *max_rel, int nthreads) {
  int64_t bad_rows = 0, bad_vals = 0, first_row = -1, first_val = -1, entries = 0;
  int64_t max_terms = 0;
  double worst = 0.0;
  int failed = 0;
  if (nthreads <= 0) nthreads = omp_get_max_threads();
  const double *gd = (const double *)g_val;
  const float *gf = (const float *)g_val;
#pragma omp parallel num_threads(nthreads)
  {
    row_scratch w;
    int ok = scratch_init(&w, n);
    int64_t br = 0, bv = 0, fr = -1, fv = -1, ne = 0, mt = 0;
    double wr = 0.0;
    if (!ok) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 64)
    for (int64_t i = r0; i < r1; ++i) {
      if (!ok) continue;
      const int64_t nt = accumulate_row(i, a_rp, a_col, a_val, b_rp, b_col, b_val,
                                        val_is_f32, &w);
      const int64_t g0 = g_rp[i - r0] - g_base, g1 = g_rp[i - r0 + 1] - g_base;
      int row_ok = (g1 - g0 == nt);
      for (int64_t e = 0; row_ok && e < nt; ++e) row_ok = (g_col[g0 + e] == w.touched[e]);
      if (!row_ok) {
        ++br;
        if (fr < 0 || i < fr) fr = i;
        continue;
      }
      ne += nt;
      for (int64_t e = 0; e < nt; ++e) {
        const int32_t c = w.touched[e];
        const double ref = w.acc[c] + w.cmp[c];
        const double g = g_val_is_f32 ? (double)gf[g0 + e] : gd[g0 + e];
        const double d = fabs(g - ref);
        const int good = exact ? (g == ref) : (d <= rtol * w.mag[c]);
        if (w.terms[c] > mt) mt = w.terms[c];
        if (ref != 0.0 && d / fabs(ref) > wr) wr = d / fabs(ref);
        if (!good) {
          ++bv;
          if (fv < 0 || g_rp[i - r0] + e < fv) fv = g_rp[i - r0] + e;
        }
      }
    }
#pragma omp critical
    {
      bad_rows += br;
      bad_vals += bv;
      entries += ne;
      if (fr >= 0 && (first_row < 0 || fr < first_row)) first_row = fr;
      if (fv >= 0 && (first_val < 0 || fv < first_val)) first_val = fv;
      if (mt > max_terms) max_terms = mt;
      if (wr > worst) worst = wr;
    }
    scratch_free(&w);
  }
  if (failed) return -1;
  report[0] = bad_rows;
  report[1] = first_row;
  report[2] = bad_vals;
  report[3] = first_val;
  report[4] = entries;
  report[5] = max_terms;
  if (max_rel) *max_rel = worst;
  return bad_rows + bad_vals;
}

int64_t oracle_prune_colnorm(int64_t m, int64_t n, const int64_t *c_rp,
                             const int32_t *c_col, const double *c_val,
                             float threshold, const int8_t *keep,
                             int64_t *out_rp, int32_t *out_col,
                             double *out_val) {
  double *colsum = (double *)calloc((size_t)(n > 0 ? n : 1), sizeof(double));
  if (!colsum) return -1;
  int64_t w = 0;
  out_rp[0] = 0;
  for (int64_t i = 0; i < m; ++i) {
    for (int64_t e = c_rp[i]; e < c_rp[i + 1]; ++e) {
      int k;
      if (keep && keep[e] >= 0)
        k = keep[e];
      else
        k = ((float)c_val[e] >= threshold);
      if (k) {
        out_col[w] = c_col[e];
        out_val[w] = c_val[e];
        colsum[c_col[e]] += c_val[e];
        ++w;
      }
    }
    out_rp[i + 1] = w;
  }
  for (int64_t e = 0; e < w; ++e) out_val[e] = out_val[e] / colsum[out_col[e]];
  free(colsum);
  return w;
}

/* MCL iteration tail (Trident page, §5.7): normalise the columns, prune the
 * normalised entries below the threshold, square the rest. */
int64_t oracle_mcl_inflate(int64_t m, int64_t n, const int64_t *c_rp,
                           const int32_t *c_col, const double *c_val,
                           double threshold, int single, const int8_t *keep,
                           int64_t *out_rp, int32_t *out_col, double *out_val) {
  double *colsum = (double *)calloc((size_t)(n > 0 ? n : 1), sizeof(double));
  if (!colsum) return -1;
  for (int64_t i = 0; i < m; ++i)
    for (int64_t e = c_rp[i]; e < c_rp[i + 1]; ++e) colsum[c_col[e]] += c_val[e];
  int64_t w = 0;
  out_rp[0] = 0;
  for (int64_t i = 0; i < m; ++i) {
    for (int64_t e = c_rp[i]; e < c_rp[i + 1]; ++e) {
      const double s = colsum[c_col[e]];
      const double y64 = s != 0.0 ? c_val[e] / s : 0.0;
      int k;
      double z;
      if (single) {
        const float y = (float)y64;
        k = y >= (float)threshold;
        z = (double)(y * y);
      } else {
        k = y64 >= threshold;
        z = y64 * y64;
      }
      if (keep && keep[e] >= 0) k = keep[e];
      if (k) {
        out_col[w] = c_col[e];
        out_val[w] = z;
        ++w;
      }
    }
    out_rp[i + 1] = w;
  }
  free(colsum);
  return w;
}

/* T = A^T by the definition T[j, i] = A[i, j]: count the entries of every
 * column, turn the counts into row starts of T, then place the entries of A
 * row by row (rising i), each at the next free position of its column. */
int oracle_transpose(int64_t m, int64_t n, const int64_t *a_rp,
                     const int32_t *a_col, const void *a_val, int val_is_f32,
                     int64_t *t_rp, int32_t *t_col, void *t_val) {
  int64_t *next = (int64_t *)calloc((size_t)(n > 0 ? n : 1), sizeof(int64_t));
  if (!next) return -1;
  const int64_t nnz = a_rp[m];
  for (int64_t e = 0; e < nnz; ++e) {
    if (a_col[e] < 0 || a_col[e] >= n) {
      free(next);
      return -2;
    }
    next[a_col[e]] += 1;
  }
  t_rp[0] = 0;
  for (int64_t j = 0; j < n; ++j) {
    t_rp[j + 1] = t_rp[j] + next[j];
    next[j] = t_rp[j];
  }
  for (int64_t i = 0; i < m; ++i) {
    for (int64_t e = a_rp[i]; e < a_rp[i + 1]; ++e) {
      const int64_t q = next[a_col[e]]++;
      t_col[q] = (int32_t)i;
      if (a_val && t_val) {
        if (val_is_f32)
          ((float *)t_val)[q] = ((const float *)a_val)[e];
        else
          ((double *)t_val)[q] = ((const double *)a_val)[e];
      }
    }
  }
  free(next);
  return 0;
}

/* MurmurHash3's 32-bit finaliser (fmix32), as published with MurmurHash3. */
static uint32_t hll_hash(uint32_t x) {
  x ^= x >> 16;
  x *= 0x85ebca6bu;
  x ^= x >> 13;
  x *= 0xc2b2ae35u;
  x ^= x >> 16;
  return x;
}

static int hll_log2(int M) { return M == 32 ? 5 : (M == 64 ? 6 : -1); }

/* Record column c in the registers. */
static void hll_add(uint8_t *regs, int M, int lg, int32_t c) {
  const uint32_t h = hll_hash((uint32_t)c);
  const uint32_t j = h & (uint32_t)(M - 1);
  const uint32_t w = h >> lg; /* 32 - lg significant bits */
  int rank = 32 - lg + 1;
  for (int b = 31 - lg; b >= 0; --b) {
    if ((w >> b) & 1u) {
      rank = (31 - lg) - b + 1;
      break;
    }
  }
  if (regs[j] < rank) regs[j] = (uint8_t)rank;
}

static double hll_value(const uint8_t *regs, int M) {
  double z = 0.0;
  int zeros = 0;
  for (int j = 0; j < M; ++j) {
    z += ldexp(1.0, -(int)regs[j]);
    zeros += regs[j] == 0;
  }
  const double alpha = M == 32 ? 0.697 : 0.709;
  double e = alpha * (double)M * (double)M / z;
  if (e <= 2.5 * M && zeros > 0) e = (double)M * log((double)M / (double)zeros);
  return e;
}

int oracle_hll_sketch(int64_t K, const int32_t *b_rp, const int32_t *b_col,
                      int M, uint8_t *regs) {
  const int lg = hll_log2(M);
  if (lg < 0) return -1;
  for (int64_t k = 0; k < K; ++k) {
    uint8_t *r = regs + k * M;
    memset(r, 0, (size_t)M);
    for (int64_t b = b_rp[k]; b < b_rp[k + 1]; ++b) hll_add(r, M, lg, b_col[b]);
  }
  return 0;
}

int oracle_hll_estimate(int64_t r0, int64_t r1, const int32_t *a_rp,
                        const int32_t *a_col, const int32_t *b_rp,
                        const int32_t *b_col, int M, double *est,
                        uint8_t *regs_out) {
  const int lg = hll_log2(M);
  if (lg < 0) return -1;
  uint8_t regs[64];
  for (int64_t i = r0; i < r1; ++i) {
    memset(regs, 0, sizeof(regs));
    for (int64_t j = a_rp[i]; j < a_rp[i + 1]; ++j) {
      const int32_t k = a_col[j];
      for (int64_t b = b_rp[k]; b < b_rp[k + 1]; ++b) hll_add(regs, M, lg, b_col[b]);
    }
    est[i - r0] = hll_value(regs, M);
    if (regs_out) memcpy(regs_out + (i - r0) * M, regs, (size_t)M);
  }
  return 0;
}
