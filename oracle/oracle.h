/*
 * CPU oracle for sparse general matrix-matrix multiplication, C = A*B, CSR.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this library; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no source with the HIP library.
 *
 * What it computes (gMAGNUS page, §II-B, Eq. 1 and Algorithm 1):
 *   C[i, j] = sum over stored pairs A[i,k], B[k,j] of A[i,k] * B[k,j].
 * An entry (i, j) exists iff at least one stored pair meets (structural
 * definition: a computed 0.0 is kept).  Columns of each row of C are emitted
 * sorted ascending without duplicates (the SortAndWrite step of Algorithm 1).
 *
 * Arithmetic: each product is rounded once to fp64 (inputs in fp32 are
 * widened first, so their products are exact), then summed in fp64 with
 * Neumaier compensation, so the returned value is close to the exact sum.
 * The library is compiled with -ffp-contract=off.
 *
 * Index conventions: row pointers of A and B are int32, column indices int32.
 * Rows are processed in [r0, r1); per-row outputs are indexed i - r0.
 */
#ifndef SPGEMM_ORACLE_H
#define SPGEMM_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* P[i - r0] = number of intermediate products of row i, the sum over k in
 * A[i,:] of nnz(B[k,:]) (stored zeros counted).  Returns the total. */
int64_t oracle_row_products(int64_t r0, int64_t r1, const int32_t *a_rp,
                            const int32_t *a_col, const int32_t *b_rp,
                            int64_t *P);

/* cnt[i - r0] = nnz(C[i,:]) = |union over k in A[i,:] of cols(B[k,:])|.
 * n = number of columns of B.  Returns 0, or -1 on allocation failure. */
int oracle_symbolic(int64_t r0, int64_t r1, int64_t n, const int32_t *a_rp,
                    const int32_t *a_col, const int32_t *b_rp,
                    const int32_t *b_col, int64_t *cnt, int nthreads);

/* Fills rows [r0, r1) of C at the local offsets c_rp[0..r1-r0] (c_rp[0] may
 * be nonzero; row i occupies [c_rp[i-r0], c_rp[i-r0+1]) ).
 * val_is_f32: 0 -> a_val/b_val are double, 1 -> float.
 * c_val: compensated fp64 value.  c_mag (optional): sum of |A[i,k]*B[k,j]|,
 * the natural scale for a summation-order tolerance.  c_terms (optional):
 * number of products summed into the entry.
 * Returns 0, -1 on allocation failure, -2 if a row's size disagrees with c_rp.
 */
int oracle_numeric(int64_t r0, int64_t r1, int64_t n, const int32_t *a_rp,
                   const int32_t *a_col, const void *a_val, const int32_t *b_rp,
                   const int32_t *b_col, const void *b_val, int val_is_f32,
                   const int64_t *c_rp, int32_t *c_col, double *c_val,
                   double *c_mag, int32_t *c_terms, int nthreads);

/* Row-by-row comparison of another implementation's C with this oracle,
 * for rows [r0, r1) of A*B, without materialising the oracle's C: every row
 * is computed as oracle_numeric computes it and compared at once.  The other
 * C is given by g_rp[0..r1-r0] (absolute offsets of rows r0..r1), and g_col,
 * g_val holding the entries from offset g_base on (g_val_is_f32 selects
 * float or double).  A row is bad when its length or any column differs; a
 * value is bad when |g - c| > rtol * sum of |terms| (exact: g != c), c being
 * the compensated oracle value.  report[0..5]: bad rows, first bad row (-1
 * if none), bad values, offset of the first bad value (-1 if none), entries
 * compared, most terms summed into one entry.  *max_rel (may be NULL): the
 * largest |g - c| / |c| over compared entries with c != 0.  Returns bad
 * rows + bad values, or -1 when out of memory. */
int64_t oracle_check_rows(int64_t r0, int64_t r1, int64_t n, const int32_t *a_rp,
                          const int32_t *a_col, const void *a_val, const int32_t *b_rp,
                          const int32_t *b_col, const void *b_val, int val_is_f32,
                          const int64_t *g_rp, int64_t g_base, const int32_t *g_col,
                          const void *g_val, int g_val_is_f32, double rtol, int exact,
                          int64_t *report, double *max_rel, int nthreads);

/* One Markov-clustering prune + column renormalisation (Trident page, §5.7):
 * keep entry (i,j) iff (float)c_val >= threshold (compared in fp32; keep[]
 * overrides the decision where keep[e] is 0 or 1, and is ignored where it is
 * -1 or keep == NULL); then divide every kept entry by the fp64 sum of the
 * kept entries of its column.  Output arrays are sized by the caller at
 * nnz(C); out_rp has m+1 entries.  Returns the number of kept entries. */
int64_t oracle_prune_colnorm(int64_t m, int64_t n, const int64_t *c_rp,
                             const int32_t *c_col, const double *c_val,
                             float threshold, const int8_t *keep,
                             int64_t *out_rp, int32_t *out_col,
                             double *out_val);

/* The rest of one Markov-clustering iteration after the expansion (Trident
 * page, §5.7): s_j = sum of every entry of column j (fp64, in row order);
 * y = C[i,j] / s_j in fp64, rounded to fp32 when single != 0 (0 when s_j is
 * 0); keep y >= threshold (compared in fp32 when single, else in fp64);
 * output y * y (computed in fp32 when single).  keep (may be NULL) overrides
 * the decision of entry e when keep[e] >= 0.  out arrays as for
 * oracle_prune_colnorm.  Returns the kept count, or -1 if out of memory. */
int64_t oracle_mcl_inflate(int64_t m, int64_t n, const int64_t *c_rp,
                           const int32_t *c_col, const double *c_val,
                           double threshold, int single, const int8_t *keep,
                           int64_t *out_rp, int32_t *out_col, double *out_val);

/* Transpose of an m x n CSR matrix: T[j, i] = A[i, j] for every stored
 * entry (the operand of the rectangular product A * A^T that the Ocean page,
 * "Ocean: Fast Estimation-Based Sparse General Matrix-Matrix Multiplication
 * on GPU", evaluates on its rectangular matrix set).  Stored entries are
 * visited row by row with rising i, so every row of T lists its column
 * indices in rising order.  a_val / t_val may be NULL (pattern only);
 * val_is_f32 selects float or double for both.  t_rp has n+1 entries; t_col
 * and t_val are sized by the caller at nnz(A).  Returns 0, -1 when out of
 * memory, -2 when a column index lies outside [0, n). */
int oracle_transpose(int64_t m, int64_t n, const int64_t *a_rp,
                     const int32_t *a_col, const void *a_val, int val_is_f32,
                     int64_t *t_rp, int32_t *t_col, void *t_val);

/* HyperLogLog size estimation (Ocean page, "Ocean: Fast Estimation-Based
 * Sparse General Matrix-Matrix Multiplication on GPU", §3: one sketch of M
 * one-byte registers per row of B, merged by element-wise maximum over the
 * B rows an A row references, then the estimate of the merged sketch).
 * Hash of a column index: the 32-bit finaliser of MurmurHash3 (fmix32).
 * Register index: the low log2(M) bits of the hash; rank: 1 + the number of
 * leading zeros of the remaining 32 - log2(M) bits (32 - log2(M) + 1 when
 * they are all zero).  Estimate (Flajolet et al.): E = alpha_M * M^2 / Z
 * with Z = sum_j 2^-r_j, alpha_32 = 0.697, alpha_64 = 0.709; when
 * E <= 2.5 M and V > 0 registers are zero, E = M * ln(M / V).
 * oracle_hll_sketch: regs[k*M + j] for the rows k of B (K rows).
 * oracle_hll_estimate: est[i - r0] for rows [r0, r1) of A*B, computed
 * from the columns of the row's products directly (no per-B-row sketches),
 * and, when regs_out is not NULL, the row's registers.  M is 32 or 64.
 * Returns 0, or -1 for an unsupported M. */
int oracle_hll_sketch(int64_t K, const int32_t *b_rp, const int32_t *b_col,
                      int M, uint8_t *regs);
int oracle_hll_estimate(int64_t r0, int64_t r1, const int32_t *a_rp,
                        const int32_t *a_col, const int32_t *b_rp,
                        const int32_t *b_col, int M, double *est,
                        uint8_t *regs_out);

#ifdef __cplusplus
}
#endif
#endif
