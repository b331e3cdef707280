// GetMagnusParams (gMAGNUS page, §III-D, Eq. 4-7): heavy threshold, dense
// accumulator width, number of chunks and multisplit levels, computed on the
// host from the column count of C, the local-memory (LDS) budget and the
// byte sizes of C's column index and value types.
//
// Readings taken where the printed formulas are garbled or ambiguous:
//  * Eq. 4.  tau = floor(s_LM / (alpha * (s_col + s_val))) with alpha = 2: a
//    numeric hash table of tau (col, val) entries at load factor 1/alpha
//    fills the LDS budget.  (The printed denominator multiplies the two type
//    sizes, which is dimensionally a byte-squared quantity.)
//  * n_denseNumeric = floor(s_LM / (s_val + 1/8)): a value array plus a one-
//    bit occupancy bitmap per column.  The final chunk width W is that count
//    floored to a power of two, so column -> chunk is a shift.
//  * n_chunksRequired = next_pow2(ceil(ncols / W)), at least 1.  Rounding the
//    count up (not down) keeps every final chunk within W columns, the
//    property the dense accumulator needs; the chunk tuples printed in the
//    page's Tables V and VI follow this rule with W = 4096 and 8192.
//  * Levels (Eq. 7): one level when n_chunksRequired <= n_chunksMax, else
//    ceil(log2 n_req / log2 n_max).  The first levels use n_chunksMax chunks
//    and the last one the remaining factor n_req / n_max^(L-1) (a quotient;
//    the printed subtraction does not reproduce the tables' tuples).
//  * n_chunksMax defaults to 32 and is a power of two >= 2.
//  * n_req == 1 means no multisplit at all (0 levels): a heavy row already
//    fits one W-wide dense accumulator.
#include <stdint.h>

#include "../../include/spgemm.h"

namespace {
int64_t floor_pow2(int64_t x) {
  int64_t p = 1;
  while (p <= x / 2) p *= 2;
  return p;
}
int64_t next_pow2(int64_t x) {
  int64_t p = 1;
  while (p < x) p *= 2;
  return p;
}
bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
int log2_exact(int64_t x) {
  int l = 0;
  while ((int64_t(1) << l) < x) ++l;
  return l;
}
}  // namespace

extern "C" spgemm_status spgemm_compute_params(int64_t ncols, int64_t lds_bytes,
                                               int32_t val_bytes, int32_t col_bytes,
                                               int32_t max_chunks_per_level,
                                               int64_t dense_width, spgemm_params* out) {
  if (!out || ncols < 0 || lds_bytes <= 0 || val_bytes <= 0 || col_bytes <= 0)
    return SPGEMM_ERR_INVALID_ARG;
  const int64_t nmax = max_chunks_per_level ? max_chunks_per_level : 32;
  if (nmax < 2 || !is_pow2(nmax)) return SPGEMM_ERR_INVALID_ARG;
  if (dense_width && !is_pow2(dense_width)) return SPGEMM_ERR_INVALID_ARG;
  spgemm_params p = {};
  const int64_t alpha = 2;
  p.tau = lds_bytes / (alpha * (int64_t)(col_bytes + val_bytes));
  p.n_dense = (8 * lds_bytes) / (8 * (int64_t)val_bytes + 1);
  if (p.tau < 1 || p.n_dense < 1) return SPGEMM_ERR_INVALID_ARG;
  p.dense_width = dense_width ? dense_width : floor_pow2(p.n_dense);
  const int64_t W = p.dense_width;
  const int64_t chunks = (ncols + W - 1) / W;
  p.chunks_required = next_pow2(chunks < 1 ? 1 : chunks);
  p.chunks_max = (int32_t)nmax;
  const int64_t nreq = p.chunks_required;
  if (nreq == 1) {
    p.levels = 0;
  } else if (nreq <= nmax) {
    p.levels = 1;
    p.v_chunks[0] = (int32_t)nreq;
  } else {
    const int lr = log2_exact(nreq), lm = log2_exact(nmax);
    const int L = (lr + lm - 1) / lm;
    if (L > 8) return SPGEMM_ERR_INVALID_ARG;
    p.levels = L;
    int64_t rest = nreq;
    for (int i = 0; i < L - 1; ++i) {
      p.v_chunks[i] = (int32_t)nmax;
      rest /= nmax;
    }
    p.v_chunks[L - 1] = (int32_t)rest;
  }
  // Chunk width after each level: the last level lands on W.
  int64_t w = W;
  for (int i = p.levels - 1; i >= 0; --i) {
    p.level_width[i] = w;
    w *= p.v_chunks[i];
  }
  *out = p;
  return SPGEMM_OK;
}
