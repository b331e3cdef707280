// Heavy-row path of gMAGNUS (gMAGNUS page, §III-A..§III-E):
//   masked CSR -> CSC of A restricted to the heavy rows (Algorithm 3 setup),
//   the outer product that expands the heavy rows into C-hat (§III-B, Eq. 2),
//   per-level histogram + heavy-first chunk partition + multisplit (§III-C),
//   dense LDS accumulation of the W-wide heavy chunks (§III-E), and the
//   per-row assembly of chunk offsets.
#include "device_common.hpp"

namespace sg {
namespace {

constexpr int kNT = 256;
inline unsigned grid_for(int64_t n, int per_block) {
  int64_t g = (n + per_block - 1) / per_block;
  return (unsigned)(g < 1 ? 1 : g);
}

// --------------------------------------------------------------- CSC of A~
// One wave per heavy row: count its entries per column.
__global__ __launch_bounds__(kNT) void k_csc_count(int64_t h, const int32_t* __restrict__ xheavy,
                                                   const int32_t* __restrict__ arp,
                                                   const int32_t* __restrict__ acol,
                                                   int32_t* __restrict__ colCnt) {
  const int64_t r = ((int64_t)blockIdx.x * kNT + threadIdx.x) / kWave;
  if (r >= h) return;
  const int32_t row = xheavy[r];
  const int64_t re = arp[row + 1];
  for (int64_t j = arp[row] + lane_id(); j < re; j += kWave) atomicAdd(&colCnt[acol[j]], 1);
}

// Scatter each heavy-row entry into its column: row = heavy index, column,
// value.  Order inside a column follows the atomics (immaterial: it only
// changes the order of segments inside a row of C-hat).
template <typename V>
__global__ __launch_bounds__(kNT) void k_csc_fill(int64_t h, const int32_t* __restrict__ xheavy,
                                                  const int32_t* __restrict__ arp,
                                                  const int32_t* __restrict__ acol,
                                                  const V* __restrict__ aval,
                                                  int64_t* __restrict__ colFill,
                                                  int32_t* __restrict__ cscRow,
                                                  int32_t* __restrict__ cscCol,
                                                  V* __restrict__ cscVal) {
  const int64_t r = ((int64_t)blockIdx.x * kNT + threadIdx.x) / kWave;
  if (r >= h) return;
  const int32_t row = xheavy[r];
  const int64_t re = arp[row + 1];
  for (int64_t j = arp[row] + lane_id(); j < re; j += kWave) {
    const int32_t k = acol[j];
    const int64_t pos = (int64_t)atomicAdd((unsigned long long*)&colFill[k], 1ull);
    cscRow[pos] = (int32_t)r;
    cscCol[pos] = k;
    cscVal[pos] = aval[j];
  }
}

__global__ __launch_bounds__(kNT) void k_entry_products(int64_t nE, const int32_t* __restrict__ cscCol,
                                                        const int32_t* __restrict__ brp,
                                                        int64_t* __restrict__ nb) {
  const int64_t e = (int64_t)blockIdx.x * kNT + threadIdx.x;
  if (e >= nE) return;
  const int32_t k = cscCol[e];
  nb[e] = (int64_t)brp[k + 1] - brp[k];
}

// Reserve, for every CSC entry (one scaled row of B), a contiguous segment
// of its C-hat row: the atomic's return value is where the segment starts.
__global__ __launch_bounds__(kNT) void k_seg_base(int64_t nE, const int32_t* __restrict__ cscRow,
                                                  const int64_t* __restrict__ nb,
                                                  int64_t* __restrict__ cursor,
                                                  int64_t* __restrict__ segBase) {
  const int64_t e = (int64_t)blockIdx.x * kNT + threadIdx.x;
  if (e >= nE) return;
  const int64_t n = nb[e];
  segBase[e] = n ? (int64_t)atomicAdd((unsigned long long*)&cursor[cscRow[e]],
                                      (unsigned long long)n)
                 : 0;
}

// ----------------------------------------------------------- outer product
// The flattened element space [0, P_h) lists, slice by slice (column k of A~
// times row k of B), one segment of nnz(B[k,:]) products per CSC entry.
// Each work group owns a static range of kOpBlock elements; each wave owns a
// contiguous quarter of it.  A wave keeps 64 consecutive CSC entries in
// registers, maps each of 64 consecutive elements to its entry by a 6-step
// binary search across lanes, and writes col_B and val_A*val_B to
// segBase[entry] + (position inside the segment).  Consecutive elements of
// a segment read consecutive B entries and write consecutive C-hat slots.
constexpr int kOpBlock = 32768;
constexpr int kXcds = 8;

template <typename V>
__global__ __launch_bounds__(kNT) void k_outer_product(int64_t Ph, const int64_t* __restrict__ entryOff,
                                                       int64_t nE, const int32_t* __restrict__ cscCol,
                                                       const V* __restrict__ cscVal,
                                                       const int64_t* __restrict__ segBase,
                                                       const int32_t* __restrict__ brp,
                                                       const int32_t* __restrict__ bcol,
                                                       const V* __restrict__ bval,
                                                       int32_t* __restrict__ outCol,
                                                       V* __restrict__ outVal) {
  constexpr int kNW = kNT / kWave;
  constexpr int kPerWave = kOpBlock / kNW;
  const int w = threadIdx.x / kWave;
  // Work groups are dealt round-robin to the 8 XCDs; give each XCD a
  // contiguous run of tiles so that the B rows shared by neighbouring tiles
  // stay in that XCD's L2.
  const int64_t perXcd = (int64_t)gridDim.x / kXcds;
  const int64_t tile = (int64_t)(blockIdx.x % kXcds) * perXcd + blockIdx.x / kXcds;
  const int64_t g0 = tile * kOpBlock;
  int64_t p = g0 + (int64_t)w * kPerWave;
  int64_t p1 = p + kPerWave;
  if (p1 > Ph) p1 = Ph;
  if (p >= p1) return;
  int64_t j = wave_last_le(entryOff, (int64_t)0, nE, p);
  while (p < p1) {
    const int64_t e = j + lane_id();
    const bool ev = e < nE;
    const int64_t off = ev ? entryOff[e] : Ph;
    int32_t bs = 0;
    V a = V(0);
    int64_t dst = 0;
    if (ev) {
      bs = brp[cscCol[e]];
      a = cscVal[e];
      dst = segBase[e];
    }
    int64_t bend = entryOff[(j + kWave < nE) ? j + kWave : nE];
    if (bend > p1) bend = p1;
    // Four windows of 64 elements per iteration: all their B loads are in
    // flight before the first store.
    constexpr int kU = 4;
    for (; p < bend; p += kWave * kU) {
      int64_t dpos[kU];
      int32_t bidx[kU];
      V av[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t q = p + u * kWave + lane_id();
        int s = 0;
#pragma unroll
        for (int step = 32; step >= 1; step >>= 1) {
          const int64_t o = __shfl(off, s + step);
          if (o <= q) s += step;
        }
        const int64_t so = __shfl(off, s);
        const int32_t sb = __shfl(bs, s);
        av[u] = __shfl(a, s);
        const int64_t sd = __shfl(dst, s);
        const int64_t r = q - so;
        dpos[u] = q < bend ? sd + r : -1;
        bidx[u] = sb + (int32_t)r;
      }
      int32_t cv[kU];
      V bv[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        cv[u] = dpos[u] >= 0 ? bcol[bidx[u]] : 0;
        bv[u] = dpos[u] >= 0 ? bval[bidx[u]] : V(0);
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (dpos[u] >= 0) {
          outCol[dpos[u]] = cv[u];
          outVal[dpos[u]] = av[u] * bv[u];
        }
      }
    }
    p = bend;
    j += kWave;
  }
}

// ------------------------------------------------------------ multisplit
// A work group owns a static range of `blockElems` elements of the level's
// input (heavy rows, or heavy chunks of the previous level, each longer than
// tau).  Local bucket of an element = (row inside the range) * v + chunk,
// chunk = col >> shift.  Bucket ids are matched across the wave with one
// ballot per bit so a single lane per bucket updates the LDS counters.
constexpr int kMsNBMax = 1024;  // LDS buckets per work group
constexpr int kMsRowsMax = 512;
constexpr int kMsItemsF64 = 8;   // elements per thread held in registers
constexpr int kMsItemsF32 = 16;

__device__ __forceinline__ int bits_for(int n) {
  int b = 0;
  while ((1 << b) < n) ++b;
  return b;
}

// Rows of the range [e0, e1): first row r0 and the row boundaries inside the
// range (rowPtr[r0+1 .. r0+nrows-1]) into bnd.  Returns nrows, or -1 when
// more than maxRows rows meet the range.
__device__ __forceinline__ int range_rows(const int64_t* __restrict__ rowPtr, int64_t R, int64_t e0,
                                          int64_t e1, int maxRows, int64_t* bnd, int64_t* s_r0,
                                          int32_t* s_nrows) {
  if (threadIdx.x < kWave) {
    const int64_t r0 = wave_last_le(rowPtr, (int64_t)0, R, e0);
    const int64_t r1 = wave_last_le(rowPtr, (int64_t)0, R, e1 - 1);
    if (lane_id() == 0) {
      *s_r0 = r0;
      *s_nrows = (int32_t)(r1 - r0 + 1);
    }
  }
  __syncthreads();
  const int nrows = *s_nrows;
  if (nrows > maxRows) return -1;
  for (int i = threadIdx.x; i < nrows - 1; i += kNT) bnd[i] = rowPtr[*s_r0 + 1 + i];
  return nrows;
}

__device__ __forceinline__ int local_row(const int64_t* bnd, int nrows, int64_t e) {
  int lo = 0, hi = nrows - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (bnd[mid] <= e)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

// Histogram: per (input row, chunk) element counts into counts[r*v + c].
__global__ __launch_bounds__(kNT) void k_histogram(int64_t E, int32_t blockElems,
                                                   const int64_t* __restrict__ rowPtr, int64_t R,
                                                   const int32_t* __restrict__ col, int shift, int v,
                                                   int maxRows, int32_t* __restrict__ counts,
                                                   int32_t* __restrict__ err) {
  __shared__ int32_t hist[kMsNBMax];
  __shared__ int64_t bnd[kMsRowsMax];
  __shared__ int64_t s_r0;
  __shared__ int32_t s_nrows;
  const int64_t e0 = (int64_t)blockIdx.x * blockElems;
  const int64_t e1 = (e0 + blockElems < E) ? e0 + blockElems : E;
  const int n = (int)(e1 - e0);
  const int nrows = range_rows(rowPtr, R, e0, e1, maxRows, bnd, &s_r0, &s_nrows);
  if (nrows < 0) {
    if (threadIdx.x == 0) flag_error(err, kErrRowsPerBlock);
    return;
  }
  const int NB = nrows * v;
  const int nbits = bits_for(NB);
  for (int i = threadIdx.x; i < NB; i += kNT) hist[i] = 0;
  __syncthreads();
  // All loads of a batch are issued before any is used.
  constexpr int kBatch = 8;
  for (int base = 0; base < n; base += kNT * kBatch) {
    int32_t cc[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int idx = base + k * kNT + threadIdx.x;
      cc[k] = idx < n ? col[e0 + idx] : 0;
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int idx = base + k * kNT + threadIdx.x;
      const bool act = idx < n;
      uint32_t b = 0;
      if (act) b = (uint32_t)(local_row(bnd, nrows, e0 + idx) * v + (cc[k] >> shift));
      const uint64_t m = match_key(b, nbits, act);
      if (act && lane_id() == ffs64(m)) atomicAdd(&hist[b], __popcll(m));
    }
  }
  __syncthreads();
  const int64_t r0 = s_r0;
  for (int i = threadIdx.x; i < NB; i += kNT) {
    const int32_t c = hist[i];
    if (c) {
      const int lr = i / v;
      atomicAdd(&counts[(r0 + lr) * v + (i - lr * v)], c);
    }
  }
}

// Multisplit (§III-C): local histogram, one global reservation per
// (row, chunk) bucket, LDS permute into bucket order, then coalesced writes
// of whole bucket runs with the column shifted into the chunk's range.
template <int ITEMS, typename V>
__global__ __launch_bounds__(kNT) void k_multisplit(int64_t E, int32_t blockElems,
                                                    const int64_t* __restrict__ rowPtr, int64_t R,
                                                    const int32_t* __restrict__ inCol,
                                                    const V* __restrict__ inVal, int shift, int v,
                                                    int32_t wmask, int maxRows,
                                                    const int32_t* __restrict__ inv,
                                                    int64_t* __restrict__ cursor,
                                                    int32_t* __restrict__ outCol,
                                                    V* __restrict__ outVal,
                                                    int32_t* __restrict__ err) {
  // LDS (sized by the host for blockElems elements and maxRows rows):
  // gbase[NB] i64 | bnd[maxRows] i64 | valBuf[blockElems] V |
  // colBuf[blockElems] i32 | hist[NB] i32 | loff[NB] i32 | bktBuf u16
  extern __shared__ __align__(16) unsigned char smem[];
  const int NBcap = maxRows * v;
  int64_t* gbase = (int64_t*)smem;
  int64_t* bnd = gbase + NBcap;
  V* valBuf = (V*)(bnd + maxRows);
  int32_t* colBuf = (int32_t*)(valBuf + blockElems);
  int32_t* hist = colBuf + blockElems;
  int32_t* loff = hist + NBcap;
  uint16_t* bktBuf = (uint16_t*)(loff + NBcap);
  __shared__ int32_t wtot[kNT / kWave];
  __shared__ int64_t s_r0;
  __shared__ int32_t s_nrows;
  const int64_t e0 = (int64_t)blockIdx.x * blockElems;
  const int64_t e1 = (e0 + blockElems < E) ? e0 + blockElems : E;
  const int n = (int)(e1 - e0);
  const int nrows = range_rows(rowPtr, R, e0, e1, maxRows, bnd, &s_r0, &s_nrows);
  if (nrows < 0) {
    if (threadIdx.x == 0) flag_error(err, kErrRowsPerBlock);
    return;
  }
  const int NB = nrows * v;
  const int nbits = bits_for(NB);
  for (int i = threadIdx.x; i < NB; i += kNT) hist[i] = 0;
  __syncthreads();

  int32_t cc[ITEMS];
  V xv[ITEMS];
  uint32_t bb[ITEMS];
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const int idx = it * kNT + threadIdx.x;
    const bool act = idx < n;
    cc[it] = 0;
    xv[it] = V(0);
    bb[it] = 0;
    if (act) {
      const int64_t e = e0 + idx;
      cc[it] = inCol[e];
      xv[it] = inVal[e];
      bb[it] = (uint32_t)(local_row(bnd, nrows, e) * v + (cc[it] >> shift));
    }
  }
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const bool act = it * kNT + (int)threadIdx.x < n;
    const uint64_t m = match_key(bb[it], nbits, act);
    if (act && lane_id() == ffs64(m)) atomicAdd(&hist[bb[it]], __popcll(m));
  }
  __syncthreads();

  // Exclusive scan of the bucket counts (4 buckets per thread).
  {
    int32_t h4[4];
    int32_t sum = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int b = threadIdx.x * 4 + k;
      h4[k] = b < NB ? hist[b] : 0;
      sum += h4[k];
    }
    int32_t tot;
    int32_t ex = block_excl_scan<kNT>(sum, wtot, &tot);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int b = threadIdx.x * 4 + k;
      if (b < NB) loff[b] = ex;
      ex += h4[k];
    }
  }
  __syncthreads();
  const int64_t r0 = s_r0;
  for (int b = threadIdx.x; b < NB; b += kNT) {
    const int32_t c = hist[b];
    if (c) {
      const int lr = b / v;
      const int32_t q = inv[(r0 + lr) * v + (b - lr * v)];
      gbase[b] = (int64_t)atomicAdd((unsigned long long*)&cursor[q], (unsigned long long)c);
    }
    hist[b] = loff[b];
  }
  __syncthreads();

#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const bool act = it * kNT + (int)threadIdx.x < n;
    const uint64_t m = match_key(bb[it], nbits, act);
    const int leader = act ? ffs64(m) : lane_id();
    int32_t base = 0;
    if (act && lane_id() == leader) base = atomicAdd(&hist[bb[it]], __popcll(m));
    base = __shfl(base, leader);
    if (act) {
      const int pos = base + __popcll(m & lanemask_lt());
      colBuf[pos] = cc[it] & wmask;
      valBuf[pos] = xv[it];
      bktBuf[pos] = (uint16_t)bb[it];
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < n; idx += kNT) {
    const int b = bktBuf[idx];
    const int64_t dest = gbase[b] + (idx - loff[b]);
    outCol[dest] = colBuf[idx];
    outVal[dest] = valBuf[idx];
  }
}

// Heavy-first placement of the chunks of one level: chunks with more than
// tau elements (only before the last level) go to the front, in any order;
// other non-empty chunks go to the back; empty chunks leave their (zeroed)
// count in the middle.  inv[q] = new position of chunk q (or -1).
__global__ __launch_bounds__(kNT) void k_partition(int64_t Q, const int32_t* __restrict__ counts,
                                                   int64_t tau, int last, int v,
                                                   const int32_t* __restrict__ inRow,
                                                   const int32_t* __restrict__ inSlot,
                                                   int32_t slotStep, int32_t* __restrict__ inv,
                                                   int32_t* __restrict__ newCnt,
                                                   int32_t* __restrict__ newRow,
                                                   int32_t* __restrict__ newSlot,
                                                   int32_t* __restrict__ ctr) {
  const int64_t q = (int64_t)blockIdx.x * kNT + threadIdx.x;
  const bool act = q < Q;
  const int32_t cnt = act ? counts[q] : 0;
  const bool heavy = act && !last && cnt > tau;
  const bool light = act && !heavy && cnt > 0;
  const uint64_t mh = __ballot(heavy), ml = __ballot(light);
  int32_t bh = 0, bl = 0;
  if (lane_id() == 0) {
    if (mh) bh = atomicAdd(&ctr[0], __popcll(mh));
    if (ml) bl = atomicAdd(&ctr[1], __popcll(ml));
  }
  bh = __shfl(bh, 0);
  bl = __shfl(bl, 0);
  int64_t pos = -1;
  if (heavy) pos = bh + __popcll(mh & lanemask_lt());
  if (light) pos = Q - 1 - (bl + __popcll(ml & lanemask_lt()));
  if (act) {
    inv[q] = (int32_t)pos;
    if (pos >= 0) {
      const int64_t r = q / v;
      const int32_t c = (int32_t)(q - r * v);
      newCnt[pos] = cnt;
      newRow[pos] = inRow ? inRow[r] : (int32_t)r;
      newSlot[pos] = (inSlot ? inSlot[r] : 0) + c * slotStep;
    }
  }
}

__global__ __launch_bounds__(kNT) void k_final_from_level(int64_t first, int64_t n,
                                                          const int64_t* __restrict__ newOff,
                                                          const int32_t* __restrict__ newCnt,
                                                          const int32_t* __restrict__ newRow,
                                                          const int32_t* __restrict__ newSlot,
                                                          int8_t buf, int64_t dst0,
                                                          int64_t* __restrict__ fcOff,
                                                          int32_t* __restrict__ fcCnt,
                                                          int32_t* __restrict__ fcRow,
                                                          int32_t* __restrict__ fcSlot,
                                                          int8_t* __restrict__ fcBuf) {
  const int64_t i = (int64_t)blockIdx.x * kNT + threadIdx.x;
  if (i >= n) return;
  const int64_t pos = first + i, d = dst0 + i;
  fcOff[d] = newOff[pos];
  fcCnt[d] = newCnt[pos];
  fcRow[d] = newRow[pos];
  fcSlot[d] = newSlot[pos];
  fcBuf[d] = buf;
}

__global__ __launch_bounds__(kNT) void k_final_from_rows(int64_t h, const int64_t* __restrict__ rowPtr,
                                                         int64_t* __restrict__ fcOff,
                                                         int32_t* __restrict__ fcCnt,
                                                         int32_t* __restrict__ fcRow,
                                                         int32_t* __restrict__ fcSlot,
                                                         int8_t* __restrict__ fcBuf) {
  const int64_t r = (int64_t)blockIdx.x * kNT + threadIdx.x;
  if (r >= h) return;
  fcOff[r] = rowPtr[r];
  fcCnt[r] = (int32_t)(rowPtr[r + 1] - rowPtr[r]);
  fcRow[r] = (int32_t)r;
  fcSlot[r] = 0;
  fcBuf[r] = 0;
}

__global__ __launch_bounds__(kNT) void k_chunk_bins(int64_t nfc, const int32_t* __restrict__ fcCnt,
                                                    int64_t lastFirst, int64_t tau,
                                                    const int32_t* __restrict__ caps, int nbins,
                                                    int denseBin, uint8_t* __restrict__ key,
                                                    int64_t* __restrict__ denseElems) {
  const int64_t i = (int64_t)blockIdx.x * kNT + threadIdx.x;
  if (i >= nfc) return;
  const int32_t c = fcCnt[i];
  if (i >= lastFirst && c > tau) {
    key[i] = (uint8_t)denseBin;
    if (denseElems) atomicAdd((unsigned long long*)denseElems, (unsigned long long)c);
    return;
  }
  int b = 0;
  while (b < nbins - 1 && c > caps[b]) ++b;
  key[i] = (uint8_t)b;
}

// ------------------------------------------------- dense LDS accumulators
// Symbolic: a W-bit LDS bitmap per chunk (read before or-ing, so repeated
// columns cost a read only), then a popcount.
__global__ __launch_bounds__(kNT) void k_dense_sym(const int32_t* __restrict__ items, ChunkList cl,
                                                   int32_t* __restrict__ err) {
  extern __shared__ __align__(16) uint32_t bm[];
  __shared__ int32_t wsum[kNT / kWave];
  const int nwords = (int)((cl.W + 31) / 32);
  const int32_t item = items[blockIdx.x];
  for (int i = threadIdx.x; i < nwords; i += kNT) bm[i] = 0;
  __syncthreads();
  const int64_t off = cl.off[item], end = off + cl.cnt[item];
  const int32_t* __restrict__ col = cl.buf[item] ? cl.col1 : cl.col0;
  for (int64_t e = off + threadIdx.x; e < end; e += kNT) {
    const int32_t c = col[e];
    const uint32_t bit = 1u << (c & 31);
    if (!(bm[c >> 5] & bit)) atomicOr(&bm[c >> 5], bit);
  }
  __syncthreads();
  int32_t mine = 0;
  for (int i = threadIdx.x; i < nwords; i += kNT) mine += __popc(bm[i]);
  mine = wave_sum(mine);
  if (lane_id() == 0) wsum[threadIdx.x / kWave] = mine;
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t t = 0;
    for (int i = 0; i < kNT / kWave; ++i) t += wsum[i];
    cl.slotNnz[(int64_t)cl.row[item] * cl.nreq + cl.slot[item]] = t;
  }
  (void)err;
}

// Numeric: val[W] + W-bit bitmap in LDS; LDS atomic adds; then every thread
// owns W/1024 consecutive columns, a work-group scan of their popcounts
// gives each thread its output position, and set bits are written in column
// order: the chunk comes out sorted and compacted.
constexpr int kDenseNT = 1024;
template <typename V>
__global__ __launch_bounds__(kDenseNT) void k_dense_num(const int32_t* __restrict__ items, ChunkList cl,
                                                        const int64_t* __restrict__ cRowOff,
                                                        int32_t* __restrict__ ccol,
                                                        V* __restrict__ cval,
                                                        int32_t* __restrict__ err) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int W = (int)cl.W;
  const int nwords = (W + 31) / 32;
  V* vals = (V*)smem;
  uint32_t* bm = (uint32_t*)(vals + W);
  int32_t* wtot = (int32_t*)(bm + nwords);
  const int32_t item = items[blockIdx.x];
  for (int i = threadIdx.x; i < W; i += kDenseNT) vals[i] = V(0);
  for (int i = threadIdx.x; i < nwords; i += kDenseNT) bm[i] = 0;
  __syncthreads();
  const int64_t off = cl.off[item], end = off + cl.cnt[item];
  const bool b1 = cl.buf[item] != 0;
  const int32_t* __restrict__ col = b1 ? cl.col1 : cl.col0;
  const V* __restrict__ val = (const V*)(b1 ? cl.val1 : cl.val0);
  constexpr int kB = 8;  // loads in flight per thread
  for (int64_t e0 = off + threadIdx.x; e0 < end; e0 += (int64_t)kDenseNT * kB) {
    int32_t cc[kB];
    V vv[kB];
#pragma unroll
    for (int k = 0; k < kB; ++k) {
      const int64_t e = e0 + (int64_t)k * kDenseNT;
      cc[k] = e < end ? col[e] : -1;
      vv[k] = e < end ? val[e] : V(0);
    }
#pragma unroll
    for (int k = 0; k < kB; ++k) {
      const int32_t c = cc[k];
      if (c >= 0) {
        atomicAdd(&vals[c], vv[k]);
        const uint32_t bit = 1u << (c & 31);
        if (!(bm[c >> 5] & bit)) atomicOr(&bm[c >> 5], bit);
      }
    }
  }
  __syncthreads();
  const int cpt = W >= kDenseNT ? W / kDenseNT : 1;  // columns per thread, <= 32
  const int c0 = threadIdx.x * cpt;
  uint32_t bits = 0;
  if (c0 < W) {
    const uint32_t word = bm[c0 >> 5];
    bits = (cpt >= 32) ? word : ((word >> (c0 & 31)) & ((1u << cpt) - 1u));
  }
  int32_t total;
  int32_t pos = block_excl_scan<kDenseNT>((int32_t)__popc(bits), wtot, &total);
  const int64_t hr = cl.row[item];
  const int64_t sidx = hr * cl.nreq + cl.slot[item];
  const int64_t base = cRowOff[cl.xheavy[hr]] + cl.slotOff[sidx];
  const int32_t want = cl.slotNnz[sidx];
  if (threadIdx.x == 0 && want != total) flag_error(err, kErrCountMismatch);
  const int32_t colBase = (int32_t)((int64_t)cl.slot[item] * cl.W);
  while (bits) {
    const int b = __ffs(bits) - 1;
    bits &= bits - 1;
    if (pos < want) {
      ccol[base + pos] = colBase + c0 + b;
      cval[base + pos] = vals[c0 + b];
    }
    ++pos;
  }
}

// One wave per heavy row: exclusive scan of its slot counts.
__global__ __launch_bounds__(kNT) void k_slot_scan(int64_t h, int64_t nreq,
                                                   const int32_t* __restrict__ slotNnz,
                                                   int64_t* __restrict__ slotOff,
                                                   const int32_t* __restrict__ xheavy,
                                                   int64_t* __restrict__ cnt) {
  const int64_t r = ((int64_t)blockIdx.x * kNT + threadIdx.x) / kWave;
  if (r >= h) return;
  int64_t carry = 0;
  for (int64_t b = 0; b < nreq; b += kWave) {
    const int64_t s = b + lane_id();
    const int64_t v = s < nreq ? slotNnz[r * nreq + s] : 0;
    const int64_t inc = wave_incl_scan(v);
    if (s < nreq) slotOff[r * nreq + s] = carry + inc - v;
    carry += __shfl(inc, kWave - 1);
  }
  if (lane_id() == 0) cnt[xheavy[r]] = carry;
}

}  // namespace

void heavy_set_attributes() {
  (void)hipFuncSetAttribute((const void*)k_multisplit<kMsItemsF64, double>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, 163840);
  (void)hipFuncSetAttribute((const void*)k_multisplit<kMsItemsF32, float>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, 163840);
  (void)hipFuncSetAttribute((const void*)k_dense_num<float>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, 163840);
  (void)hipFuncSetAttribute((const void*)k_dense_num<double>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, 163840);
  (void)hipFuncSetAttribute((const void*)k_dense_sym, hipFuncAttributeMaxDynamicSharedMemorySize,
                            163840);
}

void launch_csc_count(int64_t h, const int32_t* xheavy, const int32_t* arp, const int32_t* acol,
                      int32_t* colCnt, hipStream_t s) {
  if (h <= 0) return;
  hipLaunchKernelGGL(k_csc_count, dim3(grid_for(h * kWave, kNT)), dim3(kNT), 0, s, h, xheavy, arp,
                     acol, colCnt);
}

void launch_csc_fill(int64_t h, const int32_t* xheavy, const int32_t* arp, const int32_t* acol,
                     const void* aval, bool f64, int64_t* colFill, int32_t* cscRow,
                     int32_t* cscCol, void* cscVal, hipStream_t s) {
  if (h <= 0) return;
  if (f64)
    hipLaunchKernelGGL(k_csc_fill<double>, dim3(grid_for(h * kWave, kNT)), dim3(kNT), 0, s, h,
                       xheavy, arp, acol, (const double*)aval, colFill, cscRow, cscCol,
                       (double*)cscVal);
  else
    hipLaunchKernelGGL(k_csc_fill<float>, dim3(grid_for(h * kWave, kNT)), dim3(kNT), 0, s, h,
                       xheavy, arp, acol, (const float*)aval, colFill, cscRow, cscCol,
                       (float*)cscVal);
}

void launch_entry_products(int64_t nE, const int32_t* cscCol, const int32_t* brp, int64_t* nb,
                           hipStream_t s) {
  if (nE <= 0) return;
  hipLaunchKernelGGL(k_entry_products, dim3(grid_for(nE, kNT)), dim3(kNT), 0, s, nE, cscCol, brp,
                     nb);
}

void launch_seg_base(int64_t nE, const int32_t* cscRow, const int64_t* nb, int64_t* cursor,
                     int64_t* segBase, hipStream_t s) {
  if (nE <= 0) return;
  hipLaunchKernelGGL(k_seg_base, dim3(grid_for(nE, kNT)), dim3(kNT), 0, s, nE, cscRow, nb, cursor,
                     segBase);
}

void launch_outer_product(bool f64, int64_t Ph, const int64_t* entryOff, int64_t nE,
                          const int32_t* cscCol, const void* cscVal, const int64_t* segBase,
                          const int32_t* brp, const int32_t* bcol, const void* bval,
                          int32_t* outCol, void* outVal, hipStream_t s) {
  if (Ph <= 0) return;
  // A multiple of the XCD count; tiles past the end exit at once.
  const unsigned g = (grid_for(Ph, kOpBlock) + kXcds - 1) / kXcds * kXcds;
  if (f64)
    hipLaunchKernelGGL(k_outer_product<double>, dim3(g), dim3(kNT), 0, s, Ph, entryOff, nE, cscCol,
                       (const double*)cscVal, segBase, brp, bcol, (const double*)bval, outCol,
                       (double*)outVal);
  else
    hipLaunchKernelGGL(k_outer_product<float>, dim3(g), dim3(kNT), 0, s, Ph, entryOff, nE, cscCol,
                       (const float*)cscVal, segBase, brp, bcol, (const float*)bval, outCol,
                       (float*)outVal);
}

void multisplit_geometry(bool f64, int64_t tau, int v, int32_t* blockElems, int* maxRows) {
  int64_t G = (int64_t)kNT * (f64 ? kMsItemsF64 : kMsItemsF32);
  // A range of G elements meets at most floor((G-1)/(tau+1)) + 2 rows when
  // every row holds more than tau elements; shrink G until the buckets fit.
  auto rows_for = [&](int64_t g) { return (g - 1) / (tau + 1) + 2; };
  while (G > 64 && (rows_for(G) * v > kMsNBMax || rows_for(G) > kMsRowsMax)) G /= 2;
  *blockElems = (int32_t)G;
  *maxRows = (int)rows_for(G);
}

void launch_histogram(int64_t E, int32_t blockElems, const int64_t* rowPtr, int64_t R,
                      const int32_t* col, int shift, int v, int maxRows, int32_t* counts,
                      int32_t* err, hipStream_t s) {
  if (E <= 0) return;
  hipLaunchKernelGGL(k_histogram, dim3(grid_for(E, blockElems)), dim3(kNT), 0, s, E, blockElems,
                     rowPtr, R, col, shift, v, maxRows, counts, err);
}

void launch_partition(int64_t Q, const int32_t* counts, int64_t tau, bool last, int v,
                      const int32_t* inRow, const int32_t* inSlot, int32_t slotStep,
                      int32_t* inv, int32_t* newCnt, int32_t* newRow, int32_t* newSlot,
                      int32_t* ctr, hipStream_t s) {
  if (Q <= 0) return;
  hipLaunchKernelGGL(k_partition, dim3(grid_for(Q, kNT)), dim3(kNT), 0, s, Q, counts, tau,
                     last ? 1 : 0, v, inRow, inSlot, slotStep, inv, newCnt, newRow, newSlot, ctr);
}

void launch_multisplit(bool f64, int64_t E, int32_t blockElems, const int64_t* rowPtr,
                       int64_t R, const int32_t* inCol, const void* inVal, int shift, int v,
                       int32_t wmask, int maxRows, const int32_t* inv, int64_t* cursor,
                       int32_t* outCol, void* outVal, int32_t* err, hipStream_t s) {
  if (E <= 0) return;
  const unsigned g = grid_for(E, blockElems);
  const size_t NB = (size_t)maxRows * v;
  const size_t lds = NB * 8 + (size_t)maxRows * 8 + (size_t)blockElems * ((f64 ? 8 : 4) + 4 + 2) +
                     NB * 8 + 16;
  if (f64)
    hipLaunchKernelGGL((k_multisplit<kMsItemsF64, double>), dim3(g), dim3(kNT), lds, s, E,
                       blockElems, rowPtr, R, inCol, (const double*)inVal, shift, v, wmask,
                       maxRows, inv, cursor, outCol, (double*)outVal, err);
  else
    hipLaunchKernelGGL((k_multisplit<kMsItemsF32, float>), dim3(g), dim3(kNT), lds, s, E,
                       blockElems, rowPtr, R, inCol, (const float*)inVal, shift, v, wmask,
                       maxRows, inv, cursor, outCol, (float*)outVal, err);
}

void launch_final_from_level(int64_t first, int64_t n, const int64_t* newOff,
                             const int32_t* newCnt, const int32_t* newRow,
                             const int32_t* newSlot, int8_t buf, int64_t dst0, int64_t* fcOff,
                             int32_t* fcCnt, int32_t* fcRow, int32_t* fcSlot, int8_t* fcBuf,
                             hipStream_t s) {
  if (n <= 0) return;
  hipLaunchKernelGGL(k_final_from_level, dim3(grid_for(n, kNT)), dim3(kNT), 0, s, first, n, newOff,
                     newCnt, newRow, newSlot, buf, dst0, fcOff, fcCnt, fcRow, fcSlot, fcBuf);
}

void launch_final_from_rows(int64_t h, const int64_t* rowPtr, int64_t* fcOff, int32_t* fcCnt,
                            int32_t* fcRow, int32_t* fcSlot, int8_t* fcBuf, hipStream_t s) {
  if (h <= 0) return;
  hipLaunchKernelGGL(k_final_from_rows, dim3(grid_for(h, kNT)), dim3(kNT), 0, s, h, rowPtr, fcOff,
                     fcCnt, fcRow, fcSlot, fcBuf);
}

void launch_chunk_bins(int64_t nfc, const int32_t* fcCnt, int64_t lastFirst, int64_t tau,
                       const int32_t* caps, int nbins, int denseBin, uint8_t* key,
                       int64_t* denseElems, hipStream_t s) {
  if (nfc <= 0) return;
  hipLaunchKernelGGL(k_chunk_bins, dim3(grid_for(nfc, kNT)), dim3(kNT), 0, s, nfc, fcCnt,
                     lastFirst, tau, caps, nbins, denseBin, key, denseElems);
}

void launch_dense_sym(const int32_t* items, int64_t n, const ChunkList& cl, int32_t* err,
                      hipStream_t s) {
  if (n <= 0) return;
  const size_t lds = (size_t)((cl.W + 31) / 32) * 4;
  hipLaunchKernelGGL(k_dense_sym, dim3((unsigned)n), dim3(kNT), lds, s, items, cl, err);
}

size_t dense_num_lds(bool f64, int64_t W) {
  return (size_t)W * (f64 ? 8 : 4) + (size_t)((W + 31) / 32) * 4 + (kDenseNT / kWave) * 4;
}

void launch_dense_num(bool f64, const int32_t* items, int64_t n, const ChunkList& cl,
                      const int64_t* cRowOff, int32_t* ccol, void* cval, int32_t* err,
                      hipStream_t s) {
  if (n <= 0) return;
  const size_t lds = dense_num_lds(f64, cl.W);
  if (f64)
    hipLaunchKernelGGL(k_dense_num<double>, dim3((unsigned)n), dim3(kDenseNT), lds, s, items, cl,
                       cRowOff, ccol, (double*)cval, err);
  else
    hipLaunchKernelGGL(k_dense_num<float>, dim3((unsigned)n), dim3(kDenseNT), lds, s, items, cl,
                       cRowOff, ccol, (float*)cval, err);
}

void launch_slot_scan(int64_t h, int64_t nreq, const int32_t* slotNnz, int64_t* slotOff,
                      const int32_t* xheavy, int64_t* cnt, hipStream_t s) {
  if (h <= 0) return;
  hipLaunchKernelGGL(k_slot_scan, dim3(grid_for(h * kWave, kNT)), dim3(kNT), 0, s, h, nreq,
                     slotNnz, slotOff, xheavy, cnt);
}

}  // namespace sg
