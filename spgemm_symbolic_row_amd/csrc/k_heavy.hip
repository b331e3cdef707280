// Bookkeeping of the heavy path and the dense chunk accumulator (gMAGNUS
// page, §III-C and §III-E): heavy-first placement of each level's chunks,
// the list of final chunks, their bins, the dense LDS accumulator of W-wide
// heavy chunks, and the per-row assembly of chunk offsets.
#include <algorithm>

#include "device_common.hpp"

namespace sg {
namespace {

constexpr int kNT = 256;
inline unsigned grid_for(int64_t n, int per_block) {
  int64_t g = (n + per_block - 1) / per_block;
  return (unsigned)(g < 1 ? 1 : g);
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
  // One pair of global atomics per work group (the waves' counts added in
  // LDS first), so that a level of millions of chunks does not queue on
  // two counters.
  constexpr int NW = kNT / kWave;
  __shared__ int32_t wh[NW], wl[NW], gb[2];
  const int64_t q = (int64_t)blockIdx.x * kNT + threadIdx.x;
  const int w = threadIdx.x / kWave;
  const bool act = q < Q;
  const int32_t cnt = act ? counts[q] : 0;
  const bool heavy = act && !last && cnt > tau;
  const bool light = act && !heavy && cnt > 0;
  const uint64_t mh = __ballot(heavy), ml = __ballot(light);
  if (lane_id() == 0) {
    wh[w] = __popcll(mh);
    wl[w] = __popcll(ml);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t th = 0, tl = 0;
    for (int i = 0; i < NW; ++i) {
      th += wh[i];
      tl += wl[i];
    }
    gb[0] = th ? atomicAdd(&ctr[0], th) : 0;
    gb[1] = tl ? atomicAdd(&ctr[1], tl) : 0;
  }
  __syncthreads();
  int32_t bh = gb[0], bl = gb[1];
  for (int i = 0; i < w; ++i) {
    bh += wh[i];
    bl += wl[i];
  }
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
                                                          int8_t buf, int8_t spanLog2,
                                                          int64_t dst0,
                                                          int64_t* __restrict__ fcOff,
                                                          int32_t* __restrict__ fcCnt,
                                                          int32_t* __restrict__ fcRow,
                                                          int32_t* __restrict__ fcSlot,
                                                          int8_t* __restrict__ fcBuf,
                                                          int8_t* __restrict__ fcSpan) {
  const int64_t i = (int64_t)blockIdx.x * kNT + threadIdx.x;
  if (i >= n) return;
  const int64_t pos = first + i, d = dst0 + i;
  fcOff[d] = newOff[pos];
  fcCnt[d] = newCnt[pos];
  fcRow[d] = newRow[pos];
  fcSlot[d] = newSlot[pos];
  fcBuf[d] = buf;
  fcSpan[d] = spanLog2;
}

__global__ __launch_bounds__(kNT) void k_final_from_rows(int64_t h, const int64_t* __restrict__ rowPtr,
                                                         int64_t* __restrict__ fcOff,
                                                         int32_t* __restrict__ fcCnt,
                                                         int32_t* __restrict__ fcRow,
                                                         int32_t* __restrict__ fcSlot,
                                                         int8_t* __restrict__ fcBuf,
                                                         int8_t* __restrict__ fcSpan) {
  const int64_t r = (int64_t)blockIdx.x * kNT + threadIdx.x;
  if (r >= h) return;
  fcOff[r] = rowPtr[r];
  fcCnt[r] = (int32_t)(rowPtr[r + 1] - rowPtr[r]);
  fcRow[r] = (int32_t)r;
  fcSlot[r] = 0;
  fcBuf[r] = 0;
  fcSpan[r] = 0;
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
template <typename C>
__global__ __launch_bounds__(kNT) void k_dense_sym(const ChunkDesc* __restrict__ desc, ChunkList cl,
                                                   int32_t* __restrict__ err) {
  extern __shared__ __align__(16) uint32_t bm[];
  __shared__ int32_t wsum[kNT / kWave];
  const int nwords = (int)((cl.W + 31) / 32);
  const ChunkDesc d = desc[blockIdx.x];
  for (int i = threadIdx.x; i < nwords; i += kNT) bm[i] = 0;
  __syncthreads();
  const int64_t off = d.off, end = off + d.cnt;
  const C* __restrict__ col = (const C*)(d.buf ? cl.col1 : cl.col0);
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
    cl.slotNnz[d.base] = t;
  }
  (void)err;
}

// Numeric: val[W] and one mark per column in LDS, values added by LDS
// atomics; the marked columns, taken in column order, give the chunk sorted
// and compacted.
//
// One work group per CU holds the 128 KiB accumulator, so the kernel is
// persistent: a work group takes chunks blockIdx.x, blockIdx.x + gridDim.x,
// ..., loads the first batch of its next chunk while it writes out the
// current one, and clears only the slots the current chunk touched (the
// whole accumulator is cleared once, at the start).
constexpr int kDenseNT = 1024;
constexpr int kDenseB = 4;  // elements per thread per batch
template <typename V, typename C>
__device__ __forceinline__ void dense_load_batch(const C* __restrict__ col,
                                                 const V* __restrict__ val, int64_t e0, int64_t end,
                                                 int32_t (&cc)[kDenseB], V (&vv)[kDenseB]) {
#pragma unroll
  for (int k = 0; k < kDenseB; ++k) {
    const int64_t e = e0 + (int64_t)k * kDenseNT;
    cc[k] = e < end ? col[e] : -1;
    vv[k] = e < end ? val[e] : V(0);
  }
}
// Column marks: one byte per column when the accumulator leaves room for
// them (a plain LDS byte store per element), else one bit per column (a read
// and, for a new column, an LDS atomic OR).
template <typename V, bool kBytes>
__device__ __forceinline__ void dense_add_batch(V* vals, void* marks, const int32_t (&cc)[kDenseB],
                                                const V (&vv)[kDenseB]) {
#pragma unroll
  for (int k = 0; k < kDenseB; ++k) {
    const int32_t c = cc[k];
    if (c >= 0) {
      atomicAdd(&vals[c], vv[k]);
      if constexpr (kBytes) {
        ((unsigned char*)marks)[c] = 1;
      } else {
        uint32_t* bm = (uint32_t*)marks;
        const uint32_t bit = 1u << (c & 31);
        if (!(bm[c >> 5] & bit)) atomicOr(&bm[c >> 5], bit);
      }
    }
  }
}

// Write-out of a dense chunk in column order, then the accumulator cleared
// for the next chunk.  Wave w owns columns [w*W/16, (w+1)*W/16), lane l a
// run of cpl of them; a wave scan of the lanes' popcounts gives every lane
// its output offset, and each lane then writes its own entries in column
// order, one per step (the wave's stores of a step fall in a short stretch
// of the output).  A slot's value is cleared as it is read.  Called by the
// whole work group after a barrier that ends the accumulation.
template <typename V, bool kBytes>
__device__ __forceinline__ void dense_write_out(V* vals, uint32_t* bm, int32_t* wtot, int W,
                                                int32_t want, int64_t base, int32_t colBase,
                                                int32_t* __restrict__ ccol, V* __restrict__ cval,
                                                int32_t* __restrict__ err) {
  constexpr int kWaves = kDenseNT / kWave;
  const int w = threadIdx.x / kWave, lane = lane_id();
  const int nwords = (W + 31) / 32;
  const int cpw = (W + kWaves - 1) / kWaves;        // columns per wave
  const int cpl = cpw >= kWave ? cpw / kWave : 1;   // columns per lane, <= 32
  const int lc0 = w * cpw + lane * cpl;             // this lane's first column
  uint32_t mask = 0;
  if (lc0 < W && lane * cpl < cpw) {
    if constexpr (kBytes) {
      // cpl is a power of two; from 4 on, lc0 is a multiple of 4.  Each
      // lane owns its mark bytes, so it clears them as it reads them.
      unsigned char* mk = (unsigned char*)bm;
      if (cpl >= 4) {
        for (int k = 0; k < cpl; k += 4) {
          uint32_t* wp = (uint32_t*)(mk + lc0 + k);
          const uint32_t wd = *wp;
          *wp = 0u;
          mask |= ((wd & 1u) | ((wd >> 7) & 2u) | ((wd >> 14) & 4u) | ((wd >> 21) & 8u)) << k;
        }
      } else {
        for (int k = 0; k < cpl; ++k) {
          mask |= (uint32_t)mk[lc0 + k] << k;
          mk[lc0 + k] = 0;
        }
      }
    } else {
      const uint32_t word = bm[lc0 >> 5];
      mask = cpl >= 32 ? word : (word >> (lc0 & 31)) & ((1u << cpl) - 1u);
    }
  }
  const int32_t cntL = __popc(mask);
  const int32_t incL = wave_incl_scan(cntL);
  const int32_t exclL = incL - cntL;
  const int32_t nw = __shfl(incL, kWave - 1);
  if (lane == 0) wtot[w] = nw;
  __syncthreads();
  int32_t wbase = 0, total = 0;
  for (int i = 0; i < kWaves; ++i) {
    const int32_t t = wtot[i];
    if (i < w) wbase += t;
    total += t;
  }
  if (threadIdx.x == 0 && want != total) flag_error(err, kErrCountMismatch);
  uint32_t m = mask;
  int32_t p = wbase + exclL;
  while (__ballot(m != 0)) {
    if (m) {
      const int c = lc0 + __ffs(m) - 1;
      m &= m - 1;
      const V x = vals[c];
      vals[c] = V(0);
      if (p < want) {
        ccol[base + p] = colBase + c;
        cval[base + p] = x;
      }
      ++p;
    }
  }
  __syncthreads();
  // Byte marks were cleared as they were read; bit marks, which lanes may
  // share, are cleared here.
  if constexpr (!kBytes) {
    for (int i = threadIdx.x; i < nwords; i += kDenseNT) bm[i] = 0;
    __syncthreads();
  }
}

template <typename V, typename C, bool kBytes>
__global__ __launch_bounds__(kDenseNT) void k_dense_num(const ChunkDesc* __restrict__ desc, int64_t n,
                                                        ChunkList cl,
                                                        int32_t* __restrict__ ccol,
                                                        V* __restrict__ cval,
                                                        int32_t* __restrict__ err) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int W = (int)cl.W;
  const int nwords = (W + 31) / 32;
  // kBytes: W is a power of two from 16 on and the marks take W bytes.
  const int markWords = kBytes ? W / 4 : nwords;
  V* vals = (V*)smem;
  uint32_t* bm = (uint32_t*)(vals + W);
  int32_t* wtot = (int32_t*)(bm + markWords);
  for (int i = threadIdx.x; i < W; i += kDenseNT) vals[i] = V(0);
  for (int i = threadIdx.x; i < markWords; i += kDenseNT) bm[i] = 0;

  int64_t ci = blockIdx.x;
  int32_t cc[kDenseB];
  V vv[kDenseB];
  ChunkDesc d{};
  const C* col = (const C*)cl.col0;
  const V* val = (const V*)cl.val0;
  if (ci < n) {
    d = desc[ci];
    col = (const C*)(d.buf ? cl.col1 : cl.col0);
    val = (const V*)(d.buf ? cl.val1 : cl.val0);
    dense_load_batch(col, val, d.off + threadIdx.x, d.off + d.cnt, cc, vv);
  }
  __syncthreads();
  while (ci < n) {
    const int64_t off = d.off, end = d.off + d.cnt, base = d.base;
    const int32_t want = d.want, colBase = d.colBase;
    // The next chunk's descriptor, in flight during this chunk.
    const int64_t cn = ci + gridDim.x;
    if (cn < n) d = desc[cn];
    dense_add_batch<V, kBytes>(vals, bm, cc, vv);
    for (int64_t e0 = off + threadIdx.x + (int64_t)kDenseNT * kDenseB; e0 < end;
         e0 += (int64_t)kDenseNT * kDenseB) {
      dense_load_batch(col, val, e0, end, cc, vv);
      dense_add_batch<V, kBytes>(vals, bm, cc, vv);
    }
    __syncthreads();
    // First batch of the next chunk, in flight during the write-out.
    if (cn < n) {
      col = (const C*)(d.buf ? cl.col1 : cl.col0);
      val = (const V*)(d.buf ? cl.val1 : cl.val0);
      dense_load_batch(col, val, d.off + threadIdx.x, d.off + d.cnt, cc, vv);
    }
    dense_write_out<V, kBytes>(vals, bm, wtot, W, want, base, colBase, ccol, cval, err);
    ci = cn;
  }
}

// Dense chunks accumulated straight from A and B.  A dense chunk is one
// W-wide column slot s of a heavy row i; its elements are the products
// A[i,k] * B[k,j] with j in the slot, i.e. for every entry k of A's row i
// the run of B's row k inside the slot (B's rows are sorted, so the run is
// contiguous).  B's slot table gives the run at once: tab[k * stride + s] is
// the first position of B row k whose column is at least s * W, so the run
// is [tab[k*stride+s], tab[k*stride+s+1]).  The waves of a work group share
// the row's entries (each wave every 16th one, a lane per entry, 1024
// entries a pass).  Runs of
// at least kLong products are streamed by the whole wave, 64 products a
// piece, kLongU pieces in flight: the pieces of one pass's long runs are
// numbered by a scan of their counts, and a piece finds its run from one
// ballot, with the run's start, length and a_ik read from that lane (no
// per-product search).  The shorter runs of the pass are streamed as one
// sequence, each lane finding its run by a search across the lanes'
// offsets.  B's rows are read from the caches instead of a materialised
// intermediate.  Persistent work groups, write-out and clearing as in
// k_dense_num.
constexpr int kDirectU = 4;  // short-run pieces of 64 products in flight together
constexpr int kLongU = 4;    // long-run pieces in flight together
constexpr int kLong = 32;    // runs of at least this many products go whole-wave

__device__ __forceinline__ int32_t lane_read(int32_t x, int j) {
  return __builtin_amdgcn_readlane(x, j);
}
__device__ __forceinline__ double lane_read(double x, int j) {
  const int64_t b = __double_as_longlong(x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int32_t)(uint32_t)b, j);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int32_t)(uint32_t)(b >> 32), j);
  return __longlong_as_double((int64_t)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ float lane_read(float x, int j) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), j));
}

template <typename V, bool kBytes>
__device__ __forceinline__ void direct_add(V* vals, uint32_t* bm, int32_t c, V v, int W,
                                           int32_t* __restrict__ err) {
  if (c < 0) return;
  if (c >= W) {  // a column outside the slot: B is not canonical
    flag_error(err, kErrCsr);
    return;
  }
  atomicAdd(&vals[c], v);
  if constexpr (kBytes) {
    ((unsigned char*)bm)[c] = 1;
  } else {
    const uint32_t bit = 1u << (c & 31);
    if (!(bm[c >> 5] & bit)) atomicOr(&bm[c >> 5], bit);
  }
}

template <typename V, bool kBytes>
__global__ __launch_bounds__(kDenseNT) void k_dense_num_direct(const ChunkDesc* __restrict__ desc,
                                                               int64_t n, RowArgs a,
                                                               const int32_t* __restrict__ tab,
                                                               int64_t stride, int64_t nnzB,
                                                               int log2W,
                                                               int32_t* __restrict__ ccol,
                                                               V* __restrict__ cval,
                                                               int32_t* __restrict__ err) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int kWaves = kDenseNT / kWave;
  const int W = 1 << log2W;
  const int nwords = (W + 31) / 32;
  const int markWords = kBytes ? W / 4 : nwords;
  V* vals = (V*)smem;
  uint32_t* bm = (uint32_t*)(vals + W);
  int32_t* wtot = (int32_t*)(bm + markWords);
  for (int i = threadIdx.x; i < W; i += kDenseNT) vals[i] = V(0);
  for (int i = threadIdx.x; i < markWords; i += kDenseNT) bm[i] = 0;
  __syncthreads();
  const int w = threadIdx.x / kWave, lane = lane_id();
  const V* __restrict__ aval = (const V*)a.aval;
  const V* __restrict__ bval = (const V*)a.bval;
  const int32_t* __restrict__ bcol = a.bcol;
  for (int64_t ci = blockIdx.x; ci < n; ci += gridDim.x) {
    const ChunkDesc d = desc[ci];
    const int32_t slot = d.colBase >> log2W;
    const int32_t colBase = d.colBase;
    const int64_t rs = a.arp[d.row], re = a.arp[d.row + 1];
    for (int64_t e0 = rs; e0 < re; e0 += (int64_t)kWaves * kWave) {
      const int64_t e = e0 + (int64_t)lane * kWaves + w;
      int32_t b0 = 0, len = 0;
      V av = V(0);
      if (e < re) {
        const int32_t k = a.acol[e];
        av = aval[e];
        const int32_t* t = tab + (int64_t)k * stride + slot;
        // Clamped into B, so that no table content can send a load outside it.
        const int64_t t0 = min<int64_t>(max<int64_t>(t[0], 0), nnzB);
        const int64_t t1 = min<int64_t>(max<int64_t>(t[1], t0), nnzB);
        b0 = (int32_t)t0;
        len = (int32_t)(t1 - t0);
      }
      // Long runs: whole-wave pieces of 64 products.
      const int32_t np = len >= kLong ? (len + kWave - 1) / kWave : 0;
      const int32_t pinc = wave_incl_scan(np);
      const int32_t ptot = __shfl(pinc, kWave - 1);
      for (int32_t g0 = 0; g0 < ptot; g0 += kLongU) {
        int32_t cc[kLongU];
        V vv[kLongU];
#pragma unroll
        for (int u = 0; u < kLongU; ++u) {
          cc[u] = -1;
          vv[u] = V(0);
          const int32_t g = g0 + u;
          if (g < ptot) {  // the same for every lane
            // The run holding piece g: the first lane whose inclusive piece
            // count passes g.
            const int j = ffs64(__ballot(pinc > g));
            const int32_t rb0 = lane_read(b0, j), rlen = lane_read(len, j);
            const int32_t first = lane_read(pinc, j) - lane_read(np, j);
            const V rav = lane_read(av, j);
            const int32_t t = (g - first) * kWave + lane;
            if (t < rlen) {
              cc[u] = bcol[rb0 + t] - colBase;
              vv[u] = rav * bval[rb0 + t];
            }
          }
        }
#pragma unroll
        for (int u = 0; u < kLongU; ++u) direct_add<V, kBytes>(vals, bm, cc[u], vv[u], W, err);
      }
      // Short runs as one sequence: product q belongs to the last lane whose
      // exclusive offset is <= q (lanes with empty runs share the next
      // lane's offset, so the last one has products).
      const int32_t slen = len >= kLong ? 0 : len;
      const int32_t inc = wave_incl_scan(slen);
      const int32_t off = inc - slen;
      const int32_t total = __shfl(inc, kWave - 1);
      const int32_t sdelta = b0 - off;  // B position of product q is q + sdelta of its lane
      for (int32_t p = 0; p < total; p += kWave * kDirectU) {
        int32_t cc[kDirectU];
        V vv[kDirectU];
#pragma unroll
        for (int u = 0; u < kDirectU; ++u) {
          const int32_t q = p + u * kWave + lane;
          cc[u] = -1;
          vv[u] = V(0);
          if (p + u * kWave < total) {  // the same for every lane
            int s = 0;
#pragma unroll
            for (int step = 32; step >= 1; step >>= 1)
              if (__shfl(off, s + step) <= q) s += step;
            const int32_t bi = __shfl(sdelta, s) + q;
            const V at = __shfl(av, s);
            if (q < total) {
              cc[u] = bcol[bi] - colBase;
              vv[u] = at * bval[bi];
            }
          }
        }
#pragma unroll
        for (int u = 0; u < kDirectU; ++u) direct_add<V, kBytes>(vals, bm, cc[u], vv[u], W, err);
      }
    }
    __syncthreads();
    dense_write_out<V, kBytes>(vals, bm, wtot, W, d.want, d.base, d.colBase, ccol, cval, err);
  }
}

__global__ __launch_bounds__(kNT) void k_chunk_desc(int64_t n, const int32_t* __restrict__ order,
                                                    ChunkList cl, const int64_t* __restrict__ cRowOff,
                                                    ChunkDesc* __restrict__ desc) {
  const int64_t i = (int64_t)blockIdx.x * kNT + threadIdx.x;
  if (i >= n) return;
  const int32_t item = order[i];
  const int64_t hr = cl.row[item];
  const int64_t sidx = hr * cl.nreq + cl.slot[item];
  ChunkDesc d;
  d.off = cl.off[item];
  // Without C's row offsets (symbolic), base is the chunk's slot index.
  d.base = cRowOff ? cRowOff[cl.xheavy[hr]] + cl.slotOff[sidx] : sidx;
  d.cnt = cl.cnt[item];
  // The chunk's size: the counts of the W-wide slots it covers.
  int32_t want = 0;
  if (cRowOff) {
    const int nsl = 1 << cl.span[item];
    for (int j = 0; j < nsl; ++j) want += cl.slotNnz[sidx + j];
  }
  d.want = want;
  d.colBase = (int32_t)((int64_t)cl.slot[item] * cl.W);
  d.row = cl.xheavy[hr];
  d.buf = cl.buf[item];
  desc[i] = d;
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

// finalOf / spanOf over the W-wide slots of every final chunk.
// finalOf of a chunk accumulated straight from A and B (key == denseKey)
// is -(c + 2): the expansion skips its products.
__global__ __launch_bounds__(kNT) void k_final_map(int64_t nfc, const int32_t* __restrict__ fcRow,
                                                   const int32_t* __restrict__ fcSlot,
                                                   const int8_t* __restrict__ fcSpan, int64_t nreq,
                                                   const uint8_t* __restrict__ key, int denseKey,
                                                   int32_t* __restrict__ finalOf,
                                                   int8_t* __restrict__ spanOf) {
  const int64_t c = (int64_t)blockIdx.x * kNT + threadIdx.x;
  if (c >= nfc) return;
  const int64_t q = (int64_t)fcRow[c] * nreq + fcSlot[c];
  const int8_t sp = fcSpan[c];
  const int32_t f = (key && key[c] == denseKey) ? -(int32_t)c - 2 : (int32_t)c;
  for (int s = 0; s < (1 << sp); ++s) {
    finalOf[q + s] = f;
    spanOf[q + s] = sp;
  }
}

// Element counts of the chunks the expansion writes: 0 for the chunks taken
// straight from A and B.
__global__ __launch_bounds__(kNT) void k_stored_counts(int64_t nfc, const int32_t* __restrict__ cnt,
                                                       const uint8_t* __restrict__ key,
                                                       int denseKey, int32_t* __restrict__ out) {
  const int64_t c = (int64_t)blockIdx.x * kNT + threadIdx.x;
  if (c < nfc) out[c] = key[c] == denseKey ? 0 : cnt[c];
}

}  // namespace

void heavy_set_attributes() {
#define SG_ATTR(K) allow_max_dynamic_lds((const void*)(K))
  SG_ATTR((k_dense_num<float, int32_t, false>));
  SG_ATTR((k_dense_num<double, int32_t, false>));
  SG_ATTR((k_dense_num<float, uint16_t, false>));
  SG_ATTR((k_dense_num<double, uint16_t, false>));
  SG_ATTR((k_dense_num<float, int32_t, true>));
  SG_ATTR((k_dense_num<double, int32_t, true>));
  SG_ATTR((k_dense_num<float, uint16_t, true>));
  SG_ATTR((k_dense_num<double, uint16_t, true>));
  SG_ATTR((k_dense_num_direct<double, true>));
  SG_ATTR((k_dense_num_direct<double, false>));
  SG_ATTR((k_dense_num_direct<float, true>));
  SG_ATTR((k_dense_num_direct<float, false>));
  SG_ATTR(k_dense_sym<int32_t>);
  SG_ATTR(k_dense_sym<uint16_t>);
#undef SG_ATTR
}

void launch_partition(int64_t Q, const int32_t* counts, int64_t tau, bool last, int v,
                      const int32_t* inRow, const int32_t* inSlot, int32_t slotStep,
                      int32_t* inv, int32_t* newCnt, int32_t* newRow, int32_t* newSlot,
                      int32_t* ctr, hipStream_t s) {
  if (Q <= 0) return;
  hipLaunchKernelGGL(k_partition, dim3(grid_for(Q, kNT)), dim3(kNT), 0, s, Q, counts, tau,
                     last ? 1 : 0, v, inRow, inSlot, slotStep, inv, newCnt, newRow, newSlot, ctr);
}

void launch_final_map(int64_t nfc, const int32_t* fcRow, const int32_t* fcSlot,
                      const int8_t* fcSpan, int64_t nreq, const uint8_t* key, int denseKey,
                      int32_t* finalOf, int8_t* spanOf, hipStream_t s) {
  if (nfc <= 0) return;
  hipLaunchKernelGGL(k_final_map, dim3(grid_for(nfc, kNT)), dim3(kNT), 0, s, nfc, fcRow, fcSlot,
                     fcSpan, nreq, key, denseKey, finalOf, spanOf);
}

void launch_stored_counts(int64_t nfc, const int32_t* cnt, const uint8_t* key, int denseKey,
                          int32_t* out, hipStream_t s) {
  if (nfc <= 0) return;
  hipLaunchKernelGGL(k_stored_counts, dim3(grid_for(nfc, kNT)), dim3(kNT), 0, s, nfc, cnt, key,
                     denseKey, out);
}

void launch_final_from_level(int64_t first, int64_t n, const int64_t* newOff,
                             const int32_t* newCnt, const int32_t* newRow,
                             const int32_t* newSlot, int8_t buf, int8_t spanLog2, int64_t dst0,
                             int64_t* fcOff, int32_t* fcCnt, int32_t* fcRow, int32_t* fcSlot,
                             int8_t* fcBuf, int8_t* fcSpan, hipStream_t s) {
  if (n <= 0) return;
  hipLaunchKernelGGL(k_final_from_level, dim3(grid_for(n, kNT)), dim3(kNT), 0, s, first, n, newOff,
                     newCnt, newRow, newSlot, buf, spanLog2, dst0, fcOff, fcCnt, fcRow, fcSlot,
                     fcBuf, fcSpan);
}

void launch_final_from_rows(int64_t h, const int64_t* rowPtr, int64_t* fcOff, int32_t* fcCnt,
                            int32_t* fcRow, int32_t* fcSlot, int8_t* fcBuf, int8_t* fcSpan,
                            hipStream_t s) {
  if (h <= 0) return;
  hipLaunchKernelGGL(k_final_from_rows, dim3(grid_for(h, kNT)), dim3(kNT), 0, s, h, rowPtr, fcOff,
                     fcCnt, fcRow, fcSlot, fcBuf, fcSpan);
}

void launch_chunk_bins(int64_t nfc, const int32_t* fcCnt, int64_t lastFirst, int64_t tau,
                       const int32_t* caps, int nbins, int denseBin, uint8_t* key,
                       int64_t* denseElems, hipStream_t s) {
  if (nfc <= 0) return;
  hipLaunchKernelGGL(k_chunk_bins, dim3(grid_for(nfc, kNT)), dim3(kNT), 0, s, nfc, fcCnt,
                     lastFirst, tau, caps, nbins, denseBin, key, denseElems);
}

void launch_dense_sym(const ChunkDesc* desc, int64_t n, const ChunkList& cl, int32_t* err,
                      hipStream_t s) {
  if (n <= 0) return;
  const size_t lds = (size_t)((cl.W + 31) / 32) * 4;
  if (cl.col16)
    hipLaunchKernelGGL(k_dense_sym<uint16_t>, dim3((unsigned)n), dim3(kNT), lds, s, desc, cl, err);
  else
    hipLaunchKernelGGL(k_dense_sym<int32_t>, dim3((unsigned)n), dim3(kNT), lds, s, desc, cl, err);
}

// Byte marks when W is a power of two from 16 on (so every lane's run of
// columns is a whole number of 4-byte words, or shorter than one) and they
// fit beside the values.
static bool dense_byte_marks(bool f64, int64_t W) {
  return W >= 16 && (W & (W - 1)) == 0 &&
         W * ((f64 ? 8 : 4) + 1) + (kDenseNT / kWave) * 4 <= 163840;
}

size_t dense_num_lds(bool f64, int64_t W) {
  const size_t marks = dense_byte_marks(f64, W) ? (size_t)W : (size_t)((W + 31) / 32) * 4;
  return (size_t)W * (f64 ? 8 : 4) + marks + (kDenseNT / kWave) * 4;
}

void launch_chunk_desc(int64_t n, const int32_t* order, const ChunkList& cl,
                       const int64_t* cRowOff, ChunkDesc* desc, hipStream_t s) {
  if (n <= 0) return;
  hipLaunchKernelGGL(k_chunk_desc, dim3(grid_for(n, kNT)), dim3(kNT), 0, s, n, order, cl, cRowOff,
                     desc);
}

void launch_dense_num(bool f64, const ChunkDesc* desc, int64_t n, const ChunkList& cl,
                      int32_t* ccol, void* cval, int32_t* err, int numCUs, hipStream_t s) {
  if (n <= 0) return;
  const size_t lds = dense_num_lds(f64, cl.W);
  const bool bytes = dense_byte_marks(f64, cl.W);
  // As many work groups as fit on the device at once (LDS of a CU: 160 KiB).
  const int64_t perCU = std::max<int64_t>(1, (int64_t)163840 / (int64_t)lds);
  const unsigned g = (unsigned)std::min<int64_t>(n, std::max(numCUs, 1) * perCU);
#define L(V, C)                                                                              \
  do {                                                                                       \
    if (bytes)                                                                               \
      hipLaunchKernelGGL((k_dense_num<V, C, true>), dim3(g), dim3(kDenseNT), lds, s, desc, n,  \
                         cl, ccol, (V*)cval, err);                                           \
    else                                                                                     \
      hipLaunchKernelGGL((k_dense_num<V, C, false>), dim3(g), dim3(kDenseNT), lds, s, desc, n, \
                         cl, ccol, (V*)cval, err);                                           \
  } while (0)
  if (f64 && cl.col16) L(double, uint16_t);
  else if (f64) L(double, int32_t);
  else if (cl.col16) L(float, uint16_t);
  else L(float, int32_t);
#undef L
}

void launch_dense_num_direct(bool f64, const ChunkDesc* desc, int64_t n, int64_t W,
                             const RowArgs& a, const int32_t* slotTab, int64_t stride,
                             int64_t nnzB, int32_t* ccol, void* cval, int32_t* err, int numCUs,
                             hipStream_t s) {
  if (n <= 0) return;
  const size_t lds = dense_num_lds(f64, W);
  const bool bytes = dense_byte_marks(f64, W);
  const int64_t perCU = std::max<int64_t>(1, (int64_t)163840 / (int64_t)lds);
  const unsigned g = (unsigned)std::min<int64_t>(n, std::max(numCUs, 1) * perCU);
  int log2W = 0;
  while ((int64_t(1) << log2W) < W) ++log2W;
#define L(V, B)                                                                           \
  hipLaunchKernelGGL((k_dense_num_direct<V, B>), dim3(g), dim3(kDenseNT), lds, s, desc, n, a, \
                     slotTab, stride, nnzB, log2W, ccol, (V*)cval, err)
  if (f64 && bytes) L(double, true);
  else if (f64) L(double, false);
  else if (bytes) L(float, true);
  else L(float, false);
#undef L
}

void launch_slot_scan(int64_t h, int64_t nreq, const int32_t* slotNnz, int64_t* slotOff,
                      const int32_t* xheavy, int64_t* cnt, hipStream_t s) {
  if (h <= 0) return;
  hipLaunchKernelGGL(k_slot_scan, dim3(grid_for(h * kWave, kNT)), dim3(kNT), 0, s, h, nreq,
                     slotNnz, slotOff, xheavy, cnt);
}

}  // namespace sg
