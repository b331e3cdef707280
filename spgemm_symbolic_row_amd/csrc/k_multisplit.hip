// One level of the hierarchical multisplit (gMAGNUS page, §III-C): the
// per-(row, chunk) histogram and the multisplit kernel that reorders each
// input row into column-range chunks through LDS.
#include "device_common.hpp"

namespace sg {
namespace {

constexpr int kNT = 256;
inline unsigned grid_for(int64_t n, int per_block) {
  int64_t g = (n + per_block - 1) / per_block;
  return (unsigned)(g < 1 ? 1 : g);
}

// ------------------------------------------------------------ multisplit
// A work group owns a static range of `blockElems` elements of the level's
// input (heavy rows, or heavy chunks of the previous level, each longer than
// tau).  Local bucket of an element = (row inside the range) * v + chunk,
// chunk = col >> shift.  Bucket ids are matched across the wave with one
// ballot per bit so a single lane per bucket updates the LDS counters.
constexpr int kMsNBMax = 1024;  // LDS buckets per work group
constexpr int kMsRowsMax = 512;
constexpr int kMsItemsF64 = 4;   // elements per thread held in registers
constexpr int kMsItemsF32 = 8;
// Straight into final chunks: no LDS staging, so larger tiles.  fp64: six
// elements per thread keep the kernel at 66 VGPRs, seven waves per SIMD
// (eight elements take 84, five waves: 4% slower on R-MAT 18 and 20).
constexpr int kXfItemsF64 = 6;
constexpr int kXfItemsF32 = 8;
constexpr int kXfNBMax = 8192;   // (row, chunk) buckets per work group
constexpr int kXfEnt = 256;      // entries per tile staged in LDS

__device__ __forceinline__ int bits_for(int n) {
  int b = 0;
  while ((1 << b) < n) ++b;
  return b;
}

// Rows of tile b's range [e0, e1): its first row and row count, and the
// first row boundary inside the range, precomputed (k_tile_info); further
// boundaries (only when tau is small next to the tile) are read here.
// Returns nrows, or -1 when more than maxRows rows meet the range.
__device__ __forceinline__ int range_rows(const int64_t* __restrict__ rowPtr,
                                          const TileInfo* __restrict__ info, int64_t tile,
                                          int maxRows, int64_t* bnd, TileInfo* s_info) {
  if (threadIdx.x == 0) *s_info = info[tile];
  __syncthreads();
  const int nrows = s_info->nrows;
  if (nrows > maxRows) return -1;
  if (nrows > 1) {
    if (threadIdx.x == 0) bnd[0] = s_info->bnd0;
    for (int i = 1 + threadIdx.x; i < nrows - 1; i += kNT) bnd[i] = rowPtr[s_info->r0 + 1 + i];
  }
  return nrows;
}

// Per tile of G elements: first row, row count (rows are never empty, each
// holds more than tau elements, so the row of the tile's last element is
// the next tile's first row, or the one before it when that row starts
// exactly at the next tile), the first boundary inside the tile, and with
// blkEnt the first entry and a bound on the last.
__global__ __launch_bounds__(kNT) void k_tile_info(int64_t nTiles, int64_t E, int64_t G,
                                                   const int64_t* __restrict__ rowPtr, int64_t R,
                                                   const int32_t* __restrict__ blkRow,
                                                   const int32_t* __restrict__ blkEnt, int64_t nE,
                                                   TileInfo* __restrict__ out) {
  const int64_t b = (int64_t)blockIdx.x * kNT + threadIdx.x;
  if (b >= nTiles) return;
  const int64_t e1 = (b + 1) * G < E ? (b + 1) * G : E;
  const int64_t r0 = blkRow[b];
  int64_t r1 = (b + 1 < nTiles) ? blkRow[b + 1] : R - 1;
  if (r1 > r0 && rowPtr[r1] >= e1) r1 -= 1;
  TileInfo t;
  t.r0 = (int32_t)r0;
  t.nrows = (int32_t)(r1 - r0 + 1);
  t.t0 = blkEnt ? blkEnt[b] : 0;
  t.t1 = blkEnt ? ((b + 1 < nTiles) ? blkEnt[b + 1] : (int32_t)(nE - 1)) : 0;
  t.bnd0 = r1 > r0 ? rowPtr[r0 + 1] : 0;
  out[b] = t;
}

// out[b] = the item whose range [off[t], off[t+1]) holds element b * G, for
// every block b < nBlocks (items without elements hold no block start).
__global__ __launch_bounds__(kNT) void k_block_starts(int64_t nItems, const int64_t* __restrict__ off,
                                                      int64_t G, int64_t nBlocks,
                                                      int32_t* __restrict__ out) {
  for (int64_t t = (int64_t)blockIdx.x * kNT + threadIdx.x; t < nItems;
       t += (int64_t)gridDim.x * kNT) {
    const int64_t lo = off[t], hi = off[t + 1];
    if (hi <= lo) continue;
    int64_t b = (lo + G - 1) / G;
    const int64_t bl = (hi - 1) / G;
    for (; b <= bl && b < nBlocks; ++b) out[b] = (int32_t)t;
  }
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

// Entry of every element of the range [e0, e0 + n), as in a merge of the
// elements with the entries' first products: each entry in [t0, t1] that
// starts inside the range marks its start (the largest index wins, which
// skips entries without products), then a prefix maximum carries it
// forward.  ent[] must hold -1 on entry; t0 is the entry of element e0.
__device__ __forceinline__ void entries_of_range(int32_t* ent, int n, int64_t e0, int32_t t0,
                                                 int32_t t1, const int64_t* __restrict__ eOff,
                                                 int32_t* wtot) {
  if (threadIdx.x == 0) ent[0] = t0;
  for (int32_t t = t0 + 1 + (int32_t)threadIdx.x; t <= t1; t += kNT) {
    const int64_t pos = eOff[t] - e0;
    if (pos < n) atomicMax(&ent[(int)pos], t);
  }
  __syncthreads();
  const int cpt = (n + kNT - 1) / kNT;
  const int i0 = threadIdx.x * cpt, i1 = (i0 + cpt < n) ? i0 + cpt : n;
  int32_t run = -1;
  for (int i = i0; i < i1; ++i) {
    run = ent[i] > run ? ent[i] : run;
    ent[i] = run;
  }
  int32_t x = run;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int32_t y = __shfl_up(x, d);
    if (lane_id() >= d && y > x) x = y;
  }
  int32_t carry = __shfl_up(x, 1);
  if (lane_id() == 0) carry = -1;
  if (lane_id() == kWave - 1) wtot[threadIdx.x / kWave] = x;
  __syncthreads();
  for (int w = 0; w < (int)threadIdx.x / kWave; ++w) carry = wtot[w] > carry ? wtot[w] : carry;
  for (int i = i0; i < i1; ++i)
    if (ent[i] < carry) ent[i] = carry;
}

// Histogram: per (input row, chunk) element counts into counts[r*v + c].
__global__ __launch_bounds__(kNT) void k_histogram(int64_t E, int32_t blockElems,
                                                   const int64_t* __restrict__ rowPtr,
                                                   const TileInfo* __restrict__ info,
                                                   const int32_t* __restrict__ col, int shift, int v,
                                                   int maxRows, int32_t* __restrict__ counts,
                                                   int32_t* __restrict__ err) {
  __shared__ int32_t hist[kMsNBMax];
  __shared__ int64_t bnd[kMsRowsMax];
  __shared__ TileInfo s_info;
  const int64_t e0 = (int64_t)blockIdx.x * blockElems;
  const int64_t e1 = (e0 + blockElems < E) ? e0 + blockElems : E;
  const int n = (int)(e1 - e0);
  const int nrows = range_rows(rowPtr, info, blockIdx.x, maxRows, bnd, &s_info);
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
  const int64_t r0 = s_info.r0;
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
//
// With kExpand the input elements are not read from a C-hat array but made
// on the fly from A and B: element e of the heavy rows' row-major product
// sequence belongs to the heavy-row entry t with src.eOff[t] <= e <
// src.eOff[t+1], and is (B.col[p], a_t * B.val[p]) with p = src.eB[t] + e -
// src.eOff[t].  This is the first level fed straight from the expansion.
template <int ITEMS, typename V, bool kVals, bool kExpand>
__global__ __launch_bounds__(kNT) void k_multisplit(int64_t E, int32_t blockElems,
                                                    const int64_t* __restrict__ rowPtr,
                                                    const TileInfo* __restrict__ info,
                                                    const int32_t* __restrict__ inCol,
                                                    const V* __restrict__ inVal, ExpandSrc src,
                                                    int shift, int v,
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
  int32_t* colBuf = (int32_t*)(valBuf + (kVals ? blockElems : 0));
  int32_t* hist = colBuf + blockElems;
  int32_t* loff = hist + NBcap;
  uint16_t* bktBuf = (uint16_t*)(loff + NBcap);
  __shared__ int32_t wtot[kNT / kWave];
  __shared__ TileInfo s_info;
  // Work groups are dealt round-robin to the XCDs; each XCD gets a
  // contiguous run of tiles instead, so that neighbouring heavy rows, which
  // share B rows, are expanded under the same L2.  The grid is padded to a
  // multiple of the XCD count; padding tiles exit at once.
  const int64_t nTiles = (E + blockElems - 1) / blockElems;
  const int64_t tile = (int64_t)(blockIdx.x % kXcds) * (gridDim.x / kXcds) + blockIdx.x / kXcds;
  if (tile >= nTiles) return;
  const int64_t e0 = tile * blockElems;
  const int64_t e1 = (e0 + blockElems < E) ? e0 + blockElems : E;
  const int n = (int)(e1 - e0);
  if constexpr (kExpand) {
    // Entry marks of the elements (below), cleared before the tile
    // descriptor is read.
    for (int i = threadIdx.x; i < n; i += kNT) colBuf[i] = -1;
  }
  const int nrows = range_rows(rowPtr, info, tile, maxRows, bnd, &s_info);
  if (nrows < 0) {
    if (threadIdx.x == 0) flag_error(err, kErrRowsPerBlock);
    return;
  }
  const int NB = nrows * v;
  const int nbits = bits_for(NB);
  for (int i = threadIdx.x; i < NB; i += kNT) hist[i] = 0;
  if constexpr (kExpand) entries_of_range(colBuf, n, e0, s_info.t0, s_info.t1, src.eOff, wtot);
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
      if constexpr (kExpand) {
        const int32_t t = colBuf[idx];
        const int64_t bp = (int64_t)src.eB[t] + (e - src.eOff[t]);
        cc[it] = src.bcol[bp];
        if constexpr (kVals) xv[it] = ((const V*)src.eVal)[t] * ((const V*)src.bval)[bp];
      } else {
        cc[it] = inCol[e];
        if constexpr (kVals) xv[it] = inVal[e];
      }
      bb[it] = (uint32_t)(local_row(bnd, nrows, e) * v + (cc[it] >> shift));
    }
  }
  // Count the buckets and rank every element inside its bucket at once: one
  // lane per (wave, bucket) adds the group's size and gets its base back.
  int32_t rank[ITEMS];
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const bool act = it * kNT + (int)threadIdx.x < n;
    const uint64_t m = match_key(bb[it], nbits, act);
    const int leader = act ? ffs64(m) : lane_id();
    int32_t base = 0;
    if (act && lane_id() == leader) base = atomicAdd(&hist[bb[it]], __popcll(m));
    rank[it] = __shfl(base, leader) + __popcll(m & lanemask_lt());
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
  // Reserve each bucket's run in its chunk.  The atomics' results are only
  // needed by the final write, so they stay in registers while the LDS
  // permute runs and their latency overlaps it.
  const int64_t r0 = s_info.r0;
  constexpr int kBPT = kMsNBMax / kNT;  // buckets per thread
  unsigned long long gres[kBPT];
#pragma unroll
  for (int k = 0; k < kBPT; ++k) {
    const int b = threadIdx.x + k * kNT;
    gres[k] = 0;
    if (b < NB) {
      const int32_t c = hist[b];
      if (c) {
        const int lr = b / v;
        const int32_t q = inv[(r0 + lr) * v + (b - lr * v)];
        gres[k] = atomicAdd((unsigned long long*)&cursor[q], (unsigned long long)c);
      }
    }
  }
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const bool act = it * kNT + (int)threadIdx.x < n;
    if (act) {
      const int pos = loff[bb[it]] + rank[it];
      colBuf[pos] = cc[it] & wmask;
      if constexpr (kVals) valBuf[pos] = xv[it];
      bktBuf[pos] = (uint16_t)bb[it];
    }
  }
#pragma unroll
  for (int k = 0; k < kBPT; ++k) {
    const int b = threadIdx.x + k * kNT;
    if (b < NB) gbase[b] = (int64_t)gres[k];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < n; idx += kNT) {
    const int b = bktBuf[idx];
    const int64_t dest = gbase[b] + (idx - loff[b]);
    outCol[dest] = colBuf[idx];
    if constexpr (kVals) outVal[dest] = valBuf[idx];
  }
}


// Expansion straight into the final chunks.  With every chunk count known
// from the structure, the chunk tree of each heavy row is fixed before any
// element moves, so the levels of the multisplit (§III-C) collapse into one
// pass over the row-major product sequence: element e (made from A and B as
// above) goes to the final chunk covering its column, finalOf[row * nreq +
// slot] with slot = col >> log2W; spanOf holds that chunk's width as log2 of
// W-wide slots.  A work group's buckets are (row inside the range, first
// slot of the final chunk).
//
// The entries that start inside the range are staged in LDS at their first
// element (B offset, a_ik, row), so an element reads only B from memory: a
// wave finds each lane's entry as the last start at or before it, from one
// ballot of the start flags (and, for entries begun in an earlier 64-element
// segment, that segment's last start).  Consecutive elements that share a
// bucket (most of a scaled B row's run inside one W-wide slot) are ranked
// together: the first lane of each such group adds the group's size to the
// bucket's LDS counter.  One global reservation per bucket, then every
// element is written in place with its column made local to the chunk
// (as uint16_t when every chunk is at most 65536 columns wide).
template <int ITEMS, typename V, bool kVals, typename OC>
__global__ __launch_bounds__(kNT) void k_expand_final(int64_t E, int32_t blockElems,
                                                      const int64_t* __restrict__ rowPtr,
                                                      const TileInfo* __restrict__ info,
                                                      ExpandSrc src,
                                                      const int32_t* __restrict__ finalOf,
                                                      const int8_t* __restrict__ spanOf,
                                                      int32_t nreq, int log2W, int maxRows,
                                                      int64_t* __restrict__ cursor,
                                                      OC* __restrict__ outCol,
                                                      V* __restrict__ outVal,
                                                      int32_t* __restrict__ err) {
  // LDS (sized by the host): gbase[NB] i64 | bnd[maxRows] i64 |
  // eA[kXfEnt] V | eBase[kXfEnt] i32 | eRow[kXfEnt] i32 |
  // slotAt[blockElems] i32 | hist[NB] i32 | finS[NB] i32 | spanS[NB] i8,
  // NB = maxRows * nreq.
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int kSegs = ITEMS * (kNT / kWave);
  const int NBcap = maxRows * nreq;
  int64_t* gbase = (int64_t*)smem;
  int64_t* bnd = gbase + NBcap;
  V* eA = (V*)(bnd + maxRows);
  int32_t* eBase = (int32_t*)(eA + (kVals ? kXfEnt : 0));
  int32_t* eRow = eBase + kXfEnt;
  int32_t* slotAt = eRow + kXfEnt;
  int32_t* hist = slotAt + blockElems;
  int32_t* finS = hist + NBcap;
  int8_t* spanS = (int8_t*)(finS + NBcap);
  __shared__ int32_t segLast[kSegs];
  __shared__ TileInfo s_info;
  const int64_t nTiles = (E + blockElems - 1) / blockElems;
  const int64_t tile = (int64_t)(blockIdx.x % kXcds) * (gridDim.x / kXcds) + blockIdx.x / kXcds;
  if (tile >= nTiles) return;
  const int64_t e0 = tile * blockElems;
  const int64_t e1 = (e0 + blockElems < E) ? e0 + blockElems : E;
  const int n = (int)(e1 - e0);
  for (int i = threadIdx.x; i < n; i += kNT) slotAt[i] = -1;
  const int nrows = range_rows(rowPtr, info, tile, maxRows, bnd, &s_info);
  if (nrows < 0) {
    if (threadIdx.x == 0) flag_error(err, kErrRowsPerBlock);
    return;
  }
  const int64_t r0 = s_info.r0;
  const int32_t t0 = s_info.t0;
  const int NB = nrows * nreq;
  for (int i = threadIdx.x; i < NB; i += kNT) {
    hist[i] = 0;
    spanS[i] = spanOf[r0 * nreq + i];
    finS[i] = finalOf[r0 * nreq + i];
  }
  __syncthreads();
  // Entries with products that start inside the range (and t0, which holds
  // the range's first element) mark their first element with their index
  // j = t - t0; the first kXfEnt of them also leave their B offset relative
  // to the element index, a_ik and local row in LDS (later ones are read
  // from memory by their elements, which long tiles of very short entries
  // only need).
  // (The entry's B offset and a_ik are loaded together with its offsets, so
  // the pass waits on one round of memory latency.)
  for (int32_t t = t0 + (int32_t)threadIdx.x; t <= s_info.t1; t += kNT) {
    const int64_t o = src.eOff[t];
    const int64_t o1 = src.eOff[t + 1];
    const int32_t eb = src.eB[t];
    V ea = V(0);
    if constexpr (kVals) ea = ((const V*)src.eVal)[t];
    if (o1 == o) continue;
    const int64_t from = o > e0 ? o : e0;
    const int64_t pos = from - e0;
    if (pos >= n) continue;
    const int j = t - t0;
    slotAt[pos] = j;
    if (j < kXfEnt) {
      eRow[j] = local_row(bnd, nrows, from);
      eBase[j] = (int32_t)((int64_t)eb + e0 - o);
      if constexpr (kVals) eA[j] = ea;
    }
  }
  __syncthreads();

  // Entry start of every element: the last start flag at or before it in
  // its 64-element segment, else the last one of an earlier segment.
  const int w = threadIdx.x / kWave;
  const uint64_t le = lanemask_lt() | (1ull << lane_id());
  int32_t hp[ITEMS];
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const int idx = it * kNT + threadIdx.x;
    const bool head = idx < n && slotAt[idx] >= 0;
    const uint64_t hm = __ballot(head);
    const int segBase = it * kNT + w * kWave;
    hp[it] = (hm & le) ? segBase + last_set64(hm & le) : -1;
    if (lane_id() == 0) segLast[it * (kNT / kWave) + w] = hm ? segBase + last_set64(hm) : -1;
  }
  __syncthreads();
  // segLast becomes its own inclusive prefix maximum: the last start at or
  // before the end of each segment.
  static_assert(kSegs <= kWave, "one wave scans the segments");
  if (w == 0) {
    int32_t x = lane_id() < kSegs ? segLast[lane_id()] : -1;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int32_t y = __shfl_up(x, d);
      if (lane_id() >= d && y > x) x = y;
    }
    if (lane_id() < kSegs) segLast[lane_id()] = x;
  }
  __syncthreads();
  const int W = 1 << log2W;
  // Every lane loads (lanes past the range repeat element 0), so the loads
  // of all items are in flight together.
  int32_t lrow[ITEMS];
  uint32_t bp[ITEMS];
  V av[ITEMS];
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const int idx = it * kNT + threadIdx.x;
    // Segment 0 starts with the range's first entry, so every element of a
    // later segment without a start of its own finds one before it.
    const int sg = it * (kNT / kWave) + w - 1;
    const int h = idx < n ? (hp[it] >= 0 ? hp[it] : segLast[sg > 0 ? sg : 0]) : 0;
    const int j = slotAt[h];
    int32_t eb;
    if (j < kXfEnt) {
      eb = eBase[j];
      lrow[it] = eRow[j];
      if constexpr (kVals) av[it] = eA[j];
    } else {
      const int32_t t = t0 + j;
      const int64_t o = src.eOff[t];
      eb = (int32_t)((int64_t)src.eB[t] + e0 - o);
      lrow[it] = local_row(bnd, nrows, o > e0 ? o : e0);
      if constexpr (kVals) av[it] = ((const V*)src.eVal)[t];
    }
    bp[it] = (uint32_t)((idx < n ? idx : 0) + eb);
  }
  int32_t cc[ITEMS];
  V xv[ITEMS];
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    cc[it] = src.bcol[bp[it]];
    if constexpr (kVals) xv[it] = ((const V*)src.bval)[bp[it]];
  }
  int32_t bb[ITEMS];
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const int idx = it * kNT + threadIdx.x;
    const int lr = lrow[it];
    if constexpr (kVals) xv[it] *= av[it];
    const int32_t slot = cc[it] >> log2W;
    const int sp = spanS[lr * nreq + slot];
    cc[it] &= (W << sp) - 1;
    bb[it] = idx < n ? lr * nreq + (slot & ~((1 << sp) - 1)) : -1;
  }
  // Rank: groups of consecutive lanes with one bucket share one LDS atomic.
  int32_t rank[ITEMS];
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const bool act = bb[it] >= 0;
    const int32_t prev = __shfl_up(bb[it], 1);
    const bool head = act && (lane_id() == 0 || prev != bb[it]);
    const uint64_t heads = __ballot(head);
    const uint64_t actm = __ballot(act);
    const int h = last_set64(heads & le);
    const uint64_t above = heads & ~le;
    const int nxt = above ? ffs64(above) : 64 - __clzll((long long)actm);
    int32_t base = 0;
    if (head) base = atomicAdd(&hist[bb[it]], nxt - lane_id());
    rank[it] = __shfl(base, act ? h : lane_id()) + (lane_id() - h);
  }
  __syncthreads();
  for (int b = threadIdx.x; b < NB; b += kNT) {
    const int32_t c = hist[b];
    int64_t g = 0;
    if (c) {
      const int32_t q = finS[b];
      if (q == -1) {
        flag_error(err, kErrCountMismatch);
      } else if (q >= 0) {
        g = (int64_t)atomicAdd((unsigned long long*)&cursor[q], (unsigned long long)c);
      }  // q <= -2: a chunk taken straight from A and B, nothing written
    }
    gbase[b] = g;
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    if (bb[it] >= 0 && finS[bb[it]] >= 0) {
      const int64_t dest = gbase[bb[it]] + rank[it];
      if (dest < E) {
        outCol[dest] = (OC)cc[it];
        if constexpr (kVals) outVal[dest] = xv[it];
      }
    }
  }
}

}  // namespace

void multisplit_set_attributes() {
#define SG_ATTR(...) allow_max_dynamic_lds((const void*)__VA_ARGS__)
  SG_ATTR(k_multisplit<kMsItemsF64, double, true, false>);
  SG_ATTR(k_multisplit<kMsItemsF32, float, true, false>);
  SG_ATTR(k_multisplit<kMsItemsF32, float, false, false>);
  SG_ATTR(k_multisplit<kMsItemsF64, double, true, true>);
  SG_ATTR(k_multisplit<kMsItemsF32, float, true, true>);
  SG_ATTR(k_multisplit<kMsItemsF32, float, false, true>);
  SG_ATTR((k_expand_final<kXfItemsF64, double, true, int32_t>));
  SG_ATTR((k_expand_final<kXfItemsF32, float, true, int32_t>));
  SG_ATTR((k_expand_final<kXfItemsF32, float, false, int32_t>));
  SG_ATTR((k_expand_final<kXfItemsF64, double, true, uint16_t>));
  SG_ATTR((k_expand_final<kXfItemsF32, float, true, uint16_t>));
  SG_ATTR((k_expand_final<kXfItemsF32, float, false, uint16_t>));
#undef SG_ATTR
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

bool expand_final_geometry(bool f64, int64_t rowTau, int64_t nreq, int32_t* blockElems,
                           int* maxRows) {
  int64_t G = (int64_t)kNT * (f64 ? kXfItemsF64 : kXfItemsF32);
  auto rows_for = [&](int64_t g) { return (g - 1) / (rowTau + 1) + 2; };
  while (G > 64 && (rows_for(G) * nreq > kXfNBMax || rows_for(G) > kMsRowsMax)) G /= 2;
  *blockElems = (int32_t)G;
  *maxRows = (int)rows_for(G);
  return rows_for(G) * nreq <= kXfNBMax && rows_for(G) <= kMsRowsMax;
}

void launch_expand_final(bool f64, int64_t E, int32_t blockElems, const int64_t* rowPtr,
                         const TileInfo* info, const ExpandSrc& src, const int32_t* finalOf,
                         const int8_t* spanOf, int32_t nreq, int log2W, int maxRows,
                         int64_t* cursor, void* outCol, bool col16, void* outVal, int32_t* err,
                         hipStream_t s) {
  if (E <= 0) return;
  const unsigned g = (grid_for(E, blockElems) + kXcds - 1) / kXcds * kXcds;
  const size_t NB = (size_t)maxRows * nreq;
  const size_t vb = !outVal ? 0 : f64 ? 8 : 4;
  const size_t lds = NB * 17 + (size_t)maxRows * 8 + (size_t)kXfEnt * (vb + 8) +
                     (size_t)blockElems * 4 + 16;
#define SG_XF1(ITEMS, V, VALS, OC)                                                             \
  hipLaunchKernelGGL((k_expand_final<ITEMS, V, VALS, OC>), dim3(g), dim3(kNT), lds, s, E,        \
                     blockElems, rowPtr, info, src, finalOf, spanOf, nreq, log2W, maxRows,       \
                     cursor, (OC*)outCol, (V*)outVal, err)
#define SG_XF(ITEMS, V, VALS)                                                                  \
  do {                                                                                         \
    if (col16) SG_XF1(ITEMS, V, VALS, uint16_t);                                               \
    else SG_XF1(ITEMS, V, VALS, int32_t);                                                      \
  } while (0)
  if (!outVal) SG_XF(kXfItemsF32, float, false);
  else if (f64) SG_XF(kXfItemsF64, double, true);
  else SG_XF(kXfItemsF32, float, true);
#undef SG_XF
#undef SG_XF1
}

void launch_block_starts(int64_t nItems, const int64_t* off, int64_t G, int64_t nBlocks,
                         int32_t* out, hipStream_t s) {
  if (nItems <= 0 || nBlocks <= 0) return;
  unsigned g = grid_for(nItems, kNT);
  if (g > 65536) g = 65536;
  hipLaunchKernelGGL(k_block_starts, dim3(g), dim3(kNT), 0, s, nItems, off, G, nBlocks, out);
}

void launch_tile_info(int64_t E, int32_t blockElems, const int64_t* rowPtr, int64_t R,
                      const int32_t* blkRow, const int32_t* blkEnt, int64_t nE, TileInfo* info,
                      hipStream_t s) {
  if (E <= 0) return;
  const int64_t nTiles = (E + blockElems - 1) / blockElems;
  hipLaunchKernelGGL(k_tile_info, dim3(grid_for(nTiles, kNT)), dim3(kNT), 0, s, nTiles, E,
                     (int64_t)blockElems, rowPtr, R, blkRow, blkEnt, nE, info);
}

void launch_histogram(int64_t E, int32_t blockElems, const int64_t* rowPtr,
                      const TileInfo* info, const int32_t* col, int shift, int v, int maxRows,
                      int32_t* counts, int32_t* err, hipStream_t s) {
  if (E <= 0) return;
  hipLaunchKernelGGL(k_histogram, dim3(grid_for(E, blockElems)), dim3(kNT), 0, s, E, blockElems,
                     rowPtr, info, col, shift, v, maxRows, counts, err);
}

void launch_multisplit(bool f64, int64_t E, int32_t blockElems, const int64_t* rowPtr,
                       const TileInfo* info, const int32_t* inCol, const void* inVal,
                       const ExpandSrc* src,
                       int shift, int v, int32_t wmask, int maxRows, const int32_t* inv,
                       int64_t* cursor, int32_t* outCol, void* outVal, int32_t* err,
                       hipStream_t s) {
  if (E <= 0) return;
  const unsigned g = (grid_for(E, blockElems) + kXcds - 1) / kXcds * kXcds;
  const size_t NB = (size_t)maxRows * v;
  const size_t vb = !outVal ? 0 : f64 ? 8 : 4;
  const size_t lds = NB * 8 + (size_t)maxRows * 8 + (size_t)blockElems * (vb + 4 + 2) + NB * 8 + 16;
  const ExpandSrc none{};
  const ExpandSrc& x = src ? *src : none;
#define SG_MS(ITEMS, V, VALS, EXP)                                                              \
  hipLaunchKernelGGL((k_multisplit<ITEMS, V, VALS, EXP>), dim3(g), dim3(kNT), lds, s, E,        \
                     blockElems, rowPtr, info, inCol, (const V*)inVal, x, shift, v, wmask,     \
                     maxRows,                                                                    \
                     inv, cursor, outCol, (V*)outVal, err)
  // Columns only: the geometry of the fp32 instance.
  if (src) {
    if (!outVal) SG_MS(kMsItemsF32, float, false, true);
    else if (f64) SG_MS(kMsItemsF64, double, true, true);
    else SG_MS(kMsItemsF32, float, true, true);
  } else {
    if (!outVal) SG_MS(kMsItemsF32, float, false, false);
    else if (f64) SG_MS(kMsItemsF64, double, true, false);
    else SG_MS(kMsItemsF32, float, true, false);
  }
#undef SG_MS
}

}  // namespace sg
