// LDS hash accumulators (gMAGNUS page §III-E; Ocean page §2): light rows of C
// computed row by row with Gustavson's method (gMAGNUS §II-B, Eq. 1), and
// light chunks of the reordered heavy intermediate.  Items are binned by
// size; each bin runs `tpr` threads per item with a table of T slots.
//
//   symbolic: insert column keys into an LDS key set, count the new ones;
//   numeric:  insert-or-add (key, value) pairs with LDS atomics, compact the
//             occupied slots, bitonic-sort them by column in LDS and write
//             the sorted row (or chunk) to its place in C.
#include <algorithm>
#include <climits>

#include "device_common.hpp"

namespace sg {
namespace {

constexpr int kMaxSpt = 24;  // slots per thread held in registers by the compaction

// Value of lane j (j the same for every lane), without the LDS crossbar.
__device__ __forceinline__ float lane_read(float x, int j) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), j));
}
__device__ __forceinline__ double lane_read(double x, int j) {
  const int64_t b = __double_as_longlong(x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int32_t)(uint32_t)b, j);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int32_t)(uint32_t)(b >> 32), j);
  return __longlong_as_double((int64_t)(((uint64_t)hi << 32) | lo));
}

// Products [p0, p1) of one row of A*B in Gustavson order (entry-major): the
// flattened product index q of entry e starts at scanA[e] (row-local
// exclusive offset).  The wave keeps 64 consecutive A entries in registers
// and finds, for each of 64 consecutive products, the entry that owns it:
// when those products span at most kStreamWalk entries (two ballots tell),
// by walking these entries with lane broadcasts, else by a 6-step binary
// search across lanes (permutes through the LDS crossbar); then it loads the
// B element's column (and value).  kStreamU runs of 64 products are located and their loads issued
// before any is used, so a wave waits on one memory round trip per 256
// products, not per 64.  f(act, col, a, b, q) gets the column, the A value,
// the B value and the product index q.  Every lane runs the same iterations.
constexpr int kStreamU = 4;
constexpr int kStreamWalk = 8;  // entries a piece may span for the walk
template <bool VAL, typename V, typename F>
__device__ __forceinline__ void stream_row(const int32_t* __restrict__ scanA,
                                           const int32_t* __restrict__ acol,
                                           const V* __restrict__ aval,
                                           const int32_t* __restrict__ brp,
                                           const int32_t* __restrict__ bcol,
                                           const V* __restrict__ bval, int64_t rs,
                                           int64_t re, int32_t P, int32_t p0, int32_t p1,
                                           F&& f) {
  if (p0 >= p1) return;
  int64_t j = wave_last_le(scanA, rs, re, p0);
  int32_t p = p0;
  while (p < p1) {
    const int64_t e = j + lane_id();
    const bool ev = e < re;
    const int32_t off = ev ? scanA[e] : P;
    int32_t bs = 0;
    V a = V(0);
    if (ev) {
      bs = brp[acol[e]];
      if (VAL) a = aval[e];
    }
    int32_t bend = (j + kWave < re) ? scanA[j + kWave] : P;
    if (bend > p1) bend = p1;
    for (; p < bend; p += kWave * kStreamU) {
      bool act[kStreamU];
      int32_t cc[kStreamU], qq[kStreamU];
      V sa[kStreamU], bv[kStreamU];
#pragma unroll
      for (int u = 0; u < kStreamU; ++u) {
        const int32_t q = p + u * kWave + lane_id();
        act[u] = q < bend;
        qq[u] = q;
        cc[u] = 0;
        sa[u] = V(0);
        bv[u] = V(0);
        if (p + u * kWave < bend) {  // the same for every lane
          const int32_t pu = p + u * kWave;
          // entries owning the first and the last product of this piece
          const int lo = last_set64(__ballot(off <= pu));
          const int hi = last_set64(__ballot(off <= pu + kWave - 1));
          int32_t so, sb;
          if (hi - lo < kStreamWalk) {
            so = __builtin_amdgcn_readlane(off, lo);
            sb = __builtin_amdgcn_readlane(bs, lo);
            if (VAL) sa[u] = lane_read(a, lo);
            for (int s = lo + 1; s <= hi; ++s) {
              const int32_t os = __builtin_amdgcn_readlane(off, s);
              const int32_t bss = __builtin_amdgcn_readlane(bs, s);
              const V as = VAL ? lane_read(a, s) : V(0);
              if (os <= q) {
                so = os;
                sb = bss;
                if (VAL) sa[u] = as;
              }
            }
          } else {
            int s = 0;
#pragma unroll
            for (int step = 32; step >= 1; step >>= 1) {
              const int32_t o = __shfl(off, s + step);
              if (o <= q) s += step;
            }
            so = __shfl(off, s);
            sb = __shfl(bs, s);
            if (VAL) sa[u] = __shfl(a, s);
          }
          if (act[u]) {
            const int32_t bi = sb + (q - so);
            cc[u] = bcol[bi];
            if (VAL) bv[u] = bval[bi];
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kStreamU; ++u) f(act[u], cc[u], sa[u], bv[u], qq[u]);
    }
    p = bend;
    j += kWave;
  }
}

// ---------------------------------------------------------------- symbolic
template <int TPR, int RPB>
__global__ __launch_bounds__(TPR* RPB) void k_sym_rows(const int32_t* __restrict__ rows,
                                                       int64_t nrows, int32_t T, RowArgs a,
                                                       int64_t* __restrict__ cnt,
                                                       int32_t* __restrict__ err) {
  extern __shared__ __align__(16) unsigned char smem[];
  int32_t* keysAll = (int32_t*)smem;
  int32_t* gcount = keysAll + RPB * T;
  const int g = threadIdx.x / TPR, t = threadIdx.x % TPR;
  int32_t* keys = keysAll + g * T;
  for (int s = t; s < T; s += TPR) keys[s] = kEmptyKey;
  if (t == 0) gcount[g] = 0;
  __syncthreads();
  const int64_t ri = (int64_t)blockIdx.x * RPB + g;
  int32_t mine = 0;
  int32_t row = 0;
  if (ri < nrows) {
    row = rows[ri];
    const int64_t rs = a.arp[row], re = a.arp[row + 1];
    const int32_t P = (int32_t)a.rowP[row];
    constexpr int WPR = TPR / kWave;
    const int w = t / kWave;
    const int32_t p0 = (int32_t)((int64_t)P * w / WPR);
    const int32_t p1 = (int32_t)((int64_t)P * (w + 1) / WPR);
    stream_row<false, float>(a.scanA, a.acol, (const float*)nullptr, a.brp, a.bcol,
                             (const float*)nullptr, rs, re, P, p0, p1,
                             [&](bool act, int32_t c, float, float, int32_t) {
                               if (act && hset_insert(keys, (uint32_t)T, c, err)) ++mine;
                             });
  }
  const int32_t ws = wave_sum(mine);
  if (lane_id() == 0 && ri < nrows) atomicAdd(&gcount[g], ws);
  __syncthreads();
  if (t == 0 && ri < nrows) cnt[row] = gcount[g];
}

template <int TPR, int RPB, typename C = int32_t>
__global__ __launch_bounds__(TPR* RPB) void k_sym_chunks(const ChunkDesc* __restrict__ desc,
                                                         int64_t n, int32_t T, ChunkList cl,
                                                         int32_t* __restrict__ err) {
  extern __shared__ __align__(16) unsigned char smem[];
  int32_t* keysAll = (int32_t*)smem;
  int32_t* gcount = keysAll + RPB * T;
  const int g = threadIdx.x / TPR, t = threadIdx.x % TPR;
  int32_t* keys = keysAll + g * T;
  for (int s = t; s < T; s += TPR) keys[s] = kEmptyKey;
  if (t == 0) gcount[g] = 0;
  __syncthreads();
  const int64_t ri = (int64_t)blockIdx.x * RPB + g;
  int32_t mine = 0;
  ChunkDesc d{};
  if (ri < n) {
    d = desc[ri];
    const int64_t off = d.off;
    const int64_t end = off + d.cnt;
    const C* __restrict__ col = (const C*)(d.buf ? cl.col1 : cl.col0);
    for (int64_t e = off + t; e < end; e += TPR)
      if (hset_insert(keys, (uint32_t)T, col[e], err)) ++mine;
  }
  const int32_t ws = wave_sum(mine);
  if (lane_id() == 0 && ri < n) atomicAdd(&gcount[g], ws);
  __syncthreads();
  if (t == 0 && ri < n) cl.slotNnz[d.base] = gcount[g];
}

// ------------------------------------------------------- dense window rows
// Light rows whose products span at most 32 * window_words(cap) columns:
// rowWin[row] holds the span's first column (low 32 bits) and its length in
// 32-bit words (high bits), and an LDS bitmap over the span replaces the
// hash table.  Symbolic counts its set bits.  Numeric stages every product's
// (column, value) in LDS by product index while setting the bits, takes the
// word prefix of the popcounts (the rank of a column among the row's columns
// is its output position), then adds each staged product straight into an
// LDS array of the row's exact output size: no probing and no sort, and the
// row is written in column order.
__device__ __forceinline__ int32_t win_lo(int64_t w) { return (int32_t)(uint32_t)(w & 0xffffffff); }
__device__ __forceinline__ int32_t win_words(int64_t w) { return (int32_t)(w >> 32); }

template <int TPR, int RPB>
__global__ __launch_bounds__(TPR* RPB) void k_sym_rows_win(const int32_t* __restrict__ rows,
                                                           int64_t nrows, int32_t words, RowArgs a,
                                                           int64_t* __restrict__ cnt) {
  extern __shared__ __align__(16) uint32_t bmAll[];
  constexpr int WPR = TPR / kWave;
  __shared__ int32_t gsum[RPB * WPR];
  const int g = threadIdx.x / TPR, t = threadIdx.x % TPR, w = t / kWave;
  uint32_t* bm = bmAll + g * words;
  const int64_t ri = (int64_t)blockIdx.x * RPB + g;
  int32_t row = 0, lo = 0, nw = 0;
  if (ri < nrows) {
    row = rows[ri];
    const int64_t win = a.rowWin[row];
    lo = win_lo(win);
    nw = win_words(win);
  }
  for (int i = t; i < nw; i += TPR) bm[i] = 0;
  __syncthreads();
  if (ri < nrows) {
    const int64_t rs = a.arp[row], re = a.arp[row + 1];
    const int32_t P = (int32_t)a.rowP[row];
    const int32_t p0 = (int32_t)((int64_t)P * w / WPR);
    const int32_t p1 = (int32_t)((int64_t)P * (w + 1) / WPR);
    stream_row<false, float>(a.scanA, a.acol, (const float*)nullptr, a.brp, a.bcol,
                             (const float*)nullptr, rs, re, P, p0, p1,
                             [&](bool act, int32_t col, float, float, int32_t) {
                               if (act) {
                                 const int32_t c = col - lo;
                                 const uint32_t bit = 1u << (c & 31);
                                 if (!(bm[c >> 5] & bit)) atomicOr(&bm[c >> 5], bit);
                               }
                             });
  }
  __syncthreads();
  int32_t mine = 0;
  for (int i = t; i < nw; i += TPR) mine += __popc(bm[i]);
  mine = wave_sum(mine);
  if (lane_id() == 0) gsum[threadIdx.x / kWave] = mine;
  __syncthreads();
  if (t == 0 && ri < nrows) {
    int32_t tot = 0;
    for (int i = 0; i < WPR; ++i) tot += gsum[g * WPR + i];
    cnt[row] = tot;
  }
}

// LDS per row: vals[cap] V | pv[cap] V | bm[words] | wpre[words] |
// cols[cap] u16 | pc[cap] u16.
__host__ __device__ constexpr size_t window_group_bytes(int32_t cap, int32_t words, int vb) {
  return ((size_t)cap * (2 * vb + 4) + (size_t)words * 8 + 15) / 16 * 16;
}

template <int TPR, int RPB, typename V>
__global__ __launch_bounds__(TPR* RPB) void k_num_rows_win(const int32_t* __restrict__ rows,
                                                           int64_t nrows, int32_t words,
                                                           int32_t cap, RowArgs a,
                                                           const int64_t* __restrict__ cRowOff,
                                                           int32_t* __restrict__ ccol,
                                                           V* __restrict__ cval,
                                                           int32_t* __restrict__ err,
                                                           int64_t* __restrict__ cntOut) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int WPR = TPR / kWave;
  __shared__ int32_t wtot[RPB * WPR];
  const int g = threadIdx.x / TPR, t = threadIdx.x % TPR, w = t / kWave;
  unsigned char* base = smem + (size_t)g * window_group_bytes(cap, words, (int)sizeof(V));
  V* vals = (V*)base;
  V* pv = vals + cap;
  uint32_t* bm = (uint32_t*)(pv + cap);
  int32_t* wpre = (int32_t*)(bm + words);
  uint16_t* cols = (uint16_t*)(wpre + words);
  uint16_t* pc = cols + cap;
  const int64_t ri = (int64_t)blockIdx.x * RPB + g;
  int32_t row = 0, lo = 0, nw = 0, P = 0, want = 0;
  int64_t obase = 0;
  if (ri < nrows) {
    row = rows[ri];
    const int64_t win = a.rowWin[row];
    lo = win_lo(win);
    nw = win_words(win);
    P = (int32_t)a.rowP[row];
    if (P > cap) P = cap;
    obase = cRowOff[row];
    const int64_t wn = cRowOff[row + 1] - obase;
    want = (int32_t)(wn < cap ? wn : cap);
  }
  for (int i = t; i < nw; i += TPR) bm[i] = 0;
  for (int i = t; i < want; i += TPR) vals[i] = V(0);
  __syncthreads();
  if (ri < nrows) {
    const int64_t rs = a.arp[row], re = a.arp[row + 1];
    const int32_t p0 = (int32_t)((int64_t)P * w / WPR);
    const int32_t p1 = (int32_t)((int64_t)P * (w + 1) / WPR);
    stream_row<true, V>(a.scanA, a.acol, (const V*)a.aval, a.brp, a.bcol, (const V*)a.bval, rs,
                        re, P, p0, p1, [&](bool act, int32_t col, V av, V bv, int32_t q) {
                          if (act) {
                            const int32_t c = col - lo;
                            pc[q] = (uint16_t)c;
                            pv[q] = av * bv;
                            const uint32_t bit = 1u << (c & 31);
                            if (!(bm[c >> 5] & bit)) atomicOr(&bm[c >> 5], bit);
                          }
                        });
  }
  __syncthreads();
  // Exclusive prefix of the word popcounts: each thread owns a contiguous
  // run of words.
  const int wpt = (nw + TPR - 1) / TPR;
  const int w0 = t * wpt;
  int32_t mine = 0;
  for (int i = 0; i < wpt; ++i)
    if (w0 + i < nw) mine += __popc(bm[w0 + i]);
  const int32_t inc = wave_incl_scan(mine);
  if (lane_id() == kWave - 1) wtot[threadIdx.x / kWave] = inc;
  __syncthreads();
  int32_t before = 0, total = 0;
#pragma unroll
  for (int i = 0; i < WPR; ++i) {
    const int32_t tv = wtot[g * WPR + i];
    if (i < w) before += tv;
    total += tv;
  }
  int32_t run = before + inc - mine;
  for (int i = 0; i < wpt; ++i) {
    if (w0 + i < nw) {
      wpre[w0 + i] = run;
      run += __popc(bm[w0 + i]);
    }
  }
  __syncthreads();
  // Estimate workflows: a row with more entries than its reserved capacity
  // writes nothing and reports -1.
  const bool over = cntOut && total > want;
  if (ri < nrows && t == 0) {
    if (cntOut) cntOut[row] = over ? -1 : total;
    else if (total != want) flag_error(err, kErrCountMismatch);
  }
  if (cntOut) want = over ? 0 : total;
  for (int q = t; q < P; q += TPR) {
    const int32_t c = pc[q];
    const int32_t r = wpre[c >> 5] + __popc(bm[c >> 5] & ((1u << (c & 31)) - 1u));
    if (r < want) {
      atomicAdd(&vals[r], pv[q]);
      cols[r] = (uint16_t)c;
    }
  }
  __syncthreads();
  for (int r = t; r < want; r += TPR) {
    ccol[obase + r] = lo + cols[r];
    cval[obase + r] = vals[r];
  }
}

// ----------------------------------------------------------------- numeric
// Shared tail of the numeric kernels, part 1: compact the occupied slots of
// this group's table into [0, total) and pad [total, TPR * E) with INT_MAX.
// Returns total.  Called by every thread of the work group.
template <int TPR, int RPB, int E, typename V>
__device__ __forceinline__ int32_t compact_slots(int32_t* keys, V* vals, int32_t spt,
                                                 int32_t* wtot) {
  constexpr int WPR = TPR / kWave;
  const int g = threadIdx.x / TPR, t = threadIdx.x % TPR, w = t / kWave;
  int32_t kk[kMaxSpt];
  V vv[kMaxSpt];
  int32_t mine = 0;
#pragma unroll
  for (int s = 0; s < kMaxSpt; ++s) {
    kk[s] = kEmptyKey;
    vv[s] = V(0);
    if (s < spt) {
      const int slot = t + s * TPR;
      kk[s] = keys[slot];
      vv[s] = vals[slot];
      mine += (kk[s] != kEmptyKey);
    }
  }
  const int32_t inc = wave_incl_scan(mine);
  if (lane_id() == kWave - 1) wtot[threadIdx.x / kWave] = inc;
  __syncthreads();
  int32_t before = 0, total = 0;
#pragma unroll
  for (int i = 0; i < WPR; ++i) {
    const int32_t tv = wtot[g * WPR + i];
    if (i < w) before += tv;
    total += tv;
  }
  int32_t pos = before + inc - mine;
  __syncthreads();
#pragma unroll
  for (int s = 0; s < kMaxSpt; ++s) {
    if (s < spt && kk[s] != kEmptyKey) {
      keys[pos] = kk[s];
      vals[pos] = vv[s];
      ++pos;
    }
  }
  for (int i = total + t; i < TPR * E; i += TPR) keys[i] = INT_MAX;
  __syncthreads();
  return total;
}

// Part 2: bitonic sort of the padded entries [0, TPR * E) into registers:
// thread t ends with the entries of rank t*E .. t*E+E-1.  Of the network's
// compare-exchange distances, those below E are register swaps inside a
// thread, those below 64*E shuffles between lanes of one wave, and only the
// longer ones go through LDS with barriers (none when a wave owns the item).
// Value of lane (lane xor LD) of the wave, for the bitonic network's lane
// exchanges: within a row of 16 lanes by DPP (quad permutes for 1 and 2, row
// rotations for 4 and 8), across 16 by a swizzle inside each half wave, and
// across 32 by a permute through the LDS crossbar.
template <int LD>
__device__ __forceinline__ int32_t lane_xor(int32_t x) {
  if constexpr (LD == 1) {
    return __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
  } else if constexpr (LD == 2) {
    return __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  } else if constexpr (LD == 4) {
    const int32_t up = __builtin_amdgcn_update_dpp(x, x, 0x12C, 0xF, 0xF, false);  // row_ror:12
    const int32_t dn = __builtin_amdgcn_update_dpp(x, x, 0x124, 0xF, 0xF, false);  // row_ror:4
    return (lane_id() & 4) ? dn : up;
  } else if constexpr (LD == 8) {
    return __builtin_amdgcn_update_dpp(x, x, 0x128, 0xF, 0xF, false);  // row_ror:8
  } else if constexpr (LD == 16) {
    return __builtin_amdgcn_ds_swizzle(x, (16 << 10) | 0x1F);  // xor 16 within 32 lanes
  } else {
    return __shfl_xor(x, LD);
  }
}
template <int LD>
__device__ __forceinline__ float lane_xor_v(float x) {
  return __int_as_float(lane_xor<LD>(__float_as_int(x)));
}
template <int LD>
__device__ __forceinline__ double lane_xor_v(double x) {
  const int64_t b = __double_as_longlong(x);
  const int32_t lo = lane_xor<LD>((int32_t)(uint32_t)(b & 0xffffffff));
  const int32_t hi = lane_xor<LD>((int32_t)(b >> 32));
  return __longlong_as_double(((int64_t)hi << 32) | (int64_t)(uint32_t)lo);
}

// One compare-exchange step of the bitonic network between lanes LD apart
// (element distance j = LD * E, phase k).
template <int LD, int TPR, int E, typename V>
__device__ __forceinline__ void bitonic_lane_step(int k, int32_t (&kk)[E], V (&vv)[E]) {
  const int t = threadIdx.x % TPR;
  constexpr int j = LD * E;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int32_t ok = lane_xor<LD>(kk[e]);
    const V ov = lane_xor_v<LD>(vv[e]);
    const int i = t * E + e;
    const bool up = (i & k) == 0;
    const bool lower = (i & j) == 0;
    // In an ascending pair the lower position keeps the smaller key.
    const bool take = (lower == up) ? (ok < kk[e]) : (ok > kk[e]);
    if (take) {
      kk[e] = ok;
      vv[e] = ov;
    }
  }
}

template <int TPR, int E, typename V>
__device__ __forceinline__ void sort_to_regs(int32_t* keys, V* vals, int32_t (&kk)[E],
                                             V (&vv)[E]) {
  constexpr int NP = TPR * E;
  constexpr int kLaneSpan = kWave * E;
  const int t = threadIdx.x % TPR;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    kk[e] = keys[t * E + e];
    vv[e] = vals[t * E + e];
  }
  for (int k = 2; k <= NP; k <<= 1) {
    int j = k >> 1;
    if (j >= kLaneSpan) {
      __syncthreads();
#pragma unroll
      for (int e = 0; e < E; ++e) {
        keys[t * E + e] = kk[e];
        vals[t * E + e] = vv[e];
      }
      __syncthreads();
      for (; j >= kLaneSpan; j >>= 1) {
        for (int i = t; i < NP / 2; i += TPR) {
          const int lo = ((i & ~(j - 1)) << 1) | (i & (j - 1));
          const int hi = lo + j;
          const bool up = (lo & k) == 0;
          const int32_t ka = keys[lo], kb = keys[hi];
          if ((ka > kb) == up) {
            keys[lo] = kb;
            keys[hi] = ka;
            const V va = vals[lo];
            vals[lo] = vals[hi];
            vals[hi] = va;
          }
        }
        __syncthreads();
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        kk[e] = keys[t * E + e];
        vv[e] = vals[t * E + e];
      }
    }
    for (; j >= E; j >>= 1) {
      switch (j / E) {  // lane distance, below 64
        case 1: bitonic_lane_step<1, TPR, E, V>(k, kk, vv); break;
        case 2: bitonic_lane_step<2, TPR, E, V>(k, kk, vv); break;
        case 4: bitonic_lane_step<4, TPR, E, V>(k, kk, vv); break;
        case 8: bitonic_lane_step<8, TPR, E, V>(k, kk, vv); break;
        case 16: bitonic_lane_step<16, TPR, E, V>(k, kk, vv); break;
        default: bitonic_lane_step<32, TPR, E, V>(k, kk, vv); break;
      }
    }
#pragma unroll
    for (int jj = E / 2; jj >= 1; jj >>= 1) {
      if (jj < k) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          if ((e & jj) == 0) {
            const bool up = ((t * E + e) & k) == 0;
            if ((kk[e] > kk[e + jj]) == up) {
              const int32_t tk = kk[e];
              kk[e] = kk[e + jj];
              kk[e + jj] = tk;
              const V tv = vv[e];
              vv[e] = vv[e + jj];
              vv[e + jj] = tv;
            }
          }
        }
      }
    }
  }
}

// Radix sort of a row's compacted entries (one row per work group, at least
// 256 threads), in place of the bitonic network: the entries are sorted as
// 32-bit words (column - row minimum) << ptrBits | slot, ptrBits = bits of
// the slot index, by a least-significant-digit radix sort on 8-bit digits of
// the column part; the values stay in their slots and are gathered through
// the slot index as the sorted row is written (the indirect key-pointer sort
// the Ocean page describes for its hash accumulators, §3).  A pass ranks the
// entries of each wave stably (lanes with equal digits found by ballots, a
// running count per wave and digit), orders the waves by a prefix, and
// scatters; keys[0, total) and keys[total, 2 total) are the two buffers.
// Returns false, with nothing changed, when the words need more than 32
// bits, the row has more entries than TPR * E, or keys has no room for the
// second buffer; the caller then sorts with the network.
template <int TPR, int E, typename V>
__device__ bool radix_sorted_write(int32_t* keys, const V* vals, int32_t total, int32_t T,
                                   unsigned char* scratch, bool live, int64_t base, int32_t lim,
                                   int32_t* __restrict__ ccol, V* __restrict__ cval) {
  constexpr int WPR = TPR / kWave;
  uint16_t* wcnt = (uint16_t*)scratch;                       // [WPR][256]
  int32_t* rbase = (int32_t*)(scratch + WPR * 256 * 2);      // [256]
  int32_t* red = rbase + 256;                                // [2 * WPR]
  const int t = threadIdx.x, w = t / kWave, l = lane_id();
  if (total > TPR * E || 2 * total > T) return false;
  int32_t mn = INT_MAX, mx = -1;
  for (int i = t; i < total; i += TPR) {
    const int32_t k = keys[i];
    mn = k < mn ? k : mn;
    mx = k > mx ? k : mx;
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const int32_t a = __shfl_xor(mn, d), b = __shfl_xor(mx, d);
    mn = a < mn ? a : mn;
    mx = b > mx ? b : mx;
  }
  if (l == 0) {
    red[w] = mn;
    red[WPR + w] = mx;
  }
  __syncthreads();
  mn = INT_MAX;
  mx = -1;
#pragma unroll
  for (int i = 0; i < WPR; ++i) {
    mn = red[i] < mn ? red[i] : mn;
    mx = red[WPR + i] > mx ? red[WPR + i] : mx;
  }
  int ptrBits = 1, keyBits = 0;
  while ((1 << ptrBits) < total) ++ptrBits;
  while (keyBits < 32 && ((int64_t)1 << keyBits) <= (int64_t)mx - mn) ++keyBits;
  if (total > 0 && keyBits + ptrBits > 32) return false;  // uniform: all threads read red
  __syncthreads();  // red is read before anyone goes on
  uint32_t* src = (uint32_t*)keys;
  uint32_t* dst = src + total;
  for (int i = t; i < total; i += TPR) src[i] = ((uint32_t)(keys[i] - mn) << ptrBits) | (uint32_t)i;
  __syncthreads();
  const int passes = (keyBits + 7) / 8;
  const int64_t e0 = (int64_t)w * kWave * E + l;  // entry of item i: e0 + i * 64
  for (int p = 0; p < passes; ++p) {
    const int shift = ptrBits + 8 * p;
    const int db = keyBits - 8 * p < 8 ? keyBits - 8 * p : 8;
    const uint32_t mask = (1u << db) - 1u;
    uint16_t* my = wcnt + w * 256;
    for (int d = l; d < 256; d += kWave) my[d] = 0;
    uint32_t v[E], rank[E];
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int64_t e = e0 + (int64_t)i * kWave;
      v[i] = e < total ? src[e] : 0u;
    }
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const bool act = e0 + (int64_t)i * kWave < total;
      const uint32_t d = (v[i] >> shift) & mask;
      const uint64_t peers = match_key(d, db, act);
      uint32_t r = 0;
      if (act) {
        // The store depends on the load, and one wave's LDS accesses are
        // performed in order.
        const uint32_t before = my[d];
        r = before + (uint32_t)__popcll(peers & lanemask_lt());
        if (l == last_set64(peers)) my[d] = (uint16_t)(before + __popcll(peers));
      }
      rank[i] = r;
    }
    __syncthreads();
    // Per digit: prefix over the waves, then the digit totals' prefix.
    if (t < 256) {
      uint32_t run = 0;
      for (int u = 0; u < WPR; ++u) {
        const uint32_t c = wcnt[u * 256 + t];
        wcnt[u * 256 + t] = (uint16_t)run;
        run += c;
      }
      rbase[t] = (int32_t)run;
    }
    __syncthreads();
    if (w == 0) {
      int32_t c4[4], s4 = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c4[j] = rbase[l * 4 + j];
        s4 += c4[j];
      }
      int32_t run = wave_incl_scan(s4) - s4;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        rbase[l * 4 + j] = run;
        run += c4[j];
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < E; ++i) {
      if (e0 + (int64_t)i * kWave < total) {
        const uint32_t d = (v[i] >> shift) & mask;
        dst[rbase[d] + my[d] + rank[i]] = v[i];
      }
    }
    __syncthreads();
    uint32_t* tmp = src;
    src = dst;
    dst = tmp;
  }
  if (live) {
    const uint32_t pm = (1u << ptrBits) - 1u;
    for (int r = t; r < lim; r += TPR) {
      const uint32_t q = src[r];
      ccol[base + r] = mn + (int32_t)(q >> ptrBits);
      cval[base + r] = vals[q & pm];
    }
  }
  return true;
}

// With cntOut (size-estimate workflows), cRowOff holds each row's reserved
// capacity instead of its exact size: a row whose entries fit is written
// there and its count stored in cntOut; a row with more entries than its
// capacity, or whose table filled up, writes nothing and gets -1.
template <int TPR, int RPB, int E, typename V>
__global__ __launch_bounds__(TPR* RPB) void k_num_rows(const int32_t* __restrict__ rows,
                                                       int64_t nrows, int32_t T, int32_t spt,
                                                       RowArgs a,
                                                       const int64_t* __restrict__ cRowOff,
                                                       int32_t* __restrict__ ccol,
                                                       V* __restrict__ cval,
                                                       int32_t* __restrict__ err,
                                                       int64_t* __restrict__ cntOut) {
  extern __shared__ __align__(16) unsigned char smem[];
  V* valsAll = (V*)smem;
  int32_t* keysAll = (int32_t*)(valsAll + RPB * T);
  int32_t* wtot = keysAll + RPB * T;
  int32_t* full = wtot + RPB * (TPR / kWave);  // per row: its table filled up
  const int g = threadIdx.x / TPR, t = threadIdx.x % TPR;
  int32_t* keys = keysAll + g * T;
  V* vals = valsAll + g * T;
  for (int s = t; s < T; s += TPR) {
    keys[s] = kEmptyKey;
    vals[s] = V(0);
  }
  if (t == 0) full[g] = 0;
  int32_t* herr = cntOut ? &full[g] : err;
  __syncthreads();
  const int64_t ri = (int64_t)blockIdx.x * RPB + g;
  int32_t row = 0;
  if (ri < nrows) {
    row = rows[ri];
    const int64_t rs = a.arp[row], re = a.arp[row + 1];
    const int32_t P = (int32_t)a.rowP[row];
    constexpr int WPR = TPR / kWave;
    const int w = t / kWave;
    const int32_t p0 = (int32_t)((int64_t)P * w / WPR);
    const int32_t p1 = (int32_t)((int64_t)P * (w + 1) / WPR);
    stream_row<true, V>(a.scanA, a.acol, (const V*)a.aval, a.brp, a.bcol, (const V*)a.bval, rs,
                        re, P, p0, p1, [&](bool act, int32_t c, V av, V bv, int32_t) {
                          if (act && !(cntOut && full[g]))
                            hmap_add(keys, vals, (uint32_t)T, c, av * bv, herr);
                        });
  }
  __syncthreads();
  const int32_t total = compact_slots<TPR, RPB, E, V>(keys, vals, spt, wtot);
  int64_t base = 0;
  int32_t lim = 0;
  if (ri < nrows) {
    base = cRowOff[row];
    const int64_t want = cRowOff[row + 1] - base;
    if (cntOut) {
      const bool over = total > want || full[g] != 0;
      if (t == 0) cntOut[row] = over ? -1 : total;
      lim = over ? 0 : total;
    } else {
      if (t == 0 && want != total) flag_error(err, kErrCountMismatch);
      lim = (int32_t)(want < total ? want : total);
    }
  }
  if constexpr (RPB == 1 && TPR >= 256) {
    if (radix_sorted_write<TPR, E, V>(keys, vals, total, T, (unsigned char*)(full + RPB),
                                      ri < nrows, base, lim, ccol, cval))
      return;
  }
  int32_t kk[E];
  V vv[E];
  sort_to_regs<TPR, E, V>(keys, vals, kk, vv);
  if (ri < nrows) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int r = t * E + e;
      if (r < lim) {
        ccol[base + r] = kk[e];
        cval[base + r] = vv[e];
      }
    }
  }
}


// ------------------------------------- diagonal window plus outlier table
// Light hash-bin rows of banded or clustered matrices (the iterates of
// Markov clustering, Trident page §5.7, whose clusters lie on the diagonal)
// spread most of their products over a few thousand columns around the
// diagonal and the rest thinly over the whole row.  Such a row takes a dense
// LDS window over the kHybW columns [lo, lo + kHybW) around its diagonal
// position (a bitmap, and in numeric a value per column: no probing, no
// sort) and an LDS hash table for the other columns, its outliers.  The
// output row is the outliers below lo, then the window's columns in order,
// then the outliers above, so only the outliers are ordered (a few hundred
// at most, ranked through buckets of equal column ranges).  Symbolic
// counts both parts and stores the outlier count; numeric takes a row this
// way when the outliers fit half of a table of next_pow2(bin bound) slots
// and number at most kHybOutMax, else the row goes to the hash kernel.  (An accumulator per row chosen
// from the row's structure: gMAGNUS page §III-E, Ocean page §2.)
__device__ __forceinline__ int32_t hyb_lo(int32_t row, int64_t m, int64_t n) {
  const int64_t center = m > 0 ? (int64_t)row * n / m : 0;
  int64_t lo = center - (kHybW / 2 - 16);
  lo = lo < 0 ? 0 : lo;
  return (int32_t)(lo & ~(int64_t)31);
}

template <int TPR, int RPB>
__global__ __launch_bounds__(TPR* RPB) void k_sym_rows_hyb(const int32_t* __restrict__ rows,
                                                           int64_t nrows, int32_t T, RowArgs a,
                                                           int64_t m, int64_t n,
                                                           int64_t* __restrict__ cnt,
                                                           int32_t* __restrict__ outc,
                                                           int32_t* __restrict__ err) {
  extern __shared__ __align__(16) unsigned char smem[];
  int32_t* keysAll = (int32_t*)smem;
  uint32_t* bmAll = (uint32_t*)(keysAll + RPB * T);
  __shared__ int32_t gwin[RPB], gout[RPB];
  const int g = threadIdx.x / TPR, t = threadIdx.x % TPR;
  int32_t* keys = keysAll + g * T;
  uint32_t* bm = bmAll + g * kHybWords;
  // T is a power of two from 64 on: the keys are cleared 16 bytes a store.
  for (int s = t; s < T / 4; s += TPR)
    ((int4*)keys)[s] = make_int4(kEmptyKey, kEmptyKey, kEmptyKey, kEmptyKey);
  for (int i = t; i < kHybWords; i += TPR) bm[i] = 0;
  if (t == 0) {
    gwin[g] = 0;
    gout[g] = 0;
  }
  __syncthreads();
  const int64_t ri = (int64_t)blockIdx.x * RPB + g;
  int32_t row = 0, mine = 0;
  if (ri < nrows) {
    row = rows[ri];
    const int32_t lo = hyb_lo(row, m, n);
    const int64_t rs = a.arp[row], re = a.arp[row + 1];
    const int32_t P = (int32_t)a.rowP[row];
    constexpr int WPR = TPR / kWave;
    const int w = t / kWave;
    const int32_t p0 = (int32_t)((int64_t)P * w / WPR);
    const int32_t p1 = (int32_t)((int64_t)P * (w + 1) / WPR);
    stream_row<false, float>(a.scanA, a.acol, (const float*)nullptr, a.brp, a.bcol,
                             (const float*)nullptr, rs, re, P, p0, p1,
                             [&](bool act, int32_t c, float, float, int32_t) {
                               if (act) {
                                 const uint32_t d = (uint32_t)(c - lo);
                                 if (d < (uint32_t)kHybW) {
                                   const uint32_t bit = 1u << (d & 31);
                                   if (!(bm[d >> 5] & bit)) atomicOr(&bm[d >> 5], bit);
                                 } else if (hset_insert(keys, (uint32_t)T, c, err)) {
                                   ++mine;
                                 }
                               }
                             });
  }
  const int32_t ws = wave_sum(mine);
  if (lane_id() == 0 && ri < nrows) atomicAdd(&gout[g], ws);
  __syncthreads();
  int32_t pc = 0;
  for (int i = t; i < kHybWords; i += TPR) pc += __popc(bm[i]);
  pc = wave_sum(pc);
  if (lane_id() == 0 && ri < nrows) atomicAdd(&gwin[g], pc);
  __syncthreads();
  if (t == 0 && ri < nrows) {
    cnt[row] = gwin[g] + gout[g];
    outc[row] = gout[g];
  }
}

// LDS: vw[kHybW] V | ov[To] V | ok[To] i32 | bm[kHybWords] | wpre[kHybWords] |
// wtot[TPR / 64] | red[4] | bcnt[kHybOutMax] | bfirst[kHybOutMax].
__host__ __device__ constexpr size_t hyb_num_lds(int tpr, int32_t To, int vb) {
  return (size_t)kHybW * vb + (size_t)To * (vb + 4) + (size_t)kHybWords * 8 +
         (size_t)(tpr / kWave) * 4 + 16 + (size_t)kHybOutMax * 8;
}

template <int TPR, int E, typename V>
__global__ __launch_bounds__(TPR) void k_num_rows_hyb(const int32_t* __restrict__ rows,
                                                      int32_t To, RowArgs a, int64_t m, int64_t n,
                                                      const int64_t* __restrict__ cRowOff,
                                                      int32_t* __restrict__ ccol,
                                                      V* __restrict__ cval,
                                                      int32_t* __restrict__ err) {
  static_assert(TPR >= 256, "one row per work group");
  extern __shared__ __align__(16) unsigned char smem[];
  V* vw = (V*)smem;
  V* ov = vw + kHybW;
  int32_t* ok = (int32_t*)(ov + To);
  uint32_t* bm = (uint32_t*)(ok + To);
  int32_t* wpre = (int32_t*)(bm + kHybWords);
  int32_t* wtot = wpre + kHybWords;
  int32_t* red = wtot + TPR / kWave;  // window entries, outliers below lo
  int32_t* bcnt = red + 4;               // outliers per bucket (16-byte aligned)
  int32_t* bfirst = bcnt + kHybOutMax;   // first rank of each bucket
  int32_t* bkey = ok + To / 2;           // outlier columns gathered by bucket
  const int t = threadIdx.x;
  // Cleared 16 bytes a store: the window and the outlier values (adjacent,
  // all-zero bits), the outlier keys (kEmptyKey), the bucket counts.
  {
    float4* z = (float4*)smem;
    const int nz = (int)(((size_t)kHybW + To) * sizeof(V) / 16);
    for (int i = t; i < nz; i += TPR) z[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    int4* k4 = (int4*)ok;
    for (int i = t; i < To / 4; i += TPR) k4[i] = make_int4(kEmptyKey, kEmptyKey, kEmptyKey, kEmptyKey);
    int4* b4 = (int4*)bcnt;
    for (int i = t; i < kHybOutMax / 4; i += TPR) b4[i] = make_int4(0, 0, 0, 0);
  }
  if (t < kHybWords) bm[t] = 0;
  if (t == 0) red[1] = 0;
  __syncthreads();
  const int32_t row = rows[blockIdx.x];
  const int32_t lo = hyb_lo(row, m, n);
  {
    const int64_t rs = a.arp[row], re = a.arp[row + 1];
    const int32_t P = (int32_t)a.rowP[row];
    constexpr int WPR = TPR / kWave;
    const int w = t / kWave;
    const int32_t p0 = (int32_t)((int64_t)P * w / WPR);
    const int32_t p1 = (int32_t)((int64_t)P * (w + 1) / WPR);
    stream_row<true, V>(a.scanA, a.acol, (const V*)a.aval, a.brp, a.bcol, (const V*)a.bval, rs,
                        re, P, p0, p1, [&](bool act, int32_t c, V av, V bv, int32_t) {
                          if (act) {
                            const uint32_t d = (uint32_t)(c - lo);
                            const V x = av * bv;
                            if (d < (uint32_t)kHybW) {
                              atomicAdd(&vw[d], x);
                              const uint32_t bit = 1u << (d & 31);
                              if (!(bm[d >> 5] & bit)) atomicOr(&bm[d >> 5], bit);
                            } else {
                              hmap_add(ok, ov, (uint32_t)To, c, x, err);
                            }
                          }
                        });
  }
  __syncthreads();
  // Window ranks: exclusive prefix of the word popcounts (a lane per word).
  if (t < kWave) {
    const int32_t x = __popc(bm[t]);
    const int32_t inc = wave_incl_scan(x);
    wpre[t] = inc - x;
    if (t == kWave - 1) red[0] = inc;
  }
  // Outliers: compacted (the barriers inside also publish wpre and red[0]),
  // then ranked through kHybOutMax buckets of equal column ranges (the
  // bucket of a column is monotone in it): each outlier takes a slot in its
  // bucket, a scan of the bucket counts gives each bucket its first rank,
  // the buckets' columns are gathered there, and an outlier's rank is its
  // bucket's first rank plus the columns of its bucket below its own.
  // Routing keeps a row's outliers to kHybOutMax; a row with more (a count
  // that disagrees with symbolic) writes none and is reported by the size
  // check below.
  const int32_t nout = compact_slots<TPR, 1, E, V>(ok, ov, To / TPR, wtot);
  const bool fits = nout <= kHybOutMax;
  constexpr int kPer = (kHybOutMax + TPR - 1) / TPR;
  int32_t key[kPer], bk[kPer], slot[kPer];
  V xv[kPer];
  int32_t below = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = t + j * TPR;
    bk[j] = -1;
    if (fits && i < nout) {
      key[j] = ok[i];
      xv[j] = ov[i];
      bk[j] = (int32_t)((int64_t)key[j] * kHybOutMax / n);
      slot[j] = atomicAdd(&bcnt[bk[j]], 1);
      below += key[j] < lo;
    }
  }
  below = wave_sum(below);
  if (lane_id() == 0 && below) atomicAdd(&red[1], below);
  __syncthreads();
  {
    constexpr int kCpt = (kHybOutMax + TPR - 1) / TPR;  // bucket counters per thread
    int32_t c[kCpt], sum = 0;
#pragma unroll
    for (int j = 0; j < kCpt; ++j) {
      const int b = t * kCpt + j;
      c[j] = b < kHybOutMax ? bcnt[b] : 0;
      sum += c[j];
    }
    int32_t all;
    int32_t run = block_excl_scan<TPR>(sum, wtot, &all);
#pragma unroll
    for (int j = 0; j < kCpt; ++j) {
      const int b = t * kCpt + j;
      if (b < kHybOutMax) bfirst[b] = run;
      run += c[j];
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (bk[j] >= 0) bkey[bfirst[bk[j]] + slot[j]] = key[j];
  __syncthreads();
  const int32_t nwin = red[0], nb = red[1];
  const int64_t base = cRowOff[row];
  const int64_t want = cRowOff[row + 1] - base;
  const int32_t total = nwin + nout;
  if (t == 0 && (want != total || !fits)) flag_error(err, kErrCountMismatch);
  const int32_t lim = (int32_t)(want < total ? want : total);
  for (int c = t; c < kHybW; c += TPR) {
    const uint32_t word = bm[c >> 5];
    if ((word >> (c & 31)) & 1u) {
      const int32_t pos = nb + wpre[c >> 5] + __popc(word & ((1u << (c & 31)) - 1u));
      if (pos < lim) {
        ccol[base + pos] = lo + c;
        cval[base + pos] = vw[c];
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if (bk[j] >= 0) {
      const int32_t f = bfirst[bk[j]], e = f + bcnt[bk[j]];
      int32_t r = f;
      for (int q = f; q < e; ++q) r += bkey[q] < key[j];
      const int32_t pos = key[j] < lo ? r : r + nwin;
      if (pos < lim) {
        ccol[base + pos] = key[j];
        cval[base + pos] = xv[j];
      }
    }
  }
}

// ------------------------------------------------ ESC for short rows
// Rows of at most kEscLanes products (Ocean page, §3: an expand-sort-compact
// accumulator for short rows, several rows per work group): 32 lanes per row,
// one product per lane, a bitonic sort of (column, value) by lane exchanges,
// then equal columns are summed by a segmented scan and the last lane of
// every run writes it.  No LDS.  Symbolic (kNum false) stores the count of
// distinct columns; numeric writes the row at cRowOff[row], or, with cntOut,
// into its reserved slots (count, or -1 when it does not fit).
constexpr int kEscLanes = 32;
constexpr int kEscNT = 256;

template <int LD, typename V>
__device__ __forceinline__ void esc_step(int k, int32_t& key, V& val) {
  const int i = lane_id() % kEscLanes;
  const int32_t ok = lane_xor<LD>(key);
  const V ov = lane_xor_v<LD>(val);
  const bool up = (i & k) == 0;
  const bool lower = (i & LD) == 0;
  const bool take = (lower == up) ? (ok < key) : (ok > key);
  if (take) {
    key = ok;
    val = ov;
  }
}

template <bool kNum, typename V>
__global__ __launch_bounds__(kEscNT) void k_rows_esc(const int32_t* __restrict__ rows,
                                                     int64_t nrows, RowArgs a,
                                                     const int64_t* __restrict__ cRowOff,
                                                     int32_t* __restrict__ ccol,
                                                     V* __restrict__ cval,
                                                     int64_t* __restrict__ cnt,
                                                     int32_t* __restrict__ err,
                                                     int64_t* __restrict__ cntOut) {
  const int64_t ri = ((int64_t)blockIdx.x * kEscNT + threadIdx.x) / kEscLanes;
  const int l = lane_id() % kEscLanes;
  const bool live = ri < nrows;
  int32_t row = 0, P = 0;
  int64_t rs = 0, re = 0;
  if (live) {
    row = rows[ri];
    rs = a.arp[row];
    re = a.arp[row + 1];
    P = (int32_t)a.rowP[row];
  }
  // Product l belongs to the entry whose first product is the last at or
  // before l.  Rows of at most 32 entries: entry l of the row sits in lane l
  // and a search by shuffles finds it; longer rows (entries without products
  // pad them) search scanA in memory.
  int32_t so, sb;
  V sa = V(0);
  if (re - rs <= kEscLanes) {
    const int64_t e = rs + l;
    const bool ev = live && e < re;
    const int32_t off = ev ? a.scanA[e] : P;
    const int32_t bs = ev ? a.brp[a.acol[e]] : 0;
    V av = V(0);
    if constexpr (kNum) av = ev ? ((const V*)a.aval)[e] : V(0);
    int s = 0;
#pragma unroll
    for (int step = 16; step >= 1; step >>= 1) {
      const int idx = s + step < kEscLanes ? s + step : kEscLanes - 1;
      const int32_t o = __shfl(off, idx, kEscLanes);
      if (s + step < kEscLanes && o <= l) s += step;
    }
    so = __shfl(off, s, kEscLanes);
    sb = __shfl(bs, s, kEscLanes);
    if constexpr (kNum) sa = __shfl(av, s, kEscLanes);
  } else {
    int64_t lo = rs, hi = re - 1;
    while (lo < hi) {
      const int64_t mid = (lo + hi + 1) >> 1;
      if (a.scanA[mid] <= l) lo = mid;
      else hi = mid - 1;
    }
    so = a.scanA[lo];
    sb = a.brp[a.acol[lo]];
    if constexpr (kNum) sa = ((const V*)a.aval)[lo];
  }
  const bool act = live && l < P;
  int32_t key = INT_MAX;
  V val = V(0);
  if (act) {
    const int32_t b = sb + (l - so);
    key = a.bcol[b];
    if constexpr (kNum) val = sa * ((const V*)a.bval)[b];
  }
  // Bitonic sort of the 32 lanes (absent products sort last as INT_MAX).
#pragma unroll
  for (int k = 2; k <= kEscLanes; k <<= 1) {
    if (k >= 32) esc_step<16, V>(k, key, val);
    if (k >= 16) esc_step<8, V>(k, key, val);
    if (k >= 8) esc_step<4, V>(k, key, val);
    if (k >= 4) esc_step<2, V>(k, key, val);
    esc_step<1, V>(k, key, val);
  }
  const int32_t prev = __shfl_up(key, 1, kEscLanes);
  const bool valid = key != INT_MAX;
  const bool head = valid && (l == 0 || prev != key);
  const uint64_t heads = __ballot(head);
  const int half = (lane_id() / kEscLanes) * kEscLanes;
  const uint32_t mine = (uint32_t)(heads >> half);
  const int32_t nnz = __popc(mine);
  if constexpr (!kNum) {
    if (live && l == 0) cnt[row] = nnz;
  } else {
    // Segmented inclusive sum: a lane adds its left neighbour's partial
    // while no run starts between them.
    bool f = head;
#pragma unroll
    for (int d = 1; d < kEscLanes; d <<= 1) {
      const V y = __shfl_up(val, d, kEscLanes);
      const bool fy = __shfl_up((int)f, d, kEscLanes) != 0;
      if (l >= d && !f) val += y;
      if (l >= d) f = f || fy;
    }
    const int32_t next = __shfl_down(key, 1, kEscLanes);
    const bool tail = valid && (l == kEscLanes - 1 || next != key);
    const int32_t pos = __popc(mine & ((2u << l) - 1u)) - 1;  // run index
    if (live) {
      const int64_t base = cRowOff[row];
      const int64_t want = cRowOff[row + 1] - base;
      bool write = true;
      if (cntOut) {
        write = nnz <= want;
        if (l == 0) cntOut[row] = write ? nnz : -1;
      } else if (l == 0 && want != nnz) {
        flag_error(err, kErrCountMismatch);
      }
      if (write && tail && pos < want) {
        ccol[base + pos] = key;
        cval[base + pos] = val;
      }
    }
  }
}

// Light chunks of at most L elements (L = 32 or 64), expand-sort-compact
// as for short rows: L lanes per chunk, one element per lane, a bitonic sort
// of (chunk column, value) by lane exchanges, a segmented sum of equal
// columns, and the last lane of every run writes it.  No LDS, no table to
// clear.
template <int L, int LD, typename V>
__device__ __forceinline__ void esc_step_l(int k, int32_t& key, V& val) {
  const int i = lane_id() % L;
  const int32_t ok = lane_xor<LD>(key);
  const V ov = lane_xor_v<LD>(val);
  const bool up = (i & k) == 0;
  const bool lower = (i & LD) == 0;
  const bool take = (lower == up) ? (ok < key) : (ok > key);
  if (take) {
    key = ok;
    val = ov;
  }
}

template <int L, typename V, typename C>
__global__ __launch_bounds__(kEscNT) void k_num_chunks_esc(const ChunkDesc* __restrict__ desc,
                                                           int64_t n, ChunkList cl,
                                                           int32_t* __restrict__ ccol,
                                                           V* __restrict__ cval,
                                                           int32_t* __restrict__ err) {
  static_assert(L == 32 || L == 64, "a chunk takes half a wave or a wave");
  const int64_t ci = ((int64_t)blockIdx.x * kEscNT + threadIdx.x) / L;
  const int l = lane_id() % L;
  const bool live = ci < n;
  ChunkDesc d{};
  if (live) d = desc[ci];
  int32_t key = INT_MAX;
  V val = V(0);
  if (live && l < d.cnt) {
    const int64_t e = d.off + l;
    key = (int32_t)((const C*)(d.buf ? cl.col1 : cl.col0))[e];
    val = ((const V*)(d.buf ? cl.val1 : cl.val0))[e];
  }
  if (live && l == 0 && d.cnt > L) flag_error(err, kErrHashFull);
#pragma unroll
  for (int k = 2; k <= L; k <<= 1) {
    if (k >= 64) esc_step_l<L, 32, V>(k, key, val);
    if (k >= 32) esc_step_l<L, 16, V>(k, key, val);
    if (k >= 16) esc_step_l<L, 8, V>(k, key, val);
    if (k >= 8) esc_step_l<L, 4, V>(k, key, val);
    if (k >= 4) esc_step_l<L, 2, V>(k, key, val);
    esc_step_l<L, 1, V>(k, key, val);
  }
  const int32_t prev = __shfl_up(key, 1, L);
  const bool valid = key != INT_MAX;
  const bool head = valid && (l == 0 || prev != key);
  const uint64_t heads = __ballot(head);
  const int half = (lane_id() / L) * L;
  const uint64_t mine = L == 64 ? heads : (heads >> half) & 0xffffffffull;
  const int32_t nnz = __popcll(mine);
  bool f = head;
#pragma unroll
  for (int dd = 1; dd < L; dd <<= 1) {
    const V y = __shfl_up(val, dd, L);
    const bool fy = __shfl_up((int)f, dd, L) != 0;
    if (l >= dd && !f) val += y;
    if (l >= dd) f = f || fy;
  }
  const int32_t next = __shfl_down(key, 1, L);
  const bool tail = valid && (l == L - 1 || next != key);
  const uint64_t upto = l == 63 ? ~0ull : ((2ull << l) - 1ull);
  const int32_t pos = __popcll(mine & upto) - 1;  // run index
  if (live) {
    if (l == 0 && d.want != nnz) flag_error(err, kErrCountMismatch);
    if (tail && pos < d.want) {
      ccol[d.base + pos] = d.colBase + key;
      cval[d.base + pos] = val;
    }
  }
}

// Light chunks of at most 64 * E elements (E = 2 or 4): one wave per chunk,
// E elements per lane sorted by the bitonic network of sort_to_regs (lane
// exchanges and register swaps), then a segmented sum: inside each lane,
// across lanes for the run that continues from the lanes before, and a scan
// of the lanes' run heads gives every run its output position.
template <int E, typename V, typename C>
__global__ __launch_bounds__(kEscNT) void k_num_chunks_esc_e(const ChunkDesc* __restrict__ desc,
                                                             int64_t n, ChunkList cl,
                                                             int32_t* __restrict__ ccol,
                                                             V* __restrict__ cval,
                                                             int32_t* __restrict__ err) {
  constexpr int NP = kWave * E;
  const int64_t ci = ((int64_t)blockIdx.x * kEscNT + threadIdx.x) / kWave;
  const int l = lane_id();
  const bool live = ci < n;
  ChunkDesc d{};
  if (live) d = desc[ci];
  int32_t kk[E];
  V vv[E];
  {
    const C* __restrict__ col = (const C*)(d.buf ? cl.col1 : cl.col0);
    const V* __restrict__ val = (const V*)(d.buf ? cl.val1 : cl.val0);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = e * kWave + l;  // any order: the network sorts them all
      const bool in = live && i < d.cnt;
      kk[e] = in ? (int32_t)col[d.off + i] : INT_MAX;
      vv[e] = in ? val[d.off + i] : V(0);
    }
  }
  if (live && l == 0 && d.cnt > NP) flag_error(err, kErrHashFull);
  // Bitonic network over element index l * E + e.
  for (int k = 2; k <= NP; k <<= 1) {
    for (int j = k >> 1; j >= E; j >>= 1) {
      switch (j / E) {  // lane distance, below 64
        case 1: bitonic_lane_step<1, kWave, E, V>(k, kk, vv); break;
        case 2: bitonic_lane_step<2, kWave, E, V>(k, kk, vv); break;
        case 4: bitonic_lane_step<4, kWave, E, V>(k, kk, vv); break;
        case 8: bitonic_lane_step<8, kWave, E, V>(k, kk, vv); break;
        case 16: bitonic_lane_step<16, kWave, E, V>(k, kk, vv); break;
        default: bitonic_lane_step<32, kWave, E, V>(k, kk, vv); break;
      }
    }
#pragma unroll
    for (int jj = E / 2; jj >= 1; jj >>= 1) {
      if (jj < k) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          if ((e & jj) == 0) {
            const bool up = ((l * E + e) & k) == 0;
            if ((kk[e] > kk[e + jj]) == up) {
              const int32_t tk = kk[e];
              kk[e] = kk[e + jj];
              kk[e + jj] = tk;
              const V tv = vv[e];
              vv[e] = vv[e + jj];
              vv[e + jj] = tv;
            }
          }
        }
      }
    }
  }
  // Run heads, in-lane segmented sums, and the lanes' run-head counts.
  bool head[E];
  const int32_t prevLast = __shfl_up(kk[E - 1], 1);
  int32_t hc = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int32_t pk = e == 0 ? prevLast : kk[e - 1];
    head[e] = kk[e] != INT_MAX && ((l == 0 && e == 0) || pk != kk[e]);
    hc += head[e] ? 1 : 0;
    if (e > 0 && !head[e]) vv[e] += vv[e - 1];
  }
  // Across lanes: the partial of each lane's last run, summed over the
  // lanes before while no head separates them.
  V x = vv[E - 1];
  bool f = hc > 0;
#pragma unroll
  for (int dd = 1; dd < kWave; dd <<= 1) {
    const V y = __shfl_up(x, dd);
    const bool fy = __shfl_up((int)f, dd) != 0;
    if (l >= dd && !f) x += y;
    if (l >= dd) f = f || fy;
  }
  V incoming = __shfl_up(x, 1);
  if (l == 0) incoming = V(0);
  bool seen = false;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    seen = seen || head[e];
    if (!seen) vv[e] += incoming;
  }
  const int32_t nextFirst = __shfl_down(kk[0], 1);
  const int32_t hinc = wave_incl_scan(hc);
  const int32_t nnz = __shfl(hinc, kWave - 1);
  int32_t r = hinc - hc;  // runs that start before this lane
  if (live) {
    if (l == 0 && d.want != nnz) flag_error(err, kErrCountMismatch);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      r += head[e] ? 1 : 0;
      const int32_t nk = e < E - 1 ? kk[e + 1] : (l == kWave - 1 ? INT_MAX : nextFirst);
      const bool tail = kk[e] != INT_MAX && nk != kk[e];
      if (tail && r - 1 < d.want) {
        ccol[d.base + r - 1] = d.colBase + kk[e];
        cval[d.base + r - 1] = vv[e];
      }
    }
  }
}

template <int TPR, int RPB, int E, typename V, typename C = int32_t>
__global__ __launch_bounds__(TPR* RPB) void k_num_chunks(const ChunkDesc* __restrict__ desc,
                                                         int64_t n, int32_t T, int32_t spt,
                                                         ChunkList cl,
                                                         int32_t* __restrict__ ccol,
                                                         V* __restrict__ cval,
                                                         int32_t* __restrict__ err) {
  extern __shared__ __align__(16) unsigned char smem[];
  V* valsAll = (V*)smem;
  int32_t* keysAll = (int32_t*)(valsAll + RPB * T);
  int32_t* wtot = keysAll + RPB * T;
  const int g = threadIdx.x / TPR, t = threadIdx.x % TPR;
  int32_t* keys = keysAll + g * T;
  V* vals = valsAll + g * T;
  for (int s = t; s < T; s += TPR) {
    keys[s] = kEmptyKey;
    vals[s] = V(0);
  }
  __syncthreads();
  const int64_t ri = (int64_t)blockIdx.x * RPB + g;
  ChunkDesc d{};
  if (ri < n) {
    d = desc[ri];
    const int64_t off = d.off;
    const int64_t end = off + d.cnt;
    const bool b1 = d.buf != 0;
    const C* __restrict__ col = (const C*)(b1 ? cl.col1 : cl.col0);
    const V* __restrict__ val = (const V*)(b1 ? cl.val1 : cl.val0);
    for (int64_t e = off + t; e < end; e += TPR) hmap_add(keys, vals, (uint32_t)T, col[e], val[e], err);
  }
  __syncthreads();
  const int32_t total = compact_slots<TPR, RPB, E, V>(keys, vals, spt, wtot);
  int32_t kk[E];
  V vv[E];
  sort_to_regs<TPR, E, V>(keys, vals, kk, vv);
  if (ri < n) {
    const int64_t base = d.base;
    const int32_t want = d.want;
    if (t == 0 && want != total) flag_error(err, kErrCountMismatch);
    const int32_t lim = want < total ? want : total;
    const int32_t colBase = d.colBase;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int r = t * E + e;
      if (r < lim) {
        ccol[base + r] = colBase + kk[e];
        cval[base + r] = vv[e];
      }
    }
  }
}

// ------------------------------------------- heavy-row symbolic from A and B
// Symbolic of the heavy rows when their intermediate is too large to keep
// until numeric (the batched schedule): nnz of every W-wide column slot of a
// heavy row, taken straight from A and B with no expansion.  A work item is
// (heavy row, column window of 2^winBits columns, a multiple of W); a work
// group clears an LDS bitmap of the window, marks the columns of the row's
// products, then counts the bits of each W-wide slot, clearing the words it
// reads for the next item.  Work groups take items from a counter until
// none is left.  The per-slot counts give the chunk sizes of any chunk
// tree: a final chunk covering slots [s, s + 2^k) holds the sum of their
// counts.
//
// The products of a heavy row come almost entirely from long B rows (on
// R-MAT, 99.6% of them from B rows of 64 or more entries), so each wave
// takes an even share of the row's products and walks the A entries of that
// share in order, reading every B row's run with the whole wave, four
// columns per lane per 16-byte load; the offsets, B row starts and lengths
// of 64 entries at a time are loaded once, lane-parallel, and read back with
// lane broadcasts.
constexpr int kSymHeavyNT = 1024;
constexpr int kSymHeavyU = 2;  // 16-byte loads per lane in flight per step
constexpr int kSymHeavyG = 4;  // entries whose first loads are in flight together

__device__ __forceinline__ void mark_col(uint32_t* bm, int32_t col, int32_t w0, uint32_t wlen) {
  const uint32_t c = (uint32_t)(col - w0);
  if (c < wlen) atomicOr(&bm[c >> 5], 1u << (c & 31));
}
// Columns idx .. idx+3 of B that lie in [x0, x1) (others -1): one 16-byte
// load at a 16-byte aligned idx where the whole vector lies in B, else the
// elements one by one.
__device__ __forceinline__ int4 sym_heavy_load4(const int32_t* __restrict__ bcol, int64_t idx,
                                                int64_t x0, int64_t x1, int64_t nnzB) {
  int4 v = make_int4(-1, -1, -1, -1);
  if (idx < x1) {
    if (idx >= 0 && idx + 4 <= nnzB) {
      v = *(const int4*)(bcol + idx);
    } else {
      if (idx >= x0) v.x = bcol[idx];
      if (idx + 1 >= x0 && idx + 1 < x1) v.y = bcol[idx + 1];
      if (idx + 2 >= x0 && idx + 2 < x1) v.z = bcol[idx + 2];
      if (idx + 3 >= x0 && idx + 3 < x1) v.w = bcol[idx + 3];
    }
  }
  return v;
}
__device__ __forceinline__ void sym_heavy_mark4(uint32_t* bm, int4 v, int64_t idx, int64_t x0,
                                                int64_t x1, int32_t w0, uint32_t wlen) {
  if (idx >= x0 && idx < x1) mark_col(bm, v.x, w0, wlen);
  if (idx + 1 >= x0 && idx + 1 < x1) mark_col(bm, v.y, w0, wlen);
  if (idx + 2 >= x0 && idx + 2 < x1) mark_col(bm, v.z, w0, wlen);
  if (idx + 3 >= x0 && idx + 3 < x1) mark_col(bm, v.w, w0, wlen);
}

__global__ __launch_bounds__(kSymHeavyNT) void k_sym_heavy_rows(
    int64_t h, int32_t nwin, int32_t winBits, int32_t log2W, int64_t nreq,
    const int32_t* __restrict__ xheavy, RowArgs a, int64_t nnzB, int32_t* __restrict__ slotNnz,
    int32_t* __restrict__ next) {
  extern __shared__ uint32_t bm[];
  __shared__ int64_t item;
  constexpr int NW = kSymHeavyNT / kWave;
  const int t = threadIdx.x, w = t / kWave, lane = lane_id();
  const int32_t words = 1 << (winBits - 5);
  for (int i = t; i < words; i += kSymHeavyNT) bm[i] = 0;
  const int64_t nitems = h * nwin;
  const int32_t wps = 1 << (log2W - 5);           // bitmap words per W-wide slot
  const int32_t slots = 1 << (winBits - log2W);   // slots per window
  const int32_t* __restrict__ bcol = a.bcol;
  // elements by which bcol lies past a 16-byte boundary
  const int64_t mis = (int64_t)(((uintptr_t)bcol >> 2) & 3);
  for (;;) {
    if (t == 0) item = atomicAdd(next, 1);
    __syncthreads();
    const int64_t it = item;
    if (it >= nitems) break;  // the same for every thread
    const int64_t r = it / nwin;
    const int32_t win = (int32_t)(it - r * nwin);
    const int32_t row = xheavy[r];
    const int64_t rs = a.arp[row], re = a.arp[row + 1];
    const int32_t P = (int32_t)a.rowP[row];
    const int32_t w0 = win << winBits;
    const uint32_t wlen = 1u << winBits;
    const int32_t p0 = (int32_t)((int64_t)P * w / NW);
    const int32_t p1 = (int32_t)((int64_t)P * (w + 1) / NW);
    if (p0 < p1) {
      // Entries from the one holding product p0, 64 at a time: their
      // offsets, B row starts and ends are loaded lane-parallel and read
      // back by lane broadcasts.  Each group of kSymHeavyG entries issues the
      // first 16-byte load of every entry's run before marking any (runs are
      // mostly short), then walks what is left of each run.
      for (int64_t j = wave_last_le(a.scanA, rs, re, p0); j < re; j += kWave) {
        const int64_t e = j + lane;
        const bool ev = e < re;
        const int32_t o = ev ? a.scanA[e] : P;
        const int32_t bs = ev ? a.brp[a.acol[e]] : 0;
        int32_t on = __shfl_down(o, 1);
        if (lane == kWave - 1) on = (j + kWave < re) ? a.scanA[j + kWave] : P;
        if (__builtin_amdgcn_readlane(o, 0) >= p1) break;  // past this wave's share
        for (int q0 = 0; q0 < kWave; q0 += kSymHeavyG) {
          if (__builtin_amdgcn_readlane(o, q0) >= p1) break;
          int64_t xs[kSymHeavyG], xe[kSymHeavyG];
          int4 v[kSymHeavyG];
#pragma unroll
          for (int g = 0; g < kSymHeavyG; ++g) {
            const int q = q0 + g;
            const int32_t oe = __builtin_amdgcn_readlane(o, q);
            const int32_t one = __builtin_amdgcn_readlane(on, q);
            const int32_t be = __builtin_amdgcn_readlane(bs, q);
            // this entry's products inside [p0, p1)
            const int32_t st = oe > p0 ? oe : p0, en = one < p1 ? one : p1;
            xs[g] = en > st ? (int64_t)be + (st - oe) : 0;
            xe[g] = en > st ? (int64_t)be + (en - oe) : 0;
            v[g] = sym_heavy_load4(bcol, ((xs[g] + mis) & ~(int64_t)3) - mis + 4 * lane, xs[g],
                                   xe[g], nnzB);
          }
#pragma unroll
          for (int g = 0; g < kSymHeavyG; ++g)
            sym_heavy_mark4(bm, v[g], ((xs[g] + mis) & ~(int64_t)3) - mis + 4 * lane, xs[g],
                            xe[g], w0, wlen);
          // the rest of each run, 4 * 64 * kSymHeavyU columns a step
          for (int g = 0; g < kSymHeavyG; ++g) {
            for (int64_t base = ((xs[g] + mis) & ~(int64_t)3) - mis + 4 * kWave; base < xe[g];
                 base += 4 * kWave * kSymHeavyU) {
              int4 r[kSymHeavyU];
#pragma unroll
              for (int u = 0; u < kSymHeavyU; ++u)
                r[u] = sym_heavy_load4(bcol, base + 4 * (u * kWave + lane), xs[g], xe[g], nnzB);
#pragma unroll
              for (int u = 0; u < kSymHeavyU; ++u)
                sym_heavy_mark4(bm, r[u], base + 4 * (u * kWave + lane), xs[g], xe[g], w0, wlen);
            }
          }
        }
      }
    }
    __syncthreads();
    for (int s = w; s < slots; s += NW) {
      int32_t cnt = 0;
      for (int i = lane; i < wps; i += kWave) {
        uint32_t* q = &bm[s * wps + i];
        cnt += __popc(*q);
        *q = 0;
      }
      cnt = wave_sum(cnt);
      const int64_t gs = (int64_t)win * slots + s;
      if (lane == 0 && gs < nreq) slotNnz[r * nreq + gs] = cnt;
    }
    __syncthreads();
  }
}

template <typename K>
void set_lds_attr(K kernel) {
  allow_max_dynamic_lds((const void*)kernel);
}

}  // namespace

void light_set_attributes() {
  set_lds_attr(k_sym_heavy_rows);
  set_lds_attr(k_sym_rows<64, 4>);
  set_lds_attr(k_sym_rows<128, 2>);
  set_lds_attr(k_sym_rows<256, 1>);
  set_lds_attr(k_sym_rows<512, 1>);
  set_lds_attr(k_sym_rows<1024, 1>);
  set_lds_attr(k_sym_chunks<64, 4>);
  set_lds_attr(k_sym_chunks<128, 2>);
  set_lds_attr(k_sym_chunks<256, 1>);
  set_lds_attr(k_sym_chunks<512, 1>);
  set_lds_attr(k_sym_chunks<1024, 1>);
  set_lds_attr(k_sym_rows_win<64, 4>);
  set_lds_attr(k_sym_rows_win<128, 2>);
  set_lds_attr(k_sym_rows_win<256, 1>);
  set_lds_attr(k_sym_rows_win<512, 1>);
  set_lds_attr(k_sym_rows_win<1024, 1>);
  set_lds_attr(k_num_rows_win<64, 4, float>);
  set_lds_attr(k_num_rows_win<128, 2, float>);
  set_lds_attr(k_num_rows_win<256, 1, float>);
  set_lds_attr(k_num_rows_win<512, 1, float>);
  set_lds_attr(k_num_rows_win<1024, 1, float>);
  set_lds_attr(k_num_rows_win<64, 4, double>);
  set_lds_attr(k_num_rows_win<128, 2, double>);
  set_lds_attr(k_num_rows_win<256, 1, double>);
  set_lds_attr(k_num_rows_win<512, 1, double>);
  set_lds_attr(k_num_rows_win<1024, 1, double>);
  set_lds_attr(k_sym_chunks<64, 4, uint16_t>);
  set_lds_attr(k_sym_chunks<128, 2, uint16_t>);
  set_lds_attr(k_sym_chunks<256, 1, uint16_t>);
  set_lds_attr(k_sym_chunks<512, 1, uint16_t>);
  set_lds_attr(k_sym_chunks<1024, 1, uint16_t>);
#define SG_NUM_ATTR(V)                          \
  set_lds_attr(k_num_rows<64, 4, 1, V>);        \
  set_lds_attr(k_num_rows<64, 4, 2, V>);        \
  set_lds_attr(k_num_rows<64, 4, 4, V>);        \
  set_lds_attr(k_num_rows<128, 2, 4, V>);       \
  set_lds_attr(k_num_rows<256, 1, 4, V>);       \
  set_lds_attr(k_num_rows<512, 1, 4, V>);       \
  set_lds_attr(k_num_rows<1024, 1, 4, V>);      \
  set_lds_attr(k_num_rows<1024, 1, 8, V>);      \
  set_lds_attr(k_num_rows<1024, 1, 16, V>);     \
  set_lds_attr(k_num_chunks<64, 4, 1, V>);      \
  set_lds_attr(k_num_chunks<64, 4, 2, V>);      \
  set_lds_attr(k_num_chunks<64, 4, 4, V>);      \
  set_lds_attr(k_num_chunks<128, 2, 4, V>);     \
  set_lds_attr(k_num_chunks<256, 1, 4, V>);     \
  set_lds_attr(k_num_chunks<512, 1, 4, V>);     \
  set_lds_attr(k_num_chunks<1024, 1, 4, V>);    \
  set_lds_attr(k_num_chunks<1024, 1, 8, V>);    \
  set_lds_attr(k_num_chunks<1024, 1, 16, V>);   \
  set_lds_attr(k_num_chunks<64, 4, 1, V, uint16_t>);      \
  set_lds_attr(k_num_chunks<64, 4, 2, V, uint16_t>);      \
  set_lds_attr(k_num_chunks<64, 4, 4, V, uint16_t>);      \
  set_lds_attr(k_num_chunks<128, 2, 4, V, uint16_t>);     \
  set_lds_attr(k_num_chunks<256, 1, 4, V, uint16_t>);     \
  set_lds_attr(k_num_chunks<512, 1, 4, V, uint16_t>);     \
  set_lds_attr(k_num_chunks<1024, 1, 4, V, uint16_t>);    \
  set_lds_attr(k_num_chunks<1024, 1, 8, V, uint16_t>);    \
  set_lds_attr(k_num_chunks<1024, 1, 16, V, uint16_t>);
  SG_NUM_ATTR(float)
  SG_NUM_ATTR(double)
#undef SG_NUM_ATTR
  set_lds_attr(k_sym_rows_hyb<64, 4>);
  set_lds_attr(k_sym_rows_hyb<128, 2>);
  set_lds_attr(k_sym_rows_hyb<256, 1>);
  set_lds_attr(k_sym_rows_hyb<512, 1>);
  set_lds_attr(k_sym_rows_hyb<1024, 1>);
  set_lds_attr(k_num_rows_hyb<256, 4, float>);
  set_lds_attr(k_num_rows_hyb<512, 4, float>);
  set_lds_attr(k_num_rows_hyb<1024, 4, float>);
  set_lds_attr(k_num_rows_hyb<1024, 8, float>);
  set_lds_attr(k_num_rows_hyb<256, 4, double>);
  set_lds_attr(k_num_rows_hyb<512, 4, double>);
  set_lds_attr(k_num_rows_hyb<1024, 4, double>);
  set_lds_attr(k_num_rows_hyb<1024, 8, double>);
}

#define SG_DISPATCH_TPR(b, MACRO)                      \
  switch ((b).tpr) {                                   \
    case 64: MACRO(64, 4); break;                      \
    case 128: MACRO(128, 2); break;                    \
    case 256: MACRO(256, 1); break;                    \
    case 512: MACRO(512, 1); break;                    \
    default: MACRO(1024, 1); break;                    \
  }

void launch_sym_rows(const BinCfg& b, const int32_t* rows, int64_t nrows, const RowArgs& a,
                     int64_t* cnt, int32_t* err, hipStream_t s) {
  if (nrows <= 0) return;
  const unsigned grid = (unsigned)((nrows + b.rpb - 1) / b.rpb);
#define L(TPR, RPB)                                                                         \
  hipLaunchKernelGGL((k_sym_rows<TPR, RPB>), dim3(grid), dim3(TPR * RPB), b.lds, s, rows, nrows, \
                     b.T, a, cnt, err)
  SG_DISPATCH_TPR(b, L)
#undef L
}

void launch_sym_rows_hyb(const BinCfg& b, const int32_t* rows, int64_t nrows, const RowArgs& a,
                         int64_t m, int64_t n, int64_t* cnt, int32_t* outc, int32_t* err,
                         hipStream_t s) {
  if (nrows <= 0) return;
  const unsigned grid = (unsigned)((nrows + b.rpb - 1) / b.rpb);
  const size_t lds = (size_t)b.rpb * ((size_t)b.T * 4 + kHybWords * 4);
#define L(TPR, RPB)                                                                          \
  hipLaunchKernelGGL((k_sym_rows_hyb<TPR, RPB>), dim3(grid), dim3(TPR * RPB), lds, s, rows,   \
                     nrows, b.T, a, m, n, cnt, outc, err)
  SG_DISPATCH_TPR(b, L)
#undef L
}

size_t window_row_lds(bool numeric, bool f64, const BinCfg& b, int32_t words) {
  if (!numeric) return (size_t)b.rpb * words * 4;
  return (size_t)b.rpb * window_group_bytes(b.cap, words, f64 ? 8 : 4);
}

void launch_sym_rows_win(const BinCfg& b, int32_t words, const int32_t* rows, int64_t nrows,
                         const RowArgs& a, int64_t* cnt, hipStream_t s) {
  if (nrows <= 0) return;
  const unsigned grid = (unsigned)((nrows + b.rpb - 1) / b.rpb);
  const size_t lds = window_row_lds(false, false, b, words);
#define L(TPR, RPB)                                                                         \
  hipLaunchKernelGGL((k_sym_rows_win<TPR, RPB>), dim3(grid), dim3(TPR * RPB), lds, s, rows,  \
                     nrows, words, a, cnt)
  SG_DISPATCH_TPR(b, L)
#undef L
}

void launch_num_rows_win(const BinCfg& b, int32_t words, bool f64, const int32_t* rows,
                         int64_t nrows, const RowArgs& a, const int64_t* cRowOff, int32_t* ccol,
                         void* cval, int32_t* err, hipStream_t s, int64_t* cntOut) {
  if (nrows <= 0) return;
  const unsigned grid = (unsigned)((nrows + b.rpb - 1) / b.rpb);
  const size_t lds = window_row_lds(true, f64, b, words);
#define L(TPR, RPB)                                                                           \
  do {                                                                                       \
    if (f64)                                                                                 \
      hipLaunchKernelGGL((k_num_rows_win<TPR, RPB, double>), dim3(grid), dim3(TPR * RPB), lds, \
                         s, rows, nrows, words, b.cap, a, cRowOff, ccol, (double*)cval, err,   \
                         cntOut);                                                            \
    else                                                                                     \
      hipLaunchKernelGGL((k_num_rows_win<TPR, RPB, float>), dim3(grid), dim3(TPR * RPB), lds,  \
                         s, rows, nrows, words, b.cap, a, cRowOff, ccol, (float*)cval, err,    \
                         cntOut);                                                            \
  } while (0);
  SG_DISPATCH_TPR(b, L)
#undef L
}

void launch_sym_chunks(const BinCfg& b, const ChunkDesc* desc, int64_t n, const ChunkList& cl,
                       int32_t* err, hipStream_t s) {
  if (n <= 0) return;
  const unsigned grid = (unsigned)((n + b.rpb - 1) / b.rpb);
#define L(TPR, RPB)                                                                          \
  do {                                                                                       \
    if (cl.col16)                                                                            \
      hipLaunchKernelGGL((k_sym_chunks<TPR, RPB, uint16_t>), dim3(grid), dim3(TPR * RPB),      \
                         b.lds, s, desc, n, b.T, cl, err);                                   \
    else                                                                                     \
      hipLaunchKernelGGL((k_sym_chunks<TPR, RPB, int32_t>), dim3(grid), dim3(TPR * RPB),       \
                         b.lds, s, desc, n, b.T, cl, err);                                   \
  } while (0);
  SG_DISPATCH_TPR(b, L)
#undef L
}

// Entries per thread of the register sort: max(N, tpr) / tpr.
int sort_e(const BinCfg& b) { return (b.N > b.tpr ? b.N : b.tpr) / b.tpr; }

// (tpr, E) pairs the bins produce: tpr 64 for N <= 256 (E 1, 2, 4), tpr 128
// to 512 with N = 4 tpr, tpr 1024 with N = 4096, 8192 or 16384.
#define SG_DISPATCH_NUM(b, MACRO)                                               \
  do {                                                                          \
    const int e_ = sort_e(b);                                                   \
    if ((b).tpr == 64 && e_ == 1) MACRO(64, 4, 1);                              \
    else if ((b).tpr == 64 && e_ == 2) MACRO(64, 4, 2);                         \
    else if ((b).tpr == 64 && e_ == 4) MACRO(64, 4, 4);                         \
    else if ((b).tpr == 128 && e_ == 4) MACRO(128, 2, 4);                       \
    else if ((b).tpr == 256 && e_ == 4) MACRO(256, 1, 4);                       \
    else if ((b).tpr == 512 && e_ == 4) MACRO(512, 1, 4);                       \
    else if ((b).tpr == 1024 && e_ == 4) MACRO(1024, 1, 4);                     \
    else if ((b).tpr == 1024 && e_ == 8) MACRO(1024, 1, 8);                     \
    else if ((b).tpr == 1024 && e_ == 16) MACRO(1024, 1, 16);                   \
    else flag_unsupported = true;                                               \
  } while (0)

bool num_bin_supported(const BinCfg& b) {
  bool flag_unsupported = false;
#define NOP(TPR, RPB, E) (void)0
  SG_DISPATCH_NUM(b, NOP);
#undef NOP
  return !flag_unsupported;
}

void launch_num_rows(const BinCfg& b, bool f64, const int32_t* rows, int64_t nrows,
                     const RowArgs& a, const int64_t* cRowOff, int32_t* ccol, void* cval,
                     int32_t* err, hipStream_t s, int64_t* cntOut) {
  if (nrows <= 0) return;
  bool flag_unsupported = false;
  const unsigned grid = (unsigned)((nrows + b.rpb - 1) / b.rpb);
  if (f64) {
#define L(TPR, RPB, E)                                                                       \
  hipLaunchKernelGGL((k_num_rows<TPR, RPB, E, double>), dim3(grid), dim3(TPR * RPB), b.lds, s, \
                     rows, nrows, b.T, b.spt, a, cRowOff, ccol, (double*)cval, err, cntOut)
    SG_DISPATCH_NUM(b, L);
#undef L
  } else {
#define L(TPR, RPB, E)                                                                      \
  hipLaunchKernelGGL((k_num_rows<TPR, RPB, E, float>), dim3(grid), dim3(TPR * RPB), b.lds, s, \
                     rows, nrows, b.T, b.spt, a, cRowOff, ccol, (float*)cval, err, cntOut)
    SG_DISPATCH_NUM(b, L);
#undef L
  }
  (void)flag_unsupported;  // make_bins rejects bins without an instance
}

// The hybrid numeric's outlier table holds next_pow2(bin bound) slots (E
// per thread, as the bin's sort); a row may use half of it, and at most
// kHybOutMax (the bucket ranking's bound).
int32_t hyb_out_cap(const BinCfg& b, bool f64, int64_t lds) {
  const int E = sort_e(b);
  const bool inst = b.rpb == 1 && ((b.tpr == 256 && E == 4) || (b.tpr == 512 && E == 4) ||
                                   (b.tpr == 1024 && (E == 4 || E == 8)));
  const int32_t To = b.tpr * E;
  if (!inst || (int64_t)hyb_num_lds(b.tpr, To, f64 ? 8 : 4) > lds) return -1;
  return std::min<int32_t>(To / 2, kHybOutMax);
}

void launch_num_rows_hyb(const BinCfg& b, bool f64, const int32_t* rows, int64_t nrows,
                         const RowArgs& a, int64_t m, int64_t n, const int64_t* cRowOff,
                         int32_t* ccol, void* cval, int32_t* err, hipStream_t s) {
  if (nrows <= 0) return;
  const int E = sort_e(b);
  const int32_t To = b.tpr * E;
  const size_t lds = hyb_num_lds(b.tpr, To, f64 ? 8 : 4);
  const unsigned grid = (unsigned)nrows;
#define L(TPR, E_, V)                                                                         \
  hipLaunchKernelGGL((k_num_rows_hyb<TPR, E_, V>), dim3(grid), dim3(TPR), lds, s, rows, To, a, \
                     m, n, cRowOff, ccol, (V*)cval, err)
#define LV(V)                                 \
  do {                                        \
    if (b.tpr == 256) L(256, 4, V);           \
    else if (b.tpr == 512) L(512, 4, V);      \
    else if (E == 4) L(1024, 4, V);           \
    else L(1024, 8, V);                       \
  } while (0)
  if (f64) LV(double);
  else LV(float);
#undef LV
#undef L
}

bool launch_num_chunks_esc(int32_t cap, bool f64, const ChunkDesc* desc, int64_t n,
                           const ChunkList& cl, int32_t* ccol, void* cval, int32_t* err,
                           hipStream_t s) {
  if (cap > 256) return false;
  if (n <= 0) return true;
  if (cap > 64) {
    const unsigned g = (unsigned)((n * kWave + kEscNT - 1) / kEscNT);
#define LE(E, V, C)                                                                        \
  hipLaunchKernelGGL((k_num_chunks_esc_e<E, V, C>), dim3(g), dim3(kEscNT), 0, s, desc, n, cl, \
                     ccol, (V*)cval, err)
#define LV(E, V)              \
  do {                        \
    if (cl.col16)             \
      LE(E, V, uint16_t);     \
    else                      \
      LE(E, V, int32_t);      \
  } while (0)
    if (cap <= 128) {
      if (f64) LV(2, double);
      else LV(2, float);
    } else {
      if (f64) LV(4, double);
      else LV(4, float);
    }
#undef LV
#undef LE
    return true;
  }
  const int L = cap <= 32 ? 32 : 64;
  const unsigned grid = (unsigned)((n * L + kEscNT - 1) / kEscNT);
#define LE(LL, V, C)                                                                        \
  hipLaunchKernelGGL((k_num_chunks_esc<LL, V, C>), dim3(grid), dim3(kEscNT), 0, s, desc, n, cl, \
                     ccol, (V*)cval, err)
#define LV(LL, V)              \
  do {                         \
    if (cl.col16)              \
      LE(LL, V, uint16_t);     \
    else                       \
      LE(LL, V, int32_t);      \
  } while (0)
  if (L == 32) {
    if (f64) LV(32, double);
    else LV(32, float);
  } else {
    if (f64) LV(64, double);
    else LV(64, float);
  }
#undef LV
#undef LE
  return true;
}

void launch_num_chunks(const BinCfg& b, bool f64, const ChunkDesc* desc, int64_t n,
                       const ChunkList& cl, int32_t* ccol, void* cval, int32_t* err,
                       hipStream_t s) {
  if (n <= 0) return;
  bool flag_unsupported = false;
  const unsigned grid = (unsigned)((n + b.rpb - 1) / b.rpb);
  if (f64) {
#define L(TPR, RPB, E)                                                                         \
  do { \
  if (cl.col16)                                                                                 \
    hipLaunchKernelGGL((k_num_chunks<TPR, RPB, E, double, uint16_t>), dim3(grid),                 \
                       dim3(TPR * RPB), b.lds, s, desc, n, b.T, b.spt, cl, ccol, (double*)cval, err);  \
  else                                                                                          \
    hipLaunchKernelGGL((k_num_chunks<TPR, RPB, E, double>), dim3(grid), dim3(TPR * RPB), b.lds, s,  \
                       desc, n, b.T, b.spt, cl, ccol, (double*)cval, err); \
  } while (0)
    SG_DISPATCH_NUM(b, L);
#undef L
  } else {
#define L(TPR, RPB, E)                                                                        \
  do { \
  if (cl.col16)                                                                                \
    hipLaunchKernelGGL((k_num_chunks<TPR, RPB, E, float, uint16_t>), dim3(grid),                 \
                       dim3(TPR * RPB), b.lds, s, desc, n, b.T, b.spt, cl, ccol, (float*)cval, err);  \
  else                                                                                         \
    hipLaunchKernelGGL((k_num_chunks<TPR, RPB, E, float>), dim3(grid), dim3(TPR * RPB), b.lds, s,  \
                       desc, n, b.T, b.spt, cl, ccol, (float*)cval, err); \
  } while (0)
    SG_DISPATCH_NUM(b, L);
#undef L
  }
  (void)flag_unsupported;  // make_bins rejects bins without an instance
}

void launch_sym_rows_esc(const int32_t* rows, int64_t nrows, const RowArgs& a, int64_t* cnt,
                         hipStream_t s) {
  if (nrows <= 0) return;
  const unsigned grid = (unsigned)((nrows * kEscLanes + kEscNT - 1) / kEscNT);
  hipLaunchKernelGGL((k_rows_esc<false, float>), dim3(grid), dim3(kEscNT), 0, s, rows, nrows, a,
                     nullptr, nullptr, nullptr, cnt, nullptr, nullptr);
}

void launch_num_rows_esc(bool f64, const int32_t* rows, int64_t nrows, const RowArgs& a,
                         const int64_t* cRowOff, int32_t* ccol, void* cval, int32_t* err,
                         hipStream_t s, int64_t* cntOut) {
  if (nrows <= 0) return;
  const unsigned grid = (unsigned)((nrows * kEscLanes + kEscNT - 1) / kEscNT);
  if (f64)
    hipLaunchKernelGGL((k_rows_esc<true, double>), dim3(grid), dim3(kEscNT), 0, s, rows, nrows, a,
                       cRowOff, ccol, (double*)cval, nullptr, err, cntOut);
  else
    hipLaunchKernelGGL((k_rows_esc<true, float>), dim3(grid), dim3(kEscNT), 0, s, rows, nrows, a,
                       cRowOff, ccol, (float*)cval, nullptr, err, cntOut);
}

}  // namespace sg


namespace sg {

int32_t sym_heavy_window_bits(int64_t nreq, int32_t log2W, size_t ldsMax) {
  int32_t bits = log2W;
  while ((int64_t(1) << (bits + 1)) <= nreq * (int64_t(1) << log2W) &&
         (size_t(1) << (bits + 1 - 3)) <= ldsMax && bits < 30)
    ++bits;
  return bits;
}

void launch_sym_heavy_rows(int64_t h, int64_t nreq, int32_t log2W, const int32_t* xheavy,
                           const RowArgs& a, int64_t nnzB, int32_t* slotNnz, int32_t* next,
                           int numCUs, size_t ldsMax, hipStream_t s) {
  if (h <= 0) return;
  const int32_t winBits = sym_heavy_window_bits(nreq, log2W, ldsMax);
  const int64_t cols = nreq << log2W;
  const int32_t nwin = (int32_t)((cols + (int64_t(1) << winBits) - 1) >> winBits);
  const size_t lds = size_t(1) << (winBits - 3);
  // Work groups per CU that the bitmap leaves room for (at most two: 32 waves).
  const int perCU = lds * 2 + 4096 <= ldsMax ? 2 : 1;
  const int64_t items = h * nwin;
  const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>(items, (int64_t)numCUs * perCU));
  hipLaunchKernelGGL(k_sym_heavy_rows, dim3(grid), dim3(kSymHeavyNT), lds, s, h, nwin, winBits,
                     log2W, nreq, xheavy, a, nnzB, slotNnz, next);
}

}  // namespace sg
