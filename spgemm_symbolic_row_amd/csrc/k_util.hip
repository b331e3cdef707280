// Utility kernels: fills, device-wide exclusive scan, counting sort by bin,
// the per-row intermediate-product pass (InterOffsets of gMAGNUS Algorithm 3,
// §III-A), CSR validation and row-pointer output.
#include <climits>

#include "device_common.hpp"

namespace sg {

namespace {

constexpr int kNT = 256;

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline unsigned grid_for(int64_t n, int per_block) {
  int64_t g = cdiv(n, per_block);
  if (g < 1) g = 1;
  return (unsigned)g;
}

template <typename T>
__global__ __launch_bounds__(kNT) void k_fill(T* __restrict__ p, T v, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kNT + threadIdx.x; i < n; i += (int64_t)gridDim.x * kNT)
    p[i] = v;
}

__global__ __launch_bounds__(kNT) void k_copy_i64(int64_t* __restrict__ d, const int64_t* __restrict__ s,
                                                  int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kNT + threadIdx.x; i < n; i += (int64_t)gridDim.x * kNT)
    d[i] = s[i];
}

__global__ __launch_bounds__(kNT) void k_gather_i64(const int64_t* __restrict__ src,
                                                    const int32_t* __restrict__ idx, int64_t n,
                                                    int64_t* __restrict__ dst) {
  for (int64_t i = (int64_t)blockIdx.x * kNT + threadIdx.x; i < n; i += (int64_t)gridDim.x * kNT)
    dst[i] = src[idx[i]];
}

__global__ __launch_bounds__(kNT) void k_row_lengths(const int32_t* __restrict__ rows, int64_t n,
                                                     const int32_t* __restrict__ rp,
                                                     int64_t* __restrict__ dst) {
  for (int64_t i = (int64_t)blockIdx.x * kNT + threadIdx.x; i < n; i += (int64_t)gridDim.x * kNT) {
    const int32_t r = rows[i];
    dst[i] = rp[r + 1] - rp[r];
  }
}

// ---- exclusive scan: tile sums, one-block scan of tile sums, down-sweep ----
constexpr int kScanItems = 16;
constexpr int kScanTile = kNT * kScanItems;

template <typename TIn>
__global__ __launch_bounds__(kNT) void k_scan_reduce(const TIn* __restrict__ in, int64_t n,
                                                     int64_t* __restrict__ tileSum) {
  __shared__ int64_t wt[kNT / kWave];
  const int64_t base = (int64_t)blockIdx.x * kScanTile;
  int64_t s = 0;
#pragma unroll
  for (int k = 0; k < kScanItems; ++k) {
    const int64_t i = base + k * kNT + threadIdx.x;
    if (i < n) s += (int64_t)in[i];
  }
  int64_t tot;
  block_excl_scan<kNT>(s, wt, &tot);
  if (threadIdx.x == 0) tileSum[blockIdx.x] = tot;
}

__global__ __launch_bounds__(kNT) void k_scan_tiles(int64_t* __restrict__ t, int64_t nt) {
  __shared__ int64_t wt[kNT / kWave];
  int64_t carry = 0;
  for (int64_t base = 0; base < nt; base += kNT) {
    const int64_t i = base + threadIdx.x;
    const int64_t x = i < nt ? t[i] : 0;
    int64_t tot;
    const int64_t ex = block_excl_scan<kNT>(x, wt, &tot);
    if (i < nt) t[i] = carry + ex;
    carry += tot;
  }
}

template <typename TIn>
__global__ __launch_bounds__(kNT) void k_scan_down(const TIn* __restrict__ in, int64_t n,
                                                   const int64_t* __restrict__ tileOff,
                                                   int64_t* __restrict__ out) {
  __shared__ int64_t wt[kNT / kWave];
  const int64_t base = (int64_t)blockIdx.x * kScanTile + (int64_t)threadIdx.x * kScanItems;
  int64_t v[kScanItems];
  int64_t s = 0;
#pragma unroll
  for (int k = 0; k < kScanItems; ++k) {
    const int64_t i = base + k;
    v[k] = i < n ? (int64_t)in[i] : 0;
    s += v[k];
  }
  int64_t tot;
  int64_t run = block_excl_scan<kNT>(s, wt, &tot) + tileOff[blockIdx.x];
#pragma unroll
  for (int k = 0; k < kScanItems; ++k) {
    const int64_t i = base + k;
    if (i < n) out[i] = run;
    run += v[k];
  }
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) out[n] = tileOff[blockIdx.x] + tot;
}

template <typename TIn>
void scan_impl(const TIn* in, int64_t n, int64_t* out, int64_t* tmp, hipStream_t s) {
  if (n <= 0) {
    hipLaunchKernelGGL(k_fill<int64_t>, dim3(1), dim3(kNT), 0, s, out, (int64_t)0, (int64_t)1);
    return;
  }
  const int64_t nt = cdiv(n, kScanTile);
  hipLaunchKernelGGL(k_scan_reduce<TIn>, dim3((unsigned)nt), dim3(kNT), 0, s, in, n, tmp);
  hipLaunchKernelGGL(k_scan_tiles, dim3(1), dim3(kNT), 0, s, tmp, nt);
  hipLaunchKernelGGL(k_scan_down<TIn>, dim3((unsigned)nt), dim3(kNT), 0, s, in, n,
                     (const int64_t*)tmp, out);
}

// ---- counting sort of item indices by an 8-bit bin key ----
constexpr int kMaxBins = 64;

__global__ __launch_bounds__(kNT) void k_bin_count(const uint8_t* __restrict__ key, int64_t n,
                                                   int nbins, int32_t* __restrict__ cnt) {
  __shared__ int32_t h[kMaxBins];
  if (threadIdx.x < kMaxBins) h[threadIdx.x] = 0;
  __syncthreads();
  for (int64_t i = (int64_t)blockIdx.x * kNT + threadIdx.x; i < n; i += (int64_t)gridDim.x * kNT) {
    const int b = key[i];
    if (b < nbins) atomicAdd(&h[b], 1);
  }
  __syncthreads();
  if (threadIdx.x < nbins && h[threadIdx.x]) atomicAdd(&cnt[threadIdx.x], h[threadIdx.x]);
}

__global__ void k_bin_offsets(const int32_t* __restrict__ cnt, int nbins, int32_t* __restrict__ start,
                              int32_t* __restrict__ fill) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    int32_t r = 0;
    for (int b = 0; b < nbins; ++b) {
      start[b] = r;
      fill[b] = r;
      r += cnt[b];
    }
    start[nbins] = r;
  }
}

// One block per 4096 items: LDS histogram, one global atomic per bin for the
// block's base, then per-item positions from LDS atomics.  Order inside a
// bin is not preserved (the consumers do not depend on it).
constexpr int kBinItems = 16;
__global__ __launch_bounds__(kNT) void k_bin_scatter(const uint8_t* __restrict__ key, int64_t n,
                                                     int nbins, int32_t* __restrict__ fill,
                                                     int32_t* __restrict__ out) {
  __shared__ int32_t h[kMaxBins];
  __shared__ int32_t base[kMaxBins];
  if (threadIdx.x < kMaxBins) h[threadIdx.x] = 0;
  __syncthreads();
  const int64_t b0 = (int64_t)blockIdx.x * kNT * kBinItems;
  uint8_t kk[kBinItems];
#pragma unroll
  for (int k = 0; k < kBinItems; ++k) {
    const int64_t i = b0 + k * kNT + threadIdx.x;
    kk[k] = i < n ? key[i] : (uint8_t)255;
    if (kk[k] < nbins) atomicAdd(&h[kk[k]], 1);
  }
  __syncthreads();
  if (threadIdx.x < nbins) {
    const int32_t c = h[threadIdx.x];
    base[threadIdx.x] = c ? atomicAdd(&fill[threadIdx.x], c) : 0;
    h[threadIdx.x] = 0;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kBinItems; ++k) {
    const int64_t i = b0 + k * kNT + threadIdx.x;
    if (kk[k] < nbins) {
      const int32_t r = atomicAdd(&h[kk[k]], 1);
      out[base[kk[k]] + r] = (int32_t)i;
    }
  }
}

// ---- per-row intermediate products (InterOffsets) ----
// A group of G lanes walks one row of A: for each entry k it reads
// nnz(B[k,:]) from B.row_ptr, scans those counts across the group and
// stores the row-local exclusive offset of every entry (the flattened
// product index where that entry's scaled B row starts).  The row total is
// P_i; its bin is 0 when P_i == 0, 1 + (first cap >= P_i) when P_i <= tau,
// and nbins + 1 (heavy) otherwise.  Each lane takes kRowItems consecutive
// entries per round, so the dependent A.col -> B.row_ptr loads of several
// entries are in flight together.
// Rows of more than kLongRow entries are listed for k_row_info_long, where a
// whole work group scans one row at a time: walked by G lanes, such a row
// would take hundreds of rounds of dependent loads (power-law matrices hold
// rows of 10^4 entries).
// The totals are reduced per work group in LDS and written as one partial
// per work group (part[blockIdx.x * 8 + i]); k_row_stats folds them, so no
// two work groups update the same global address.
constexpr int kRowItems = 4;
constexpr int kLongRow = 1024;
constexpr int kLongNT = 1024;
constexpr int kLongItems = 4;
constexpr int kRowInfoBlocks = 2048;
constexpr int kLongBlocks = 256;

struct RowTotals {
  unsigned long long P, Ph, Ah, Max, H, L, W;
  int32_t Wm[64];  // widest window of each bin, in 32-bit words
  int32_t caps[64];
};

__device__ __forceinline__ void totals_init(RowTotals& t, const int32_t* caps, int nbins) {
  if (threadIdx.x == 0) t.P = t.Ph = t.Ah = t.Max = t.H = t.L = t.W = 0;
  if (threadIdx.x < 64) {
    t.Wm[threadIdx.x] = 0;
    t.caps[threadIdx.x] = threadIdx.x < nbins ? caps[threadIdx.x] : INT_MAX;
  }
}

__device__ __forceinline__ int light_bin(const RowTotals& t, int64_t p, int64_t tau, int nbins) {
  int lb = 0;
  if (p > 0 && p <= tau)
    while (lb < nbins - 1 && p > t.caps[lb]) ++lb;
  return lb;
}

// Bin, window and totals of one row (called by one lane per row).
__device__ __forceinline__ void finish_row(RowTotals& t, int64_t row, int64_t p, int64_t alen,
                                           int lb, int32_t lo, int32_t hi, int64_t tau,
                                           int nbins, int winBins, int64_t* __restrict__ rowP,
                                           uint8_t* __restrict__ rowBin,
                                           int64_t* __restrict__ rowWin) {
  rowP[row] = p;
  uint8_t bin;
  if (p == 0) {
    bin = 0;
  } else if (p > tau) {
    bin = (uint8_t)(nbins + 1);
    atomicAdd(&t.Ph, (unsigned long long)p);
    atomicAdd(&t.Ah, (unsigned long long)alen);
    atomicAdd(&t.H, 1ull);
  } else {
    bin = (uint8_t)(1 + lb);
    const int64_t span = (int64_t)hi - lo + 1;
    if (lb < winBins && span <= 32 * (int64_t)window_words(t.caps[lb])) {
      bin = (uint8_t)(nbins + 2 + lb);
      rowWin[row] = ((span + 31) / 32) << 32 | (int64_t)(uint32_t)lo;
      atomicMax(&t.Wm[lb], (int32_t)((span + 31) / 32));
      atomicAdd(&t.W, (unsigned long long)p);
    }
    atomicAdd(&t.L, 1ull);
  }
  rowBin[row] = bin;
  atomicAdd(&t.P, (unsigned long long)p);
  atomicMax(&t.Max, (unsigned long long)p);
}

__device__ __forceinline__ void totals_write(const RowTotals& t, int64_t* __restrict__ q,
                                             int winBins, int32_t* __restrict__ winMax) {
  if (threadIdx.x == 0) {
    q[kStatProducts] = (int64_t)t.P;
    q[kStatHeavyProducts] = (int64_t)t.Ph;
    q[kStatHeavyANnz] = (int64_t)t.Ah;
    q[kStatMaxRowProducts] = (int64_t)t.Max;
    q[kStatHeavyRows] = (int64_t)t.H;
    q[kStatLightRows] = (int64_t)t.L;
    q[kStatDenseElems] = (int64_t)t.W;
  }
  // Widest window of each bin, for the LDS the window kernels reserve.
  if (threadIdx.x < winBins && t.Wm[threadIdx.x] > 0)
    atomicMax(&winMax[threadIdx.x], t.Wm[threadIdx.x]);
}

template <int G>
__global__ __launch_bounds__(kNT) void k_row_info(int64_t m, const int32_t* __restrict__ arp,
                                                  const int32_t* __restrict__ acol,
                                                  const int32_t* __restrict__ brp,
                                                  const int2* __restrict__ bSpan, int64_t tau,
                                                  const int32_t* __restrict__ caps, int nbins,
                                                  int64_t* __restrict__ rowP,
                                                  int32_t* __restrict__ scanA,
                                                  uint8_t* __restrict__ rowBin,
                                                  int64_t* __restrict__ rowWin, int winBins,
                                                  int32_t* __restrict__ winMax,
                                                  int64_t* __restrict__ part,
                                                  int32_t* __restrict__ longCount,
                                                  int32_t* __restrict__ longRows) {
  __shared__ RowTotals tot;
  totals_init(tot, caps, nbins);
  __syncthreads();
  const int gl = threadIdx.x % G;
  const int64_t rowsPerPass = (int64_t)gridDim.x * (kNT / G);
  for (int64_t row = ((int64_t)blockIdx.x * kNT + threadIdx.x) / G; row < m; row += rowsPerPass) {
    const int64_t rs = arp[row], re = arp[row + 1];
    if (re - rs > kLongRow) {
      if (gl == 0) longRows[atomicAdd(longCount, 1)] = (int32_t)row;
      continue;
    }
    int64_t p = 0;
    for (int64_t b = rs; b < re; b += G * kRowItems) {
      const int64_t j0 = b + (int64_t)gl * kRowItems;
      int32_t k[kRowItems];
      int64_t nb[kRowItems];
#pragma unroll
      for (int u = 0; u < kRowItems; ++u) k[u] = j0 + u < re ? acol[j0 + u] : -1;
      int64_t sum = 0;
#pragma unroll
      for (int u = 0; u < kRowItems; ++u) {
        nb[u] = k[u] >= 0 ? (int64_t)brp[k[u] + 1] - brp[k[u]] : 0;
        sum += nb[u];
      }
      int64_t inc = sum;
#pragma unroll
      for (int d = 1; d < G; d <<= 1) {
        const int64_t t = __shfl_up(inc, d, G);
        if (gl >= d) inc += t;
      }
      int64_t ex = p + inc - sum;
#pragma unroll
      for (int u = 0; u < kRowItems; ++u) {
        if (j0 + u < re) scanA[j0 + u] = (int32_t)ex;
        ex += nb[u];
      }
      p += __shfl(inc, G - 1, G);
    }
    // Light rows of a bin with dense windows: span of the row's products,
    // from the first column of its first-starting B row to the last column
    // of its last-ending one (B rows are sorted; empty ones hold an empty
    // span).
    const int lb = light_bin(tot, p, tau, nbins);
    int32_t lo = INT_MAX, hi = -1;
    if (p > 0 && p <= tau && lb < winBins) {
      for (int64_t b = rs; b < re; b += G * kRowItems) {
        int32_t k[kRowItems];
#pragma unroll
        for (int u = 0; u < kRowItems; ++u) {
          const int64_t j = b + gl + (int64_t)u * G;
          k[u] = j < re ? acol[j] : -1;
        }
#pragma unroll
        for (int u = 0; u < kRowItems; ++u) {
          if (k[u] >= 0) {
            const int2 sp = bSpan[k[u]];
            lo = sp.x < lo ? sp.x : lo;
            hi = sp.y > hi ? sp.y : hi;
          }
        }
      }
#pragma unroll
      for (int d = 1; d < G; d <<= 1) {
        const int32_t l2 = __shfl_xor(lo, d, G), h2 = __shfl_xor(hi, d, G);
        lo = l2 < lo ? l2 : lo;
        hi = h2 > hi ? h2 : hi;
      }
    }
    if (gl == 0)
      finish_row(tot, row, p, re - rs, lb, lo, hi, tau, nbins, winBins, rowP, rowBin, rowWin);
  }
  __syncthreads();
  totals_write(tot, part + (int64_t)blockIdx.x * 8, winBins, winMax);
}

// The rows k_row_info listed: one work group per row, kLongItems
// consecutive entries per thread per round, a work-group scan per round.
// Writes its partials after the short-row grid's.
__global__ __launch_bounds__(kLongNT) void k_row_info_long(
    const int32_t* __restrict__ longCount, const int32_t* __restrict__ longRows,
    const int32_t* __restrict__ arp, const int32_t* __restrict__ acol,
    const int32_t* __restrict__ brp, const int2* __restrict__ bSpan, int64_t tau,
    const int32_t* __restrict__ caps, int nbins, int64_t* __restrict__ rowP,
    int32_t* __restrict__ scanA, uint8_t* __restrict__ rowBin, int64_t* __restrict__ rowWin,
    int winBins, int32_t* __restrict__ winMax, int64_t* __restrict__ part) {
  __shared__ RowTotals tot;
  __shared__ int64_t wtot[kLongNT / kWave];
  __shared__ int32_t wlo[kLongNT / kWave], whi[kLongNT / kWave];
  totals_init(tot, caps, nbins);
  __syncthreads();
  const int32_t cnt = *longCount;
  for (int32_t i = blockIdx.x; i < cnt; i += gridDim.x) {
    const int64_t row = longRows[i];
    const int64_t rs = arp[row], re = arp[row + 1];
    int64_t p = 0;
    for (int64_t b = rs; b < re; b += (int64_t)kLongNT * kLongItems) {
      const int64_t j0 = b + (int64_t)threadIdx.x * kLongItems;
      int32_t k[kLongItems];
      int64_t nb[kLongItems];
#pragma unroll
      for (int u = 0; u < kLongItems; ++u) k[u] = j0 + u < re ? acol[j0 + u] : -1;
      int64_t sum = 0;
#pragma unroll
      for (int u = 0; u < kLongItems; ++u) {
        nb[u] = k[u] >= 0 ? (int64_t)brp[k[u] + 1] - brp[k[u]] : 0;
        sum += nb[u];
      }
      int64_t total;
      int64_t ex = p + block_excl_scan<kLongNT>(sum, wtot, &total);
#pragma unroll
      for (int u = 0; u < kLongItems; ++u) {
        if (j0 + u < re) scanA[j0 + u] = (int32_t)ex;
        ex += nb[u];
      }
      p += total;
    }
    const int lb = light_bin(tot, p, tau, nbins);
    int32_t lo = INT_MAX, hi = -1;
    if (p > 0 && p <= tau && lb < winBins) {
      for (int64_t j = rs + threadIdx.x; j < re; j += kLongNT) {
        const int2 sp = bSpan[acol[j]];
        lo = sp.x < lo ? sp.x : lo;
        hi = sp.y > hi ? sp.y : hi;
      }
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) {
        const int32_t l2 = __shfl_xor(lo, d), h2 = __shfl_xor(hi, d);
        lo = l2 < lo ? l2 : lo;
        hi = h2 > hi ? h2 : hi;
      }
      if (lane_id() == 0) {
        wlo[threadIdx.x / kWave] = lo;
        whi[threadIdx.x / kWave] = hi;
      }
      __syncthreads();
      for (int w = 0; w < kLongNT / kWave; ++w) {
        lo = wlo[w] < lo ? wlo[w] : lo;
        hi = whi[w] > hi ? whi[w] : hi;
      }
    }
    if (threadIdx.x == 0)
      finish_row(tot, row, p, re - rs, lb, lo, hi, tau, nbins, winBins, rowP, rowBin, rowWin);
    __syncthreads();
  }
  __syncthreads();
  totals_write(tot, part + (int64_t)blockIdx.x * 8, winBins, winMax);
}

// First and last column of every B row (rows are sorted).
__global__ __launch_bounds__(kNT) void k_b_span(int64_t K, const int32_t* __restrict__ brp,
                                                const int32_t* __restrict__ bcol,
                                                int2* __restrict__ span) {
  const int64_t k = (int64_t)blockIdx.x * kNT + threadIdx.x;
  if (k >= K) return;
  const int32_t b0 = brp[k], b1 = brp[k + 1];
  span[k] = b1 > b0 ? make_int2(bcol[b0], bcol[b1 - 1]) : make_int2(INT_MAX, -1);
}

// One work group folds the nb partials of k_row_info into stats (added to
// what stats holds; the maximum is taken).
__global__ __launch_bounds__(kNT) void k_row_stats(int64_t nb, const int64_t* __restrict__ part,
                                                   int64_t* __restrict__ stats) {
  __shared__ int64_t red[kNT / kWave];
  const int ids[7] = {kStatProducts, kStatHeavyProducts, kStatHeavyANnz, kStatMaxRowProducts,
                      kStatHeavyRows, kStatLightRows, kStatDenseElems};
  for (int q = 0; q < 7; ++q) {
    const int id = ids[q];
    const bool isMax = id == kStatMaxRowProducts;
    int64_t x = 0;
    for (int64_t b = threadIdx.x; b < nb; b += kNT) {
      const int64_t y = part[b * 8 + id];
      x = isMax ? (y > x ? y : x) : x + y;
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      const int64_t y = __shfl_xor(x, d);
      x = isMax ? (y > x ? y : x) : x + y;
    }
    if (lane_id() == 0) red[threadIdx.x / kWave] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
      int64_t t = stats[id];
      for (int w = 0; w < kNT / kWave; ++w) t = isMax ? (red[w] > t ? red[w] : t) : t + red[w];
      stats[id] = t;
    }
    __syncthreads();
  }
}

// ---- CSR validation: one thread per row ----
__global__ __launch_bounds__(kNT) void k_validate(int64_t rows, int64_t cols, int64_t nnz,
                                                  const int32_t* __restrict__ rp,
                                                  const int32_t* __restrict__ col,
                                                  int32_t* __restrict__ err) {
  const int64_t i = (int64_t)blockIdx.x * kNT + threadIdx.x;
  if (i >= rows) return;
  const int64_t a = rp[i], b = rp[i + 1];
  bool ok = (a >= 0) && (b >= a) && (b <= nnz);
  if (i == 0 && a != 0) ok = false;
  if (i == rows - 1 && b != nnz) ok = false;
  if (ok) {
    int64_t prev = -1;
    for (int64_t e = a; e < b; ++e) {
      const int64_t c = col[e];
      if (c < 0 || c >= cols || c <= prev) {
        ok = false;
        break;
      }
      prev = c;
    }
  }
  if (!ok) flag_error(err, kErrCsr);
}

__global__ __launch_bounds__(kNT) void k_write_rowptr(const int64_t* __restrict__ off, int64_t n,
                                                      void* __restrict__ out, int is64) {
  for (int64_t i = (int64_t)blockIdx.x * kNT + threadIdx.x; i < n; i += (int64_t)gridDim.x * kNT) {
    if (is64)
      ((int64_t*)out)[i] = off[i];
    else
      ((int32_t*)out)[i] = (int32_t)off[i];
  }
}

__global__ __launch_bounds__(kNT) void k_numeric_row_bins(int64_t m, const int64_t* __restrict__ cnt,
                                                          const uint8_t* __restrict__ rowBin,
                                                          int heavyBin,
                                                          const int32_t* __restrict__ caps,
                                                          int nbins, int escKey,
                                                          const int32_t* __restrict__ outc,
                                                          const int32_t* __restrict__ hybCap,
                                                          int hybSymMin, int hybKey,
                                                          uint8_t* __restrict__ key) {
  const int64_t i = (int64_t)blockIdx.x * kNT + threadIdx.x;
  if (i >= m) return;
  const int rb = rowBin[i];
  if (rb == 0 || rb == heavyBin) {
    key[i] = 255;
    return;
  }
  if (rb == 1 && escKey >= 0) {  // at most caps[0] <= 32 products: ESC
    key[i] = (uint8_t)escKey;
    return;
  }
  if (rb > heavyBin) {  // dense window rows: bin by products, after the hash bins
    key[i] = (uint8_t)(nbins + rb - heavyBin - 1);
    return;
  }
  const int64_t c = cnt[i];
  int b = 0;
  while (b < nbins - 1 && c > caps[b]) ++b;
  if (outc && rb >= hybSymMin && outc[i] <= hybCap[b]) {
    key[i] = (uint8_t)(hybKey + b);
    return;
  }
  key[i] = (uint8_t)b;
}

struct SmallI32 {
  int32_t v[64];
};
__global__ void k_set_small(int32_t* __restrict__ dst, SmallI32 vals, int n) {
  if ((int)threadIdx.x < n) dst[threadIdx.x] = vals.v[threadIdx.x];
}

// tail = (ctr[0], ctr[1], newOff[ctr[0]]): a multisplit level's heavy and
// light chunk counts and the heavy chunks' element total.
__global__ void k_level_tail(const int32_t* __restrict__ ctr, const int64_t* __restrict__ newOff,
                             int64_t* __restrict__ tail) {
  if (threadIdx.x == 0) {
    tail[0] = ctr[0];
    tail[1] = ctr[1];
    tail[2] = newOff[ctr[0]];
  }
}

}  // namespace

void launch_set_small_i32(int32_t* dst, const int32_t* vals, int n, hipStream_t s) {
  if (n <= 0) return;
  SmallI32 sv{};
  for (int i = 0; i < n && i < 64; ++i) sv.v[i] = vals[i];
  hipLaunchKernelGGL(k_set_small, dim3(1), dim3(64), 0, s, dst, sv, n < 64 ? n : 64);
}
void launch_level_tail(const int32_t* ctr, const int64_t* newOff, int64_t* tail, hipStream_t s) {
  hipLaunchKernelGGL(k_level_tail, dim3(1), dim3(64), 0, s, ctr, newOff, tail);
}

void launch_fill_i32(int32_t* p, int32_t v, int64_t n, hipStream_t s) {
  if (n <= 0) return;
  unsigned g = grid_for(n, kNT * 4);
  if (g > 65536) g = 65536;
  hipLaunchKernelGGL(k_fill<int32_t>, dim3(g), dim3(kNT), 0, s, p, v, n);
}
void launch_fill_i64(int64_t* p, int64_t v, int64_t n, hipStream_t s) {
  if (n <= 0) return;
  unsigned g = grid_for(n, kNT * 4);
  if (g > 65536) g = 65536;
  hipLaunchKernelGGL(k_fill<int64_t>, dim3(g), dim3(kNT), 0, s, p, v, n);
}
void launch_fill_i8(int8_t* p, int8_t v, int64_t n, hipStream_t s) {
  if (n <= 0) return;
  unsigned g = grid_for(n, kNT * 4);
  if (g > 65536) g = 65536;
  hipLaunchKernelGGL(k_fill<int8_t>, dim3(g), dim3(kNT), 0, s, p, v, n);
}
void launch_copy_i64(int64_t* dst, const int64_t* src, int64_t n, hipStream_t s) {
  if (n <= 0) return;
  unsigned g = grid_for(n, kNT * 4);
  if (g > 65536) g = 65536;
  hipLaunchKernelGGL(k_copy_i64, dim3(g), dim3(kNT), 0, s, dst, src, n);
}
void launch_gather_i64(const int64_t* src, const int32_t* idx, int64_t n, int64_t* dst,
                       hipStream_t s) {
  if (n <= 0) return;
  unsigned g = grid_for(n, kNT * 4);
  if (g > 65536) g = 65536;
  hipLaunchKernelGGL(k_gather_i64, dim3(g), dim3(kNT), 0, s, src, idx, n, dst);
}

void launch_row_lengths(int64_t n, const int32_t* rows, const int32_t* rp, int64_t* dst,
                        hipStream_t s) {
  if (n <= 0) return;
  unsigned g = grid_for(n, kNT * 4);
  if (g > 65536) g = 65536;
  hipLaunchKernelGGL(k_row_lengths, dim3(g), dim3(kNT), 0, s, rows, n, rp, dst);
}

int64_t scan_tmp_elems(int64_t n) { return cdiv(n > 0 ? n : 1, kScanTile); }

void launch_scan_i64(const int64_t* in, int64_t n, int64_t* out, int64_t* tmp, hipStream_t s) {
  scan_impl<int64_t>(in, n, out, tmp, s);
}
void launch_scan_i32(const int32_t* in, int64_t n, int64_t* out, int64_t* tmp, hipStream_t s) {
  scan_impl<int32_t>(in, n, out, tmp, s);
}

void launch_bin_sort(const uint8_t* key, int64_t n, int nbins, int32_t* cnt, int32_t* fill,
                     int32_t* start, int32_t* out, hipStream_t s) {
  launch_fill_i32(cnt, 0, nbins, s);
  if (n > 0) {
    unsigned g = grid_for(n, kNT * 4);
    if (g > 65536) g = 65536;
    hipLaunchKernelGGL(k_bin_count, dim3(g), dim3(kNT), 0, s, key, n, nbins, cnt);
  }
  hipLaunchKernelGGL(k_bin_offsets, dim3(1), dim3(64), 0, s, (const int32_t*)cnt, nbins, start,
                     fill);
  if (n > 0) {
    hipLaunchKernelGGL(k_bin_scatter, dim3(grid_for(n, kNT * kBinItems)), dim3(kNT), 0, s, key,
                       n, nbins, fill, out);
  }
}

namespace {
unsigned row_info_grid(int64_t m) {
  unsigned g = grid_for(m * 16, kNT);
  return g > (unsigned)kRowInfoBlocks ? (unsigned)kRowInfoBlocks : g;
}
}  // namespace

int64_t row_info_partials(int64_t m, int64_t nnzA) {
  // partials of both grids, the long-row count, the long-row list
  return ((int64_t)row_info_grid(m) + kLongBlocks) * 8 + 1 + (nnzA / kLongRow + 2) / 2;
}

void launch_row_info(int64_t m, int64_t nnzA, const int32_t* arp, const int32_t* acol,
                     const int32_t* brp, const int2* bSpan, int64_t tau, const int32_t* caps,
                     int nbins, int64_t* rowP, int32_t* scanA, uint8_t* rowBin, int64_t* rowWin,
                     int winBins, int32_t* winMax, int64_t* part, int64_t* stats,
                     hipStream_t s) {
  if (m <= 0) return;
  constexpr int G = 16;
  const unsigned g = row_info_grid(m);
  int64_t* partLong = part + (int64_t)g * 8;
  int32_t* longCount = (int32_t*)(part + ((int64_t)g + kLongBlocks) * 8);
  int32_t* longRows = longCount + 2;
  (void)nnzA;
  launch_fill_i32(longCount, 0, 1, s);
  hipLaunchKernelGGL(k_row_info<G>, dim3(g), dim3(kNT), 0, s, m, arp, acol, brp, bSpan, tau, caps,
                     nbins, rowP, scanA, rowBin, rowWin, rowWin ? winBins : 0, winMax, part,
                     longCount, longRows);
  hipLaunchKernelGGL(k_row_info_long, dim3(kLongBlocks), dim3(kLongNT), 0, s, longCount, longRows,
                     arp, acol, brp, bSpan, tau, caps, nbins, rowP, scanA, rowBin, rowWin,
                     rowWin ? winBins : 0, winMax, partLong);
  hipLaunchKernelGGL(k_row_stats, dim3(1), dim3(kNT), 0, s, (int64_t)g + kLongBlocks, part, stats);
}

void launch_b_span(int64_t K, const int32_t* brp, const int32_t* bcol, int2* span, hipStream_t s) {
  if (K <= 0) return;
  hipLaunchKernelGGL(k_b_span, dim3(grid_for(K, kNT)), dim3(kNT), 0, s, K, brp, bcol, span);
}

void launch_validate(int64_t rows, int64_t cols, int64_t nnz, const int32_t* rp,
                     const int32_t* col, int32_t* err, hipStream_t s) {
  if (rows <= 0) return;
  hipLaunchKernelGGL(k_validate, dim3(grid_for(rows, kNT)), dim3(kNT), 0, s, rows, cols, nnz, rp,
                     col, err);
}

void launch_write_rowptr(const int64_t* off, int64_t n, void* out, int is64, hipStream_t s) {
  if (n <= 0) return;
  unsigned g = grid_for(n, kNT * 4);
  if (g > 65536) g = 65536;
  hipLaunchKernelGGL(k_write_rowptr, dim3(g), dim3(kNT), 0, s, off, n, out, is64);
}

void launch_numeric_row_bins(int64_t m, const int64_t* cnt, const uint8_t* rowBin,
                             int heavyBin, const int32_t* caps, int nbins, uint8_t* key,
                             hipStream_t s, int escKey, const int32_t* outc,
                             const int32_t* hybCap, int hybSymMin, int hybKey) {
  if (m <= 0) return;
  hipLaunchKernelGGL(k_numeric_row_bins, dim3(grid_for(m, kNT)), dim3(kNT), 0, s, m, cnt, rowBin,
                     heavyBin, caps, nbins, escKey, outc, hybCap, hybSymMin, hybKey, key);
}

}  // namespace sg
