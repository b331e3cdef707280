// CSR transpose, T = A^T, for the rectangular products A * A^T (the Ocean
// page, "Ocean: Fast Estimation-Based Sparse General Matrix-Matrix
// Multiplication on GPU", evaluates them on its rectangular matrix set) and
// for restriction-type operands (Trident page, §5.4).
//
// The entries of A are sorted on their column index by a stable
// least-significant-digit radix sort that carries each entry's row and value.
// A stores its entries row by row with rising rows, so stability leaves every
// row of T with rising column indices.  A pass handles one digit of at most
// kTrMaxBits bits:
//   k_tr_hist  : per tile of kTrTile entries, the count of every digit value;
//   scan       : digit-major over (digit, tile), giving every tile its first
//                output position for every digit value;
//   k_tr_pass  : every wave ranks its entries stably (a match of equal digits
//                across the wave, then a running count per wave and digit in
//                LDS), waves are ordered by a prefix over the work group, and
//                each entry is written to its position.
// The row pointers of T come from binary searches over the sorted columns.
#include <algorithm>

#include "device_common.hpp"

namespace sg {
namespace {

constexpr int kTrNT = 512;
constexpr int kTrNW = kTrNT / kWave;
constexpr int kTrItems = 16;
constexpr int kTrWaveElems = kWave * kTrItems;
constexpr int kTrTile = kTrNT * kTrItems;
constexpr int kTrMaxBits = 10;  // digit width cap: 1024 counters per wave
constexpr int kTrMaxBins = 1 << kTrMaxBits;

// Row index of every stored entry: one wave per row, clamped to [0, nnz).
template <typename RP>
__global__ __launch_bounds__(256) void k_tr_rows(int64_t m, const RP* __restrict__ rp,
                                                 int64_t nnz, int32_t* __restrict__ rows) {
  constexpr int WPB = 256 / kWave;
  const int64_t nw = (int64_t)gridDim.x * WPB;
  for (int64_t r = (int64_t)blockIdx.x * WPB + threadIdx.x / kWave; r < m; r += nw) {
    int64_t s = (int64_t)rp[r], e = (int64_t)rp[r + 1];
    s = s < 0 ? 0 : s;
    e = e > nnz ? nnz : e;
    for (int64_t j = s + lane_id(); j < e; j += kWave) rows[j] = (int32_t)r;
  }
}

// Digit counts of one tile, written digit-major: hist[d * tiles + t].  With
// err set, column indices outside [0, n) raise kErrCsr (the sort itself stays
// in bounds for any key: every position comes from these same counts).
__global__ __launch_bounds__(kTrNT) void k_tr_hist(int64_t nnz, const uint32_t* __restrict__ key,
                                                   int shift, int bits, int64_t tiles, int64_t n,
                                                   int32_t* __restrict__ hist,
                                                   int32_t* __restrict__ err) {
  __shared__ int32_t h[kTrMaxBins];
  const int nb = 1 << bits;
  const uint32_t mask = (uint32_t)nb - 1u;
  for (int d = threadIdx.x; d < nb; d += kTrNT) h[d] = 0;
  __syncthreads();
  const int64_t t = blockIdx.x;
  bool bad = false;
#pragma unroll 4
  for (int i = 0; i < kTrItems; ++i) {
    const int64_t e = t * kTrTile + (int64_t)i * kTrNT + threadIdx.x;
    if (e < nnz) {
      const uint32_t k = key[e];
      bad |= (int64_t)k >= n;  // negative indices read as large unsigned values
      atomicAdd(&h[(k >> shift) & mask], 1);
    }
  }
  if (err && __ballot(bad) != 0 && lane_id() == 0) flag_error(err, kErrCsr);
  __syncthreads();
  for (int d = threadIdx.x; d < nb; d += kTrNT) hist[(int64_t)d * tiles + t] = h[d];
}

// One stable scatter pass.  Entry e of tile t is held by wave w, lane l,
// item i with e = t*kTrTile + w*kTrWaveElems + i*64 + l, so a wave visits its
// entries in storage order item by item, and waves cover consecutive ranges.
// kout may be null (keys not needed after this pass).
template <typename V, bool kVals>
__global__ __launch_bounds__(kTrNT) void k_tr_pass(
    int64_t nnz, const uint32_t* __restrict__ kin, const int32_t* __restrict__ rin,
    const V* __restrict__ vin, int shift, int bits, int64_t tiles,
    const int64_t* __restrict__ off, uint32_t* __restrict__ kout, int32_t* __restrict__ rout,
    V* __restrict__ vout) {
  __shared__ uint32_t wc[kTrNW * kTrMaxBins];  // per wave and digit: count, then prefix
  __shared__ int64_t base[kTrMaxBins];         // first output position of each digit
  const int nb = 1 << bits;
  const uint32_t mask = (uint32_t)nb - 1u;
  const int64_t t = blockIdx.x;
  for (int i = threadIdx.x; i < kTrNW * nb; i += kTrNT) wc[(i / nb) * kTrMaxBins + i % nb] = 0;
  for (int d = threadIdx.x; d < nb; d += kTrNT) base[d] = off[(int64_t)d * tiles + t];
  const int w = threadIdx.x / kWave, l = lane_id();
  const int64_t e0 = t * kTrTile + (int64_t)w * kTrWaveElems + l;
  uint32_t key[kTrItems];
  int32_t row[kTrItems];
  V val[kTrItems];
#pragma unroll
  for (int i = 0; i < kTrItems; ++i) {
    const int64_t e = e0 + (int64_t)i * kWave;
    const bool act = e < nnz;
    key[i] = act ? kin[e] : 0u;
    row[i] = act ? rin[e] : 0;
    if constexpr (kVals) val[i] = act ? vin[e] : V(0);
  }
  __syncthreads();
  uint32_t* my = wc + w * kTrMaxBins;
  uint32_t rank[kTrItems];
#pragma unroll
  for (int i = 0; i < kTrItems; ++i) {
    const bool act = e0 + (int64_t)i * kWave < nnz;
    const uint32_t d = (key[i] >> shift) & mask;
    const uint64_t peers = match_key(d, bits, act);
    uint32_t r = 0;
    if (act) {
      // Every lane of the group reads the running count before its highest
      // lane advances it; the store depends on the load, and one wave's LDS
      // accesses are performed in order.
      const uint32_t before = my[d];
      r = before + (uint32_t)__popcll(peers & lanemask_lt());
      if (l == last_set64(peers)) my[d] = before + (uint32_t)__popcll(peers);
    }
    rank[i] = r;
  }
  __syncthreads();
  for (int d = threadIdx.x; d < nb; d += kTrNT) {
    uint32_t run = 0;
#pragma unroll
    for (int v = 0; v < kTrNW; ++v) {
      const uint32_t c = wc[v * kTrMaxBins + d];
      wc[v * kTrMaxBins + d] = run;
      run += c;
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kTrItems; ++i) {
    if (e0 + (int64_t)i * kWave < nnz) {
      const uint32_t d = (key[i] >> shift) & mask;
      const int64_t q = base[d] + (int64_t)my[d] + rank[i];
      if (kout) kout[q] = key[i];
      rout[q] = row[i];
      if constexpr (kVals) vout[q] = val[i];
    }
  }
}

// trp[j] = number of sorted keys below j (lower bound), for j in [0, n].
template <typename RP>
__global__ __launch_bounds__(256) void k_tr_rowptr(int64_t n, int64_t nnz,
                                                   const uint32_t* __restrict__ key,
                                                   RP* __restrict__ trp) {
  for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j <= n;
       j += (int64_t)gridDim.x * 256) {
    int64_t lo = 0, hi = nnz;
    while (lo < hi) {
      const int64_t mid = (lo + hi) >> 1;
      if ((int64_t)key[mid] < j) lo = mid + 1;
      else hi = mid;
    }
    trp[j] = (RP)lo;
  }
}

inline unsigned capped_grid(int64_t items, int per_block) {
  const int64_t g = (items + per_block - 1) / per_block;
  return (unsigned)(g < 1 ? 1 : (g > 65536 ? 65536 : g));
}

template <typename V, bool kVals>
void launch_pass(int64_t nnz, const uint32_t* kin, const int32_t* rin, const void* vin,
                 int shift, int bits, int64_t tiles, const int64_t* off, uint32_t* kout,
                 int32_t* rout, void* vout, hipStream_t s) {
  hipLaunchKernelGGL((k_tr_pass<V, kVals>), dim3((unsigned)tiles), dim3(kTrNT), 0, s, nnz, kin,
                     rin, (const V*)vin, shift, bits, tiles, off, kout, rout, (V*)vout);
}

}  // namespace

TransposePlan transpose_plan(int64_t n, int64_t nnz) {
  TransposePlan tp{};
  int total = 1;
  while (total < 31 && ((int64_t)1 << total) < n) ++total;
  tp.passes = (total + kTrMaxBits - 1) / kTrMaxBits;
  tp.digitBits = (total + tp.passes - 1) / tp.passes;
  tp.totalBits = total;
  tp.tiles = (nnz + kTrTile - 1) / kTrTile;
  tp.histElems = ((int64_t)1 << tp.digitBits) * tp.tiles;
  return tp;
}

void launch_transpose(const TransposePlan& tp, int64_t m, int64_t n, int64_t nnz, const void* arp,
                      int arp64, const int32_t* acol, const void* aval, int valBytes,
                      void* trp, int trp64, int32_t* tcol, void* tval, int32_t* rows[2],
                      uint32_t* keys[2], void* vals[2], int32_t* hist, int64_t* off,
                      int64_t* scanTmp, int32_t* err, hipStream_t s) {
  if (nnz > 0) {
    if (arp64)
      hipLaunchKernelGGL((k_tr_rows<int64_t>), dim3(capped_grid(m, 4)), dim3(256), 0, s, m,
                         (const int64_t*)arp, nnz, rows[1]);
    else
      hipLaunchKernelGGL((k_tr_rows<int32_t>), dim3(capped_grid(m, 4)), dim3(256), 0, s, m,
                         (const int32_t*)arp, nnz, rows[1]);
    for (int p = 0; p < tp.passes; ++p) {
      const int shift = p * tp.digitBits;
      const int bits = std::min(tp.digitBits, tp.totalBits - shift);
      const bool last = p == tp.passes - 1;
      const uint32_t* kin = p == 0 ? (const uint32_t*)acol : keys[(p - 1) & 1];
      const int32_t* rin = rows[(p + 1) & 1];
      const void* vin = p == 0 ? aval : vals[(p - 1) & 1];
      uint32_t* kout = keys[p & 1];
      int32_t* rout = last ? tcol : rows[p & 1];
      void* vout = last ? tval : vals[p & 1];
      hipLaunchKernelGGL(k_tr_hist, dim3((unsigned)tp.tiles), dim3(kTrNT), 0, s, nnz, kin, shift,
                         bits, tp.tiles, n, hist, p == 0 ? err : nullptr);
      const int64_t hn = ((int64_t)1 << bits) * tp.tiles;
      launch_scan_i32(hist, hn, off, scanTmp, s);
      if (!aval)
        launch_pass<float, false>(nnz, kin, rin, nullptr, shift, bits, tp.tiles, off, kout, rout,
                                  nullptr, s);
      else if (valBytes == 8)
        launch_pass<double, true>(nnz, kin, rin, vin, shift, bits, tp.tiles, off, kout, rout,
                                  vout, s);
      else
        launch_pass<float, true>(nnz, kin, rin, vin, shift, bits, tp.tiles, off, kout, rout, vout,
                                 s);
    }
  }
  const uint32_t* sorted = keys[(tp.passes - 1) & 1];
  if (trp64)
    hipLaunchKernelGGL((k_tr_rowptr<int64_t>), dim3(capped_grid(n + 1, 256)), dim3(256), 0, s, n,
                       nnz, sorted, (int64_t*)trp);
  else
    hipLaunchKernelGGL((k_tr_rowptr<int32_t>), dim3(capped_grid(n + 1, 256)), dim3(256), 0, s, n,
                       nnz, sorted, (int32_t*)trp);
}

}  // namespace sg
