// Outer-product expansion of the heavy rows (gMAGNUS page, §III-B, Eq. 2 and
// the outer-product kernel): the masked CSR -> CSC of A restricted to the
// heavy rows, the reservation of one C-hat segment per CSC entry, and the
// expansion itself.
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

template <typename V, bool kVals>
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
      if constexpr (kVals) a = cscVal[e];
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
        if constexpr (kVals) av[u] = __shfl(a, s);
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
        if constexpr (kVals) bv[u] = dpos[u] >= 0 ? bval[bidx[u]] : V(0);
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (dpos[u] >= 0) {
          outCol[dpos[u]] = cv[u];
          if constexpr (kVals) outVal[dpos[u]] = av[u] * bv[u];
        }
      }
    }
    p = bend;
    j += kWave;
  }
}

// Heavy-row entries in row order: B row start, A value and flattened product
// offset of each (entry t of the batch; rowEntry: entry prefix over the
// batch's rows, absolute; chatRowPtr: product prefix over them, from 0).
// One thread per entry, so rows of 10^4 entries spread over the grid: a wave
// finds the row of its first entry by a search over rowEntry, each lane walks
// forward from there.  offset = product start of the row + the row-local
// offset the row pass stored in scanA.
template <typename V>
__global__ __launch_bounds__(kNT) void k_expand_entries(
    int64_t nE, int64_t hb, const int32_t* __restrict__ rows,
    const int64_t* __restrict__ rowEntry, const int64_t* __restrict__ chatRowPtr,
    const int32_t* __restrict__ arp, const int32_t* __restrict__ acol,
    const V* __restrict__ aval, const int32_t* __restrict__ brp,
    const int32_t* __restrict__ scanA, int32_t* __restrict__ eB, int64_t* __restrict__ eOff,
    V* __restrict__ eVal) {
  const int64_t t0 = ((int64_t)blockIdx.x * kNT + threadIdx.x) / kWave * kWave;
  if (t0 >= nE) return;
  const int64_t base = rowEntry[0];
  int64_t q = wave_last_le(rowEntry, 0, hb, t0 + base);
  const int64_t t = t0 + lane_id();
  if (t >= nE) return;
  while (q + 1 < hb && rowEntry[q + 1] <= t + base) ++q;
  const int32_t row = rows[q];
  const int64_t j = arp[row] + (t + base - rowEntry[q]);
  eB[t] = brp[acol[j]];
  eOff[t] = chatRowPtr[q] + scanA[j];
  if (eVal) eVal[t] = aval[j];
  if (t == nE - 1) eOff[nE] = chatRowPtr[hb];
}

}  // namespace

void launch_expand_entries(bool f64, int64_t nE, int64_t hb, const int32_t* rows,
                           const int64_t* rowEntry, const int64_t* chatRowPtr,
                           const int32_t* arp, const int32_t* acol, const void* aval,
                           const int32_t* brp, const int32_t* scanA, int32_t* eB, int64_t* eOff,
                           void* eVal, hipStream_t s) {
  if (hb <= 0 || nE <= 0) return;
  const unsigned g = grid_for(nE, kNT);
  if (f64)
    hipLaunchKernelGGL(k_expand_entries<double>, dim3(g), dim3(kNT), 0, s, nE, hb, rows, rowEntry,
                       chatRowPtr, arp, acol, (const double*)aval, brp, scanA, eB, eOff,
                       (double*)eVal);
  else
    hipLaunchKernelGGL(k_expand_entries<float>, dim3(g), dim3(kNT), 0, s, nE, hb, rows, rowEntry,
                       chatRowPtr, arp, acol, (const float*)aval, brp, scanA, eB, eOff,
                       (float*)eVal);
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
  if (!outVal)  // columns only
    hipLaunchKernelGGL((k_outer_product<float, false>), dim3(g), dim3(kNT), 0, s, Ph, entryOff, nE,
                       cscCol, (const float*)nullptr, segBase, brp, bcol, (const float*)nullptr,
                       outCol, (float*)nullptr);
  else if (f64)
    hipLaunchKernelGGL((k_outer_product<double, true>), dim3(g), dim3(kNT), 0, s, Ph, entryOff, nE,
                       cscCol, (const double*)cscVal, segBase, brp, bcol, (const double*)bval,
                       outCol, (double*)outVal);
  else
    hipLaunchKernelGGL((k_outer_product<float, true>), dim3(g), dim3(kNT), 0, s, Ph, entryOff, nE,
                       cscCol, (const float*)cscVal, segBase, brp, bcol, (const float*)bval, outCol,
                       (float*)outVal);
}

}  // namespace sg
