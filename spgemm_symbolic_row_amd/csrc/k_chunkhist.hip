// Element counts of every heavy row per W-wide column chunk, from the
// structure of A and B alone (gMAGNUS page, §III-C, the histogram that
// sizes each level's chunks).
//
// Row i's intermediate products in chunk f number
//     sum over k in A_i of |{ j in B_k : j >> log2(W) == f }|,
// and B_k's columns are sorted, so they fall into runs of equal chunk.  The
// runs of every B row are listed once; a heavy row then adds up the runs of
// its A entries in LDS.  That touches at most min(nnz(B_k), n_req) runs per
// A entry instead of every product, and gives the same integers the pass
// over the expanded columns counts.  Every level's counts are sums of these
// over a chunk's range of W-wide pieces.
#include "device_common.hpp"

namespace sg {
namespace {

constexpr int kNT = 256;
inline unsigned grid_for(int64_t n, int per_block, unsigned cap = 65536) {
  int64_t g = (n + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (unsigned)g;
}

// flags[t] = 1 where B's element t starts a run (its chunk differs from the
// previous element's); row starts are added by k_run_row_starts.
__global__ __launch_bounds__(kNT) void k_run_flags(int64_t nnz, const int32_t* __restrict__ col,
                                                   int shift, int32_t* __restrict__ flags) {
  for (int64_t t = (int64_t)blockIdx.x * kNT + threadIdx.x; t < nnz;
       t += (int64_t)gridDim.x * kNT)
    flags[t] = (t == 0 || (col[t] >> shift) != (col[t - 1] >> shift)) ? 1 : 0;
}

__global__ __launch_bounds__(kNT) void k_run_row_starts(int64_t K, const int32_t* __restrict__ rp,
                                                        int32_t* __restrict__ flags) {
  const int64_t k = (int64_t)blockIdx.x * kNT + threadIdx.x;
  if (k >= K) return;
  const int32_t a = rp[k];
  if (a < rp[k + 1]) flags[a] = 1;
}

// runIdx = exclusive scan of flags (nnz + 1 entries).
__global__ __launch_bounds__(kNT) void k_run_fill(int64_t nnz, const int32_t* __restrict__ col,
                                                  int shift, const int32_t* __restrict__ flags,
                                                  const int64_t* __restrict__ runIdx,
                                                  int32_t* __restrict__ runChunk,
                                                  int32_t* __restrict__ runStart) {
  for (int64_t t = (int64_t)blockIdx.x * kNT + threadIdx.x; t < nnz;
       t += (int64_t)gridDim.x * kNT) {
    if (flags[t]) {
      const int64_t r = runIdx[t];
      runChunk[r] = col[t] >> shift;
      runStart[r] = (int32_t)t;
    }
  }
}

// runPtr[k] = first run of B row k (k in [0, K]); runStart[total] = nnz.
__global__ __launch_bounds__(kNT) void k_run_row_ptr(int64_t K, int64_t nnz,
                                                     const int32_t* __restrict__ rp,
                                                     const int64_t* __restrict__ runIdx,
                                                     int32_t* __restrict__ runPtr,
                                                     int32_t* __restrict__ runStart) {
  const int64_t k = (int64_t)blockIdx.x * kNT + threadIdx.x;
  if (k > K) return;
  runPtr[k] = (int32_t)runIdx[rp[k]];
  if (k == K) runStart[runIdx[nnz]] = (int32_t)nnz;
}

// B's slot table from its runs: tab[k * (nreq + 1) + f] = first position of
// B row k whose column lies in slot f or later (the row's end when none
// does), for f in [0, nreq].  One thread per B row writes its nreq + 1
// cells once each, in rising slot order.
__global__ __launch_bounds__(kNT) void k_slot_table(int64_t K, int32_t nreq,
                                                    const int32_t* __restrict__ rp,
                                                    const int32_t* __restrict__ runPtr,
                                                    const int32_t* __restrict__ runChunk,
                                                    const int32_t* __restrict__ runStart,
                                                    int32_t* __restrict__ tab) {
  const int64_t k = (int64_t)blockIdx.x * kNT + threadIdx.x;
  if (k >= K) return;
  int32_t* t = tab + k * (int64_t)(nreq + 1);
  int32_t f = 0;
  const int32_t q1 = runPtr[k + 1];
  for (int32_t q = runPtr[k]; q < q1; ++q) {
    const int32_t c = min(runChunk[q], nreq - 1);
    const int32_t pos = runStart[q];
    for (; f <= c; ++f) t[f] = pos;
  }
  const int32_t end = rp[k + 1];
  for (; f <= nreq; ++f) t[f] = end;
}

// Chunk histogram of the heavy rows.  A work item is a part of at most
// kHistPart consecutive A entries of one heavy row (a row of more entries
// is cut into several parts, so one long row does not hold up the launch);
// itemPtr[i] is the first item of heavy row i.  A work group keeps LDS
// counters for the n_req chunks.  Its waves take the part's entries in turn,
// kHistU at a time, and the lanes of a wave take the runs of one entry's B
// row, which all lie in different chunks, so the LDS adds of one
// instruction never meet at one counter.  A row of one part stores its
// counts; the parts of a longer row add theirs into zeroed counts.
constexpr int kHistU = 4;
constexpr int kHistPart = 256;
__global__ __launch_bounds__(kNT) void k_chunk_hist_rows(int64_t h, const int64_t* __restrict__ itemPtr,
                                                         const int32_t* __restrict__ rows,
                                                         const int32_t* __restrict__ arp,
                                                         const int32_t* __restrict__ acol,
                                                         const int32_t* __restrict__ runPtr,
                                                         const int32_t* __restrict__ runChunk,
                                                         const int32_t* __restrict__ runStart,
                                                         int32_t nreq, int32_t* __restrict__ CH) {
  extern __shared__ int32_t ch[];
  constexpr int NW = kNT / kWave;
  const int64_t item = blockIdx.x;
  if (item >= itemPtr[h]) return;  // the same for the whole work group
  // The heavy row of this item: the last i with itemPtr[i] <= item.
  const int64_t i = wave_last_le(itemPtr, 0, h + 1, item);
  const int64_t part = item - itemPtr[i];
  const bool whole = itemPtr[i + 1] - itemPtr[i] == 1;
  for (int f = threadIdx.x; f < nreq; f += kNT) ch[f] = 0;
  __syncthreads();
  const int32_t r = rows[i];
  const int32_t a0 = arp[r] + (int32_t)(part * kHistPart);
  const int32_t a1 = min(arp[r + 1], a0 + kHistPart);
  const int w = threadIdx.x / kWave, lane = lane_id();
  for (int32_t e0 = a0 + w; e0 < a1; e0 += NW * kHistU) {
    int32_t q0[kHistU], nq[kHistU];
#pragma unroll
    for (int u = 0; u < kHistU; ++u) {
      const int32_t e = e0 + u * NW;
      q0[u] = 0;
      nq[u] = 0;
      if (e < a1) {  // the same for every lane
        const int32_t k = acol[e];
        q0[u] = runPtr[k];
        nq[u] = runPtr[k + 1] - q0[u];
      }
    }
    int32_t c[kHistU], d[kHistU];
#pragma unroll
    for (int u = 0; u < kHistU; ++u) {
      c[u] = -1;
      d[u] = 0;
      if (lane < nq[u]) {
        const int32_t q = q0[u] + lane;
        c[u] = runChunk[q];
        d[u] = runStart[q + 1] - runStart[q];
      }
    }
#pragma unroll
    for (int u = 0; u < kHistU; ++u)
      if (c[u] >= 0) atomicAdd(&ch[c[u]], d[u]);
    // B rows with more than 64 runs (more than 64 chunks per row)
#pragma unroll
    for (int u = 0; u < kHistU; ++u) {
      for (int32_t j = kWave + lane; j < nq[u]; j += kWave) {
        const int32_t q = q0[u] + j;
        atomicAdd(&ch[runChunk[q]], runStart[q + 1] - runStart[q]);
      }
    }
  }
  __syncthreads();
  int32_t* out = CH + i * nreq;
  for (int f = threadIdx.x; f < nreq; f += kNT) {
    if (whole) out[f] = ch[f];
    else if (ch[f]) atomicAdd(&out[f], ch[f]);
  }
}

// Items of every heavy row: ceil(entries / kHistPart), at least one.
__global__ __launch_bounds__(kNT) void k_hist_parts(int64_t h, const int64_t* __restrict__ annz,
                                                    int64_t* __restrict__ parts) {
  const int64_t i = (int64_t)blockIdx.x * kNT + threadIdx.x;
  if (i >= h) return;
  const int64_t e = annz[i + 1] - annz[i];
  parts[i] = e <= kHistPart ? 1 : (e + kHistPart - 1) / kHistPart;
}

// counts[q*v + c] = elements of level row q in its sub-chunk c: the sum of
// `span` consecutive W-wide counts of the row, starting at the row's first
// W-wide piece plus c * span.
__global__ __launch_bounds__(kNT) void k_level_counts(int64_t Q, int v, int32_t span, int32_t nreq,
                                                      const int32_t* __restrict__ inRow,
                                                      const int32_t* __restrict__ inSlot,
                                                      const int32_t* __restrict__ CH,
                                                      int32_t* __restrict__ counts) {
  for (int64_t q = (int64_t)blockIdx.x * kNT + threadIdx.x; q < Q; q += (int64_t)gridDim.x * kNT) {
    const int64_t r = q / v;
    const int32_t c = (int32_t)(q - r * v);
    const int64_t row = inRow ? inRow[r] : r;
    const int32_t s0 = (inSlot ? inSlot[r] : 0) + c * span;
    const int32_t* p = CH + row * nreq + s0;
    int32_t sum = 0;
    for (int32_t f = 0; f < span; ++f) sum += p[f];
    counts[q] = sum;
  }
}

}  // namespace

void launch_b_runs(int64_t K, int64_t nnzB, const int32_t* brp, const int32_t* bcol, int shift,
                   int32_t* flags, int64_t* runIdx, int64_t* scanTmp, int32_t* runPtr,
                   int32_t* runChunk, int32_t* runStart, hipStream_t s) {
  if (nnzB > 0) {
    hipLaunchKernelGGL(k_run_flags, dim3(grid_for(nnzB, kNT * 4)), dim3(kNT), 0, s, nnzB, bcol,
                       shift, flags);
    if (K > 0)
      hipLaunchKernelGGL(k_run_row_starts, dim3(grid_for(K, kNT, 1u << 30)), dim3(kNT), 0, s, K,
                         brp, flags);
  }
  launch_scan_i32(flags, nnzB, runIdx, scanTmp, s);
  if (nnzB > 0)
    hipLaunchKernelGGL(k_run_fill, dim3(grid_for(nnzB, kNT * 4)), dim3(kNT), 0, s, nnzB, bcol,
                       shift, flags, runIdx, runChunk, runStart);
  hipLaunchKernelGGL(k_run_row_ptr, dim3(grid_for(K + 1, kNT, 1u << 30)), dim3(kNT), 0, s, K,
                     nnzB, brp, runIdx, runPtr, runStart);
}

void launch_slot_table(int64_t K, int32_t nreq, const int32_t* brp, const int32_t* runPtr,
                       const int32_t* runChunk, const int32_t* runStart, int32_t* tab,
                       hipStream_t s) {
  if (K <= 0) return;
  hipLaunchKernelGGL(k_slot_table, dim3(grid_for(K, kNT, 1u << 30)), dim3(kNT), 0, s, K, nreq, brp,
                     runPtr, runChunk, runStart, tab);
}

void launch_chunk_hist_rows(int64_t hb, int64_t nAh, const int64_t* annz, const int32_t* rows,
                            const int32_t* arp, const int32_t* acol, const int32_t* runPtr,
                            const int32_t* runChunk, const int32_t* runStart, int32_t nreq,
                            int32_t* CH, int64_t* parts, int64_t* itemPtr, int64_t* scanTmp,
                            hipStream_t s) {
  if (hb <= 0) return;
  hipLaunchKernelGGL(k_hist_parts, dim3(grid_for(hb, kNT, 1u << 30)), dim3(kNT), 0, s, hb, annz,
                     parts);
  launch_scan_i64(parts, hb, itemPtr, scanTmp, s);
  launch_fill_i32(CH, 0, hb * nreq, s);
  // Items: one per row plus one per kHistPart entries, at most.
  const int64_t maxItems = hb + nAh / kHistPart + 1;
  hipLaunchKernelGGL(k_chunk_hist_rows, dim3((unsigned)maxItems), dim3(kNT), (size_t)nreq * 4, s,
                     hb, itemPtr, rows, arp, acol, runPtr, runChunk, runStart, nreq, CH);
}

void launch_level_counts(int64_t Q, int v, int32_t span, int32_t nreq, const int32_t* inRow,
                         const int32_t* inSlot, const int32_t* CH, int32_t* counts,
                         hipStream_t s) {
  if (Q <= 0) return;
  hipLaunchKernelGGL(k_level_counts, dim3(grid_for(Q, kNT)), dim3(kNT), 0, s, Q, v, span, nreq,
                     inRow, inSlot, CH, counts);
}

}  // namespace sg
