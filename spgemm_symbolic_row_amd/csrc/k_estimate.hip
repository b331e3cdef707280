// Size prediction without the symbolic pass, for light rows (Ocean page,
// "Ocean: Fast Estimation-Based Sparse General Matrix-Matrix Multiplication
// on GPU", §3 and Table 1):
//   upper bound  : a row reserves P_i output slots (its product count);
//   estimation   : a HyperLogLog sketch of M one-byte registers per row of B,
//                  merged by element-wise maximum over the B rows an A row
//                  references; the row reserves min(P_i, ceil(coef * E))
//                  slots, E the merged sketch's estimate.
// The numeric pass then writes every light row into its reserved slots and
// reports its count; rows that did not fit are computed again with P_i slots;
// a compaction copies the rows into C once its row pointers are known.
//
// Hash of a column index: MurmurHash3's 32-bit finaliser.  Register index:
// the low log2(M) bits; rank: 1 + the leading zeros of the other 32 - log2(M)
// bits.  E = alpha_M * M^2 / sum_j 2^-r_j (alpha_32 = 0.697, alpha_64 =
// 0.709), or M * ln(M / V) when E <= 2.5 M and V registers are zero (the
// host passes that value for every V, so no logarithm runs on the device).
#include "device_common.hpp"

namespace sg {
namespace {

constexpr int kNT = 256;
constexpr int kWPB = kNT / kWave;

inline unsigned capped_grid(int64_t items, int per_block) {
  const int64_t g = (items + per_block - 1) / per_block;
  return (unsigned)(g < 1 ? 1 : (g > 65536 ? 65536 : g));
}

__device__ __forceinline__ uint32_t hll_hash(uint32_t x) {
  x ^= x >> 16;
  x *= 0x85ebca6bu;
  x ^= x >> 13;
  x *= 0xc2b2ae35u;
  x ^= x >> 16;
  return x;
}

// Register and rank of one column.
__device__ __forceinline__ void hll_slot(int32_t c, int lg, uint32_t* j, uint32_t* rank) {
  const uint32_t h = hll_hash((uint32_t)c);
  *j = h & ((1u << lg) - 1u);
  const uint32_t w = h >> lg;  // 32 - lg significant bits
  *rank = w ? (uint32_t)(__clz((int)w) - lg + 1) : (uint32_t)(32 - lg + 1);
}

__device__ __forceinline__ bool light_bin(int rb, int heavyBin) {
  return rb != 0 && rb != heavyBin;
}

// Estimate of a wave's merged registers (lane j < M holds register j).
__device__ __forceinline__ double hll_value(uint32_t reg, int M, const double* lc) {
  const bool mine = lane_id() < M;
  double z = mine ? ldexp(1.0, -(int)reg) : 0.0;
  z = wave_sum(z);  // sums of powers of two down to 2^-33: exact in fp64
  const int zeros = __popcll(__ballot(mine && reg == 0));
  const double alpha = M == 32 ? 0.697 : 0.709;
  double e = alpha * (double)M * (double)M / z;
  if (e <= 2.5 * M && zeros > 0) e = lc[zeros];
  return e;
}

// One wave per row of B: the row's registers in LDS, then M bytes out.
__global__ __launch_bounds__(kNT) void k_hll_sketch(int64_t K, const int32_t* __restrict__ brp,
                                                    const int32_t* __restrict__ bcol, int lg,
                                                    uint8_t* __restrict__ regs) {
  __shared__ uint32_t r[kWPB][kWave];
  const int w = threadIdx.x / kWave, l = lane_id();
  const int M = 1 << lg;
  const int64_t nw = (int64_t)gridDim.x * kWPB;
  for (int64_t k = (int64_t)blockIdx.x * kWPB + w; k < K; k += nw) {
    r[w][l] = 0;
    const int32_t b0 = brp[k], b1 = brp[k + 1];
    for (int32_t b = b0 + l; b < b1; b += kWave) {
      uint32_t j, rank;
      hll_slot(bcol[b], lg, &j, &rank);
      atomicMax(&r[w][j], rank);
    }
    if (l < M) regs[k * M + l] = (uint8_t)r[w][l];
  }
}

// One wave per light row: merge the sketches of the row's B rows (lane j
// keeps register j), estimate, and reserve min(P_i, ceil(coef * E)) slots
// (at least one).  est (optional) receives E.
__global__ __launch_bounds__(kNT) void k_hll_capacity(
    int64_t m, const int32_t* __restrict__ arp, const int32_t* __restrict__ acol,
    const uint8_t* __restrict__ regs, int lg, const double* __restrict__ lc, double coef,
    const int64_t* __restrict__ rowP, const uint8_t* __restrict__ rowBin, int heavyBin,
    int64_t* __restrict__ cap, double* __restrict__ est) {
  const int l = lane_id();
  const int M = 1 << lg;
  const int64_t nw = (int64_t)gridDim.x * kWPB;
  for (int64_t i = (int64_t)blockIdx.x * kWPB + threadIdx.x / kWave; i < m; i += nw) {
    if (!light_bin(rowBin[i], heavyBin)) continue;
    const int32_t j0 = arp[i], j1 = arp[i + 1];
    uint32_t reg = 0;
    int32_t j = j0;
    // Four entries per round keep four register loads in flight.
    for (; j + 4 <= j1; j += 4) {
      const int32_t k0 = acol[j], k1 = acol[j + 1], k2 = acol[j + 2], k3 = acol[j + 3];
      if (l < M) {
        const uint32_t a0 = regs[(int64_t)k0 * M + l], a1 = regs[(int64_t)k1 * M + l];
        const uint32_t a2 = regs[(int64_t)k2 * M + l], a3 = regs[(int64_t)k3 * M + l];
        reg = max(reg, max(max(a0, a1), max(a2, a3)));
      }
    }
    for (; j < j1; ++j) {
      const int32_t k = acol[j];
      if (l < M) reg = max(reg, (uint32_t)regs[(int64_t)k * M + l]);
    }
    const double e = hll_value(reg, M, lc);
    if (l == 0) {
      const int64_t P = rowP[i];
      int64_t c = (int64_t)ceil(coef * e);
      c = c < P ? c : P;
      cap[i] = P > 0 ? (c > 1 ? c : 1) : 0;
      if (est) est[i] = e;
    }
  }
}

// Estimate of listed rows straight from their products' columns (no B
// sketches): the row sample of the workflow selection.  Rows of more than
// maxP products (heavy rows, sized exactly by the chunk path) get 0.
__global__ __launch_bounds__(kNT) void k_hll_rows_direct(
    int64_t ns, const int32_t* __restrict__ rows, const int32_t* __restrict__ arp,
    const int32_t* __restrict__ acol, const int32_t* __restrict__ brp,
    const int32_t* __restrict__ bcol, const int64_t* __restrict__ rowP, int64_t maxP, int lg,
    const double* __restrict__ lc, double* __restrict__ est) {
  __shared__ uint32_t r[kWPB][kWave];
  const int w = threadIdx.x / kWave, l = lane_id();
  const int M = 1 << lg;
  const int64_t nw = (int64_t)gridDim.x * kWPB;
  for (int64_t s = (int64_t)blockIdx.x * kWPB + w; s < ns; s += nw) {
    const int64_t i = rows[s];
    if (rowP[i] > maxP) {
      if (l == 0) est[s] = 0.0;
      continue;
    }
    r[w][l] = 0;
    for (int32_t j = arp[i]; j < arp[i + 1]; ++j) {
      const int32_t k = acol[j];
      for (int32_t b = brp[k] + l; b < brp[k + 1]; b += kWave) {
        uint32_t q, rank;
        hll_slot(bcol[b], lg, &q, &rank);
        atomicMax(&r[w][q], rank);
      }
    }
    const uint32_t reg = l < M ? r[w][l] : 0u;
    const double e = hll_value(reg, M, lc);
    if (l == 0) est[s] = e;
  }
}

// Upper bound: every light row reserves P_i slots.
__global__ __launch_bounds__(kNT) void k_ub_capacity(int64_t m, const int64_t* __restrict__ rowP,
                                                     const uint8_t* __restrict__ rowBin,
                                                     int heavyBin, int64_t* __restrict__ cap) {
  const int64_t i = (int64_t)blockIdx.x * kNT + threadIdx.x;
  if (i < m && light_bin(rowBin[i], heavyBin)) cap[i] = rowP[i];
}

// Light rows that did not fit (count -1): reserve P_i slots in a second pass
// and give them the numeric key of their product bin; other rows get 0 slots
// and no key.  *nOver receives the number of such rows.
__global__ __launch_bounds__(kNT) void k_overflow_rows(int64_t m, const int64_t* __restrict__ cnt,
                                                       const int64_t* __restrict__ rowP,
                                                       const uint8_t* __restrict__ rowBin,
                                                       int heavyBin, int nbins,
                                                       int64_t* __restrict__ cap2,
                                                       uint8_t* __restrict__ key,
                                                       int32_t* __restrict__ nOver) {
  const int64_t i = (int64_t)blockIdx.x * kNT + threadIdx.x;
  bool over = false;
  if (i < m) {
    const int rb = rowBin[i];
    over = light_bin(rb, heavyBin) && cnt[i] < 0;
    cap2[i] = over ? rowP[i] : 0;
    // hash rows 1..nbins -> keys 0..nbins-1; window rows -> nbins.. (as the
    // numeric binning of the exact workflow)
    key[i] = over ? (uint8_t)(rb < heavyBin ? rb - 1 : nbins + rb - heavyBin - 1) : (uint8_t)255;
  }
  const uint64_t b = __ballot(over);
  if (lane_id() == 0 && b) atomicAdd(nOver, __popcll(b));
}

// Row counts of C: light rows from the estimate workflow's numeric pass
// (first or second), heavy rows as the symbolic pass left them.  Light rows
// redone in the second pass take their source offset from off2, marked by
// bit 62.
__global__ __launch_bounds__(kNT) void k_merge_counts(int64_t m, const uint8_t* __restrict__ rowBin,
                                                      int heavyBin, const int64_t* __restrict__ cnt1,
                                                      const int64_t* __restrict__ cnt2,
                                                      const int64_t* __restrict__ off2,
                                                      int64_t* __restrict__ srcOff,
                                                      int64_t* __restrict__ cnt) {
  const int64_t i = (int64_t)blockIdx.x * kNT + threadIdx.x;
  if (i >= m || !light_bin(rowBin[i], heavyBin)) return;
  const int64_t c1 = cnt1[i];
  if (c1 >= 0 || !cnt2) {
    cnt[i] = c1 < 0 ? 0 : c1;
  } else {
    cnt[i] = cnt2[i] < 0 ? 0 : cnt2[i];
    srcOff[i] = off2[i] | ((int64_t)1 << 62);
  }
}

// Copy every light row from its reserved slots to its place in C (one wave
// per row).
template <typename V>
__global__ __launch_bounds__(kNT) void k_compact_rows(
    int64_t m, const uint8_t* __restrict__ rowBin, int heavyBin,
    const int64_t* __restrict__ srcOff, const int64_t* __restrict__ cnt,
    const int64_t* __restrict__ cRowOff, const int32_t* __restrict__ col1,
    const V* __restrict__ val1, const int32_t* __restrict__ col2, const V* __restrict__ val2,
    int32_t* __restrict__ ccol, V* __restrict__ cval) {
  const int64_t nw = (int64_t)gridDim.x * kWPB;
  for (int64_t i = (int64_t)blockIdx.x * kWPB + threadIdx.x / kWave; i < m; i += nw) {
    if (!light_bin(rowBin[i], heavyBin)) continue;
    const int64_t so = srcOff[i];
    const bool second = (so >> 62) & 1;
    const int64_t src = so & (((int64_t)1 << 62) - 1);
    const int32_t* sc = second ? col2 : col1;
    const V* sv = second ? val2 : val1;
    const int64_t n = cnt[i], dst = cRowOff[i];
    for (int64_t e = lane_id(); e < n; e += kWave) {
      ccol[dst + e] = sc[src + e];
      cval[dst + e] = sv[src + e];
    }
  }
}

}  // namespace

void launch_hll_sketch(int64_t K, const int32_t* brp, const int32_t* bcol, int lg, uint8_t* regs,
                       hipStream_t s) {
  if (K <= 0) return;
  hipLaunchKernelGGL(k_hll_sketch, dim3(capped_grid(K, kWPB)), dim3(kNT), 0, s, K, brp, bcol, lg,
                     regs);
}

void launch_hll_capacity(int64_t m, const int32_t* arp, const int32_t* acol, const uint8_t* regs,
                         int lg, const double* lc, double coef, const int64_t* rowP,
                         const uint8_t* rowBin, int heavyBin, int64_t* cap, double* est,
                         hipStream_t s) {
  if (m <= 0) return;
  hipLaunchKernelGGL(k_hll_capacity, dim3(capped_grid(m, kWPB)), dim3(kNT), 0, s, m, arp, acol,
                     regs, lg, lc, coef, rowP, rowBin, heavyBin, cap, est);
}

void launch_hll_rows_direct(int64_t ns, const int32_t* rows, const int32_t* arp,
                            const int32_t* acol, const int32_t* brp, const int32_t* bcol,
                            const int64_t* rowP, int64_t maxP, int lg, const double* lc,
                            double* est, hipStream_t s) {
  if (ns <= 0) return;
  hipLaunchKernelGGL(k_hll_rows_direct, dim3(capped_grid(ns, kWPB)), dim3(kNT), 0, s, ns, rows,
                     arp, acol, brp, bcol, rowP, maxP, lg, lc, est);
}

void launch_ub_capacity(int64_t m, const int64_t* rowP, const uint8_t* rowBin, int heavyBin,
                        int64_t* cap, hipStream_t s) {
  if (m <= 0) return;
  hipLaunchKernelGGL(k_ub_capacity, dim3((unsigned)((m + kNT - 1) / kNT)), dim3(kNT), 0, s, m,
                     rowP, rowBin, heavyBin, cap);
}

void launch_overflow_rows(int64_t m, const int64_t* cnt, const int64_t* rowP,
                          const uint8_t* rowBin, int heavyBin, int nbins, int64_t* cap2,
                          uint8_t* key, int32_t* nOver, hipStream_t s) {
  if (m <= 0) return;
  hipLaunchKernelGGL(k_overflow_rows, dim3((unsigned)((m + kNT - 1) / kNT)), dim3(kNT), 0, s, m,
                     cnt, rowP, rowBin, heavyBin, nbins, cap2, key, nOver);
}

void launch_merge_counts(int64_t m, const uint8_t* rowBin, int heavyBin, const int64_t* cnt1,
                         const int64_t* cnt2, const int64_t* off2, int64_t* srcOff, int64_t* cnt,
                         hipStream_t s) {
  if (m <= 0) return;
  hipLaunchKernelGGL(k_merge_counts, dim3((unsigned)((m + kNT - 1) / kNT)), dim3(kNT), 0, s, m,
                     rowBin, heavyBin, cnt1, cnt2, off2, srcOff, cnt);
}

void launch_compact_rows(bool f64, int64_t m, const uint8_t* rowBin, int heavyBin,
                         const int64_t* srcOff, const int64_t* cnt, const int64_t* cRowOff,
                         const int32_t* col1, const void* val1, const int32_t* col2,
                         const void* val2, int32_t* ccol, void* cval, hipStream_t s) {
  if (m <= 0) return;
  const dim3 g(capped_grid(m, kWPB)), b(kNT);
  if (f64)
    hipLaunchKernelGGL(k_compact_rows<double>, g, b, 0, s, m, rowBin, heavyBin, srcOff, cnt,
                       cRowOff, col1, (const double*)val1, col2, (const double*)val2, ccol,
                       (double*)cval);
  else
    hipLaunchKernelGGL(k_compact_rows<float>, g, b, 0, s, m, rowBin, heavyBin, srcOff, cnt,
                       cRowOff, col1, (const float*)val1, col2, (const float*)val2, ccol,
                       (float*)cval);
}

}  // namespace sg
