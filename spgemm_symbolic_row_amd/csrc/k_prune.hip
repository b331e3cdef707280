// One Markov-clustering prune and column renormalisation (Trident page,
// "Communication-Avoiding SpGEMM via Trident Partitioning", §5.7): entries
// below the threshold are dropped, then every column is divided by the sum
// of its kept entries.  The comparison is made in the value type; column
// sums are accumulated in fp64 and each kept value is rounded once.
#include "device_common.hpp"

namespace sg {
namespace {

constexpr int kNT = 256;

template <typename RP>
__device__ __forceinline__ int64_t rp_at(const void* rp, int64_t i) {
  return (int64_t)((const RP*)rp)[i];
}

// Column sums are aggregated per work group before they reach global memory:
// a work group takes kPruneRows consecutive rows (one wave per row at a
// time), adds every kept value into an LDS table keyed by column, and then
// adds each distinct column's partial sum once with a global atomic.  Rows
// close to each other usually share most columns (clustered graphs, banded
// matrices), so far fewer global atomics are issued; a value whose column
// finds no free slot within kPruneProbes probes goes to global memory
// directly (once the table is full, the columns met only once, such as the
// scattered inter-cluster entries of a clustered graph, take this path
// after a few probes, while the shared columns already sit in the table).
// A wave loads kPruneU runs of 64 entries (columns and values together)
// before it uses any of them.  Kept counts per row are exact integers
// either way.
constexpr int kPruneNT = 512;
constexpr int kPruneRows = 64;
constexpr int kPruneSlots = 4096;
constexpr int kPruneProbes = 4;
constexpr int kPruneU = 4;

__device__ __forceinline__ bool colsum_add_lds(int32_t* keys, double* vals, int32_t key, double v) {
  uint32_t s = hash_slot(key, kPruneSlots);
  for (int probe = 0; probe < kPruneProbes; ++probe) {
    const int32_t cur = lds_load_relaxed(&keys[s]);
    if (cur == key) {
      atomicAdd(&vals[s], v);
      return true;
    }
    if (cur == kEmptyKey) {
      const int32_t old = atomicCAS(&keys[s], kEmptyKey, key);
      if (old == kEmptyKey || old == key) {
        atomicAdd(&vals[s], v);
        return true;
      }
    }
    s = (s + 1 == kPruneSlots) ? 0 : s + 1;
  }
  return false;
}

template <typename V, typename RP>
__global__ __launch_bounds__(kPruneNT) void k_prune_count(int64_t m, const void* __restrict__ rp,
                                                          const int32_t* __restrict__ col,
                                                          const V* __restrict__ val, V thr,
                                                          int64_t* __restrict__ keep,
                                                          double* __restrict__ colsum) {
  __shared__ int32_t keys[kPruneSlots];
  __shared__ double vals[kPruneSlots];
  for (int i = threadIdx.x; i < kPruneSlots; i += kPruneNT) {
    keys[i] = kEmptyKey;
    vals[i] = 0.0;
  }
  __syncthreads();
  const int64_t r0 = (int64_t)blockIdx.x * kPruneRows;
  const int w = threadIdx.x / kWave;
  for (int64_t r = r0 + w; r < r0 + kPruneRows && r < m; r += kPruneNT / kWave) {
    const int64_t a = rp_at<RP>(rp, r), b = rp_at<RP>(rp, r + 1);
    int64_t kept = 0;
    for (int64_t base = a; base < b; base += kWave * kPruneU) {
      V x[kPruneU];
      int32_t c[kPruneU];
      bool act[kPruneU];
#pragma unroll
      for (int u = 0; u < kPruneU; ++u) {
        const int64_t e = base + u * kWave + lane_id();
        act[u] = e < b;
        x[u] = act[u] ? val[e] : V(0);
        c[u] = act[u] ? col[e] : 0;
      }
#pragma unroll
      for (int u = 0; u < kPruneU; ++u) {
        const bool k = act[u] && x[u] >= thr;
        if (k && !colsum_add_lds(keys, vals, c[u], (double)x[u]))
          unsafeAtomicAdd(&colsum[c[u]], (double)x[u]);
        kept += __popcll(__ballot(k));
      }
    }
    if (lane_id() == 0) keep[r] = kept;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kPruneSlots; i += kPruneNT) {
    const int32_t c = keys[i];
    if (c != kEmptyKey) unsafeAtomicAdd(&colsum[c], vals[i]);
  }
}

// One wave per row: order-preserving compaction of the kept entries.  As in
// the count, a wave loads kPruneU runs of 64 entries, then gathers their
// column sums, then writes.
template <typename V, typename RP>
__global__ __launch_bounds__(kNT) void k_prune_fill(int64_t m, const void* __restrict__ rp,
                                                    const int32_t* __restrict__ col,
                                                    const V* __restrict__ val, V thr,
                                                    const int64_t* __restrict__ outOff,
                                                    const double* __restrict__ colsum,
                                                    int32_t* __restrict__ ocol,
                                                    V* __restrict__ oval) {
  const int64_t r = ((int64_t)blockIdx.x * kNT + threadIdx.x) / kWave;
  if (r >= m) return;
  const int64_t a = rp_at<RP>(rp, r), b = rp_at<RP>(rp, r + 1);
  int64_t w = outOff[r];
  for (int64_t base = a; base < b; base += kWave * kPruneU) {
    V x[kPruneU];
    int32_t c[kPruneU];
    bool k[kPruneU];
    double cs[kPruneU];
#pragma unroll
    for (int u = 0; u < kPruneU; ++u) {
      const int64_t e = base + u * kWave + lane_id();
      const bool act = e < b;
      x[u] = act ? val[e] : V(0);
      c[u] = act ? col[e] : 0;
      k[u] = act && x[u] >= thr;
    }
#pragma unroll
    for (int u = 0; u < kPruneU; ++u) cs[u] = k[u] ? colsum[c[u]] : 1.0;
#pragma unroll
    for (int u = 0; u < kPruneU; ++u) {
      const uint64_t mk = __ballot(k[u]);
      if (k[u]) {
        const int64_t pos = w + __popcll(mk & lanemask_lt());
        ocol[pos] = c[u];
        oval[pos] = (V)((double)x[u] / cs[u]);
      }
      w += __popcll(mk);
    }
  }
}

// ------------------------------------------------------------ MCL inflation
// One Markov-clustering iteration after the expansion (Trident page, §5.7):
// columns normalised to sum 1, entries below the threshold dropped, the rest
// squared.  The column sums s_j of all entries come from k_prune_count with
// no threshold; y = x / s_j is formed in fp64 and rounded once to the value
// type (0 for a zero column sum), kept when y >= threshold in the value type,
// and written as y * y in the value type (one more rounding).
template <typename V>
__device__ __forceinline__ V mcl_normalised(V x, double s) {
  return s != 0.0 ? (V)((double)x / s) : V(0);
}

// One wave per row: kept entries per row.
template <typename V, typename RP>
__global__ __launch_bounds__(kNT) void k_mcl_count(int64_t m, const void* __restrict__ rp,
                                                   const int32_t* __restrict__ col,
                                                   const V* __restrict__ val, V thr,
                                                   const double* __restrict__ colsum,
                                                   int64_t* __restrict__ keep) {
  const int64_t r = ((int64_t)blockIdx.x * kNT + threadIdx.x) / kWave;
  if (r >= m) return;
  const int64_t a = rp_at<RP>(rp, r), b = rp_at<RP>(rp, r + 1);
  int64_t kept = 0;
  for (int64_t base = a; base < b; base += kWave * kPruneU) {
    V x[kPruneU];
    int32_t c[kPruneU];
    bool act[kPruneU];
#pragma unroll
    for (int u = 0; u < kPruneU; ++u) {
      const int64_t e = base + u * kWave + lane_id();
      act[u] = e < b;
      x[u] = act[u] ? val[e] : V(0);
      c[u] = act[u] ? col[e] : 0;
    }
    double cs[kPruneU];
#pragma unroll
    for (int u = 0; u < kPruneU; ++u) cs[u] = act[u] ? colsum[c[u]] : 0.0;
#pragma unroll
    for (int u = 0; u < kPruneU; ++u)
      kept += __popcll(__ballot(act[u] && mcl_normalised(x[u], cs[u]) >= thr));
  }
  if (lane_id() == 0) keep[r] = kept;
}

// One wave per row: order-preserving compaction of the kept entries, squared.
template <typename V, typename RP>
__global__ __launch_bounds__(kNT) void k_mcl_fill(int64_t m, const void* __restrict__ rp,
                                                  const int32_t* __restrict__ col,
                                                  const V* __restrict__ val, V thr,
                                                  const int64_t* __restrict__ outOff,
                                                  const double* __restrict__ colsum,
                                                  int32_t* __restrict__ ocol,
                                                  V* __restrict__ oval) {
  const int64_t r = ((int64_t)blockIdx.x * kNT + threadIdx.x) / kWave;
  if (r >= m) return;
  const int64_t a = rp_at<RP>(rp, r), b = rp_at<RP>(rp, r + 1);
  int64_t w = outOff[r];
  for (int64_t base = a; base < b; base += kWave * kPruneU) {
    V x[kPruneU];
    int32_t c[kPruneU];
    bool act[kPruneU];
#pragma unroll
    for (int u = 0; u < kPruneU; ++u) {
      const int64_t e = base + u * kWave + lane_id();
      act[u] = e < b;
      x[u] = act[u] ? val[e] : V(0);
      c[u] = act[u] ? col[e] : 0;
    }
    double cs[kPruneU];
#pragma unroll
    for (int u = 0; u < kPruneU; ++u) cs[u] = act[u] ? colsum[c[u]] : 0.0;
#pragma unroll
    for (int u = 0; u < kPruneU; ++u) {
      const V y = act[u] ? mcl_normalised(x[u], cs[u]) : V(0);
      const bool k = act[u] && y >= thr;
      const uint64_t mk = __ballot(k);
      if (k) {
        const int64_t pos = w + __popcll(mk & lanemask_lt());
        ocol[pos] = c[u];
        oval[pos] = y * y;
      }
      w += __popcll(mk);
    }
  }
}

inline unsigned grid_rows(int64_t m) { return (unsigned)((m * kWave + kNT - 1) / kNT); }

}  // namespace

void launch_prune_count(int64_t m, const void* rp, int rp64, const int32_t* col, const void* val,
                        bool f64, double thr, int64_t* keepCnt, double* colsum,
                        hipStream_t s) {
  if (m <= 0) return;
  const dim3 g((unsigned)((m + kPruneRows - 1) / kPruneRows)), b(kPruneNT);
  if (f64) {
    if (rp64)
      hipLaunchKernelGGL((k_prune_count<double, int64_t>), g, b, 0, s, m, rp, col,
                         (const double*)val, thr, keepCnt, colsum);
    else
      hipLaunchKernelGGL((k_prune_count<double, int32_t>), g, b, 0, s, m, rp, col,
                         (const double*)val, thr, keepCnt, colsum);
  } else {
    if (rp64)
      hipLaunchKernelGGL((k_prune_count<float, int64_t>), g, b, 0, s, m, rp, col,
                         (const float*)val, (float)thr, keepCnt, colsum);
    else
      hipLaunchKernelGGL((k_prune_count<float, int32_t>), g, b, 0, s, m, rp, col,
                         (const float*)val, (float)thr, keepCnt, colsum);
  }
}

void launch_prune_fill(int64_t m, const void* rp, int rp64, const int32_t* col, const void* val,
                       bool f64, double thr, const int64_t* outOff, const double* colsum,
                       int32_t* ocol, void* oval, hipStream_t s) {
  if (m <= 0) return;
  const dim3 g(grid_rows(m)), b(kNT);
  if (f64) {
    if (rp64)
      hipLaunchKernelGGL((k_prune_fill<double, int64_t>), g, b, 0, s, m, rp, col,
                         (const double*)val, thr, outOff, colsum, ocol, (double*)oval);
    else
      hipLaunchKernelGGL((k_prune_fill<double, int32_t>), g, b, 0, s, m, rp, col,
                         (const double*)val, thr, outOff, colsum, ocol, (double*)oval);
  } else {
    if (rp64)
      hipLaunchKernelGGL((k_prune_fill<float, int64_t>), g, b, 0, s, m, rp, col,
                         (const float*)val, (float)thr, outOff, colsum, ocol, (float*)oval);
    else
      hipLaunchKernelGGL((k_prune_fill<float, int32_t>), g, b, 0, s, m, rp, col,
                         (const float*)val, (float)thr, outOff, colsum, ocol, (float*)oval);
  }
}

void launch_mcl_count(int64_t m, const void* rp, int rp64, const int32_t* col, const void* val,
                      bool f64, double thr, const double* colsum, int64_t* keep, hipStream_t s) {
  if (m <= 0) return;
  const dim3 g(grid_rows(m)), b(kNT);
#define L(V, RP)                                                                              \
  hipLaunchKernelGGL((k_mcl_count<V, RP>), g, b, 0, s, m, rp, col, (const V*)val, (V)thr,   \
                     colsum, keep)
  if (f64 && rp64) L(double, int64_t);
  else if (f64) L(double, int32_t);
  else if (rp64) L(float, int64_t);
  else L(float, int32_t);
#undef L
}

void launch_mcl_fill(int64_t m, const void* rp, int rp64, const int32_t* col, const void* val,
                     bool f64, double thr, const int64_t* outOff, const double* colsum,
                     int32_t* ocol, void* oval, hipStream_t s) {
  if (m <= 0) return;
  const dim3 g(grid_rows(m)), b(kNT);
#define L(V, RP)                                                                              \
  hipLaunchKernelGGL((k_mcl_fill<V, RP>), g, b, 0, s, m, rp, col, (const V*)val, (V)thr,    \
                     outOff, colsum, ocol, (V*)oval)
  if (f64 && rp64) L(double, int64_t);
  else if (f64) L(double, int32_t);
  else if (rp64) L(float, int64_t);
  else L(float, int32_t);
#undef L
}

}  // namespace sg
