// One Markov-clustering prune and column renormalisation (Trident page,
// "Communication-Avoiding SpGEMM via Trident Partitioning", §5.7): entries
// below the threshold are dropped, then every column is divided by the sum
// of its kept entries.  The comparison is made in the value type; column
// sums are accumulated in fp64; an fp64 kept value is divided by its column
// sum and rounded once, an fp32 one multiplied by the fp32-rounded
// reciprocal of the sum (relative error below 2^-22).
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

template <int SLOTS = kPruneSlots>
__device__ __forceinline__ bool colsum_add_lds(int32_t* keys, double* vals, int32_t key, double v) {
  uint32_t s = hash_slot(key, SLOTS);
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
    s = (s + 1 == SLOTS) ? 0 : s + 1;
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

// The same count with no global add per column: the LDS table's misses
// (mostly columns met once by the work group, such as entries between
// clusters) are kept in an LDS list, and at the end the work group counts
// the list and its table's columns per bucket of 2^log2Cols columns,
// reserves each bucket's range with one global add, and writes them there as
// (column, fp64 value); k_colsum_buckets then adds each bucket up in LDS.  A
// full list or bucket falls back to the global add.
constexpr int kPruneBNT = 1024;
constexpr int kPruneBRows = 40;
constexpr int kPruneBSlots = 4096;
constexpr int kMissCap = 8192;
constexpr int kMaxBuckets = 1024;
constexpr int kBucketSplit = 4;  // work groups per bucket in k_colsum_buckets

template <typename V, typename RP>
__global__ __launch_bounds__(kPruneBNT) void k_prune_count_b(int64_t m, const void* __restrict__ rp,
                                                             const int32_t* __restrict__ col,
                                                             const V* __restrict__ val, V thr,
                                                             int64_t* __restrict__ keep,
                                                             double* __restrict__ colsum,
                                                             int32_t nb, int log2Cols, int64_t cap,
                                                             unsigned long long* __restrict__ fill,
                                                             int32_t* __restrict__ bcol,
                                                             double* __restrict__ bval) {
  __shared__ int32_t keys[kPruneBSlots];
  __shared__ double vals[kPruneBSlots];
  __shared__ int32_t missCol[kMissCap];
  __shared__ V missVal[kMissCap];
  __shared__ int32_t hist[kMaxBuckets];
  __shared__ int64_t base[kMaxBuckets];
  __shared__ int32_t nMiss;
  for (int i = threadIdx.x; i < kPruneBSlots; i += kPruneBNT) {
    keys[i] = kEmptyKey;
    vals[i] = 0.0;
  }
  for (int i = threadIdx.x; i < nb; i += kPruneBNT) hist[i] = 0;
  if (threadIdx.x == 0) nMiss = 0;
  __syncthreads();
  const int64_t r0 = (int64_t)blockIdx.x * kPruneBRows;
  const int w = threadIdx.x / kWave;
  for (int64_t r = r0 + w; r < r0 + kPruneBRows && r < m; r += kPruneBNT / kWave) {
    const int64_t a = rp_at<RP>(rp, r), b = rp_at<RP>(rp, r + 1);
    int64_t kept = 0;
    for (int64_t e0 = a; e0 < b; e0 += kWave * kPruneU) {
      V x[kPruneU];
      int32_t c[kPruneU];
      bool act[kPruneU];
#pragma unroll
      for (int u = 0; u < kPruneU; ++u) {
        const int64_t e = e0 + u * kWave + lane_id();
        act[u] = e < b;
        x[u] = act[u] ? val[e] : V(0);
        c[u] = act[u] ? col[e] : 0;
      }
#pragma unroll
      for (int u = 0; u < kPruneU; ++u) {
        const bool k = act[u] && x[u] >= thr;
        if (k && !colsum_add_lds<kPruneBSlots>(keys, vals, c[u], (double)x[u])) {
          const int at = atomicAdd(&nMiss, 1);
          if (at < kMissCap) {
            missCol[at] = c[u];
            missVal[at] = x[u];
          } else {
            unsafeAtomicAdd(&colsum[c[u]], (double)x[u]);
          }
        }
        kept += __popcll(__ballot(k));
      }
    }
    if (lane_id() == 0) keep[r] = kept;
  }
  __syncthreads();
  // Bucket counts of the table's columns and of the list, one reservation
  // per bucket, then both written out.
  const int nm = min(nMiss, kMissCap);
  for (int i = threadIdx.x; i < kPruneBSlots + nm; i += kPruneBNT) {
    const int32_t c = i < kPruneBSlots ? keys[i] : missCol[i - kPruneBSlots];
    if (c == kEmptyKey) continue;
    const uint32_t bk = (uint32_t)c >> log2Cols;
    if (bk < (uint32_t)nb) atomicAdd(&hist[bk], 1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nb; i += kPruneBNT) {
    const int32_t h = hist[i];
    base[i] = h ? (int64_t)atomicAdd(&fill[i * kFillStride], (unsigned long long)h) : 0;
    hist[i] = 0;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kPruneBSlots + nm; i += kPruneBNT) {
    int32_t c;
    double v;
    if (i < kPruneBSlots) {
      c = keys[i];
      v = vals[i];
    } else {
      c = missCol[i - kPruneBSlots];
      v = (double)missVal[i - kPruneBSlots];
    }
    if (c == kEmptyKey) continue;
    const uint32_t bk = (uint32_t)c >> log2Cols;
    const int64_t p = bk < (uint32_t)nb ? base[bk] + atomicAdd(&hist[bk], 1) : cap;
    if (p < cap) {
      bcol[bk * cap + p] = c;
      bval[bk * cap + p] = v;
    } else {
      unsafeAtomicAdd(&colsum[c], v);
    }
  }
}

// kBucketSplit work groups per bucket, each adding its share of the
// bucket's entries up in LDS (fp64) and each column's partial sum into
// colsum.
constexpr int kSumNT = 1024;
__global__ __launch_bounds__(kSumNT) void k_colsum_buckets(int64_t n, int log2Cols, int64_t cap,
                                                              const unsigned long long* __restrict__ fill,
                                                              const int32_t* __restrict__ bcol,
                                                              const double* __restrict__ bval,
                                                              double* __restrict__ colsum) {
  extern __shared__ __align__(16) unsigned char smem[];
  double* sums = (double*)smem;
  const int cols = 1 << log2Cols;
  const int64_t bk = blockIdx.x / kBucketSplit;
  const int part = blockIdx.x % kBucketSplit;
  const int64_t c0 = bk << log2Cols;
  for (int j = threadIdx.x; j < cols; j += kSumNT) sums[j] = 0.0;
  __syncthreads();
  const int64_t cnt = min<int64_t>((int64_t)fill[bk * kFillStride], cap);
  const int64_t i0 = cnt * part / kBucketSplit, i1 = cnt * (part + 1) / kBucketSplit;
  const int32_t* bc = bcol + bk * cap;
  const double* bv = bval + bk * cap;
  for (int64_t i = i0 + threadIdx.x; i < i1; i += kSumNT) {
    const int64_t j = (int64_t)bc[i] - c0;
    if (j >= 0 && j < cols) atomicAdd(&sums[j], bv[i]);
  }
  __syncthreads();
  for (int j = threadIdx.x; j < cols; j += kSumNT) {
    const int64_t c = c0 + j;
    if (c < n && sums[j] != 0.0) unsafeAtomicAdd(&colsum[c], sums[j]);
  }
}

// fp32 values: the reciprocal of every column sum, rounded to fp32 (0 for
// an empty column), so that the fill gathers 4 bytes per kept entry from a
// table half the size of the sums.
__global__ __launch_bounds__(kNT) void k_colsum_recip(int64_t n, const double* __restrict__ colsum,
                                                      float* __restrict__ inv) {
  const int64_t j = (int64_t)blockIdx.x * kNT + threadIdx.x;
  if (j < n) inv[j] = colsum[j] != 0.0 ? (float)(1.0 / colsum[j]) : 0.0f;
}

template <typename V>
__device__ __forceinline__ V prune_scaled(V x, double cs) {
  return (V)((double)x / cs);
}
__device__ __forceinline__ float prune_scaled(float x, float inv) { return x * inv; }

// One wave per row: order-preserving compaction of the kept entries.  As in
// the count, a wave loads kPruneU runs of 64 entries, then gathers their
// column scales (fp64 sums, or fp32 reciprocals of them for fp32 values),
// then writes.
template <typename V, typename RP, typename S>
__global__ __launch_bounds__(kNT) void k_prune_fill(int64_t m, const void* __restrict__ rp,
                                                    const int32_t* __restrict__ col,
                                                    const V* __restrict__ val, V thr,
                                                    const int64_t* __restrict__ outOff,
                                                    const S* __restrict__ colsum,
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
    S cs[kPruneU];
#pragma unroll
    for (int u = 0; u < kPruneU; ++u) {
      const int64_t e = base + u * kWave + lane_id();
      const bool act = e < b;
      x[u] = act ? val[e] : V(0);
      c[u] = act ? col[e] : 0;
      k[u] = act && x[u] >= thr;
    }
#pragma unroll
    for (int u = 0; u < kPruneU; ++u) cs[u] = k[u] ? colsum[c[u]] : S(1);
#pragma unroll
    for (int u = 0; u < kPruneU; ++u) {
      const uint64_t mk = __ballot(k[u]);
      if (k[u]) {
        const int64_t pos = w + __popcll(mk & lanemask_lt());
        ocol[pos] = c[u];
        oval[pos] = prune_scaled(x[u], cs[u]);
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

bool prune_buckets_fit(int64_t n, int* log2Cols, int32_t* nb) {
  int lg = 11;
  while (lg < 14 && ((n + ((int64_t)1 << lg) - 1) >> lg) > kMaxBuckets) ++lg;
  const int64_t b = (n + ((int64_t)1 << lg) - 1) >> lg;
  if (n <= 0 || b > kMaxBuckets) return false;
  *log2Cols = lg;
  *nb = (int32_t)b;
  return true;
}

void launch_prune_count_b(int64_t m, int64_t n, const void* rp, int rp64, const int32_t* col,
                          const void* val, bool f64, double thr, int64_t* keepCnt, double* colsum,
                          int32_t nb, int log2Cols, int64_t cap, unsigned long long* fill,
                          int32_t* bcol, double* bval, hipStream_t s) {
  if (m <= 0) return;
  const dim3 g((unsigned)((m + kPruneBRows - 1) / kPruneBRows)), b(kPruneBNT);
#define L(V, RP)                                                                               \
  hipLaunchKernelGGL((k_prune_count_b<V, RP>), g, b, 0, s, m, rp, col, (const V*)val, (V)thr,   \
                     keepCnt, colsum, nb, log2Cols, cap, fill, bcol, bval)
  if (f64 && rp64) L(double, int64_t);
  else if (f64) L(double, int32_t);
  else if (rp64) L(float, int64_t);
  else L(float, int32_t);
#undef L
  const size_t lds = sizeof(double) << log2Cols;
  hipLaunchKernelGGL(k_colsum_buckets, dim3((unsigned)nb * kBucketSplit), dim3(kSumNT), lds, s,
                     n, log2Cols, cap, fill, bcol, bval, colsum);
}

void launch_colsum_recip(int64_t n, const double* colsum, float* inv, hipStream_t s) {
  if (n <= 0) return;
  hipLaunchKernelGGL(k_colsum_recip, dim3((unsigned)((n + kNT - 1) / kNT)), dim3(kNT), 0, s, n,
                     colsum, inv);
}

void launch_prune_fill(int64_t m, const void* rp, int rp64, const int32_t* col, const void* val,
                       bool f64, double thr, const int64_t* outOff, const double* colsum,
                       const float* inv, int32_t* ocol, void* oval, hipStream_t s) {
  if (m <= 0) return;
  const dim3 g(grid_rows(m)), b(kNT);
  if (f64) {
    if (rp64)
      hipLaunchKernelGGL((k_prune_fill<double, int64_t, double>), g, b, 0, s, m, rp, col,
                         (const double*)val, thr, outOff, colsum, ocol, (double*)oval);
    else
      hipLaunchKernelGGL((k_prune_fill<double, int32_t, double>), g, b, 0, s, m, rp, col,
                         (const double*)val, thr, outOff, colsum, ocol, (double*)oval);
  } else {
    if (rp64)
      hipLaunchKernelGGL((k_prune_fill<float, int64_t, float>), g, b, 0, s, m, rp, col,
                         (const float*)val, (float)thr, outOff, inv, ocol, (float*)oval);
    else
      hipLaunchKernelGGL((k_prune_fill<float, int32_t, float>), g, b, 0, s, m, rp, col,
                         (const float*)val, (float)thr, outOff, inv, ocol, (float*)oval);
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
