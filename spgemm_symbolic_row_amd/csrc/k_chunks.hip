// Accumulation of the final chunks of the heavy rows (gMAGNUS page, §III-E),
// exploiting that a chunk's local columns lie in [0, width) with width a
// power of two no larger than a few tens of thousands:
//
//   symbolic: an LDS bitmap of `width` bits per chunk; each element sets its
//             column's bit (reading first, so repeats cost a read only); the
//             chunk's nnz is the bitmap's popcount.
//   numeric (light chunks): an LDS hash of (column, value) with LDS atomic
//             adds; a new key also sets its column's bit.  A prefix popcount
//             over the bitmap words then gives every occupied slot its rank
//             among the chunk's columns, i.e. its position in the sorted
//             output, so no sort is needed.
// Heavy W-wide chunks use the dense accumulator in k_heavy.hip.
#include "device_common.hpp"

namespace sg {
namespace {

template <int TPC, int CPB, typename C = int32_t>
__global__ __launch_bounds__(TPC* CPB) void k_sym_chunks_bitmap(const ChunkDesc* __restrict__ desc,
                                                                int64_t n, int32_t words,
                                                                ChunkList cl) {
  extern __shared__ __align__(16) uint32_t bmAll[];
  __shared__ int32_t gsum[CPB * (TPC / kWave)];
  const int g = threadIdx.x / TPC, t = threadIdx.x % TPC;
  uint32_t* bm = bmAll + g * words;
  for (int i = t; i < words; i += TPC) bm[i] = 0;
  __syncthreads();
  const int64_t ci = (int64_t)blockIdx.x * CPB + g;
  ChunkDesc d{};
  if (ci < n) {
    d = desc[ci];
    const int64_t off = d.off, end = off + d.cnt;
    const C* __restrict__ col = (const C*)(d.buf ? cl.col1 : cl.col0);
    constexpr int kB = 8;  // loads in flight per thread
    for (int64_t e0 = off + t; e0 < end; e0 += (int64_t)TPC * kB) {
      int32_t cc[kB];
#pragma unroll
      for (int k = 0; k < kB; ++k) {
        const int64_t e = e0 + (int64_t)k * TPC;
        cc[k] = e < end ? col[e] : -1;
      }
#pragma unroll
      for (int k = 0; k < kB; ++k) {
        const int32_t c = cc[k];
        if (c >= 0) {
          const uint32_t bit = 1u << (c & 31);
          if (!(bm[c >> 5] & bit)) atomicOr(&bm[c >> 5], bit);
        }
      }
    }
  }
  __syncthreads();
  int32_t mine = 0;
  for (int i = t; i < words; i += TPC) mine += __popc(bm[i]);
  mine = wave_sum(mine);
  if (lane_id() == 0) gsum[threadIdx.x / kWave] = mine;
  __syncthreads();
  if (t == 0 && ci < n) {
    int32_t tot = 0;
    for (int i = 0; i < TPC / kWave; ++i) tot += gsum[g * (TPC / kWave) + i];
    cl.slotNnz[d.base] = tot;
  }
}

// Symbolic of the dense chunks: one persistent 1024-thread work group per
// half CU walks its chunks, and the first batch of the next chunk's columns
// (and its descriptor) is in flight while the current marks are counted and
// cleared.  A column is marked by a plain LDS byte store (no read, no atomic:
// every writer stores the same 1), and the chunk's nnz is the number of
// marked bytes.
constexpr int kSymPT = 1024;
constexpr int kSymB = 8;  // columns per thread per batch
template <typename C>
__global__ __launch_bounds__(kSymPT) void k_sym_chunks_persist(const ChunkDesc* __restrict__ desc,
                                                               int64_t n, int32_t width,
                                                               ChunkList cl) {
  // width: the dense chunks' width, a multiple of 16; marks[width] bytes.
  extern __shared__ __align__(16) uint4 mk4[];
  unsigned char* mk = (unsigned char*)mk4;
  __shared__ int32_t gsum[kSymPT / kWave];
  const int nv = width / 16;
  for (int i = threadIdx.x; i < nv; i += kSymPT) mk4[i] = uint4{0, 0, 0, 0};
  int64_t ci = blockIdx.x;
  ChunkDesc d{};
  int32_t cc[kSymB];
  const C* col = (const C*)cl.col0;
  auto load = [&](int64_t e0, int64_t end) {
#pragma unroll
    for (int k = 0; k < kSymB; ++k) {
      const int64_t e = e0 + (int64_t)k * kSymPT;
      cc[k] = e < end ? (int32_t)col[e] : -1;
    }
  };
  auto mark = [&]() {
#pragma unroll
    for (int k = 0; k < kSymB; ++k) {
      const int32_t c = cc[k];
      if ((uint32_t)c < (uint32_t)width) mk[c] = 1;
    }
  };
  if (ci < n) {
    d = desc[ci];
    col = (const C*)(d.buf ? cl.col1 : cl.col0);
    load(d.off + threadIdx.x, d.off + d.cnt);
  }
  __syncthreads();
  while (ci < n) {
    const int64_t off = d.off, end = off + d.cnt, slot = d.base;
    const int64_t cn = ci + gridDim.x;
    if (cn < n) d = desc[cn];
    mark();
    for (int64_t e0 = off + threadIdx.x + (int64_t)kSymPT * kSymB; e0 < end;
         e0 += (int64_t)kSymPT * kSymB) {
      load(e0, end);
      mark();
    }
    __syncthreads();
    if (cn < n) {
      col = (const C*)(d.buf ? cl.col1 : cl.col0);
      load(d.off + threadIdx.x, d.off + d.cnt);
    }
    // Marks are 0 or 1, so the popcount of the bytes counts them.
    int32_t mine = 0;
    for (int i = threadIdx.x; i < nv; i += kSymPT) {
      const uint4 x = mk4[i];
      mine += __popc(x.x) + __popc(x.y) + __popc(x.z) + __popc(x.w);
      mk4[i] = uint4{0, 0, 0, 0};
    }
    mine = wave_sum(mine);
    if (lane_id() == 0) gsum[threadIdx.x / kWave] = mine;
    __syncthreads();
    if (threadIdx.x == 0) {
      int32_t tot = 0;
      for (int i = 0; i < kSymPT / kWave; ++i) tot += gsum[i];
      cl.slotNnz[slot] = tot;
    }
    ci = cn;
  }
}

template <typename V>
__device__ __forceinline__ void hmap_add_mark(int32_t* keys, V* vals, uint32_t* bm, uint32_t T,
                                              int32_t key, V v, int32_t* err) {
  uint32_t s = hash_slot(key, T);
  for (uint32_t probe = 0; probe < T; ++probe) {
    const int32_t cur = lds_load_relaxed(&keys[s]);
    if (cur == key) {
      atomicAdd(&vals[s], v);
      return;
    }
    if (cur == kEmptyKey) {
      const int32_t old = atomicCAS(&keys[s], kEmptyKey, key);
      if (old == kEmptyKey) atomicOr(&bm[key >> 5], 1u << (key & 31));
      if (old == kEmptyKey || old == key) {
        atomicAdd(&vals[s], v);
        return;
      }
    }
    s = (s + 1 == T) ? 0 : s + 1;
  }
  flag_error(err, kErrHashFull);
}

// LDS per chunk group: vals[T], keys[T], bitmap[words], word prefix[words].
template <typename V>
__host__ __device__ constexpr size_t rank_group_bytes(int32_t T, int32_t words) {
  return (size_t)T * sizeof(V) + (size_t)T * 4 + (size_t)words * 8;
}

template <int TPC, int CPB, typename V, typename C = int32_t>
__global__ __launch_bounds__(TPC* CPB) void k_num_chunks_rank(const ChunkDesc* __restrict__ desc,
                                                              int64_t n, int32_t T, int32_t words,
                                                              ChunkList cl,
                                                              int32_t* __restrict__ ccol,
                                                              V* __restrict__ cval,
                                                              int32_t* __restrict__ err) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int WPG = TPC / kWave;
  __shared__ int32_t wtot[CPB * WPG];
  const int g = threadIdx.x / TPC, t = threadIdx.x % TPC, w = t / kWave;
  unsigned char* base = smem + (size_t)g * rank_group_bytes<V>(T, words);
  V* vals = (V*)base;
  int32_t* keys = (int32_t*)(vals + T);
  uint32_t* bm = (uint32_t*)(keys + T);
  int32_t* wpre = (int32_t*)(bm + words);
  for (int s = t; s < T; s += TPC) {
    keys[s] = kEmptyKey;
    vals[s] = V(0);
  }
  for (int i = t; i < words; i += TPC) bm[i] = 0;
  __syncthreads();
  const int64_t ci = (int64_t)blockIdx.x * CPB + g;
  ChunkDesc d{};
  if (ci < n) {
    d = desc[ci];
    const int64_t off = d.off, end = off + d.cnt;
    const bool b1 = d.buf != 0;
    const C* __restrict__ col = (const C*)(b1 ? cl.col1 : cl.col0);
    const V* __restrict__ val = (const V*)(b1 ? cl.val1 : cl.val0);
    constexpr int kB = 4;  // loads in flight per thread
    for (int64_t e0 = off + t; e0 < end; e0 += (int64_t)TPC * kB) {
      int32_t cc[kB];
      V vv[kB];
#pragma unroll
      for (int k = 0; k < kB; ++k) {
        const int64_t e = e0 + (int64_t)k * TPC;
        cc[k] = e < end ? col[e] : -1;
        vv[k] = e < end ? val[e] : V(0);
      }
#pragma unroll
      for (int k = 0; k < kB; ++k)
        if (cc[k] >= 0) hmap_add_mark(keys, vals, bm, (uint32_t)T, cc[k], vv[k], err);
    }
  }
  __syncthreads();
  // Exclusive prefix of the word popcounts: each thread owns a contiguous
  // run of words.
  const int wpt = (words + TPC - 1) / TPC;
  const int w0 = t * wpt;
  int32_t mine = 0;
  for (int i = 0; i < wpt; ++i)
    if (w0 + i < words) mine += __popc(bm[w0 + i]);
  const int32_t inc = wave_incl_scan(mine);
  if (lane_id() == kWave - 1) wtot[threadIdx.x / kWave] = inc;
  __syncthreads();
  int32_t before = 0, total = 0;
#pragma unroll
  for (int i = 0; i < WPG; ++i) {
    const int32_t tv = wtot[g * WPG + i];
    if (i < w) before += tv;
    total += tv;
  }
  int32_t run = before + inc - mine;
  for (int i = 0; i < wpt; ++i) {
    if (w0 + i < words) {
      wpre[w0 + i] = run;
      run += __popc(bm[w0 + i]);
    }
  }
  __syncthreads();
  if (ci < n) {
    const int64_t obase = d.base;
    const int32_t want = d.want;
    if (t == 0 && want != total) flag_error(err, kErrCountMismatch);
    const int32_t colBase = d.colBase;
    for (int s = t; s < T; s += TPC) {
      const int32_t k = keys[s];
      if (k != kEmptyKey) {
        const int32_t r = wpre[k >> 5] + __popc(bm[k >> 5] & ((1u << (k & 31)) - 1u));
        if (r < want) {
          ccol[obase + r] = colBase + k;
          cval[obase + r] = vals[s];
        }
      }
    }
  }
}

// Light chunks with their elements held in registers (at most TPC * KB per
// chunk): the columns set bits of a chunk-width bitmap, the word prefix of
// its popcounts gives every column its rank among the chunk's distinct
// columns, and each element adds its value straight into slot rank of a
// dense LDS array of the chunk's exact output size.  Ranks follow column
// order, so the output is written sorted and coalesced, with no hash table
// and no probing.
__host__ __device__ constexpr size_t direct_group_bytes(int32_t cap, int32_t words, int vb) {
  return ((size_t)cap * vb + (size_t)words * 8 + (size_t)cap * 2 + 15) / 16 * 16;
}

template <int TPC, int CPB, int KB, typename V, typename C = int32_t>
__global__ __launch_bounds__(TPC* CPB) void k_num_chunks_direct(const ChunkDesc* __restrict__ desc,
                                                                int64_t n, int32_t cap,
                                                                int32_t words, ChunkList cl,
                                                                int32_t* __restrict__ ccol,
                                                                V* __restrict__ cval,
                                                                int32_t* __restrict__ err) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int WPG = TPC / kWave;
  __shared__ int32_t wtot[CPB * WPG];
  const int g = threadIdx.x / TPC, t = threadIdx.x % TPC, w = t / kWave;
  unsigned char* base = smem + (size_t)g * direct_group_bytes(cap, words, (int)sizeof(V));
  V* vals = (V*)base;
  uint32_t* bm = (uint32_t*)(vals + cap);
  int32_t* wpre = (int32_t*)(bm + words);
  uint16_t* cols = (uint16_t*)(wpre + words);
  const int64_t ci = (int64_t)blockIdx.x * CPB + g;
  ChunkDesc d{};
  int32_t cc[KB];
  V vv[KB];
  if (ci < n) d = desc[ci];
  {
    const int64_t end = d.off + d.cnt;
    const bool b1 = d.buf != 0;
    const C* __restrict__ col = (const C*)(b1 ? cl.col1 : cl.col0);
    const V* __restrict__ val = (const V*)(b1 ? cl.val1 : cl.val0);
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int64_t e = d.off + t + (int64_t)k * TPC;
      cc[k] = e < end ? col[e] : -1;
      vv[k] = e < end ? val[e] : V(0);
    }
  }
  if (t == 0 && d.cnt > (int64_t)TPC * KB) flag_error(err, kErrHashFull);
  const int32_t want = d.want < cap ? d.want : cap;
  for (int i = t; i < words; i += TPC) bm[i] = 0;
  for (int i = t; i < want; i += TPC) vals[i] = V(0);
  __syncthreads();
#pragma unroll
  for (int k = 0; k < KB; ++k)
    if (cc[k] >= 0) atomicOr(&bm[cc[k] >> 5], 1u << (cc[k] & 31));
  __syncthreads();
  // Exclusive prefix of the word popcounts: each thread owns a contiguous
  // run of words.
  const int wpt = (words + TPC - 1) / TPC;
  const int w0 = t * wpt;
  int32_t mine = 0;
  for (int i = 0; i < wpt; ++i)
    if (w0 + i < words) mine += __popc(bm[w0 + i]);
  const int32_t inc = wave_incl_scan(mine);
  if (lane_id() == kWave - 1) wtot[threadIdx.x / kWave] = inc;
  __syncthreads();
  int32_t before = 0, total = 0;
#pragma unroll
  for (int i = 0; i < WPG; ++i) {
    const int32_t tv = wtot[g * WPG + i];
    if (i < w) before += tv;
    total += tv;
  }
  int32_t run = before + inc - mine;
  for (int i = 0; i < wpt; ++i) {
    if (w0 + i < words) {
      wpre[w0 + i] = run;
      run += __popc(bm[w0 + i]);
    }
  }
  __syncthreads();
  if (ci < n && t == 0 && total != d.want) flag_error(err, kErrCountMismatch);
#pragma unroll
  for (int k = 0; k < KB; ++k) {
    const int32_t c = cc[k];
    if (c >= 0) {
      const int32_t r = wpre[c >> 5] + __popc(bm[c >> 5] & ((1u << (c & 31)) - 1u));
      if (r < want) {
        atomicAdd(&vals[r], vv[k]);
        cols[r] = (uint16_t)c;
      }
    }
  }
  __syncthreads();
  if (ci < n) {
    const int64_t obase = d.base;
    const int32_t colBase = d.colBase;
    for (int r = t; r < want; r += TPC) {
      ccol[obase + r] = colBase + cols[r];
      cval[obase + r] = vals[r];
    }
  }
}

}  // namespace

void chunks_set_attributes() {
#define SG_ATTR(K) allow_max_dynamic_lds((const void*)(K))
  SG_ATTR((k_sym_chunks_bitmap<64, 4>));
  SG_ATTR((k_sym_chunks_bitmap<256, 1>));
  SG_ATTR((k_sym_chunks_bitmap<1024, 1>));
  SG_ATTR((k_sym_chunks_bitmap<64, 4, uint16_t>));
  SG_ATTR((k_sym_chunks_bitmap<256, 1, uint16_t>));
  SG_ATTR((k_sym_chunks_bitmap<1024, 1, uint16_t>));
  SG_ATTR(k_sym_chunks_persist<int32_t>);
  SG_ATTR(k_sym_chunks_persist<uint16_t>);
  SG_ATTR((k_num_chunks_rank<64, 4, float>));
  SG_ATTR((k_num_chunks_rank<64, 4, float, uint16_t>));
  SG_ATTR((k_num_chunks_rank<128, 2, float>));
  SG_ATTR((k_num_chunks_rank<128, 2, float, uint16_t>));
  SG_ATTR((k_num_chunks_rank<256, 1, float>));
  SG_ATTR((k_num_chunks_rank<256, 1, float, uint16_t>));
  SG_ATTR((k_num_chunks_rank<512, 1, float>));
  SG_ATTR((k_num_chunks_rank<512, 1, float, uint16_t>));
  SG_ATTR((k_num_chunks_rank<1024, 1, float>));
  SG_ATTR((k_num_chunks_rank<1024, 1, float, uint16_t>));
  SG_ATTR((k_num_chunks_rank<64, 4, double>));
  SG_ATTR((k_num_chunks_rank<64, 4, double, uint16_t>));
  SG_ATTR((k_num_chunks_rank<128, 2, double>));
  SG_ATTR((k_num_chunks_rank<128, 2, double, uint16_t>));
  SG_ATTR((k_num_chunks_rank<256, 1, double>));
  SG_ATTR((k_num_chunks_rank<256, 1, double, uint16_t>));
  SG_ATTR((k_num_chunks_rank<512, 1, double>));
  SG_ATTR((k_num_chunks_rank<512, 1, double, uint16_t>));
  SG_ATTR((k_num_chunks_rank<1024, 1, double>));
  SG_ATTR((k_num_chunks_rank<1024, 1, double, uint16_t>));
#define SG_DIR(V) \
  SG_ATTR((k_num_chunks_direct<64, 4, 1, V>));  \
  SG_ATTR((k_num_chunks_direct<64, 4, 2, V>));  \
  SG_ATTR((k_num_chunks_direct<64, 4, 4, V>));  \
  SG_ATTR((k_num_chunks_direct<128, 2, 4, V>)); \
  SG_ATTR((k_num_chunks_direct<256, 1, 4, V>)); \
  SG_ATTR((k_num_chunks_direct<256, 1, 8, V>)); \
  SG_ATTR((k_num_chunks_direct<512, 1, 4, V>)); \
  SG_ATTR((k_num_chunks_direct<512, 1, 8, V>)); \
  SG_ATTR((k_num_chunks_direct<512, 1, 16, V>)); \
  SG_ATTR((k_num_chunks_direct<1024, 1, 4, V>)); \
  SG_ATTR((k_num_chunks_direct<1024, 1, 8, V>)); \
  SG_ATTR((k_num_chunks_direct<1024, 1, 16, V>))
  SG_DIR(float);
  SG_DIR(double);
#undef SG_DIR
#define SG_DIR(V) \
  SG_ATTR((k_num_chunks_direct<64, 4, 1, V, uint16_t>));  \
  SG_ATTR((k_num_chunks_direct<64, 4, 2, V, uint16_t>));  \
  SG_ATTR((k_num_chunks_direct<64, 4, 4, V, uint16_t>));  \
  SG_ATTR((k_num_chunks_direct<128, 2, 4, V, uint16_t>)); \
  SG_ATTR((k_num_chunks_direct<256, 1, 4, V, uint16_t>)); \
  SG_ATTR((k_num_chunks_direct<256, 1, 8, V, uint16_t>)); \
  SG_ATTR((k_num_chunks_direct<512, 1, 4, V, uint16_t>)); \
  SG_ATTR((k_num_chunks_direct<512, 1, 8, V, uint16_t>)); \
  SG_ATTR((k_num_chunks_direct<512, 1, 16, V, uint16_t>)); \
  SG_ATTR((k_num_chunks_direct<1024, 1, 4, V, uint16_t>)); \
  SG_ATTR((k_num_chunks_direct<1024, 1, 8, V, uint16_t>)); \
  SG_ATTR((k_num_chunks_direct<1024, 1, 16, V, uint16_t>))
  SG_DIR(float);
  SG_DIR(double);
#undef SG_DIR
#undef SG_ATTR
}

size_t direct_chunk_lds(bool f64, int32_t cap, int32_t words, int rpb) {
  return (size_t)rpb * direct_group_bytes(cap, words, f64 ? 8 : 4);
}

bool launch_num_chunks_direct(const BinCfg& b, bool f64, const ChunkDesc* desc, int64_t n,
                              int32_t words, size_t ldsMax, const ChunkList& cl, int32_t* ccol,
                              void* cval, int32_t* err, hipStream_t s) {
  const int kb = (int)((b.cap + b.tpr - 1) / b.tpr);
  const size_t lds = direct_chunk_lds(f64, b.cap, words, b.rpb);
  if (kb > 16 || (b.tpr < 1024 && b.tpr * 4 < b.cap) || lds > ldsMax) return false;
  if (n <= 0) return true;
  // Grid and LDS follow the instance's chunks per block (CPB), which may
  // differ from the bin's rows per block; an instance whose LDS would not
  // fit is not launched.
#define L1(TPC, CPB, KB, V, C)                                                                 \
  do {                                                                                         \
    const size_t ldsI = direct_chunk_lds(f64, b.cap, words, CPB);                              \
    if (ldsI > ldsMax || (int64_t)(TPC) * (KB) < b.cap) return false;                          \
    hipLaunchKernelGGL((k_num_chunks_direct<TPC, CPB, KB, V, C>),                              \
                       dim3((unsigned)((n + (CPB) - 1) / (CPB))), dim3((TPC) * (CPB)), ldsI, s, \
                       desc, n, b.cap, words, cl, ccol, (V*)cval, err);                         \
  } while (0)
#define L(TPC, CPB, KB)                                                                        \
  do {                                                                                         \
    if (f64 && cl.col16) L1(TPC, CPB, KB, double, uint16_t);                                   \
    else if (f64) L1(TPC, CPB, KB, double, int32_t);                                           \
    else if (cl.col16) L1(TPC, CPB, KB, float, uint16_t);                                      \
    else L1(TPC, CPB, KB, float, int32_t);                                                     \
  } while (0)
  switch (b.tpr) {
    case 64:
      if (kb <= 1) L(64, 4, 1);
      else if (kb <= 2) L(64, 4, 2);
      else L(64, 4, 4);
      break;
    case 128: L(128, 2, 4); break;
    case 256: L(256, 1, 4); break;
    case 512: L(256, 1, 8); break;
    default: {
      // 512 threads with more elements each: more chunks in flight per CU.
      const int kb2 = (int)((b.cap + 511) / 512);
      if (kb2 <= 8) L(512, 1, 8);
      else if (kb2 <= 16) L(512, 1, 16);
      else L(1024, 1, 16);
      break;
    }
  }
#undef L
#undef L1
  return true;
}

size_t rank_chunk_lds(bool f64, int32_t T, int32_t words, int rpb) {
  return (size_t)rpb * (f64 ? rank_group_bytes<double>(T, words) : rank_group_bytes<float>(T, words));
}

void launch_sym_chunks_bitmap(int sizeClass, const ChunkDesc* desc, int64_t n, int32_t words,
                              const ChunkList& cl, hipStream_t s) {
  if (n <= 0) return;
#define L(TPC, CPB, G, LDS)                                                                     \
  do {                                                                                          \
    if (cl.col16)                                                                               \
      hipLaunchKernelGGL((k_sym_chunks_bitmap<TPC, CPB, uint16_t>), dim3(G), dim3(TPC * CPB),   \
                         LDS, s, desc, n, words, cl);                                           \
    else                                                                                        \
      hipLaunchKernelGGL((k_sym_chunks_bitmap<TPC, CPB, int32_t>), dim3(G), dim3(TPC * CPB),    \
                         LDS, s, desc, n, words, cl);                                           \
  } while (0)
  if (sizeClass == 0)
    L(64, 4, (unsigned)((n + 3) / 4), (size_t)4 * words * 4);
  else if (sizeClass == 1)
    L(256, 1, (unsigned)n, (size_t)words * 4);
  else
    L(1024, 1, (unsigned)n, (size_t)words * 4);
#undef L
}

void launch_sym_chunks_persist(const ChunkDesc* desc, int64_t n, const ChunkList& cl,
                               int numCUs, hipStream_t s) {
  if (n <= 0) return;
  // Two 1024-thread work groups fill a CU's waves.
  const unsigned g = (unsigned)std::min<int64_t>(n, (int64_t)std::max(numCUs, 1) * 2);
  const int32_t width = (int32_t)((cl.W + 15) / 16 * 16);
  const size_t lds = (size_t)width;
  if (cl.col16)
    hipLaunchKernelGGL(k_sym_chunks_persist<uint16_t>, dim3(g), dim3(kSymPT), lds, s, desc, n,
                       width, cl);
  else
    hipLaunchKernelGGL(k_sym_chunks_persist<int32_t>, dim3(g), dim3(kSymPT), lds, s, desc, n,
                       width, cl);
}

void launch_num_chunks_rank(const BinCfg& b, bool f64, const ChunkDesc* desc, int64_t n,
                            int32_t words, const ChunkList& cl, int32_t* ccol, void* cval,
                            int32_t* err, hipStream_t s) {
  if (n <= 0) return;
  const unsigned grid = (unsigned)((n + b.rpb - 1) / b.rpb);
  const size_t lds = rank_chunk_lds(f64, b.T, words, b.rpb);
#define L1(TPC, CPB, V, C)                                                                     \
  hipLaunchKernelGGL((k_num_chunks_rank<TPC, CPB, V, C>), dim3(grid), dim3(TPC * CPB), lds, s,  \
                     desc, n, b.T, words, cl, ccol, (V*)cval, err)
#define L(TPC, CPB)                                                                            \
  do {                                                                                         \
    if (f64 && cl.col16) L1(TPC, CPB, double, uint16_t);                                       \
    else if (f64) L1(TPC, CPB, double, int32_t);                                               \
    else if (cl.col16) L1(TPC, CPB, float, uint16_t);                                          \
    else L1(TPC, CPB, float, int32_t);                                                         \
  } while (0)
  switch (b.tpr) {
    case 64: L(64, 4); break;
    case 128: L(128, 2); break;
    case 256: L(256, 1); break;
    case 512: L(512, 1); break;
    default: L(1024, 1); break;
  }
#undef L
#undef L1
}

}  // namespace sg
