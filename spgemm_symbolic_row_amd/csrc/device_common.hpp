// Device-side helpers shared by the kernel translation units: wave64
// primitives, searches over sorted offset arrays, LDS hash insertion and the
// work-group scans used by the accumulators and the multisplit.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.hpp"

namespace sg {

// XCDs of an MI355X; work groups are dealt to them round-robin.
constexpr int kXcds = 8;

constexpr int kWave = 64;

// LDS of one work group on gfx950.
constexpr int kLdsPerGroup = 163840;

// Lets `kernel` take as much dynamic LDS as a work group's LDS leaves beside
// the kernel's static LDS, and leaves the thread's HIP error state clear.
inline void allow_max_dynamic_lds(const void* kernel) {
  hipFuncAttributes fa{};
  size_t st = 0;
  if (hipFuncGetAttributes(&fa, kernel) == hipSuccess) st = fa.sharedSizeBytes;
  (void)hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)(kLdsPerGroup - (int)st));
  (void)hipGetLastError();
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }
__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l ? (~0ull >> (64 - l)) : 0ull;
}
__device__ __forceinline__ int ffs64(uint64_t m) { return __ffsll((unsigned long long)m) - 1; }
__device__ __forceinline__ int last_set64(uint64_t m) { return 63 - __clzll((long long)m); }

template <typename T>
__device__ __forceinline__ T wave_incl_scan(T x) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    T t = __shfl_up(x, d);
    if (lane_id() >= d) x += t;
  }
  return x;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d);
  return x;
}

// Largest index j in [lo, hi) with a[j] <= key, for non-decreasing a with
// a[lo] <= key.  Executed by a whole wave (all lanes get the answer).  Each
// round samples 64 evenly spaced positions and narrows the range 64-fold.
template <typename T, typename K>
__device__ __forceinline__ int64_t wave_last_le(const T* __restrict__ a, int64_t lo,
                                                int64_t hi, K key) {
  while (hi - lo > kWave) {
    const int64_t span = hi - lo;
    const int64_t pos = lo + (span * lane_id()) / kWave;
    const uint64_t m = __ballot((int64_t)a[pos] <= (int64_t)key);
    const int last = last_set64(m);
    const int64_t nlo = lo + (span * last) / kWave;
    const int64_t nhi = (last == kWave - 1) ? hi : lo + (span * (last + 1)) / kWave;
    lo = nlo;
    hi = nhi;
  }
  const int64_t e = lo + lane_id();
  const uint64_t m = __ballot(e < hi && (int64_t)a[e] <= (int64_t)key);
  return lo + last_set64(m);
}

// Lanes (among `act`) holding the same key, compared on its low `nbits`
// bits: the wave64 equivalent of a match-any, built from one ballot per bit.
__device__ __forceinline__ uint64_t match_key(uint32_t key, int nbits, bool act) {
  uint64_t m = __ballot(act);
  for (int i = 0; i < nbits; ++i) {
    const bool bit = (key >> i) & 1u;
    const uint64_t b = __ballot(act && bit);
    m &= bit ? b : ~b;
  }
  return m;
}

// Slot of a column key in a table of T slots: multiplicative hash, then the
// high 32 bits of hash*T, which maps uniformly onto [0, T) for any T.
__device__ __forceinline__ uint32_t hash_slot(int32_t key, uint32_t T) {
  const uint32_t h = (uint32_t)key * 2654435761u;
  return (uint32_t)(((uint64_t)h * T) >> 32);
}

__device__ __forceinline__ int32_t lds_load_relaxed(int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ void flag_error(int32_t* err, int32_t bit) {
  atomicOr(err, bit);
}

// Insert `key` into an LDS key set with linear probing.  Returns true when
// the key was new.  A full table (never the case when T exceeds the number
// of distinct keys, which the binning guarantees) raises ERR_HASH_FULL.
__device__ __forceinline__ bool hset_insert(int32_t* keys, uint32_t T, int32_t key,
                                            int32_t* err) {
  uint32_t s = hash_slot(key, T);
  for (uint32_t probe = 0; probe < T; ++probe) {
    // One compare-and-swap per probe: it claims an empty slot and reports
    // the key already held by a taken one.
    const int32_t old = atomicCAS(&keys[s], kEmptyKey, key);
    if (old == kEmptyKey) return true;
    if (old == key) return false;
    s = (s + 1 == T) ? 0 : s + 1;
  }
  flag_error(err, kErrHashFull);
  return false;
}

// Add v to the value of `key` in an LDS (key, value) table, inserting the
// key on first use.
template <typename V>
__device__ __forceinline__ void hmap_add(int32_t* keys, V* vals, uint32_t T, int32_t key,
                                         V v, int32_t* err) {
  uint32_t s = hash_slot(key, T);
  for (uint32_t probe = 0; probe < T; ++probe) {
    const int32_t old = atomicCAS(&keys[s], kEmptyKey, key);
    if (old == kEmptyKey || old == key) {
      atomicAdd(&vals[s], v);
      return;
    }
    s = (s + 1 == T) ? 0 : s + 1;
  }
  flag_error(err, kErrHashFull);
}

// Exclusive scan of one value per thread across a work group of NT threads
// (NT a multiple of 64, at most 1024).  `wtot` is LDS scratch of NT/64
// entries.  Returns the exclusive prefix; *total receives the sum.  Must be
// called by every thread of the work group.
template <int NT, typename T>
__device__ __forceinline__ T block_excl_scan(T x, T* wtot, T* total) {
  constexpr int NW = NT / kWave;
  const int w = threadIdx.x / kWave;
  const T inc = wave_incl_scan(x);
  if (lane_id() == kWave - 1) wtot[w] = inc;
  __syncthreads();
  T before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const T t = wtot[i];
    if (i < w) before += t;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + inc - x;
}

}  // namespace sg
