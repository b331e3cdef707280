// Host orchestration of the C ABI (include/spgemm.h): the gMAGNUS end-to-end
// schedule (gMAGNUS page, §III-A, Algorithm 3) on one GPU.
//
//   plan      setup phase: validation, parameters (§III-D), intermediate
//             products per row (InterOffsets), light/heavy split and size
//             bins; one host sync to learn the bin sizes.
//   symbolic  light rows: LDS hash symbolic per bin (light stream);
//             heavy rows: masked CSR->CSC, outer product, multisplit levels,
//             chunk symbolic (heavy stream); then C.rowPtr by a scan and one
//             sync for nnz(C).
//   numeric   light rows and heavy chunks accumulated in LDS, written sorted.
//
// Light and heavy work run on two internal streams forked from, and joined
// back into, the caller's stream with events.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/spgemm.h"
#include "internal.hpp"

using namespace sg;

namespace {

struct Error {
  spgemm_status st;
  std::string msg;
};

thread_local std::string g_thread_error;

#define HIP_CHECK(expr)                                                            \
  do {                                                                             \
    hipError_t e_ = (expr);                                                        \
    if (e_ != hipSuccess)                                                          \
      throw Error{SPGEMM_ERR_HIP, std::string(#expr) + ": " + hipGetErrorString(e_)}; \
  } while (0)

inline void check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) throw Error{SPGEMM_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e)};
}

int64_t next_pow2(int64_t x) {
  int64_t p = 1;
  while (p < x) p *= 2;
  return p;
}
int log2_exact(int64_t x) {
  int l = 0;
  while ((int64_t(1) << l) < x) ++l;
  return l;
}
double now_ms() {
  return std::chrono::duration<double, std::milli>(
             std::chrono::steady_clock::now().time_since_epoch())
      .count();
}

int tpr_for(int64_t cap) {
  if (cap <= 256) return 64;
  if (cap <= 512) return 128;
  if (cap <= 1024) return 256;
  if (cap <= 2048) return 512;
  return 1024;
}

// Size classes of the LDS hash accumulators: caps 32, 64, ... below tau, then
// tau itself.  Symbolic tables hold keys only (4 bytes a slot); numeric
// tables hold (key, value) pairs and must also fit the sort of
// next_pow2(cap) entries.  Both lists share their caps, so a bin index found
// from an element count is valid in either.
void make_bins(int64_t tau, int64_t lds, int val_bytes, std::vector<BinCfg>* sym,
               std::vector<BinCfg>* num) {
  std::vector<int64_t> caps;
  for (int64_t c = 32; c < tau; c *= 2) caps.push_back(c);
  caps.push_back(tau);
  for (int64_t cap : caps) {
    const int tpr = tpr_for(cap);
    const int rpb = tpr >= 256 ? 1 : 256 / tpr;
    BinCfg s{};
    s.cap = (int32_t)cap;
    s.tpr = tpr;
    s.rpb = rpb;
    s.T = (int32_t)std::max<int64_t>(next_pow2(2 * cap), tpr);
    s.spt = s.T / tpr;
    s.N = (int32_t)next_pow2(cap);
    s.lds = (size_t)rpb * s.T * 4 + rpb * 4;
    if ((int64_t)s.lds > lds)
      throw Error{SPGEMM_ERR_INVALID_ARG, "symbolic hash table does not fit the LDS budget"};
    sym->push_back(s);

    BinCfg n = s;
    const int slot = 4 + val_bytes;
    const int64_t N = next_pow2(cap);
    int64_t T = std::max<int64_t>(next_pow2(2 * cap), tpr);
    const int64_t extra = (int64_t)(tpr * rpb / 64) * 4 + (int64_t)rpb * 4 +
                          (int64_t)num_rows_radix_bytes(tpr, rpb);
    while (T > tpr && (int64_t)rpb * T * slot + extra > lds) T -= tpr;
    if (T < N || T <= cap || T / tpr > 24)
      throw Error{SPGEMM_ERR_INVALID_ARG, "numeric hash table does not fit the LDS budget"};
    n.T = (int32_t)T;
    n.spt = (int32_t)(T / tpr);
    n.N = (int32_t)N;
    n.lds = (size_t)rpb * T * slot + extra;
    if (!num_bin_supported(n))
      throw Error{SPGEMM_ERR_INVALID_ARG, "no numeric kernel for this bin size"};
    num->push_back(n);
  }
}

// Light-chunk numeric bins for the bitmap-rank accumulator: the same caps
// as make_bins, tables sized to leave room for the chunk-width bitmap and
// its word prefix.
void make_rank_bins(int64_t lds, bool f64, int32_t words, const std::vector<BinCfg>& sym,
                    std::vector<BinCfg>* out) {
  for (const BinCfg& s : sym) {
    BinCfg b = s;
    int64_t T = std::max<int64_t>(next_pow2(2 * (int64_t)s.cap), s.tpr);
    while (T > s.cap + 1 && (int64_t)rank_chunk_lds(f64, (int32_t)T, words, s.rpb) > lds)
      T = T * 15 / 16;
    if ((int64_t)rank_chunk_lds(f64, (int32_t)T, words, s.rpb) > lds || T <= s.cap)
      throw Error{SPGEMM_ERR_INVALID_ARG, "chunk hash table does not fit the LDS budget"};
    b.T = (int32_t)T;
    b.lds = rank_chunk_lds(f64, b.T, words, s.rpb);
    out->push_back(b);
  }
}

// Side streams for the light and heavy work, one pair per device, created on
// first use and kept for the life of the process: workspace freed on a side
// stream is then reused by the next product's allocations on it.
struct SideStreams {
  hipStream_t sl = nullptr, sh = nullptr, sd = nullptr;
};
SideStreams side_streams(int device) {
  static SideStreams pool[64];
  SideStreams& ss = pool[device & 63];
  if (!ss.sl) {
    HIP_CHECK(hipStreamCreateWithFlags(&ss.sl, hipStreamNonBlocking));
    HIP_CHECK(hipStreamCreateWithFlags(&ss.sh, hipStreamNonBlocking));
    HIP_CHECK(hipStreamCreateWithFlags(&ss.sd, hipStreamNonBlocking));
  }
  return ss;
}

// Per-device workspace arena.  One plan at a time bump-allocates from a
// single device block that persists across products, so repeated products
// of similar size allocate nothing.  The block grows (between plans) to the
// largest workspace demand seen.  A plan that finds the arena busy, or runs
// out of it, falls back to stream-ordered allocation.  `done` is recorded on
// the last user's stream after all its streams joined; the next user's
// stream waits for it before touching the memory.
struct Arena {
  std::mutex mu;
  char* base = nullptr;
  size_t cap = 0;
  size_t highWater = 0;
  bool busy = false;
  hipEvent_t done = nullptr;
  bool doneValid = false;
};
Arena g_arena[64];

// Per-device region for the heavy intermediate (the outer-product and
// multisplit buffers): one block, sized to the largest batch seen and reused
// by every batch of every product, with the same one-user-at-a-time and
// `done` protocol as the arena.  Kept apart from the arena so that the
// intermediate, the largest allocation by far, is never split or cached in
// pieces that a later, larger batch cannot use.
struct Region {
  std::mutex mu;
  char* base = nullptr;
  size_t cap = 0;
  bool busy = false;
  hipEvent_t done = nullptr;
  bool doneValid = false;
};
Region g_region[64];

// Return the stream-ordered pool's cached memory to the device (after all
// queued work), so that a large block can be allocated in its place.
void trim_pool(int device) {
  hipMemPool_t pool;
  if (hipDeviceGetDefaultMemPool(&pool, device) == hipSuccess) {
    HIP_CHECK(hipDeviceSynchronize());
    (void)hipMemPoolTrimTo(pool, 0);
  }
  (void)hipGetLastError();
}

// Small pinned host buffers for readbacks, one set per host thread.
struct Pinned {
  int64_t* stats = nullptr;  // 32 entries
  int32_t* bins = nullptr;   // 128 entries
};
Pinned& pinned() {
  thread_local Pinned pb;
  if (!pb.stats) {
    HIP_CHECK(hipHostMalloc((void**)&pb.stats, sizeof(int64_t) * 32, hipHostMallocDefault));
    HIP_CHECK(hipHostMalloc((void**)&pb.bins, sizeof(int32_t) * 128, hipHostMallocDefault));
  }
  return pb;
}

// One batch of heavy rows after expansion: its intermediate buffers and
// final chunk list, ordered by numeric bin.
struct Batch {
  int64_t hb0 = 0, hb1 = 0, Pb = 0;
  int32_t* bufCol[2] = {nullptr, nullptr};
  void* bufVal[2] = {nullptr, nullptr};
  int64_t nfc = 0, lastFirst = 0, denseChunks = 0;
  int64_t* fcOff = nullptr;
  int32_t *fcCnt = nullptr, *fcRow = nullptr, *fcSlot = nullptr, *fcOrder = nullptr;
  int8_t* fcBuf = nullptr;
  int8_t* fcSpan = nullptr;  // log2 of the W-wide slots each chunk covers
  std::vector<int32_t> fcBinStart;
  int64_t levelElems[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  bool denseDirect = false;  // dense chunks taken straight from A and B
};

}  // namespace

struct spgemm_plan_s {
  // inputs
  int64_t m = 0, k = 0, n = 0, nnzA = 0, nnzB = 0;
  const int32_t *arp = nullptr, *acol = nullptr, *brp = nullptr, *bcol = nullptr;
  const void *aval = nullptr, *bval = nullptr;
  bool f64 = true;
  spgemm_options opts{};
  hipStream_t stream = nullptr, sl = nullptr, sh = nullptr;
  hipStream_t sd = nullptr;  // dense chunks, beside the light chunks on sh
  hipEvent_t evFork = nullptr, evL = nullptr, evH = nullptr, evD0 = nullptr, evD1 = nullptr;
  int device = 0;
  int64_t lds = 0, tau = 0, rowTau = 0;  // chunk and row heavy thresholds
  int numCUs = 0;
  spgemm_params params{};
  int state = 0;  // 0 planned, 1 symbolic done, 2 numeric done, -1 failed
  std::string err;
  std::vector<std::pair<void*, hipStream_t>> allocs;
  Arena* arena = nullptr;   // held from plan to destroy, or null
  Region* region = nullptr; // held from the first heavy batch to destroy, or null
  char* heavyBuf = nullptr; // the heavy intermediate buffers of the current batch
  size_t arenaUsed = 0, demand = 0;
  std::vector<BinCfg> symBins, numBins, rankBins;
  int32_t chunkWords = 0;  // bitmap words of the widest final chunk (0: hash fallback)
  int NS = 0;  // number of hash bins
  int winBins = 0;  // leading light bins whose rows may take the dense window
  int hybSymBin = 0;  // first symbolic bin of the hybrid kernel (NS: none)
  // device arrays
  int32_t *dSymCaps = nullptr;
  int32_t* dHybCap = nullptr;  // per numeric bin: outliers a hybrid row may have (-1: none)
  int32_t* outc = nullptr;     // outlier count of every row of a hybrid symbolic bin
  int64_t *rowP = nullptr, *cnt = nullptr, *stats = nullptr, *cRowOff = nullptr, *scanTmp = nullptr;
  int32_t *scanA = nullptr, *rowOrder = nullptr, *numOrder = nullptr, *errWord = nullptr;
  int64_t* rowWin = nullptr;  // dense-window rows: first column and span words
  int32_t* winMax = nullptr;  // widest window of each light bin, in words
  std::vector<int32_t> winWords;
  int32_t *binCnt = nullptr, *binFill = nullptr, *binStart = nullptr;
  uint8_t *rowBin = nullptr, *numKey = nullptr;
  // pinned host mirrors
  int64_t* hStats = nullptr;   // kNumStats + 8
  int32_t* hBins = nullptr;    // 128
  // host copies
  std::vector<int32_t> rowBinStart, numBinStart;
  // heavy path
  int64_t h = 0, Ph = 0, nAh = 0, nreq = 1;
  const int32_t* xheavy = nullptr;
  std::vector<int64_t> hChat, hAnnz;                   // scans over heavy rows
  std::vector<std::pair<int64_t, int64_t>> batches;   // heavy-row ranges of numeric
  bool symVals = true;   // symbolic expands values too (one batch, kept)
  Batch kept{};          // the expansion symbolic leaves for numeric (one batch)
  bool haveKept = false;
  ChunkDesc* keptDesc = nullptr;  // numeric's chunk descriptors for `kept`
  size_t wsCur = 0;      // workspace bytes currently held
  int32_t* CH = nullptr; // per heavy row, elements per W-wide chunk (or null)
  // Dense chunks accumulated straight from A and B (option dense_direct),
  // with B's slot table: (nreq + 1) run starts per B row.
  bool useDD = false;
  const int32_t* slotTab = nullptr;
  int64_t* dAnnz = nullptr; // scan of the heavy rows' A lengths (h + 1)
  bool fused = false;    // the first level is fed straight from A and B
  bool direct = false;   // one pass straight into the final chunks
  bool col16 = false;    // final chunk columns stored as uint16_t
  int32_t* slotNnz = nullptr;
  int64_t* slotOff = nullptr;
  int64_t nnzC = 0;
  // Size prediction of the light rows: 0 symbolic pass, 1 upper bound, 2
  // HyperLogLog estimate (Ocean page, §3, Table 1).  With 1 or 2 the light
  // rows are computed during spgemm_symbolic into reserved slots (tcol1,
  // tval1 at tmpOff; rows that did not fit again into tcol2, tval2) and
  // copied into C by spgemm_numeric.
  int wf = 0;
  int hllLg = 0;
  int64_t *capL = nullptr, *tmpOff = nullptr, *cnt1 = nullptr, *cnt2 = nullptr, *off2 = nullptr;
  double* estL = nullptr;
  int32_t *tcol1 = nullptr, *tcol2 = nullptr;
  void *tval1 = nullptr, *tval2 = nullptr;
  std::vector<double> hLc;
  spgemm_stats st{};
  struct PhaseRec {
    int id;
    hipEvent_t a, b;
  };
  std::vector<PhaseRec> phases;
};

namespace {

void* plan_alloc(spgemm_plan_t p, size_t bytes, hipStream_t s) {
  if (bytes == 0) bytes = 16;
  bytes = (bytes + 255) & ~size_t(255);
  p->wsCur += bytes;
  p->demand = std::max(p->demand, p->wsCur);
  if (p->arena && p->arenaUsed + bytes <= p->arena->cap) {
    void* ptr = p->arena->base + p->arenaUsed;
    p->arenaUsed += bytes;
    return ptr;
  }
  void* ptr = nullptr;
  if (p->opts.alloc) {
    ptr = p->opts.alloc(bytes, (void*)s, p->opts.alloc_ctx);
    // The callback reports failure by NULL; a HIP error state it may leave
    // behind in this thread is not the library's and must not be taken for
    // a failed launch.
    (void)hipGetLastError();
  } else if (hipMallocAsync(&ptr, bytes, s) != hipSuccess) {
    (void)hipGetLastError();
    ptr = nullptr;
  }
  if (!ptr)
    throw Error{SPGEMM_ERR_OOM, "device allocation of " + std::to_string(bytes) + " bytes failed"};
  p->allocs.push_back({ptr, s});
  return ptr;
}
template <typename T>
T* alloc_n(spgemm_plan_t p, int64_t n, hipStream_t s) {
  return (T*)plan_alloc(p, (size_t)std::max<int64_t>(n, 1) * sizeof(T), s);
}

// Frees every workspace buffer on the stream that allocated it.  Callers
// first make the caller's stream and both side streams wait for each other.
void release(spgemm_plan_t p) {
  for (auto& a : p->allocs) {
    if (p->opts.alloc) {
      if (p->opts.free) p->opts.free(a.first, (void*)a.second, p->opts.alloc_ctx);
      (void)hipGetLastError();  // not the library's error state
    } else {
      (void)hipFreeAsync(a.first, a.second);
    }
  }
  p->allocs.clear();
}

// Workspace marks: everything allocated after a mark is given back by
// ws_reset, in stream order on `s` (the only stream that used it), so the
// next batch reuses the same memory.
struct WsMark {
  size_t arenaUsed, wsCur, nAllocs;
};
WsMark ws_mark(spgemm_plan_t p) { return WsMark{p->arenaUsed, p->wsCur, p->allocs.size()}; }
void ws_reset(spgemm_plan_t p, const WsMark& mk, hipStream_t s) {
  for (size_t i = mk.nAllocs; i < p->allocs.size(); ++i) {
    auto& a = p->allocs[i];
    if (p->opts.alloc) {
      if (p->opts.free) p->opts.free(a.first, (void*)s, p->opts.alloc_ctx);
      (void)hipGetLastError();  // not the library's error state
    } else {
      HIP_CHECK(hipFreeAsync(a.first, s));
    }
  }
  p->allocs.resize(mk.nAllocs);
  p->arenaUsed = mk.arenaUsed;
  p->wsCur = mk.wsCur;
}

// Optional GPU timing of kernel phases: an event pair recorded on the
// stream the phase's kernels are launched on.
int ph_begin(spgemm_plan_t p, int id, hipStream_t s) {
  if (!p->opts.profile) return -1;
  spgemm_plan_s::PhaseRec r{id, nullptr, nullptr};
  HIP_CHECK(hipEventCreate(&r.a));
  HIP_CHECK(hipEventCreate(&r.b));
  p->phases.push_back(r);
  HIP_CHECK(hipEventRecord(r.a, s));
  return (int)p->phases.size() - 1;
}
void ph_end(spgemm_plan_t p, int idx, hipStream_t s) {
  if (idx < 0) return;
  HIP_CHECK(hipEventRecord(p->phases[idx].b, s));
}
void ph_collect(spgemm_plan_t p) {
  for (int i = 0; i < 16; ++i) {
    p->st.phase_ms[i] = 0;
    p->st.phase_windows[i] = 0;
    p->st.phase_min_ms[i] = 0;
  }
  for (auto& r : p->phases) {
    HIP_CHECK(hipEventSynchronize(r.b));
    float ms = 0;
    HIP_CHECK(hipEventElapsedTime(&ms, r.a, r.b));
    p->st.phase_ms[r.id] += ms;
    if (p->st.phase_windows[r.id] == 0 || ms < p->st.phase_min_ms[r.id])
      p->st.phase_min_ms[r.id] = ms;
    p->st.phase_windows[r.id] += 1;
  }
}

// Take the device's arena if it is free, growing it to the largest demand
// seen so far.  The plan's stream waits for the previous user to finish.
void arena_acquire(spgemm_plan_t p) {
  if (p->opts.alloc) return;
  Arena& a = g_arena[p->device & 63];
  std::lock_guard<std::mutex> lk(a.mu);
  if (a.busy) return;
  if (a.cap < a.highWater) {
    if (a.doneValid) HIP_CHECK(hipEventSynchronize(a.done));
    if (a.base) HIP_CHECK(hipFree(a.base));
    a.base = nullptr;
    a.cap = 0;
    trim_pool(p->device);
    if (hipMalloc((void**)&a.base, a.highWater) == hipSuccess) {
      a.cap = a.highWater;
    } else {
      (void)hipGetLastError();
      a.base = nullptr;
    }
  }
  if (!a.done) HIP_CHECK(hipEventCreateWithFlags(&a.done, hipEventDisableTiming));
  if (a.doneValid) HIP_CHECK(hipStreamWaitEvent(p->stream, a.done, 0));
  a.busy = true;
  p->arena = &a;
}

// Give the arena back: called after the plan's streams have joined into
// the caller's stream, so `done` covers all of the plan's work.
void arena_release(spgemm_plan_t p) {
  if (!p->arena) return;
  Arena& a = *p->arena;
  std::lock_guard<std::mutex> lk(a.mu);
  a.highWater = std::max(a.highWater, p->demand);
  if (hipEventRecord(a.done, p->stream) == hipSuccess) a.doneValid = true;
  a.busy = false;
  p->arena = nullptr;
}

// The heavy intermediate block of `bytes`: the device region if it is free
// (grown first if needed), else an ordinary workspace allocation.
char* heavy_region(spgemm_plan_t p, size_t bytes) {
  if (!p->opts.alloc) {
    Region& r = g_region[p->device & 63];
    std::lock_guard<std::mutex> lk(r.mu);
    if (!r.busy) {
      if (!r.done) HIP_CHECK(hipEventCreateWithFlags(&r.done, hipEventDisableTiming));
      if (r.cap < bytes) {
        if (r.doneValid) HIP_CHECK(hipEventSynchronize(r.done));
        if (r.base) HIP_CHECK(hipFree(r.base));
        r.base = nullptr;
        r.cap = 0;
        trim_pool(p->device);
        if (hipMalloc((void**)&r.base, bytes) == hipSuccess) {
          r.cap = bytes;
        } else {
          (void)hipGetLastError();
          r.base = nullptr;
        }
      }
      if (r.base) {
        if (r.doneValid) HIP_CHECK(hipStreamWaitEvent(p->sh, r.done, 0));
        r.busy = true;
        p->region = &r;
        return r.base;
      }
    }
  }
  return (char*)plan_alloc(p, bytes, p->sh);
}

// Bytes of the region the device would give this plan without growing.
size_t region_free(spgemm_plan_t p) {
  if (p->opts.alloc) return 0;
  Region& r = g_region[p->device & 63];
  std::lock_guard<std::mutex> lk(r.mu);
  return r.busy ? 0 : r.cap;
}

void region_release(spgemm_plan_t p) {
  if (!p->region) return;
  Region& r = *p->region;
  std::lock_guard<std::mutex> lk(r.mu);
  if (hipEventRecord(r.done, p->stream) == hipSuccess) r.doneValid = true;
  r.busy = false;
  p->region = nullptr;
}

void fork(spgemm_plan_t p) {
  if (p->sl == p->stream) return;
  HIP_CHECK(hipEventRecord(p->evFork, p->stream));
  HIP_CHECK(hipStreamWaitEvent(p->sl, p->evFork, 0));
  HIP_CHECK(hipStreamWaitEvent(p->sh, p->evFork, 0));
}
void join(spgemm_plan_t p) {
  if (p->sl == p->stream) return;
  HIP_CHECK(hipEventRecord(p->evL, p->sl));
  HIP_CHECK(hipEventRecord(p->evH, p->sh));
  HIP_CHECK(hipEventRecord(p->evD1, p->sd));
  HIP_CHECK(hipStreamWaitEvent(p->stream, p->evL, 0));
  HIP_CHECK(hipStreamWaitEvent(p->stream, p->evH, 0));
  HIP_CHECK(hipStreamWaitEvent(p->stream, p->evD1, 0));
}

void check_device_errors(spgemm_plan_t p, int32_t word) {
  if (word & kErrCsr) throw Error{SPGEMM_ERR_INVALID_CSR, "input is not canonical CSR"};
  if (word & kErrHashFull) throw Error{SPGEMM_ERR_INTERNAL, "an LDS hash table overflowed"};
  if (word & kErrRowsPerBlock)
    throw Error{SPGEMM_ERR_INTERNAL, "multisplit work group met more rows than sized for"};
  if (word & kErrCountMismatch)
    throw Error{SPGEMM_ERR_INTERNAL, "numeric and symbolic sizes disagree"};
  if (word) throw Error{SPGEMM_ERR_INTERNAL, "device status word " + std::to_string(word)};
  (void)p;
}

int32_t read_err(spgemm_plan_t p, hipStream_t s) {
  HIP_CHECK(hipMemcpyAsync(p->hBins + 120, p->errWord, 4, hipMemcpyDeviceToHost, s));
  HIP_CHECK(hipStreamSynchronize(s));
  return p->hBins[120];
}

RowArgs row_args(spgemm_plan_t p) {
  return RowArgs{p->arp, p->acol, p->aval, p->brp, p->bcol, p->bval, p->scanA, p->rowP, p->rowWin};
}

// Largest value held in an int32 index (options.index_limit lowers it for
// tests of the overflow checks).
int64_t index_limit(spgemm_plan_t p) {
  return p->opts.index_limit > 0 ? std::min<int64_t>(p->opts.index_limit, INT32_MAX) : INT32_MAX;
}

// ------------------------------------------------------------------ plan
void do_plan(spgemm_plan_t p) {
  const double t0 = now_ms();
  HIP_CHECK(hipGetDevice(&p->device));
  int ldsDev = 0;
  HIP_CHECK(hipDeviceGetAttribute(&ldsDev, hipDeviceAttributeMaxSharedMemoryPerBlock, p->device));
  HIP_CHECK(hipDeviceGetAttribute(&p->numCUs, hipDeviceAttributeMultiprocessorCount, p->device));
  p->lds = p->opts.lds_budget ? p->opts.lds_budget : ldsDev;
  if (p->lds > ldsDev || p->lds < 4096)
    throw Error{SPGEMM_ERR_INVALID_ARG, "lds_budget must lie in [4096, LDS per work group]"};
  const int vb = p->f64 ? 8 : 4;
  spgemm_status ps = spgemm_compute_params(p->n, p->lds, vb, 4, p->opts.max_chunks_per_level,
                                           p->opts.dense_width, &p->params);
  if (ps != SPGEMM_OK) throw Error{ps, "parameter selection failed"};
  p->tau = p->params.tau;
  if (p->opts.heavy_threshold) {
    if (p->opts.heavy_threshold < 1 || p->opts.heavy_threshold > p->params.tau)
      throw Error{SPGEMM_ERR_INVALID_ARG, "heavy_threshold must lie in [1, LDS-derived tau]"};
    p->tau = p->opts.heavy_threshold;
  }
  // Light rows up to tau / 3 products: a numeric table of 2 slots per product
  // then takes at most a third of the LDS, so three rows share a CU.  Larger
  // rows run faster through the heavy path (measured on gfx950).
  p->rowTau = p->opts.heavy_row_threshold ? p->opts.heavy_row_threshold
              : p->opts.heavy_threshold   ? p->tau
                                          : std::max<int64_t>(p->tau / 3, 1);
  if (p->rowTau < 1 || p->rowTau > p->tau)
    throw Error{SPGEMM_ERR_INVALID_ARG, "heavy_row_threshold must lie in [1, tau]"};
  if ((int64_t)dense_num_lds(p->f64, p->params.dense_width) > ldsDev ||
      p->params.dense_width > 32768)
    throw Error{SPGEMM_ERR_INVALID_ARG, "dense width does not fit the LDS"};
  if (p->opts.mem_budget < 0) throw Error{SPGEMM_ERR_INVALID_ARG, "mem_budget must be >= 0"};
  if (p->opts.index_limit < 0) throw Error{SPGEMM_ERR_INVALID_ARG, "index_limit must be >= 0"};
  if (p->opts.workflow < 0 || p->opts.workflow > 3)
    throw Error{SPGEMM_ERR_INVALID_ARG, "workflow must lie in [0, 3]"};
  if (p->opts.hll_registers != 0 && p->opts.hll_registers != 32 && p->opts.hll_registers != 64)
    throw Error{SPGEMM_ERR_INVALID_ARG, "hll_registers must be 0, 32 or 64"};
  if (p->opts.hll_coef_pct < 0) throw Error{SPGEMM_ERR_INVALID_ARG, "hll_coef_pct must be >= 0"};
  make_bins(p->tau, p->lds, vb, &p->symBins, &p->numBins);
  p->NS = (int)p->symBins.size();
  if (3 * p->NS + 2 > 60) throw Error{SPGEMM_ERR_INVALID_ARG, "too many bins"};
  // Dense windows for light rows unless turned off or a bin's window does
  // not fit the LDS budget.
  p->winBins = 0;
  if (!p->opts.light_hash_only)
    while (p->winBins < p->NS &&
           (int64_t)window_row_lds(true, p->f64, p->symBins[p->winBins],
                                   window_words(p->symBins[p->winBins].cap)) <= p->lds)
      ++p->winBins;

  static bool attrs = false;
  if (!attrs) {
    light_set_attributes();
    heavy_set_attributes();
    multisplit_set_attributes();
    chunks_set_attributes();
    attrs = true;
  }
  // Nothing before this point launched work of this plan: an error state
  // left in this thread by earlier, unrelated calls is not this plan's.
  (void)hipGetLastError();
  if (!p->opts.alloc) {
    // Keep freed workspace in the stream-ordered pool for the next product
    // instead of returning it to the driver at every synchronisation.
    static int poolDevice = -1;
    if (poolDevice != p->device) {
      hipMemPool_t pool;
      if (hipDeviceGetDefaultMemPool(&pool, p->device) == hipSuccess) {
        uint64_t thr = UINT64_MAX;
        (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &thr);
      }
      (void)hipGetLastError();
      poolDevice = p->device;
    }
  }

  if (p->opts.single_stream) {
    p->sl = p->sh = p->sd = p->stream;
  } else {
    const SideStreams ss = side_streams(p->device);
    p->sl = ss.sl;
    p->sh = ss.sh;
    p->sd = ss.sd;
    HIP_CHECK(hipEventCreateWithFlags(&p->evD0, hipEventDisableTiming));
    HIP_CHECK(hipEventCreateWithFlags(&p->evD1, hipEventDisableTiming));
    HIP_CHECK(hipEventCreateWithFlags(&p->evFork, hipEventDisableTiming));
    HIP_CHECK(hipEventCreateWithFlags(&p->evL, hipEventDisableTiming));
    HIP_CHECK(hipEventCreateWithFlags(&p->evH, hipEventDisableTiming));
  }
  p->hStats = pinned().stats;
  p->hBins = pinned().bins;
  arena_acquire(p);

  hipStream_t s = p->stream;
  const int64_t m = p->m;
  p->errWord = alloc_n<int32_t>(p, 4, s);
  p->stats = alloc_n<int64_t>(p, kNumStats, s);
  launch_fill_i32(p->errWord, 0, 4, s);
  launch_fill_i64(p->stats, 0, kNumStats, s);

  if (p->opts.validate) {
    launch_validate(p->m, p->k, p->nnzA, p->arp, p->acol, p->errWord, s);
    launch_validate(p->k, p->n, p->nnzB, p->brp, p->bcol, p->errWord, s);
    check_launch("validate");
    check_device_errors(p, read_err(p, s));
  }

  // Bin caps reach the device as kernel arguments (no copy to wait for).
  std::vector<int32_t> caps(p->NS);
  for (int b = 0; b < p->NS; ++b) caps[b] = p->symBins[b].cap;
  p->dSymCaps = alloc_n<int32_t>(p, 64, s);
  launch_set_small_i32(p->dSymCaps, caps.data(), p->NS, s);
  // Hybrid light rows (diagonal window plus outlier table) from the first
  // bin of at least kHybMinCap products, unless every light row is to take
  // the hash table.
  p->hybSymBin = p->NS;
  if (!p->opts.light_hash_only)
    for (int b = 0; b < p->NS; ++b)
      if (p->symBins[b].cap >= kHybMinCap) {
        p->hybSymBin = b;
        break;
      }
  std::vector<int32_t> hcap(p->NS, -1);
  for (int b = 0; b < p->NS; ++b) hcap[b] = hyb_out_cap(p->numBins[b], p->f64, p->lds);
  p->dHybCap = alloc_n<int32_t>(p, 64, s);
  launch_set_small_i32(p->dHybCap, hcap.data(), p->NS, s);

  p->rowP = alloc_n<int64_t>(p, m, s);
  p->cnt = alloc_n<int64_t>(p, m, s);
  p->scanA = alloc_n<int32_t>(p, p->nnzA, s);
  p->rowBin = alloc_n<uint8_t>(p, m, s);
  if (p->winBins) {
    p->rowWin = alloc_n<int64_t>(p, m, s);
    p->winMax = alloc_n<int32_t>(p, 64, s);
    launch_fill_i32(p->winMax, 0, 64, s);
  }
  p->rowOrder = alloc_n<int32_t>(p, m, s);
  p->binCnt = alloc_n<int32_t>(p, 64, s);
  p->binFill = alloc_n<int32_t>(p, 64, s);
  p->binStart = alloc_n<int32_t>(p, 65, s);
  launch_fill_i64(p->cnt, 0, m, s);
  const int ph = ph_begin(p, SPGEMM_PH_ROW_INFO, s);
  int64_t* part = alloc_n<int64_t>(p, row_info_partials(m, p->nnzA), s);
  int2* bSpan = nullptr;
  if (p->winBins) {
    bSpan = alloc_n<int2>(p, std::max<int64_t>(p->k, 1), s);
    launch_b_span(p->k, p->brp, p->bcol, bSpan, s);
  }
  launch_row_info(m, p->nnzA, p->arp, p->acol, p->brp, bSpan, p->rowTau, p->dSymCaps, p->NS, p->rowP,
                  p->scanA, p->rowBin, p->rowWin, p->winBins, p->winMax, part, p->stats, s);
  // 0 empty, 1..NS hash bins, NS+1 heavy, NS+2..2NS+1 dense-window bins
  const int nkeys = 2 * p->NS + 2;
  launch_bin_sort(p->rowBin, m, nkeys, p->binCnt, p->binFill, p->binStart, p->rowOrder, s);
  ph_end(p, ph, s);
  check_launch("plan kernels");
  HIP_CHECK(hipMemcpyAsync(p->hStats, p->stats, sizeof(int64_t) * kNumStats, hipMemcpyDeviceToHost, s));
  HIP_CHECK(hipMemcpyAsync(p->hBins, p->binStart, sizeof(int32_t) * (nkeys + 1), hipMemcpyDeviceToHost, s));
  if (p->winBins)
    HIP_CHECK(hipMemcpyAsync(p->hBins + 64, p->winMax, sizeof(int32_t) * p->NS,
                             hipMemcpyDeviceToHost, s));
  HIP_CHECK(hipStreamSynchronize(s));
  p->rowBinStart.assign(p->hBins, p->hBins + nkeys + 1);
  p->winWords.assign(p->NS, 0);
  if (p->winBins) std::copy(p->hBins + 64, p->hBins + 64 + p->NS, p->winWords.begin());
  p->st.products = p->hStats[kStatProducts];
  p->st.heavy_products = p->Ph = p->hStats[kStatHeavyProducts];
  p->st.heavy_a_nnz = p->nAh = p->hStats[kStatHeavyANnz];
  p->st.max_row_products = p->hStats[kStatMaxRowProducts];
  p->st.heavy_rows = p->h = p->hStats[kStatHeavyRows];
  p->st.light_rows = p->hStats[kStatLightRows];
  p->st.params = p->params;
  p->st.params.tau = p->tau;
  p->st.heavy_row_threshold = p->rowTau;
  p->st.chunk_col_bytes = 4;
  p->xheavy = p->rowOrder + p->rowBinStart[p->NS + 1];
  p->nreq = p->params.chunks_required;
  // Row-local product offsets (scanA) and chunk counts are int32.
  if (p->st.max_row_products > index_limit(p))
    throw Error{SPGEMM_ERR_INDEX_OVERFLOW,
                "a row has " + std::to_string(p->st.max_row_products) +
                    " intermediate products, beyond the 32-bit row-local product offsets"};
  p->st.ms_plan = now_ms() - t0;
}

// -------------------------------------------------------------- symbolic
// ---------------------------------------------------------------- heavy
// Heavy rows are processed in batches of consecutive heavy rows whose
// intermediate fits the memory budget.  With one batch the expansion made by
// symbolic is kept for numeric (gMAGNUS Alg. 3); with several, symbolic
// keeps only the chunk counts and numeric expands every batch again.

size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

// Intermediate buffers that hold `Pb` elements at once: one, or two for
// ping-pong between levels.  The outer product fills one that the first
// level reads; fed straight from A and B, one level needs only its output.
int heavy_nbuf(spgemm_plan_t p) {
  const int L = p->params.levels;
  if (L == 0 || p->direct) return 1;
  return (p->fused && L == 1) ? 1 : 2;
}
size_t heavy_buf_bytes(spgemm_plan_t p, int64_t Pb, bool vals) {
  const size_t n = (size_t)std::max<int64_t>(Pb, 1);
  const size_t pair = align256(n * (p->col16 ? 2 : 4)) + (vals ? align256(n * (p->f64 ? 8 : 4)) : 0);
  return heavy_nbuf(p) * pair;
}

// Consecutive heavy rows whose C-hat rows together hold at most `cap`
// elements (at least one row each); returns the largest batch's elements.
int64_t cut_batches(spgemm_plan_t p, int64_t cap, std::vector<std::pair<int64_t, int64_t>>* out) {
  out->clear();
  int64_t r0 = 0, maxPb = 0;
  while (r0 < p->h) {
    int64_t r1 = r0 + 1;
    while (r1 < p->h && p->hChat[r1 + 1] - p->hChat[r0] <= cap) ++r1;
    out->push_back({r0, r1});
    maxPb = std::max(maxPb, p->hChat[r1] - p->hChat[r0]);
    r0 = r1;
  }
  return maxPb;
}

// Per heavy row: products (C-hat row length) and nnz of its A row, both
// scanned, copied to the host; then the batch boundaries.
void heavy_prepare(spgemm_plan_t p) {
  hipStream_t s = p->sh;
  const int64_t h = p->h;
  int64_t* tmp = alloc_n<int64_t>(p, scan_tmp_elems(h) + 1, s);
  int64_t* hv = alloc_n<int64_t>(p, h, s);
  p->dAnnz = alloc_n<int64_t>(p, h + 1, s);
  launch_row_lengths(h, p->xheavy, p->arp, hv, s);
  launch_scan_i64(hv, h, p->dAnnz, tmp, s);
  check_launch("heavy prepare");
  // Bytes of intermediate per heavy element: one or two (col, val) buffers.
  const int64_t vb = p->f64 ? 8 : 4;
  int64_t budget = p->opts.mem_budget;
  if (!budget) {
    size_t freeB = 0, totalB = 0;
    HIP_CHECK(hipMemGetInfo(&freeB, &totalB));
    int64_t avail = (int64_t)freeB + (int64_t)region_free(p);
    if (p->arena) avail += (int64_t)(p->arena->cap - p->arenaUsed);
    budget = std::max<int64_t>(avail * 45 / 100, (int64_t)1 << 30);
  }
  // Chunk counts come from the structure unless asked otherwise or too wide
  // for LDS.  With them the whole chunk tree is known before any element
  // moves: the elements go straight to their final chunks when one work
  // group's (row, chunk) buckets fit its LDS, else the first level is fed
  // straight from A and B.
  const bool structCounts =
      p->params.levels > 0 && !p->opts.histogram_from_data && p->nreq <= 8192;
  int32_t xfElems = 0;
  int xfRows = 0;
  const bool xfFits = expand_final_geometry(p->f64, p->rowTau, p->nreq, &xfElems, &xfRows);
  p->direct = structCounts && p->opts.expansion == 0 && xfFits;
  p->fused = structCounts && !p->direct && p->opts.expansion != 1;
  // Straight into final chunks at most 65536 columns wide, a local column
  // takes two bytes.
  p->col16 = p->direct && p->params.level_width[0] <= 65536;
  p->st.chunk_col_bytes = p->col16 ? 2 : 4;
  const int64_t nbuf = heavy_nbuf(p);
  // Numeric needs columns and values.  If that takes one batch, symbolic
  // expands with values and numeric reuses the result (gMAGNUS Algorithm
  // 3); otherwise symbolic counts every heavy row's W-wide slots straight
  // from A and B (no expansion) and numeric expands each batch.
  const int64_t cap = std::max<int64_t>(budget / (nbuf * (4 + vb)), 1);
  int64_t maxNum = p->Ph;
  if (p->Ph <= cap) {
    // One batch: only the totals (known since plan) are needed on the host.
    p->hChat.assign(h + 1, 0);
    p->hAnnz.assign(h + 1, 0);
    p->hChat[h] = p->Ph;
    p->hAnnz[h] = p->nAh;
    p->batches.assign(1, {0, h});
  } else {
    // Batch cuts need every heavy row's product prefix on the host.
    int64_t* pref = alloc_n<int64_t>(p, h + 1, s);
    p->hChat.assign(h + 1, 0);
    p->hAnnz.assign(h + 1, 0);
    launch_gather_i64(p->rowP, p->xheavy, h, hv, s);
    launch_scan_i64(hv, h, pref, tmp, s);
    HIP_CHECK(hipMemcpyAsync(p->hChat.data(), pref, sizeof(int64_t) * (h + 1),
                             hipMemcpyDeviceToHost, s));
    HIP_CHECK(hipMemcpyAsync(p->hAnnz.data(), p->dAnnz, sizeof(int64_t) * (h + 1),
                             hipMemcpyDeviceToHost, s));
    check_launch("heavy batch cuts");
    HIP_CHECK(hipStreamSynchronize(s));
    maxNum = cut_batches(p, cap, &p->batches);
  }
  const int64_t bytes = (int64_t)heavy_buf_bytes(p, maxNum, true);
  p->symVals = p->batches.size() == 1;
  p->st.batches = (int64_t)p->batches.size();
  p->heavyBuf = heavy_region(p, (size_t)bytes);

  // Chunk counts of every heavy row from the structure, for all levels.
  const int64_t nreq = p->nreq;
  if (structCounts) {
    p->CH = alloc_n<int32_t>(p, h * nreq, s);
    const int64_t nnzB = p->nnzB;
    // B's slot table ((nreq + 1) run starts per B row) for the dense chunks
    // taken straight from A and B (option dense_direct), when it takes at
    // most 1 GiB; else those chunks are expanded as usual.
    const int64_t tabElems = p->k * (nreq + 1);
    p->useDD = p->opts.dense_direct && p->direct && tabElems * 4 <= ((int64_t)1 << 30);
    int32_t* tab = p->useDD ? alloc_n<int32_t>(p, tabElems, s) : nullptr;
    const int ph = ph_begin(p, SPGEMM_PH_CHUNK_HIST, s);
    const WsMark mk = ws_mark(p);
    int32_t* runPtr = alloc_n<int32_t>(p, p->k + 1, s);
    int32_t* runChunk = alloc_n<int32_t>(p, nnzB, s);
    int32_t* runStart = alloc_n<int32_t>(p, nnzB + 1, s);
    int32_t* flags = alloc_n<int32_t>(p, nnzB, s);
    int64_t* runIdx = alloc_n<int64_t>(p, nnzB + 1, s);
    int64_t* stmp = alloc_n<int64_t>(p, scan_tmp_elems(nnzB) + 1, s);
    launch_b_runs(p->k, nnzB, p->brp, p->bcol, log2_exact(p->params.dense_width), flags, runIdx,
                  stmp, runPtr, runChunk, runStart, s);
    int64_t* parts = alloc_n<int64_t>(p, h, s);
    int64_t* itemPtr = alloc_n<int64_t>(p, h + 1, s);
    int64_t* htmp = alloc_n<int64_t>(p, scan_tmp_elems(h) + 1, s);
    launch_chunk_hist_rows(h, p->nAh, p->dAnnz, p->xheavy, p->arp, p->acol, runPtr, runChunk,
                           runStart, (int32_t)nreq, p->CH, parts, itemPtr, htmp, s);
    if (tab) launch_slot_table(p->k, (int32_t)nreq, p->brp, runPtr, runChunk, runStart, tab, s);
    check_launch("chunk histogram");
    ws_reset(p, mk, s);
    p->slotTab = tab;
    ph_end(p, ph, s);
  }
}

// Expand heavy rows [hb0, hb1): CSC, outer product, multisplit levels, the
// final chunk list and its numeric bins.
void expand_batch(spgemm_plan_t p, int64_t hb0, int64_t hb1, bool countStats, bool vals, Batch* B) {
  hipStream_t s = p->sh;
  const int64_t hb = hb1 - hb0;
  const int64_t Pb = p->hChat[hb1] - p->hChat[hb0];
  const int64_t nE = p->hAnnz[hb1] - p->hAnnz[hb0];
  const int32_t* xb = p->xheavy + hb0;
  const bool f64 = p->f64;
  const size_t vb = f64 ? 8 : 4;
  const int64_t W = p->params.dense_width;
  *B = Batch{};
  B->hb0 = hb0;
  B->hb1 = hb1;
  B->Pb = Pb;
  int64_t* tmp = alloc_n<int64_t>(p, scan_tmp_elems(std::max<int64_t>({hb, nE, p->k, 1}) + 1), s);
  const int phCsc = ph_begin(p, SPGEMM_PH_CSC, s);

  // C-hat row pointers of the batch: scan of its rows' product counts.
  int64_t* hP = alloc_n<int64_t>(p, hb, s);
  int64_t* chatRowPtr = alloc_n<int64_t>(p, hb + 1, s);
  launch_gather_i64(p->rowP, xb, hb, hP, s);
  launch_scan_i64(hP, hb, chatRowPtr, tmp, s);

  const int L = p->params.levels;
  {
    char* q = p->heavyBuf;
    const size_t n = (size_t)std::max<int64_t>(Pb, 1);
    for (int b = 0; b < heavy_nbuf(p); ++b) {
      B->bufCol[b] = (int32_t*)q;
      q += align256(n * (p->col16 ? 2 : 4));
      if (vals) {
        B->bufVal[b] = q;
        q += align256(n * vb);
      }
    }
  }
  ExpandSrc src{};
  if (p->fused || p->direct) {
    // The heavy rows' A entries in row order with their product offsets:
    // the first multisplit level makes its elements from these.
    int32_t* eB = alloc_n<int32_t>(p, nE, s);
    int64_t* eOff = alloc_n<int64_t>(p, nE + 1, s);
    void* eVal = vals ? plan_alloc(p, std::max<int64_t>(nE, 1) * vb, s) : nullptr;
    launch_expand_entries(f64, nE, hb, xb, p->dAnnz + hb0, chatRowPtr, p->arp, p->acol, p->aval,
                          p->brp, p->scanA, eB, eOff, eVal, s);
    src = ExpandSrc{eOff, eB, eVal, p->bcol, vals ? p->bval : nullptr, nE};
    ph_end(p, phCsc, s);
  } else {
  // Masked CSR -> CSC of A restricted to the batch's heavy rows.
  int32_t* colCnt = alloc_n<int32_t>(p, p->k, s);
  int64_t* colPtr = alloc_n<int64_t>(p, p->k + 1, s);
  int64_t* colFill = alloc_n<int64_t>(p, p->k, s);
  int32_t* cscRow = alloc_n<int32_t>(p, nE, s);
  int32_t* cscCol = alloc_n<int32_t>(p, nE, s);
  void* cscVal = plan_alloc(p, std::max<int64_t>(nE, 1) * vb, s);
  launch_fill_i32(colCnt, 0, p->k, s);
  launch_csc_count(hb, xb, p->arp, p->acol, colCnt, s);
  launch_scan_i32(colCnt, p->k, colPtr, tmp, s);
  launch_copy_i64(colFill, colPtr, p->k, s);
  launch_csc_fill(hb, xb, p->arp, p->acol, p->aval, f64, colFill, cscRow, cscCol, cscVal, s);

  // Flattened element offsets of the CSC entries and their C-hat segments.
  int64_t* nb = alloc_n<int64_t>(p, nE, s);
  int64_t* entryOff = alloc_n<int64_t>(p, nE + 1, s);
  int64_t* cursor = alloc_n<int64_t>(p, hb, s);
  int64_t* segBase = alloc_n<int64_t>(p, nE, s);
  launch_entry_products(nE, cscCol, p->brp, nb, s);
  launch_scan_i64(nb, nE, entryOff, tmp, s);
  launch_copy_i64(cursor, chatRowPtr, hb, s);
  launch_seg_base(nE, cscRow, nb, cursor, segBase, s);
  ph_end(p, phCsc, s);

  // Outer product into buffer 0.
  const int phOp = ph_begin(p, SPGEMM_PH_OUTER_PRODUCT, s);
  launch_outer_product(f64, Pb, entryOff, nE, cscCol, cscVal, segBase, p->brp, p->bcol, p->bval,
                       B->bufCol[0], B->bufVal[0], s);
  ph_end(p, phOp, s);
  check_launch("outer product");
  }

  struct Piece {
    int64_t first, n;
    const int64_t* newOff;
    const int32_t *newCnt, *newRow, *newSlot;
    int8_t buf, spanLog2;
  };
  std::vector<Piece> pieces;
  bool completed = (L == 0);
  int64_t R = hb, E = Pb;
  const int64_t* rowPtr = chatRowPtr;
  const int32_t *inRow = nullptr, *inSlot = nullptr;
  // Buffer the level reads (none when fed from A and B; with the direct
  // expansion the levels only shape the chunk tree).
  int cur = p->fused ? 1 : 0;
  for (int l = 0; l < L; ++l) {
    B->levelElems[l] = E;
    const int v = p->params.v_chunks[l];
    const int64_t w = p->params.level_width[l];
    const int shift = log2_exact(w);
    const int64_t Q = R * v;
    if (Q >= INT32_MAX) throw Error{SPGEMM_ERR_INDEX_OVERFLOW, "too many chunks in one level"};
    const bool last = (l == L - 1);
    int32_t* counts = alloc_n<int32_t>(p, Q, s);
    int32_t* inv = alloc_n<int32_t>(p, Q, s);
    int32_t* newCnt = alloc_n<int32_t>(p, Q, s);
    int32_t* newRow = alloc_n<int32_t>(p, Q, s);
    int32_t* newSlot = alloc_n<int32_t>(p, Q, s);
    int64_t* newOff = alloc_n<int64_t>(p, Q + 1, s);
    int64_t* cur64 = alloc_n<int64_t>(p, Q, s);
    int32_t* ctr = alloc_n<int32_t>(p, 2, s);
    int64_t* ltmp = alloc_n<int64_t>(p, scan_tmp_elems(Q) + 1, s);
    if (!p->CH) launch_fill_i32(counts, 0, Q, s);
    launch_fill_i32(newCnt, 0, Q, s);
    launch_fill_i32(ctr, 0, 2, s);
    int32_t blockElems = 0;
    int maxRows = 0;
    TileInfo* info = nullptr;
    if (!p->direct) {
      // Rows of the first level are heavy rows (more than rowTau elements),
      // of later levels heavy chunks (more than tau).
      multisplit_geometry(f64 && vals, l == 0 ? p->rowTau : p->tau, v, &blockElems, &maxRows);
      // First row (and, fed from A and B, first entry) of every work group.
      const int64_t nBlk = (E + blockElems - 1) / blockElems;
      int32_t* blkRow = alloc_n<int32_t>(p, nBlk, s);
      int32_t* blkEnt = nullptr;
      info = alloc_n<TileInfo>(p, nBlk, s);
      launch_block_starts(R, rowPtr, blockElems, nBlk, blkRow, s);
      if (p->fused && l == 0) {
        blkEnt = alloc_n<int32_t>(p, nBlk, s);
        launch_block_starts(src.nE, src.eOff, blockElems, nBlk, blkEnt, s);
      }
      launch_tile_info(E, blockElems, rowPtr, R, blkRow, blkEnt, src.nE, info, s);
    }
    const int phH = ph_begin(p, SPGEMM_PH_HISTOGRAM, s);
    if (p->CH)
      launch_level_counts(Q, v, (int32_t)(w / W), (int32_t)p->nreq, inRow, inSlot,
                          p->CH + hb0 * p->nreq, counts, s);
    else
      launch_histogram(E, blockElems, rowPtr, info, B->bufCol[cur], shift, v, maxRows, counts,
                       p->errWord, s);
    ph_end(p, phH, s);
    launch_partition(Q, counts, p->tau, last, v, inRow, inSlot, (int32_t)(w / W), inv, newCnt,
                     newRow, newSlot, ctr, s);
    launch_scan_i32(newCnt, Q, newOff, ltmp, s);
    launch_copy_i64(cur64, newOff, Q, s);
    const int out = p->direct ? 0 : 1 - cur;
    if (!p->direct) {
      const bool direct = p->fused && l == 0;
      const int phM = ph_begin(p, direct ? SPGEMM_PH_EXPAND_SPLIT : SPGEMM_PH_MULTISPLIT, s);
      launch_multisplit(f64, E, blockElems, rowPtr, info, direct ? nullptr : B->bufCol[cur],
                        direct ? nullptr : B->bufVal[cur], direct ? &src : nullptr, shift, v,
                        (int32_t)(w - 1), maxRows, inv, cur64, B->bufCol[out], B->bufVal[out],
                        p->errWord, s);
      ph_end(p, phM, s);
    }
    check_launch("multisplit level");
    // nH, nL and the heavy chunks' element total newOff[nH], in one readback
    int64_t* tail = alloc_n<int64_t>(p, 3, s);
    launch_level_tail(ctr, newOff, tail, s);
    HIP_CHECK(hipMemcpyAsync(p->hStats + 16, tail, 24, hipMemcpyDeviceToHost, s));
    HIP_CHECK(hipStreamSynchronize(s));
    const int64_t nH = p->hStats[16], nL = p->hStats[17];
    const int64_t nextE = nH > 0 ? p->hStats[18] : 0;
    pieces.push_back(Piece{Q - nL, nL, newOff, newCnt, newRow, newSlot, (int8_t)out,
                           (int8_t)log2_exact(w / W)});
    if (last) completed = true;
    if (nH == 0) break;
    R = nH;
    E = nextE;
    rowPtr = newOff;
    inRow = newRow;
    inSlot = newSlot;
    cur = out;
  }

  // Final chunk list: light chunks of every level, then the W-wide chunks
  // of the last level (or the heavy rows themselves with no multisplit).
  int64_t nfc = 0;
  for (auto& pc : pieces) nfc += pc.n;
  if (L == 0) nfc = hb;
  B->nfc = nfc;
  B->fcOff = alloc_n<int64_t>(p, nfc, s);
  B->fcCnt = alloc_n<int32_t>(p, nfc, s);
  B->fcRow = alloc_n<int32_t>(p, nfc, s);
  B->fcSlot = alloc_n<int32_t>(p, nfc, s);
  B->fcBuf = alloc_n<int8_t>(p, nfc, s);
  B->fcSpan = alloc_n<int8_t>(p, nfc, s);
  if (L == 0) {
    launch_final_from_rows(hb, chatRowPtr, B->fcOff, B->fcCnt, B->fcRow, B->fcSlot, B->fcBuf,
                           B->fcSpan, s);
    B->lastFirst = 0;
  } else {
    int64_t dst = 0;
    for (auto& pc : pieces) {
      launch_final_from_level(pc.first, pc.n, pc.newOff, pc.newCnt, pc.newRow, pc.newSlot, pc.buf,
                              pc.spanLog2, dst, B->fcOff, B->fcCnt, B->fcRow, B->fcSlot,
                              B->fcBuf, B->fcSpan, s);
      dst += pc.n;
    }
    B->lastFirst = completed ? nfc - pieces.back().n : nfc;
  }
  // Numeric bins: W-wide chunks with more than tau elements (or W/2, if
  // smaller) go to the dense accumulator; the rest by element count.  Below
  // that the light chunk kernels (register sort, bitmap rank) beat zeroing
  // and scanning W columns: with W/8 in place of tau, 9% more time per
  // product at R-MAT 18 (fp64, W = 16384) and 5% at R-MAT 20.
  uint8_t* key = alloc_n<uint8_t>(p, nfc, s);
  B->fcOrder = alloc_n<int32_t>(p, nfc, s);
  int32_t* bc = alloc_n<int32_t>(p, 64, s);
  int32_t* bf = alloc_n<int32_t>(p, 64, s);
  int32_t* bs = alloc_n<int32_t>(p, 65, s);
  const int64_t denseMin = std::min<int64_t>(p->tau, W / 2);
  launch_chunk_bins(nfc, B->fcCnt, B->lastFirst, denseMin, p->dSymCaps, p->NS, p->NS, key,
                    countStats ? p->stats + kStatDenseElems : nullptr, s);
  launch_bin_sort(key, nfc, p->NS + 1, bc, bf, bs, B->fcOrder, s);
  HIP_CHECK(hipMemcpyAsync(p->hBins + 64, bs, sizeof(int32_t) * (p->NS + 2), hipMemcpyDeviceToHost, s));
  HIP_CHECK(hipStreamSynchronize(s));
  B->fcBinStart.assign(p->hBins + 64, p->hBins + 64 + p->NS + 2);
  B->denseChunks = B->fcBinStart[p->NS + 1] - B->fcBinStart[p->NS];
  if (p->direct) {
    // Final chunks back to back in buffer 0, in list order; every product
    // goes straight to the final chunk covering its column.
    const int phX = ph_begin(p, vals ? SPGEMM_PH_EXPAND_FINAL : SPGEMM_PH_SYM_HEAVY, s);
    // With values, dense chunks are accumulated straight from A and B: the
    // expansion skips their products and they take no space.
    B->denseDirect = vals && p->useDD;
    const int32_t* stored = B->fcCnt;
    if (B->denseDirect) {
      int32_t* sc = alloc_n<int32_t>(p, nfc, s);
      launch_stored_counts(nfc, B->fcCnt, key, p->NS, sc, s);
      stored = sc;
    }
    int64_t* fcOff = alloc_n<int64_t>(p, nfc + 1, s);
    int64_t* ftmp = alloc_n<int64_t>(p, scan_tmp_elems(nfc) + 1, s);
    launch_scan_i32(stored, nfc, fcOff, ftmp, s);
    B->fcOff = fcOff;
    launch_fill_i8(B->fcBuf, 0, nfc, s);
    const int64_t nslot = hb * p->nreq;
    int32_t* finalOf = alloc_n<int32_t>(p, nslot, s);
    int8_t* spanOf = alloc_n<int8_t>(p, nslot, s);
    launch_fill_i32(finalOf, -1, nslot, s);
    launch_fill_i8(spanOf, 0, nslot, s);
    launch_final_map(nfc, B->fcRow, B->fcSlot, B->fcSpan, p->nreq,
                     B->denseDirect ? key : nullptr, p->NS, finalOf, spanOf, s);
    int64_t* fcCursor = alloc_n<int64_t>(p, nfc, s);
    launch_copy_i64(fcCursor, fcOff, nfc, s);
    int32_t blockElems = 0;
    int maxRows = 0;
    if (!expand_final_geometry(f64 && vals, p->rowTau, p->nreq, &blockElems, &maxRows))
      throw Error{SPGEMM_ERR_INTERNAL, "direct expansion geometry"};
    const int64_t nBlk = (Pb + blockElems - 1) / blockElems;
    int32_t* blkRow = alloc_n<int32_t>(p, nBlk, s);
    int32_t* blkEnt = alloc_n<int32_t>(p, nBlk, s);
    TileInfo* info = alloc_n<TileInfo>(p, nBlk, s);
    launch_block_starts(hb, chatRowPtr, blockElems, nBlk, blkRow, s);
    launch_block_starts(src.nE, src.eOff, blockElems, nBlk, blkEnt, s);
    launch_tile_info(Pb, blockElems, chatRowPtr, hb, blkRow, blkEnt, src.nE, info, s);
    launch_expand_final(f64, Pb, blockElems, chatRowPtr, info, src, finalOf, spanOf,
                        (int32_t)p->nreq, log2_exact(W), maxRows, fcCursor, B->bufCol[0],
                        p->col16, vals ? B->bufVal[0] : nullptr, p->errWord, s);
    ph_end(p, phX, s);
    check_launch("direct expansion");
  }
}

ChunkList chunk_list(spgemm_plan_t p, const Batch& B) {
  return ChunkList{B.fcOff, B.fcCnt, B.fcRow, B.fcSlot, B.fcBuf, B.bufCol[0], B.bufCol[1],
                   B.bufVal[0], B.bufVal[1], p->params.dense_width, p->nreq,
                   p->xheavy + B.hb0, p->slotOff + B.hb0 * p->nreq,
                   p->slotNnz + B.hb0 * p->nreq, p->col16 ? 1 : 0, B.fcSpan};
}

// Chunk symbolic: per-chunk nnz into the batch's slots.
// Light chunks take the bitmap kernels (no sort: a chunk's columns are
// ranked by prefix popcounts over its width) when the bitmap is small next
// to the hash table of the chunk's bin; small chunks of wide levels take the
// hash kernels, whose cost follows the element count, not the width.
bool sym_bitmap(spgemm_plan_t p, int b) {
  return p->chunkWords && p->chunkWords <= 2 * (int64_t)p->symBins[b].cap;
}
bool num_bitmap(spgemm_plan_t p, int b) {
  return p->chunkWords && p->chunkWords <= 4 * (int64_t)p->symBins[b].cap;
}

// Chunk symbolic: per-chunk nnz into the batch's slots.
void symbolic_batch(spgemm_plan_t p, const Batch& B) {
  hipStream_t s = p->sh;
  const ChunkList cl = chunk_list(p, B);
  ChunkDesc* desc = alloc_n<ChunkDesc>(p, B.nfc, s);
  launch_chunk_desc(B.nfc, B.fcOrder, cl, nullptr, desc, s);
  const int ph = ph_begin(p, SPGEMM_PH_SYM_CHUNK_HASH, s);
  for (int b = 0; b < p->NS; ++b) {
    const int64_t a = B.fcBinStart[b], e = B.fcBinStart[b + 1];
    if (!sym_bitmap(p, b)) launch_sym_chunks(p->symBins[b], desc + a, e - a, cl, p->errWord, s);
  }
  ph_end(p, ph, s);
  const int phD = ph_begin(p, SPGEMM_PH_SYM_CHUNK_DENSE, s);
  for (int b = 0; b < p->NS; ++b) {
    const int64_t a = B.fcBinStart[b], e = B.fcBinStart[b + 1];
    const int64_t cap = p->symBins[b].cap;
    if (sym_bitmap(p, b))
      launch_sym_chunks_bitmap(cap <= 256 ? 0 : cap <= 4096 ? 1 : 2, desc + a, e - a,
                               p->chunkWords, cl, s);
  }
  const int64_t a = B.fcBinStart[p->NS], e = B.fcBinStart[p->NS + 1];
  if (p->chunkWords)
    launch_sym_chunks_persist(desc + a, e - a, cl, p->numCUs, s);
  else
    launch_dense_sym(desc + a, e - a, cl, p->errWord, s);
  ph_end(p, phD, s);
  check_launch("chunk symbolic");
}

void numeric_batch(spgemm_plan_t p, const Batch& B, int32_t* ccol, void* cval,
                   ChunkDesc* desc = nullptr) {
  hipStream_t s = p->sh;
  const ChunkList cl = chunk_list(p, B);
  // Descriptors of the chunks in bin order, gathered once (into space
  // reserved by symbolic for the kept batch).
  if (!desc) desc = alloc_n<ChunkDesc>(p, B.nfc, s);
  launch_chunk_desc(B.nfc, B.fcOrder, cl, p->cRowOff, desc, s);
  // Dense chunks on their own stream, launched first (one persistent work
  // group per CU), while the light chunks' kernels fill the rest of the
  // device from the heavy stream; the heavy stream waits for both.
  hipStream_t sd = p->sd;
  if (sd != s) {
    HIP_CHECK(hipEventRecord(p->evD0, s));
    HIP_CHECK(hipStreamWaitEvent(sd, p->evD0, 0));
  }
  {
    const int64_t st = B.fcBinStart[p->NS], en = B.fcBinStart[p->NS + 1];
    const int phD = ph_begin(p, SPGEMM_PH_NUM_CHUNK_DENSE, sd);
    if (B.denseDirect)
      launch_dense_num_direct(p->f64, desc + st, en - st, p->params.dense_width, row_args(p),
                              p->slotTab, p->nreq + 1, p->nnzB, ccol, cval,
                              p->errWord, p->numCUs, sd);
    else
      launch_dense_num(p->f64, desc + st, en - st, cl, ccol, cval, p->errWord, p->numCUs, sd);
    ph_end(p, phD, sd);
    if (sd != s) HIP_CHECK(hipEventRecord(p->evD1, sd));
  }
  const int ph = ph_begin(p, SPGEMM_PH_NUM_CHUNK_HASH, s);
  for (int b = 0; b < p->NS; ++b) {
    const int64_t st = B.fcBinStart[b], en = B.fcBinStart[b + 1];
    // Up to 256 elements: sorted in registers; then the bitmap-rank or the
    // hash accumulators.
    if (launch_num_chunks_esc(p->symBins[b].cap, p->f64, desc + st, en - st, cl, ccol, cval,
                              p->errWord, s))
      continue;
    if (num_bitmap(p, b)) {
      if (!launch_num_chunks_direct(p->symBins[b], p->f64, desc + st, en - st, p->chunkWords,
                                    (size_t)p->lds, cl, ccol, cval, p->errWord, s))
        launch_num_chunks_rank(p->rankBins[b], p->f64, desc + st, en - st, p->chunkWords, cl, ccol,
                               cval, p->errWord, s);
    } else {
      launch_num_chunks(p->numBins[b], p->f64, desc + st, en - st, cl, ccol, cval, p->errWord, s);
    }
  }
  ph_end(p, ph, s);
  if (s != p->sd) HIP_CHECK(hipStreamWaitEvent(s, p->evD1, 0));
  check_launch("chunk numeric");
}

void heavy_symbolic(spgemm_plan_t p) {
  hipStream_t s = p->sh;
  const int64_t h = p->h, W = p->params.dense_width;
  const int L = p->params.levels;
  heavy_prepare(p);
  p->slotNnz = alloc_n<int32_t>(p, h * p->nreq, s);
  p->slotOff = alloc_n<int64_t>(p, h * p->nreq, s);
  launch_fill_i32(p->slotNnz, 0, h * p->nreq, s);
  // Bitmap chunk symbolic and rank numeric when the widest final chunk (the
  // first level's width, or W with no multisplit) is at most 64 Kbit.
  const int64_t maxWidth = L == 0 ? W : p->params.level_width[0];
  if (maxWidth <= 65536) {
    p->chunkWords = (int32_t)((maxWidth + 31) / 32);
    make_rank_bins(p->lds, p->f64, p->chunkWords, p->symBins, &p->rankBins);
  }
  p->st.final_chunks = 0;
  p->st.dense_chunks = 0;
  if (p->symVals && !p->useDD) {
    // One batch (gMAGNUS Algorithm 3): expand with values, count every final
    // chunk, keep the chunks for numeric.
    Batch B;
    expand_batch(p, p->batches[0].first, p->batches[0].second, true, true, &B);
    symbolic_batch(p, B);
    p->st.final_chunks += B.nfc;
    p->st.dense_chunks += B.denseChunks;
    for (int l = 0; l < 8; ++l) p->st.level_elems[l] += B.levelElems[l];
    p->kept = B;
    p->haveKept = true;
    // numeric's descriptors, reserved now so that numeric allocates nothing
    p->keptDesc = alloc_n<ChunkDesc>(p, B.nfc, s);
    launch_slot_scan(h, p->nreq, p->slotNnz, p->slotOff, p->xheavy, p->cnt, s);
  } else {
    // Every heavy row's W-wide slots counted straight from A and B, on the
    // dense chunks' stream (idle until numeric); meanwhile the heavy stream
    // expands the first batch with values (only its light chunks with
    // dense_direct), which numeric takes as it is.  Symbolic ends by joining
    // both streams.
    hipStream_t sy = p->sd;
    if (sy != s) {
      HIP_CHECK(hipEventRecord(p->evD0, s));
      HIP_CHECK(hipStreamWaitEvent(sy, p->evD0, 0));
    }
    const int ph = ph_begin(p, SPGEMM_PH_SYM_HEAVY, sy);
    int32_t* next = alloc_n<int32_t>(p, 1, sy);
    launch_fill_i32(next, 0, 1, sy);
    launch_sym_heavy_rows(h, p->nreq, log2_exact(W), p->xheavy, row_args(p), p->nnzB,
                          p->slotNnz, next, p->numCUs, (size_t)p->lds, sy);
    ph_end(p, ph, sy);
    launch_slot_scan(h, p->nreq, p->slotNnz, p->slotOff, p->xheavy, p->cnt, sy);
    Batch B;
    expand_batch(p, p->batches[0].first, p->batches[0].second, true, true, &B);
    p->st.final_chunks += B.nfc;
    p->st.dense_chunks += B.denseChunks;
    for (int l = 0; l < 8; ++l) p->st.level_elems[l] += B.levelElems[l];
    p->kept = B;
    p->haveKept = true;
    p->keptDesc = alloc_n<ChunkDesc>(p, B.nfc, s);
  }
  check_launch("heavy symbolic");
}

void heavy_numeric(spgemm_plan_t p, int32_t* ccol, void* cval) {
  // The first batch was expanded in symbolic; the others are expanded here,
  // one after another, each into the same memory.
  if (p->haveKept) numeric_batch(p, p->kept, ccol, cval, p->keptDesc);
  for (size_t i = p->haveKept ? 1 : 0; i < p->batches.size(); ++i) {
    const auto& bt = p->batches[i];
    const WsMark mk = ws_mark(p);
    Batch B;
    expand_batch(p, bt.first, bt.second, true, true, &B);
    numeric_batch(p, B, ccol, cval);
    p->st.final_chunks += B.nfc;
    p->st.dense_chunks += B.denseChunks;
    for (int l = 0; l < 8; ++l) p->st.level_elems[l] += B.levelElems[l];
    ws_reset(p, mk, p->sh);
  }
}

// Rows of the first product bin (at most 32 products) by expand-sort-compact.
bool esc_on(spgemm_plan_t p) {
  return !p->opts.light_no_esc && p->symBins[0].cap <= 32;
}

// ------------------------------------------------- size-estimate workflows
// Registers per sketch: 32 while the expansion ratio products / nnz(A) is
// below 48, else 64 (Ocean page, parameter settings), unless set.
int hll_lg(spgemm_plan_t p) {
  int M = p->opts.hll_registers;
  if (M == 0) M = p->st.products < 48 * std::max<int64_t>(p->nnzA, 1) ? 32 : 64;
  if (M != 32 && M != 64) throw Error{SPGEMM_ERR_INVALID_ARG, "hll_registers must be 0, 32 or 64"};
  return M == 32 ? 5 : 6;
}

// M * ln(M / V) for V = 0..M, the small-count estimate, on the device.
const double* hll_table(spgemm_plan_t p, int lg, hipStream_t s) {
  const int M = 1 << lg;
  p->hLc.assign(M + 1, 0.0);
  for (int v = 1; v <= M; ++v) p->hLc[v] = (double)M * std::log((double)M / (double)v);
  double* d = alloc_n<double>(p, M + 1, s);
  HIP_CHECK(hipMemcpyAsync(d, p->hLc.data(), sizeof(double) * (M + 1), hipMemcpyHostToDevice, s));
  HIP_CHECK(hipStreamSynchronize(s));  // the host table may change with the next call
  return d;
}

// Ocean's Table 1 on this plan: upper bound below 64 products per row;
// HyperLogLog when products / nnz(A) >= 8 and the compression ratio of a row
// sample (products / estimated nnz over 3% of the rows, 600 to 10,000, evenly
// spaced; heavy rows, which keep the exact chunk path, left out) is >= 8;
// else the symbolic pass.
int select_workflow(spgemm_plan_t p, hipStream_t s) {
  const int64_t m = p->m, P = p->st.products;
  if (P < 64 * m) return 1;
  if (P < 8 * p->nnzA) return 0;
  const int lg = hll_lg(p);
  const int64_t ns = std::min<int64_t>(m, std::min<int64_t>(10000, std::max<int64_t>(
                                                                     600, std::llround(0.03 * m))));
  std::vector<int32_t> hrows(ns);
  for (int64_t j = 0; j < ns; ++j) hrows[j] = (int32_t)((j * m) / ns);
  int32_t* rows = alloc_n<int32_t>(p, ns, s);
  double* est = alloc_n<double>(p, ns, s);
  int64_t* pr = alloc_n<int64_t>(p, ns, s);
  HIP_CHECK(hipMemcpyAsync(rows, hrows.data(), sizeof(int32_t) * ns, hipMemcpyHostToDevice, s));
  const double* lc = hll_table(p, lg, s);
  launch_hll_rows_direct(ns, rows, p->arp, p->acol, p->brp, p->bcol, p->rowP, p->rowTau, lg, lc,
                         est, s);
  launch_gather_i64(p->rowP, rows, ns, pr, s);
  check_launch("row sample estimate");
  std::vector<double> he(ns);
  std::vector<int64_t> hp(ns);
  HIP_CHECK(hipMemcpyAsync(he.data(), est, sizeof(double) * ns, hipMemcpyDeviceToHost, s));
  HIP_CHECK(hipMemcpyAsync(hp.data(), pr, sizeof(int64_t) * ns, hipMemcpyDeviceToHost, s));
  HIP_CHECK(hipStreamSynchronize(s));
  double sp = 0, se = 0;
  for (int64_t j = 0; j < ns; ++j) {
    if (hp[j] > p->rowTau) continue;
    sp += (double)hp[j];
    se += he[j];
  }
  p->st.sampled_cr = se > 0 ? sp / se : 0.0;
  return p->st.sampled_cr >= 8.0 ? 2 : 0;
}

// Light rows without the symbolic pass: reserve slots (upper bound or
// estimate), compute every light row into them, redo the rows that did not
// fit with P_i slots, and leave each light row's count in p->cnt.
void estimate_light(spgemm_plan_t p, const RowArgs& a) {
  hipStream_t s = p->sl;
  const int64_t m = p->m;
  const int heavyBin = p->NS + 1;
  const int phL = ph_begin(p, SPGEMM_PH_SYM_LIGHT, s);
  p->capL = alloc_n<int64_t>(p, m, s);
  p->tmpOff = alloc_n<int64_t>(p, m + 1, s);
  p->cnt1 = alloc_n<int64_t>(p, m, s);
  int64_t* tmp = alloc_n<int64_t>(p, scan_tmp_elems(m) + 1, s);
  uint8_t* key = alloc_n<uint8_t>(p, m, s);
  int32_t* order = alloc_n<int32_t>(p, m, s);
  launch_fill_i64(p->capL, 0, m, s);
  launch_fill_i64(p->cnt1, 0, m, s);
  if (p->wf == 1) {
    launch_ub_capacity(m, p->rowP, p->rowBin, heavyBin, p->capL, s);
  } else {
    const int lg = p->hllLg = hll_lg(p);
    const int M = 1 << lg;
    p->st.hll_registers = M;
    const double coef = p->opts.hll_coef_pct ? p->opts.hll_coef_pct / 100.0 : (M == 32 ? 2.0 : 1.5);
    uint8_t* regs = alloc_n<uint8_t>(p, std::max<int64_t>(p->k, 1) * M, s);
    p->estL = alloc_n<double>(p, m, s);
    launch_fill_i64((int64_t*)p->estL, 0, m, s);  // +0.0 has an all-zero bit pattern
    const double* lc = hll_table(p, lg, s);
    launch_hll_sketch(p->k, p->brp, p->bcol, lg, regs, s);
    launch_hll_capacity(m, p->arp, p->acol, regs, lg, lc, coef, p->rowP, p->rowBin, heavyBin,
                        p->capL, p->estL, s);
  }
  launch_scan_i64(p->capL, m, p->tmpOff, tmp, s);
  launch_numeric_row_bins(m, p->capL, p->rowBin, heavyBin, p->dSymCaps, p->NS, key, s,
                          esc_on(p) ? 2 * p->NS : -1);
  launch_bin_sort(key, m, 2 * p->NS + 1, p->binCnt, p->binFill, p->binStart, order, s);
  check_launch("light capacities");
  std::vector<int32_t> bins(2 * p->NS + 2);
  int64_t total = 0;
  HIP_CHECK(hipMemcpyAsync(&total, p->tmpOff + m, 8, hipMemcpyDeviceToHost, s));
  HIP_CHECK(hipMemcpyAsync(bins.data(), p->binStart, sizeof(int32_t) * bins.size(),
                           hipMemcpyDeviceToHost, s));
  HIP_CHECK(hipStreamSynchronize(s));
  p->st.light_capacity = total;
  const int vb = p->f64 ? 8 : 4;
  p->tcol1 = alloc_n<int32_t>(p, std::max<int64_t>(total, 1), s);
  p->tval1 = plan_alloc(p, (size_t)std::max<int64_t>(total, 1) * vb, s);
  auto run = [&](const std::vector<int32_t>& bs, const int64_t* off, int32_t* tc, void* tv,
                 int64_t* cntOut) {
    launch_num_rows_esc(p->f64, order + bs[2 * p->NS], bs[2 * p->NS + 1] - bs[2 * p->NS], a, off,
                        tc, tv, p->errWord, s, cntOut);
    for (int b = 0; b < p->NS; ++b) {
      launch_num_rows(p->numBins[b], p->f64, order + bs[b], bs[b + 1] - bs[b], a, off, tc, tv,
                      p->errWord, s, cntOut);
      const int64_t ws = bs[p->NS + b], we = bs[p->NS + b + 1];
      if (we > ws)
        launch_num_rows_win(p->symBins[b], p->winWords[b], p->f64, order + ws, we - ws, a, off,
                            tc, tv, p->errWord, s, cntOut);
    }
  };
  run(bins, p->tmpOff, p->tcol1, p->tval1, p->cnt1);
  check_launch("light numeric into reserved slots");
  // Rows that did not fit (estimates only; P_i slots always suffice).
  int32_t nOver = 0;
  if (p->wf == 2) {
    int32_t* dOver = alloc_n<int32_t>(p, 1, s);
    int64_t* cap2 = alloc_n<int64_t>(p, m, s);
    launch_fill_i32(dOver, 0, 1, s);
    launch_overflow_rows(m, p->cnt1, p->rowP, p->rowBin, heavyBin, p->NS, cap2, key, dOver, s);
    HIP_CHECK(hipMemcpyAsync(&nOver, dOver, 4, hipMemcpyDeviceToHost, s));
    HIP_CHECK(hipStreamSynchronize(s));
    if (nOver > 0) {
      p->off2 = alloc_n<int64_t>(p, m + 1, s);
      p->cnt2 = alloc_n<int64_t>(p, m, s);
      launch_fill_i64(p->cnt2, 0, m, s);
      launch_scan_i64(cap2, m, p->off2, tmp, s);
      launch_bin_sort(key, m, 2 * p->NS + 1, p->binCnt, p->binFill, p->binStart, order, s);
      int64_t total2 = 0;
      HIP_CHECK(hipMemcpyAsync(&total2, p->off2 + m, 8, hipMemcpyDeviceToHost, s));
      HIP_CHECK(hipMemcpyAsync(bins.data(), p->binStart, sizeof(int32_t) * bins.size(),
                               hipMemcpyDeviceToHost, s));
      HIP_CHECK(hipStreamSynchronize(s));
      p->tcol2 = alloc_n<int32_t>(p, std::max<int64_t>(total2, 1), s);
      p->tval2 = plan_alloc(p, (size_t)std::max<int64_t>(total2, 1) * vb, s);
      run(bins, p->off2, p->tcol2, p->tval2, p->cnt2);
      check_launch("light numeric of rows that did not fit");
    }
  }
  p->st.overflow_rows = nOver;
  launch_merge_counts(m, p->rowBin, heavyBin, p->cnt1, nOver ? p->cnt2 : nullptr, p->off2,
                      p->tmpOff, p->cnt, s);
  ph_end(p, phL, s);
  check_launch("light counts");
}

void do_symbolic(spgemm_plan_t p, void* dRowPtr, int64_t* nnzC) {
  const double t0 = now_ms();
  hipStream_t s = p->stream;
  p->wf = p->opts.workflow == 3 ? select_workflow(p, s) : p->opts.workflow;
  p->st.workflow = p->wf;
  if (p->wf == 0 && p->hybSymBin < p->NS) p->outc = alloc_n<int32_t>(p, p->m, s);
  fork(p);
  const RowArgs a = row_args(p);
  if (p->wf == 0) {
    const int phL = ph_begin(p, SPGEMM_PH_SYM_LIGHT, p->sl);
    for (int b = 0; b < p->NS; ++b) {
      const int64_t st = p->rowBinStart[b + 1], en = p->rowBinStart[b + 2];
      if (b == 0 && esc_on(p))
        launch_sym_rows_esc(p->rowOrder + st, en - st, a, p->cnt, p->sl);
      else if (b >= p->hybSymBin)
        launch_sym_rows_hyb(p->symBins[b], p->rowOrder + st, en - st, a, p->m, p->n, p->cnt,
                            p->outc, p->errWord, p->sl);
      else
        launch_sym_rows(p->symBins[b], p->rowOrder + st, en - st, a, p->cnt, p->errWord, p->sl);
      const int64_t ws = p->rowBinStart[p->NS + 2 + b], we = p->rowBinStart[p->NS + 3 + b];
      if (we > ws)
        launch_sym_rows_win(p->symBins[b], p->winWords[b], p->rowOrder + ws, we - ws, a, p->cnt,
                            p->sl);
    }
    ph_end(p, phL, p->sl);
    check_launch("light symbolic");
  }
  if (p->h > 0) heavy_symbolic(p);
  // After the heavy batches (their workspace marks), so the light rows'
  // reserved slots stay allocated until destroy.
  if (p->wf != 0) estimate_light(p, a);
  join(p);

  const int64_t m = p->m;
  p->cRowOff = alloc_n<int64_t>(p, m + 1, s);
  p->scanTmp = alloc_n<int64_t>(p, scan_tmp_elems(m) + 1, s);
  p->numKey = alloc_n<uint8_t>(p, m, s);
  p->numOrder = alloc_n<int32_t>(p, m, s);
  const int phR = ph_begin(p, SPGEMM_PH_ROWPTR, s);
  launch_scan_i64(p->cnt, m, p->cRowOff, p->scanTmp, s);
  // numeric keys: hash bins, dense-window bins, ESC, hybrid bins
  const int nkeys = 3 * p->NS + 1;
  if (p->wf == 0) {
    launch_numeric_row_bins(m, p->cnt, p->rowBin, p->NS + 1, p->dSymCaps, p->NS, p->numKey, s,
                            esc_on(p) ? 2 * p->NS : -1, p->outc, p->dHybCap,
                            p->hybSymBin + 1, 2 * p->NS + 1);
    launch_bin_sort(p->numKey, m, nkeys, p->binCnt, p->binFill, p->binStart, p->numOrder, s);
  } else {
    launch_fill_i32(p->binStart, 0, nkeys + 1, s);  // light rows are done
  }
  ph_end(p, phR, s);
  check_launch("row pointer scan");
  HIP_CHECK(hipMemcpyAsync(p->hStats + 20, p->cRowOff + m, 8, hipMemcpyDeviceToHost, s));
  HIP_CHECK(hipMemcpyAsync(p->hBins, p->binStart, sizeof(int32_t) * (nkeys + 1), hipMemcpyDeviceToHost, s));
  HIP_CHECK(hipMemcpyAsync(p->hBins + 120, p->errWord, 4, hipMemcpyDeviceToHost, s));
  HIP_CHECK(hipMemcpyAsync(p->hStats, p->stats, sizeof(int64_t) * kNumStats, hipMemcpyDeviceToHost, s));
  HIP_CHECK(hipStreamSynchronize(s));
  check_device_errors(p, p->hBins[120]);
  p->numBinStart.assign(p->hBins, p->hBins + nkeys + 1);
  p->st.hybrid_rows = p->numBinStart[nkeys] - p->numBinStart[2 * p->NS + 1];
  p->nnzC = p->hStats[20];
  p->st.nnz_c = p->nnzC;
  p->st.lds_dense_products = p->hStats[kStatDenseElems];
  p->st.lds_hash_products = p->st.products - p->st.lds_dense_products;
  p->st.global_products = 0;
  if (!p->opts.rowptr64 && p->nnzC > index_limit(p))
    throw Error{SPGEMM_ERR_INDEX_OVERFLOW,
                "nnz(C) = " + std::to_string(p->nnzC) +
                    " exceeds the int32 row pointers; request rowptr64"};
  launch_write_rowptr(p->cRowOff, m + 1, dRowPtr, p->opts.rowptr64 ? 1 : 0, s);
  check_launch("row pointer write");
  *nnzC = p->nnzC;
  p->st.ms_symbolic = now_ms() - t0;
}

void do_numeric(spgemm_plan_t p, int32_t* ccol, void* cval) {
  const double t0 = now_ms();
  fork(p);
  const RowArgs a = row_args(p);
  const int phL = ph_begin(p, SPGEMM_PH_NUM_LIGHT, p->sl);
  if (p->wf != 0)
    launch_compact_rows(p->f64, p->m, p->rowBin, p->NS + 1, p->tmpOff, p->cnt, p->cRowOff,
                        p->tcol1, p->tval1, p->tcol2, p->tval2, ccol, cval, p->sl);
  if (p->wf == 0)
    launch_num_rows_esc(p->f64, p->numOrder + p->numBinStart[2 * p->NS],
                        p->numBinStart[2 * p->NS + 1] - p->numBinStart[2 * p->NS], a, p->cRowOff,
                        ccol, cval, p->errWord, p->sl);
  for (int b = 0; p->wf == 0 && b < p->NS; ++b) {
    const int64_t st = p->numBinStart[b], en = p->numBinStart[b + 1];
    launch_num_rows(p->numBins[b], p->f64, p->numOrder + st, en - st, a, p->cRowOff, ccol, cval,
                    p->errWord, p->sl);
    const int64_t ws = p->numBinStart[p->NS + b], we = p->numBinStart[p->NS + b + 1];
    if (we > ws)
      launch_num_rows_win(p->symBins[b], p->winWords[b], p->f64, p->numOrder + ws, we - ws, a,
                          p->cRowOff, ccol, cval, p->errWord, p->sl);
    const int64_t hs = p->numBinStart[2 * p->NS + 1 + b], he = p->numBinStart[2 * p->NS + 2 + b];
    if (he > hs)
      launch_num_rows_hyb(p->numBins[b], p->f64, p->numOrder + hs, he - hs, a, p->m, p->n,
                          p->cRowOff, ccol, cval, p->errWord, p->sl);
  }
  ph_end(p, phL, p->sl);
  check_launch("light numeric");
  if (p->h > 0) heavy_numeric(p, ccol, cval);
  join(p);
  if (p->opts.debug_device_error)
    launch_fill_i32(p->errWord, (int32_t)p->opts.debug_device_error, 1, p->stream);
  p->st.ms_numeric = now_ms() - t0;
}

template <typename F>
spgemm_status guarded(spgemm_plan_t p, F&& f) {
  try {
    f();
    return SPGEMM_OK;
  } catch (const Error& e) {
    if (p) {
      p->err = e.msg;
      p->state = -1;
    }
    g_thread_error = e.msg;
    return e.st;
  } catch (const std::exception& e) {
    if (p) {
      p->err = e.what();
      p->state = -1;
    }
    g_thread_error = e.what();
    return SPGEMM_ERR_INTERNAL;
  }
}

void destroy_plan(spgemm_plan_t p) {
  if (!p) return;
  if (p->sl && p->sl != p->stream && p->evL) {
    // Every stream waits for every other before any buffer is freed, so a
    // free on one stream never overtakes a use on another.
    (void)hipEventRecord(p->evL, p->sl);
    (void)hipEventRecord(p->evH, p->sh);
    (void)hipEventRecord(p->evD1, p->sd);
    (void)hipEventRecord(p->evFork, p->stream);
    (void)hipStreamWaitEvent(p->stream, p->evL, 0);
    (void)hipStreamWaitEvent(p->stream, p->evH, 0);
    (void)hipStreamWaitEvent(p->stream, p->evD1, 0);
    (void)hipStreamWaitEvent(p->sd, p->evL, 0);
    (void)hipStreamWaitEvent(p->sd, p->evH, 0);
    (void)hipStreamWaitEvent(p->sd, p->evFork, 0);
    (void)hipStreamWaitEvent(p->sl, p->evH, 0);
    (void)hipStreamWaitEvent(p->sl, p->evD1, 0);
    (void)hipStreamWaitEvent(p->sl, p->evFork, 0);
    (void)hipStreamWaitEvent(p->sh, p->evL, 0);
    (void)hipStreamWaitEvent(p->sh, p->evD1, 0);
    (void)hipStreamWaitEvent(p->sh, p->evFork, 0);
  }
  arena_release(p);
  region_release(p);
  release(p);
  if (!p->phases.empty()) (void)hipStreamSynchronize(p->stream);
  for (auto& r : p->phases) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  if (p->evD0) (void)hipEventDestroy(p->evD0);
  if (p->evD1) (void)hipEventDestroy(p->evD1);
  if (p->evFork) (void)hipEventDestroy(p->evFork);
  if (p->evL) (void)hipEventDestroy(p->evL);
  if (p->evH) (void)hipEventDestroy(p->evH);
  delete p;
}

}  // namespace

// ====================================================================== ABI
extern "C" {

spgemm_status spgemm_plan(spgemm_plan_t* out, int64_t m, int64_t k, int64_t n,
                          const int32_t* dA_row_ptr, const int32_t* dA_col, const void* dA_val,
                          int64_t nnzA, const int32_t* dB_row_ptr, const int32_t* dB_col,
                          const void* dB_val, int64_t nnzB, spgemm_dtype dtype,
                          const spgemm_options* opts, void* stream) {
  if (!out) {
    g_thread_error = "out is NULL";
    return SPGEMM_ERR_INVALID_ARG;
  }
  *out = nullptr;
  if (m < 0 || k < 0 || n < 0 || nnzA < 0 || nnzB < 0 || (dtype != SPGEMM_F32 && dtype != SPGEMM_F64)) {
    g_thread_error = "negative size or bad dtype";
    return SPGEMM_ERR_INVALID_ARG;
  }
  if (!dA_row_ptr || !dB_row_ptr || (nnzA > 0 && (!dA_col || !dA_val)) ||
      (nnzB > 0 && (!dB_col || !dB_val))) {
    g_thread_error = "null device pointer";
    return SPGEMM_ERR_INVALID_ARG;
  }
  if (m >= INT32_MAX || k >= INT32_MAX || n >= INT32_MAX || nnzA > INT32_MAX || nnzB > INT32_MAX) {
    g_thread_error = "a size exceeds the int32 index range";
    return SPGEMM_ERR_INDEX_OVERFLOW;
  }
  spgemm_plan_t p = new spgemm_plan_s();
  p->m = m;
  p->k = k;
  p->n = n;
  p->nnzA = nnzA;
  p->nnzB = nnzB;
  p->arp = dA_row_ptr;
  p->acol = dA_col;
  p->aval = dA_val;
  p->brp = dB_row_ptr;
  p->bcol = dB_col;
  p->bval = dB_val;
  p->f64 = dtype == SPGEMM_F64;
  if (opts) p->opts = *opts;
  p->stream = (hipStream_t)stream;
  spgemm_status st = guarded(p, [&] { do_plan(p); });
  if (st != SPGEMM_OK) {
    g_thread_error = p->err;
    destroy_plan(p);
    return st;
  }
  *out = p;
  return SPGEMM_OK;
}

spgemm_status spgemm_symbolic(spgemm_plan_t p, void* dC_row_ptr, int64_t* nnzC) {
  if (!p || !nnzC || !dC_row_ptr) return SPGEMM_ERR_INVALID_ARG;
  if (p->state != 0) {
    p->err = "symbolic must follow a successful plan, once";
    return SPGEMM_ERR_STATE;
  }
  spgemm_status st = guarded(p, [&] { do_symbolic(p, dC_row_ptr, nnzC); });
  if (st == SPGEMM_OK) p->state = 1;
  return st;
}

spgemm_status spgemm_numeric(spgemm_plan_t p, int32_t* dC_col, void* dC_val) {
  if (!p) return SPGEMM_ERR_INVALID_ARG;
  if (p->state != 1) {
    p->err = "numeric must follow a successful symbolic, once";
    return SPGEMM_ERR_STATE;
  }
  if (p->nnzC > 0 && (!dC_col || !dC_val)) return SPGEMM_ERR_INVALID_ARG;
  spgemm_status st = guarded(p, [&] { do_numeric(p, dC_col, dC_val); });
  if (st == SPGEMM_OK) p->state = 2;
  return st;
}

spgemm_status spgemm_row_estimates(spgemm_plan_t p, int64_t* dCap, double* dEst) {
  if (!p) return SPGEMM_ERR_INVALID_ARG;
  if (p->state < 1 || p->wf == 0) {
    p->err = "row estimates exist after spgemm_symbolic with workflow 1 or 2";
    return SPGEMM_ERR_STATE;
  }
  if (dEst && p->wf != 2) {
    p->err = "estimates exist with workflow 2 only";
    return SPGEMM_ERR_INVALID_ARG;
  }
  return guarded(p, [&] {
    if (dCap)
      HIP_CHECK(hipMemcpyAsync(dCap, p->capL, sizeof(int64_t) * p->m, hipMemcpyDeviceToDevice,
                               p->stream));
    if (dEst)
      HIP_CHECK(hipMemcpyAsync(dEst, p->estL, sizeof(double) * p->m, hipMemcpyDeviceToDevice,
                               p->stream));
  });
}

spgemm_status spgemm_wait(spgemm_plan_t p) {
  if (!p) return SPGEMM_ERR_INVALID_ARG;
  return guarded(p, [&] {
    if (p->sl && p->sl != p->stream) {
      HIP_CHECK(hipStreamSynchronize(p->sl));
      HIP_CHECK(hipStreamSynchronize(p->sh));
    }
    const int32_t word = read_err(p, p->stream);
    p->st.device_errors = word;
    check_device_errors(p, word);
  });
}

spgemm_status spgemm_get_stats(spgemm_plan_t p, spgemm_stats* out) {
  if (!p || !out) return SPGEMM_ERR_INVALID_ARG;
  spgemm_status st = guarded(p, [&] {
    if (p->state >= 1) {
      const int32_t word = read_err(p, p->stream);
      p->st.device_errors = word;
      if (p->opts.profile) ph_collect(p);
      if (p->state >= 2 && p->h > 0 && !p->symVals) {
        // the batched schedule bins the chunks (and counts the dense
        // accumulators' products) in numeric
        HIP_CHECK(hipMemcpyAsync(p->hStats + 24, p->stats + kStatDenseElems, 8,
                                 hipMemcpyDeviceToHost, p->stream));
        HIP_CHECK(hipStreamSynchronize(p->stream));
        p->st.lds_dense_products = p->hStats[24];
        p->st.lds_hash_products = p->st.products - p->st.lds_dense_products;
      }
      check_device_errors(p, word);
    }
  });
  *out = p->st;
  return st;
}

void spgemm_destroy(spgemm_plan_t p) { destroy_plan(p); }

const char* spgemm_status_string(spgemm_status s) {
  switch (s) {
    case SPGEMM_OK: return "ok";
    case SPGEMM_ERR_INVALID_ARG: return "invalid argument";
    case SPGEMM_ERR_INVALID_CSR: return "input is not canonical CSR";
    case SPGEMM_ERR_INDEX_OVERFLOW: return "index overflow";
    case SPGEMM_ERR_OOM: return "out of device memory";
    case SPGEMM_ERR_HIP: return "HIP runtime error";
    case SPGEMM_ERR_STATE: return "call order violated";
    case SPGEMM_ERR_INTERNAL: return "internal capacity check failed";
  }
  return "unknown status";
}

const char* spgemm_last_error(spgemm_plan_t p) {
  return p ? p->err.c_str() : g_thread_error.c_str();
}

}  // extern "C"

// ============================================================ prune / renorm
struct spgemm_prune_s {
  int64_t m = 0, n = 0;
  const void* rp = nullptr;
  int rp64 = 0;
  const int32_t* col = nullptr;
  const void* val = nullptr;
  bool f64 = false;
  double thr = 0;
  bool mcl = false;  // normalise, prune, square (else prune, normalise)
  hipStream_t stream = nullptr;
  int64_t *keep = nullptr, *off = nullptr, *tmp = nullptr;
  double* colsum = nullptr;
  float* inv = nullptr;     // fp32 values: reciprocals of the column sums
  void* buckets = nullptr;  // column buckets of the count (fill, columns, values)
  int64_t nnzOut = 0;
  int state = 0;
  std::string err;
  int64_t* hbuf = nullptr;
};

namespace {
void prune_free(spgemm_prune_t p) {
  if (!p) return;
  for (void* ptr : {(void*)p->keep, (void*)p->off, (void*)p->tmp, (void*)p->colsum, p->buckets})
    if (ptr) (void)hipFreeAsync(ptr, p->stream);
  if (p->hbuf) {
    (void)hipStreamSynchronize(p->stream);
    (void)hipHostFree(p->hbuf);
  }
  delete p;
}
}  // namespace

namespace {
spgemm_status prune_count(bool mcl, spgemm_prune_t* out, int64_t m, int64_t n,
                          const void* dC_row_ptr, int32_t c_rowptr64, const int32_t* dC_col,
                          const void* dC_val, spgemm_dtype dtype, double threshold,
                          void* dOut_row_ptr, int32_t out_rowptr64, int64_t* nnzOut,
                          void* stream) {
  if (!out || !nnzOut || !dC_row_ptr || !dOut_row_ptr || m < 0 || n < 0 ||
      (dtype != SPGEMM_F32 && dtype != SPGEMM_F64)) {
    g_thread_error = "invalid argument";
    return SPGEMM_ERR_INVALID_ARG;
  }
  *out = nullptr;
  spgemm_prune_t p = new spgemm_prune_s();
  p->m = m;
  p->n = n;
  p->rp = dC_row_ptr;
  p->rp64 = c_rowptr64;
  p->col = dC_col;
  p->val = dC_val;
  p->f64 = dtype == SPGEMM_F64;
  p->thr = threshold;
  p->mcl = mcl;
  p->stream = (hipStream_t)stream;
  try {
    hipStream_t s = p->stream;
    HIP_CHECK(hipHostMalloc((void**)&p->hbuf, 64, hipHostMallocDefault));
    HIP_CHECK(hipMallocAsync((void**)&p->keep, sizeof(int64_t) * std::max<int64_t>(m, 1), s));
    HIP_CHECK(hipMallocAsync((void**)&p->off, sizeof(int64_t) * (m + 1), s));
    HIP_CHECK(hipMallocAsync((void**)&p->tmp, sizeof(int64_t) * (scan_tmp_elems(m) + 1), s));
    // column sums (fp64), then for fp32 values their reciprocals (fp32)
    HIP_CHECK(hipMallocAsync((void**)&p->colsum,
                             (sizeof(double) + (p->f64 ? 0 : sizeof(float))) *
                                 std::max<int64_t>(n, 1),
                             s));
    if (!p->f64) p->inv = (float*)(p->colsum + std::max<int64_t>(n, 1));
    launch_fill_i64((int64_t*)p->colsum, 0, n, s);  // +0.0 has an all-zero bit pattern
    // Column buckets for the count's column sums (each work group's LDS
    // table and the entries it misses): room for min(nnz(C), 2^29) entries
    // spread evenly (full buckets fall back to global adds).
    int log2Cols = 0;
    int32_t nb = 0;
    int64_t cap = 0;
    unsigned long long* fill = nullptr;
    int32_t* bcol = nullptr;
    double* bval = nullptr;
    if (m > 0 && prune_buckets_fit(n, &log2Cols, &nb)) {
      HIP_CHECK(hipMemcpyAsync(p->hbuf, (const char*)p->rp + m * (p->rp64 ? 8 : 4),
                               p->rp64 ? 8 : 4, hipMemcpyDeviceToHost, s));
      HIP_CHECK(hipStreamSynchronize(s));
      const int64_t nnzC = p->rp64 ? p->hbuf[0] : (int64_t)((const int32_t*)p->hbuf)[0];
      cap = (std::min<int64_t>(nnzC, (int64_t)1 << 29) + nb - 1) / nb;
      if (cap > 0) {
        const size_t bytes = 8 * kFillStride * (size_t)nb + (size_t)nb * cap * 12;
        HIP_CHECK(hipMallocAsync(&p->buckets, bytes, s));
        fill = (unsigned long long*)p->buckets;
        bval = (double*)(fill + kFillStride * (size_t)nb);
        bcol = (int32_t*)(bval + (size_t)nb * cap);
        launch_fill_i64((int64_t*)fill, 0, kFillStride * nb, s);
      }
    }
    auto count = [&](double thr) {
      if (fill)
        launch_prune_count_b(m, n, p->rp, p->rp64, p->col, p->val, p->f64, thr, p->keep,
                             p->colsum, nb, log2Cols, cap, fill, bcol, bval, s);
      else
        launch_prune_count(m, p->rp, p->rp64, p->col, p->val, p->f64, thr, p->keep, p->colsum,
                           s);
    };
    if (mcl) {
      // Column sums of every entry, then the kept count of every row.
      count(-INFINITY);
      launch_mcl_count(m, p->rp, p->rp64, p->col, p->val, p->f64, p->thr, p->colsum, p->keep, s);
    } else {
      count(p->thr);
      if (p->inv) launch_colsum_recip(n, p->colsum, p->inv, s);
    }
    launch_scan_i64(p->keep, m, p->off, p->tmp, s);
    check_launch("prune count");
    HIP_CHECK(hipMemcpyAsync(p->hbuf, p->off + m, 8, hipMemcpyDeviceToHost, s));
    HIP_CHECK(hipStreamSynchronize(s));
    p->nnzOut = p->hbuf[0];
    if (p->buckets) {  // only the count uses them
      HIP_CHECK(hipFreeAsync(p->buckets, s));
      p->buckets = nullptr;
    }
    if (!out_rowptr64 && p->nnzOut > INT32_MAX)
      throw Error{SPGEMM_ERR_INDEX_OVERFLOW, "kept entries exceed INT32_MAX"};
    launch_write_rowptr(p->off, m + 1, dOut_row_ptr, out_rowptr64 ? 1 : 0, s);
    check_launch("prune row pointers");
  } catch (const Error& e) {
    g_thread_error = e.msg;
    prune_free(p);
    return e.st;
  }
  *nnzOut = p->nnzOut;
  *out = p;
  return SPGEMM_OK;
}

}  // namespace

extern "C" spgemm_status spgemm_prune_colnorm_count(
    spgemm_prune_t* out, int64_t m, int64_t n, const void* dC_row_ptr, int32_t c_rowptr64,
    const int32_t* dC_col, const void* dC_val, spgemm_dtype dtype, double threshold,
    void* dOut_row_ptr, int32_t out_rowptr64, int64_t* nnzOut, void* stream) {
  return prune_count(false, out, m, n, dC_row_ptr, c_rowptr64, dC_col, dC_val, dtype, threshold,
                     dOut_row_ptr, out_rowptr64, nnzOut, stream);
}

extern "C" spgemm_status spgemm_mcl_inflate_count(
    spgemm_prune_t* out, int64_t m, int64_t n, const void* dC_row_ptr, int32_t c_rowptr64,
    const int32_t* dC_col, const void* dC_val, spgemm_dtype dtype, double threshold,
    void* dOut_row_ptr, int32_t out_rowptr64, int64_t* nnzOut, void* stream) {
  return prune_count(true, out, m, n, dC_row_ptr, c_rowptr64, dC_col, dC_val, dtype, threshold,
                     dOut_row_ptr, out_rowptr64, nnzOut, stream);
}

namespace {
spgemm_status prune_fill(bool mcl, spgemm_prune_t p, int32_t* dOut_col, void* dOut_val) {
  if (!p) return SPGEMM_ERR_INVALID_ARG;
  if (p->mcl != mcl) return SPGEMM_ERR_STATE;
  if (p->state != 0) return SPGEMM_ERR_STATE;
  if (p->nnzOut > 0 && (!dOut_col || !dOut_val)) return SPGEMM_ERR_INVALID_ARG;
  try {
    if (mcl)
      launch_mcl_fill(p->m, p->rp, p->rp64, p->col, p->val, p->f64, p->thr, p->off, p->colsum,
                      dOut_col, dOut_val, p->stream);
    else
      launch_prune_fill(p->m, p->rp, p->rp64, p->col, p->val, p->f64, p->thr, p->off,
                        p->colsum, p->inv, dOut_col, dOut_val, p->stream);
    check_launch("prune fill");
  } catch (const Error& e) {
    p->err = e.msg;
    g_thread_error = e.msg;
    return e.st;
  }
  p->state = 1;
  return SPGEMM_OK;
}
}  // namespace

extern "C" spgemm_status spgemm_prune_colnorm_fill(spgemm_prune_t p, int32_t* dOut_col,
                                                   void* dOut_val) {
  return prune_fill(false, p, dOut_col, dOut_val);
}

extern "C" spgemm_status spgemm_mcl_inflate_fill(spgemm_prune_t p, int32_t* dOut_col,
                                                 void* dOut_val) {
  return prune_fill(true, p, dOut_col, dOut_val);
}

extern "C" void spgemm_prune_destroy(spgemm_prune_t p) { prune_free(p); }

// ================================================================ transpose
namespace sg {

// Validation shared by both transpose entry points; 0 when the arguments
// are usable, else the status (message in g_thread_error).
spgemm_status transpose_check_args(int64_t m, int64_t n, int64_t nnz, const void* dA_row_ptr,
                                   const int32_t* dA_col, const void* dA_val,
                                   spgemm_dtype dtype, void* dT_row_ptr, int32_t t_rowptr64,
                                   int32_t* dT_col, void* dT_val) {
  if (m < 0 || n < 0 || nnz < 0 || !dT_row_ptr || (m > 0 && !dA_row_ptr) ||
      (nnz > 0 && (!dA_col || !dT_col || (dA_val && !dT_val))) ||
      (dtype != SPGEMM_F32 && dtype != SPGEMM_F64)) {
    g_thread_error = "invalid argument";
    return SPGEMM_ERR_INVALID_ARG;
  }
  if (m > INT32_MAX || n > INT32_MAX || (!t_rowptr64 && nnz > INT32_MAX)) {
    g_thread_error = "size exceeds the int32 index range";
    return SPGEMM_ERR_INDEX_OVERFLOW;
  }
  return SPGEMM_OK;
}

namespace {
struct TrLayout {
  TransposePlan tp;
  int64_t szRows, szKeys, szVals, szHist, szOff, szTmp, total;
  int nVals;
  bool multi;
};
TrLayout transpose_layout(int64_t n, int64_t nnz, int vb, bool vals) {
  TrLayout L{};
  L.tp = transpose_plan(n, nnz);
  auto al = [](int64_t b) { return (b + 255) & ~(int64_t)255; };
  const int64_t ent = std::max<int64_t>(nnz, 1);
  L.multi = L.tp.passes > 1;
  L.szRows = al(4 * ent);
  L.szKeys = al(4 * ent);
  L.szVals = al((int64_t)vb * ent);
  L.nVals = vals ? (L.tp.passes > 2 ? 2 : (L.multi ? 1 : 0)) : 0;
  L.szHist = al(4 * std::max<int64_t>(L.tp.histElems, 1));
  L.szOff = al(8 * (L.tp.histElems + 1));
  L.szTmp = al(8 * (scan_tmp_elems(L.tp.histElems) + 1));
  L.total = L.szRows * (L.multi ? 2 : 1) + L.szKeys * (L.multi ? 2 : 1) + L.szVals * L.nVals +
            L.szHist + L.szOff + L.szTmp + 256;
  return L;
}
}  // namespace

int64_t transpose_workspace_bytes(int64_t n, int64_t nnz, spgemm_dtype dtype, bool vals) {
  return transpose_layout(n, nnz, dtype == SPGEMM_F64 ? 8 : 4, vals).total;
}

// The transpose with its temporaries carved from `ws` (at least
// transpose_workspace_bytes): enqueues everything on `s`, then blocks once
// to read the column check.  Every piece of `ws` that must start at zero is
// cleared by a kernel here.
spgemm_status transpose_run(int64_t m, int64_t n, int64_t nnz, const void* dA_row_ptr,
                            int32_t a_rowptr64, const int32_t* dA_col, const void* dA_val,
                            spgemm_dtype dtype, void* dT_row_ptr, int32_t t_rowptr64,
                            int32_t* dT_col, void* dT_val, char* ws, hipStream_t s) {
  const int vb = dtype == SPGEMM_F64 ? 8 : 4;
  const TrLayout L = transpose_layout(n, nnz, vb, dA_val != nullptr);
  try {
    char* q = ws;
    auto take = [&](int64_t b) {
      char* r = q;
      q += b;
      return r;
    };
    int32_t* rows[2] = {nullptr, nullptr};
    uint32_t* keys[2] = {nullptr, nullptr};
    void* vals[2] = {nullptr, nullptr};
    rows[1] = (int32_t*)take(L.szRows);
    if (L.multi) rows[0] = (int32_t*)take(L.szRows);
    keys[0] = (uint32_t*)take(L.szKeys);
    if (L.multi) keys[1] = (uint32_t*)take(L.szKeys);
    for (int i = 0; i < L.nVals; ++i) vals[i] = take(L.szVals);
    int32_t* hist = (int32_t*)take(L.szHist);
    int64_t* off = (int64_t*)take(L.szOff);
    int64_t* tmp = (int64_t*)take(L.szTmp);
    int32_t* err = (int32_t*)take(256);
    launch_fill_i32(err, 0, 1, s);
    launch_transpose(L.tp, m, n, nnz, dA_row_ptr, a_rowptr64, dA_col, dA_val, vb, dT_row_ptr,
                     t_rowptr64, dT_col, dT_val, rows, keys, vals, hist, off, tmp, err, s);
    check_launch("transpose");
    int32_t herr = 0;
    HIP_CHECK(hipMemcpyAsync(&herr, err, sizeof(herr), hipMemcpyDeviceToHost, s));
    HIP_CHECK(hipStreamSynchronize(s));
    if (herr & kErrCsr) throw Error{SPGEMM_ERR_INVALID_CSR, "column index outside [0, n)"};
  } catch (const Error& e) {
    g_thread_error = e.msg;
    return e.st;
  }
  return SPGEMM_OK;
}

void set_thread_error(const char* msg) { g_thread_error = msg; }

}  // namespace sg

extern "C" spgemm_status spgemm_transpose(int64_t m, int64_t n, int64_t nnz,
                                          const void* dA_row_ptr, int32_t a_rowptr64,
                                          const int32_t* dA_col, const void* dA_val,
                                          spgemm_dtype dtype, void* dT_row_ptr,
                                          int32_t t_rowptr64, int32_t* dT_col, void* dT_val,
                                          void* stream) {
  spgemm_status st = transpose_check_args(m, n, nnz, dA_row_ptr, dA_col, dA_val, dtype,
                                          dT_row_ptr, t_rowptr64, dT_col, dT_val);
  if (st != SPGEMM_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  const int64_t total = transpose_workspace_bytes(n, nnz, dtype, dA_val != nullptr);
  // One allocation, carved into 256-byte aligned pieces.
  char* buf = nullptr;
  if (hipMallocAsync((void**)&buf, (size_t)total, s) != hipSuccess) {
    (void)hipGetLastError();
    g_thread_error = "device allocation failed";
    return SPGEMM_ERR_OOM;
  }
  st = transpose_run(m, n, nnz, dA_row_ptr, a_rowptr64, dA_col, dA_val, dtype, dT_row_ptr,
                     t_rowptr64, dT_col, dT_val, buf, s);
  (void)hipFreeAsync(buf, s);
  return st;
}
