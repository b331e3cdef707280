// Declarations shared between the host orchestrator (api.cpp) and the kernel
// translation units.  Every launcher enqueues on the given stream and
// returns without synchronising.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/spgemm.h"

namespace sg {

constexpr int32_t kEmptyKey = -1;

// Bits of the plan's device status word.
enum : int32_t {
  kErrHashFull = 1,       // an LDS hash table ran out of slots
  kErrCsr = 2,            // validation found a non-canonical input
  kErrRowsPerBlock = 4,   // a multisplit work group met more rows than sized for
  kErrCountMismatch = 8,  // numeric produced a row/chunk size != symbolic
};

// Indices of the per-plan int64 counters filled by the row-information pass.
enum : int {
  kStatProducts = 0,
  kStatHeavyProducts = 1,
  kStatHeavyANnz = 2,
  kStatMaxRowProducts = 3,
  kStatHeavyRows = 4,
  kStatLightRows = 5,
  kStatDenseElems = 6,
  kNumStats = 8,
};

// One LDS hash-accumulator bin: items with size <= cap run with `tpr`
// threads each, `rpb` items per work group, a table of T = tpr*spt slots and
// (numeric) a sort of N = next_pow2(cap) entries.
struct BinCfg {
  int32_t cap;
  int32_t tpr;
  int32_t rpb;
  int32_t spt;
  int32_t T;
  int32_t N;
  size_t lds;  // dynamic LDS bytes per work group
};

struct RowArgs {
  const int32_t* arp;
  const int32_t* acol;
  const void* aval;
  const int32_t* brp;
  const int32_t* bcol;
  const void* bval;
  const int32_t* scanA;  // row-local exclusive product offset of each A entry
  const int64_t* rowP;   // products per row
  const int64_t* rowWin; // dense-window rows: first product column (low 32
                         // bits) and span in 32-bit words (high bits)
};

// Dense window of a light row (gMAGNUS page §III-E: any local-memory
// accumulator; Ocean page §2: hash-based and dense accumulators chosen per
// row): a row whose products span at most 32 * window_words(cap) columns,
// cap being its bin's product bound, is accumulated in an LDS bitmap over
// [lo, lo + 32 * words) and a dense array indexed by bitmap rank instead of a
// hash table.  The bitmap (16 bytes per product of the bin's bound) stays
// within a small multiple of the hash table it replaces, and at most 65536
// columns wide.
// LDS the light numeric kernel reserves for the radix sort of a row's
// entries (one row per work group, at least 256 threads): per wave 256
// 16-bit digit counters, 256 digit bases, and a min/max per wave.
__host__ __device__ inline size_t num_rows_radix_bytes(int tpr, int rpb) {
  return (rpb == 1 && tpr >= 256) ? (size_t)(tpr / 64) * 256 * 2 + 256 * 4 + (size_t)(tpr / 64) * 8
                                  : 0;
}

// Diagonal window of the hybrid light-row accumulator (window plus outlier
// table): columns per row, and bitmap words.
constexpr int kHybW = 2048;
constexpr int kHybWords = kHybW / 32;
// Symbolic bins from this product bound on take the hybrid kernel.
constexpr int64_t kHybMinCap = 512;
// Outliers a row may have to take the hybrid numeric kernel.
constexpr int32_t kHybOutMax = 512;

__host__ __device__ inline int32_t window_words(int64_t cap) {
  return (int32_t)(4 * cap < 2048 ? 4 * cap : 2048);
}

// Final chunks of the heavy rows, in the order they were listed.  Chunk c
// holds cnt[c] elements at off[c] of buffer buf[c]; it belongs to heavy row
// row[c] and covers the W-wide column slots starting at slot[c] (its column
// base is slot[c] * W).
struct ChunkList {
  const int64_t* off;
  const int32_t* cnt;
  const int32_t* row;
  const int32_t* slot;
  const int8_t* buf;
  const void* col0;       // final columns: int32_t, or uint16_t with col16
  const void* col1;
  const void* val0;
  const void* val1;
  int64_t W;
  int64_t nreq;           // W-wide slots per heavy row
  const int32_t* xheavy;  // heavy row index -> row of C
  const int64_t* slotOff; // exclusive offset of each slot inside its row
  int32_t* slotNnz;       // nnz per slot: of the chunk starting there (the
                          // chunk symbolic kernels; 0 in its other slots),
                          // or of the slot alone (heavy-row symbolic)
  int32_t col16;          // chunk columns stored as uint16_t
  const int8_t* span;     // log2 of the W-wide slots each chunk covers
};

// Everything a numeric chunk kernel needs about one final chunk, gathered
// once per batch in the order the kernels take the chunks: where its
// elements are, where its entries go, and how many there are.
struct ChunkDesc {
  int64_t off;      // first element in its buffer
  int64_t base;     // first output position in C
  int32_t cnt;      // elements
  int32_t want;     // distinct columns (from symbolic)
  int32_t colBase;  // global column of local column 0
  int32_t buf;      // buffer holding the elements (0 or 1)
  int32_t row;      // row of C (and of A) the chunk belongs to
};


// What a multisplit work group needs to know about its tile of elements.
struct TileInfo {
  int32_t r0, nrows;  // first row meeting the tile, rows meeting it
  int32_t t0, t1;     // first entry, bound on the last (fed from A and B)
  int64_t bnd0;       // first row boundary inside the tile (nrows > 1)
};

// ---- k_util.hip ----
// dst[0..n) = vals[0..n) for n <= 64, the values passed as kernel arguments.
void launch_set_small_i32(int32_t* dst, const int32_t* vals, int n, hipStream_t s);
// tail[0..3) = (ctr[0], ctr[1], newOff[ctr[0]]).
void launch_level_tail(const int32_t* ctr, const int64_t* newOff, int64_t* tail, hipStream_t s);
void launch_fill_i32(int32_t* p, int32_t v, int64_t n, hipStream_t s);
void launch_fill_i64(int64_t* p, int64_t v, int64_t n, hipStream_t s);
void launch_fill_i8(int8_t* p, int8_t v, int64_t n, hipStream_t s);
void launch_copy_i64(int64_t* dst, const int64_t* src, int64_t n, hipStream_t s);
// out[i] = sum_{j<i} in[j] for i in [0, n]; out has n+1 entries.  tmp needs
// scan_tmp_elems(n) int64 entries.
int64_t scan_tmp_elems(int64_t n);
void launch_scan_i64(const int64_t* in, int64_t n, int64_t* out, int64_t* tmp, hipStream_t s);
void launch_scan_i32(const int32_t* in, int64_t n, int64_t* out, int64_t* tmp, hipStream_t s);
// Counting sort of item indices by an 8-bit key (keys >= nbins are dropped).
// cnt/fill: nbins int32 scratch; start: nbins+1 int32 (bin offsets).
void launch_bin_sort(const uint8_t* key, int64_t n, int nbins, int32_t* cnt, int32_t* fill,
                     int32_t* start, int32_t* out, hipStream_t s);
// Scratch entries (int64) launch_row_info needs for its per-work-group
// partials and its list of long rows.
int64_t row_info_partials(int64_t m, int64_t nnzA);
// rowWin (null: no window bins) receives, for light rows of the first
// winBins bins whose products fit their bin's window, the span's first
// column and its length in 32-bit words (see RowArgs); those rows get bin
// nbins + 2 + b instead of 1 + b; winMax[b] (zeroed by the caller) receives
// the widest window of bin b in words.
// bSpan: first and last column of every B row (launch_b_span), needed with
// rowWin.
void launch_b_span(int64_t K, const int32_t* brp, const int32_t* bcol, int2* span, hipStream_t s);
void launch_row_info(int64_t m, int64_t nnzA, const int32_t* arp, const int32_t* acol,
                     const int32_t* brp, const int2* bSpan, int64_t tau, const int32_t* caps,
                     int nbins,
                     int64_t* rowP, int32_t* scanA, uint8_t* rowBin, int64_t* rowWin,
                     int winBins, int32_t* winMax, int64_t* part, int64_t* stats,
                     hipStream_t s);
void launch_validate(int64_t rows, int64_t cols, int64_t nnz, const int32_t* rp,
                     const int32_t* col, int32_t* err, hipStream_t s);
void launch_write_rowptr(const int64_t* off, int64_t n, void* out, int is64, hipStream_t s);
void launch_gather_i64(const int64_t* src, const int32_t* idx, int64_t n, int64_t* dst,
                       hipStream_t s);
// dst[i] = rp[rows[i] + 1] - rp[rows[i]]
void launch_row_lengths(int64_t n, const int32_t* rows, const int32_t* rp, int64_t* dst,
                        hipStream_t s);
// key[i] = bin of cnt[rows[i]] among caps[0..nbins) (first cap >= value), for
// light rows; heavy rows (rowBin == heavyBin) get 255; with escKey >= 0,
// rows of the first product bin (at most 32 products) get escKey.
// With outc: a row of a symbolic bin from hybSymMin on (its outlier count
// in outc) whose outliers fit hybCap[b] of its numeric bin b gets hybKey + b.
void launch_numeric_row_bins(int64_t m, const int64_t* cnt, const uint8_t* rowBin,
                             int heavyBin, const int32_t* caps, int nbins, uint8_t* key,
                             hipStream_t s, int escKey = -1, const int32_t* outc = nullptr,
                             const int32_t* hybCap = nullptr, int hybSymMin = 0,
                             int hybKey = 0);

// ---- k_light.hip ----
void light_set_attributes();
// Dense-window light rows (window_words(b.cap) bitmap words per row); LDS
// bytes per work group of the symbolic or numeric kernel.
// `words`: the widest window among the rows (at most window_words(b.cap)).
size_t window_row_lds(bool numeric, bool f64, const BinCfg& b, int32_t words);
void launch_sym_rows_win(const BinCfg& b, int32_t words, const int32_t* rows, int64_t nrows,
                         const RowArgs& a, int64_t* cnt, hipStream_t s);
// cntOut (size-estimate workflows): cRowOff holds capacities; each row's
// count, or -1 when it did not fit, goes to cntOut (no device error).
void launch_num_rows_win(const BinCfg& b, int32_t words, bool f64, const int32_t* rows,
                         int64_t nrows, const RowArgs& a, const int64_t* cRowOff, int32_t* ccol,
                         void* cval, int32_t* err, hipStream_t s, int64_t* cntOut = nullptr);
void launch_sym_rows(const BinCfg& b, const int32_t* rows, int64_t nrows, const RowArgs& a,
                     int64_t* cnt, int32_t* err, hipStream_t s);
// Hybrid light rows (diagonal window plus outlier table): symbolic for every
// row of a hash bin, storing its count and its outlier count; numeric for
// the rows whose outliers fit half of the bin's outlier table.
void launch_sym_rows_hyb(const BinCfg& b, const int32_t* rows, int64_t nrows, const RowArgs& a,
                         int64_t m, int64_t n, int64_t* cnt, int32_t* outc, int32_t* err,
                         hipStream_t s);
// Outliers a row may have to take the hybrid numeric kernel of bin b, or -1
// when the kernel has no instance for b or does not fit the LDS budget.
int32_t hyb_out_cap(const BinCfg& b, bool f64, int64_t lds);
void launch_num_rows_hyb(const BinCfg& b, bool f64, const int32_t* rows, int64_t nrows,
                         const RowArgs& a, int64_t m, int64_t n, const int64_t* cRowOff,
                         int32_t* ccol, void* cval, int32_t* err, hipStream_t s);
// Rows of at most 32 products (the first product bin) by expand-sort-compact
// in 32 lanes each: count of distinct columns, or the sorted row (cntOut as
// for launch_num_rows).
void launch_sym_rows_esc(const int32_t* rows, int64_t nrows, const RowArgs& a, int64_t* cnt,
                         hipStream_t s);
void launch_num_rows_esc(bool f64, const int32_t* rows, int64_t nrows, const RowArgs& a,
                         const int64_t* cRowOff, int32_t* ccol, void* cval, int32_t* err,
                         hipStream_t s, int64_t* cntOut = nullptr);
void launch_num_rows(const BinCfg& b, bool f64, const int32_t* rows, int64_t nrows,
                     const RowArgs& a, const int64_t* cRowOff, int32_t* ccol, void* cval,
                     int32_t* err, hipStream_t s, int64_t* cntOut = nullptr);
void launch_sym_chunks(const BinCfg& b, const ChunkDesc* desc, int64_t n, const ChunkList& cl,
                       int32_t* err, hipStream_t s);
// Heavy-row symbolic straight from A and B (batched schedule): per heavy
// row r and W-wide slot s, slotNnz[r * nreq + s] = distinct columns of the
// row's products inside the slot.  `next` is one int32, zeroed by the caller.
// Windows of 2^winBits columns (a power of two from W up to what ldsMax
// bytes of bitmap hold, at most nreq * W).
int32_t sym_heavy_window_bits(int64_t nreq, int32_t log2W, size_t ldsMax);
void launch_sym_heavy_rows(int64_t h, int64_t nreq, int32_t log2W, const int32_t* xheavy,
                           const RowArgs& a, int64_t nnzB, int32_t* slotNnz, int32_t* next,
                           int numCUs, size_t ldsMax, hipStream_t s);
// Whether a numeric bin's (tpr, sort size) has a kernel instance.
bool num_bin_supported(const BinCfg& b);
void launch_num_chunks(const BinCfg& b, bool f64, const ChunkDesc* desc, int64_t n,
                       const ChunkList& cl, int32_t* ccol, void* cval, int32_t* err,
                       hipStream_t s);
// Light chunks of at most 256 elements by expand-sort-compact in registers
// (false, with nothing launched, for a larger cap).
bool launch_num_chunks_esc(int32_t cap, bool f64, const ChunkDesc* desc, int64_t n,
                           const ChunkList& cl, int32_t* ccol, void* cval, int32_t* err,
                           hipStream_t s);

// ---- k_outer.hip, k_multisplit.hip, k_heavy.hip ----
void heavy_set_attributes();
void multisplit_set_attributes();
void launch_csc_count(int64_t h, const int32_t* xheavy, const int32_t* arp, const int32_t* acol,
                      int32_t* colCnt, hipStream_t s);
void launch_csc_fill(int64_t h, const int32_t* xheavy, const int32_t* arp, const int32_t* acol,
                     const void* aval, bool f64, int64_t* colFill, int32_t* cscRow,
                     int32_t* cscCol, void* cscVal, hipStream_t s);
void launch_entry_products(int64_t nE, const int32_t* cscCol, const int32_t* brp, int64_t* nb,
                           hipStream_t s);
void launch_seg_base(int64_t nE, const int32_t* cscRow, const int64_t* nb, int64_t* cursor,
                     int64_t* segBase, hipStream_t s);
void launch_outer_product(bool f64, int64_t Ph, const int64_t* entryOff, int64_t nE,
                          const int32_t* cscCol, const void* cscVal, const int64_t* segBase,
                          const int32_t* brp, const int32_t* bcol, const void* bval,
                          int32_t* outCol, void* outVal, hipStream_t s);
// Multisplit levels.  Input rows r in [0, R) hold elements
// [rowPtr[r], rowPtr[r+1]) whose chunk is col >> shift (< v).
// Elements per multisplit work group and the most input rows such a range
// can meet, for rows of more than tau elements and v chunks per row.
void multisplit_geometry(bool f64, int64_t tau, int v, int32_t* blockElems, int* maxRows);
// out[b] = the item t with off[t] <= b * G < off[t+1], for b < nBlocks: the
// first row (or entry) of each multisplit work group.
void launch_block_starts(int64_t nItems, const int64_t* off, int64_t G, int64_t nBlocks,
                         int32_t* out, hipStream_t s);
// info[b] for the tiles of blockElems elements (blkRow/blkEnt from
// launch_block_starts; blkEnt may be null).
void launch_tile_info(int64_t E, int32_t blockElems, const int64_t* rowPtr, int64_t R,
                      const int32_t* blkRow, const int32_t* blkEnt, int64_t nE, TileInfo* info,
                      hipStream_t s);
void launch_histogram(int64_t E, int32_t blockElems, const int64_t* rowPtr,
                      const TileInfo* info, const int32_t* col, int shift, int v, int maxRows,
                      int32_t* counts, int32_t* err, hipStream_t s);
// Runs of equal W-wide chunk in B's rows (chunk = col >> shift): runPtr[K+1],
// runChunk/runStart[runs + 1]; flags[nnzB] and runIdx[nnzB + 1] are scratch.
void launch_b_runs(int64_t K, int64_t nnzB, const int32_t* brp, const int32_t* bcol, int shift,
                   int32_t* flags, int64_t* runIdx, int64_t* scanTmp, int32_t* runPtr,
                   int32_t* runChunk, int32_t* runStart, hipStream_t s);
// CH[i][f] = products of row rows[i] in W-wide chunk f (nreq <= 16384).
// B's slot table (k_slot_table): (nreq + 1) run starts per B row.
void launch_slot_table(int64_t K, int32_t nreq, const int32_t* brp, const int32_t* runPtr,
                       const int32_t* runChunk, const int32_t* runStart, int32_t* tab,
                       hipStream_t s);
// annz: scan of the heavy rows' A lengths (hb + 1), nAh its total; parts
// (hb), itemPtr (hb + 1) and scanTmp (scan_tmp_elems(hb) + 1) are workspace.
void launch_chunk_hist_rows(int64_t hb, int64_t nAh, const int64_t* annz, const int32_t* rows,
                            const int32_t* arp, const int32_t* acol, const int32_t* runPtr,
                            const int32_t* runChunk, const int32_t* runStart, int32_t nreq,
                            int32_t* CH, int64_t* parts, int64_t* itemPtr, int64_t* scanTmp,
                            hipStream_t s);
// finalOf[row * nreq + slot] = the final chunk covering W-wide slot `slot`
// of batch row `row`, or -(chunk + 2) when key[chunk] == denseKey (a chunk
// accumulated straight from A and B, whose products the expansion skips;
// key may be null), spanOf[...] = that chunk's width as log2 of W-wide
// slots (slots of no chunk are left as they are).
void launch_final_map(int64_t nfc, const int32_t* fcRow, const int32_t* fcSlot,
                      const int8_t* fcSpan, int64_t nreq, const uint8_t* key, int denseKey,
                      int32_t* finalOf, int8_t* spanOf, hipStream_t s);
// out[c] = key[c] == denseKey ? 0 : cnt[c].
void launch_stored_counts(int64_t nfc, const int32_t* cnt, const uint8_t* key, int denseKey,
                          int32_t* out, hipStream_t s);
// One level's (row, chunk) counts as sums of `span` W-wide counts.
void launch_level_counts(int64_t Q, int v, int32_t span, int32_t nreq, const int32_t* inRow,
                         const int32_t* inSlot, const int32_t* CH, int32_t* counts,
                         hipStream_t s);
void launch_partition(int64_t Q, const int32_t* counts, int64_t tau, bool last, int v,
                      const int32_t* inRow, const int32_t* inSlot, int32_t slotStep,
                      int32_t* inv, int32_t* newCnt, int32_t* newRow, int32_t* newSlot,
                      int32_t* ctr, hipStream_t s);
// Source of a multisplit fed straight from the expansion: the heavy rows'
// A entries in row order, with the first product of each (eOff, nE + 1
// entries), its B row start and its A value.
struct ExpandSrc {
  const int64_t* eOff;
  const int32_t* eB;
  const void* eVal;
  const int32_t* bcol;
  const void* bval;
  int64_t nE;
};
// Heavy-row expansion straight into the final chunks (chunk tree known from
// the structure): tile geometry, false when (rows per tile) x nreq buckets
// cannot fit.
bool expand_final_geometry(bool f64, int64_t rowTau, int64_t nreq, int32_t* blockElems,
                           int* maxRows);
void launch_expand_final(bool f64, int64_t E, int32_t blockElems, const int64_t* rowPtr,
                         const TileInfo* info, const ExpandSrc& src, const int32_t* finalOf,
                         const int8_t* spanOf, int32_t nreq, int log2W, int maxRows,
                         int64_t* cursor, void* outCol, bool col16, void* outVal, int32_t* err,
                         hipStream_t s);
// One multisplit level.  inCol/inVal: the level's input, or src (not null)
// to make the elements from A and B.  outVal null: columns only.
void launch_multisplit(bool f64, int64_t E, int32_t blockElems, const int64_t* rowPtr,
                       const TileInfo* info, const int32_t* inCol, const void* inVal, const ExpandSrc* src,
                       int shift, int v, int32_t wmask, int maxRows, const int32_t* inv,
                       int64_t* cursor, int32_t* outCol, void* outVal, int32_t* err,
                       hipStream_t s);
// Heavy-row entries of rows[0..hb) in row order: entry t of local row q sits
// at rowEntry[q] - rowEntry[0] + (j - arp[rows[q]]); eB = B row start, nb =
// products, eVal = A value.
// eOff receives nE + 1 flattened product offsets (eOff[nE] = chatRowPtr[hb]).
void launch_expand_entries(bool f64, int64_t nE, int64_t hb, const int32_t* rows,
                           const int64_t* rowEntry, const int64_t* chatRowPtr,
                           const int32_t* arp, const int32_t* acol, const void* aval,
                           const int32_t* brp, const int32_t* scanA, int32_t* eB, int64_t* eOff,
                           void* eVal, hipStream_t s);
// Final-chunk descriptors: from a level's light positions [first, first+n)
// or, when there is no multisplit, from the heavy rows themselves.
void launch_final_from_level(int64_t first, int64_t n, const int64_t* newOff,
                             const int32_t* newCnt, const int32_t* newRow,
                             const int32_t* newSlot, int8_t buf, int8_t spanLog2, int64_t dst0,
                             int64_t* fcOff, int32_t* fcCnt, int32_t* fcRow, int32_t* fcSlot,
                             int8_t* fcBuf, int8_t* fcSpan, hipStream_t s);
void launch_final_from_rows(int64_t h, const int64_t* rowPtr, int64_t* fcOff, int32_t* fcCnt,
                            int32_t* fcRow, int32_t* fcSlot, int8_t* fcBuf, int8_t* fcSpan,
                            hipStream_t s);
// Bin of each final chunk: dense when it is W wide (list positions
// >= lastFirst hold the W-wide chunks) and has more than tau elements, else
// the hash bin of its element count.
void launch_chunk_bins(int64_t nfc, const int32_t* fcCnt, int64_t lastFirst, int64_t tau,
                       const int32_t* caps, int nbins, int denseBin, uint8_t* key,
                       int64_t* denseElems, hipStream_t s);
void launch_dense_sym(const ChunkDesc* desc, int64_t n, const ChunkList& cl, int32_t* err,
                      hipStream_t s);
void launch_dense_num(bool f64, const ChunkDesc* desc, int64_t n, const ChunkList& cl,
                      int32_t* ccol, void* cval, int32_t* err, int numCUs, hipStream_t s);
// desc[i] for the chunk order[i], i < n; with cRowOff null (symbolic) base
// is the chunk's slot index and want is 0.
void launch_chunk_desc(int64_t n, const int32_t* order, const ChunkList& cl,
                       const int64_t* cRowOff, ChunkDesc* desc, hipStream_t s);
size_t dense_num_lds(bool f64, int64_t W);
// Dense chunks (W-wide, one column slot of a heavy row each) accumulated
// straight from A and B through B's slot runs; desc as for launch_dense_num.
void launch_dense_num_direct(bool f64, const ChunkDesc* desc, int64_t n, int64_t W,
                             const RowArgs& a, const int32_t* slotTab, int64_t stride,
                             int64_t nnzB, int32_t* ccol, void* cval, int32_t* err, int numCUs,
                             hipStream_t s);
// Per heavy row: exclusive scan of its nreq slot counts -> slotOff, and the
// row total -> cnt[xheavy[r]].
void launch_slot_scan(int64_t h, int64_t nreq, const int32_t* slotNnz, int64_t* slotOff,
                      const int32_t* xheavy, int64_t* cnt, hipStream_t s);

// ---- k_chunks.hip ----
void chunks_set_attributes();
size_t rank_chunk_lds(bool f64, int32_t T, int32_t words, int rpb);
// Chunk symbolic by bitmap with persistent work groups (dense chunks).
void launch_sym_chunks_persist(const ChunkDesc* desc, int64_t n, const ChunkList& cl,
                               int numCUs, hipStream_t s);
// Light-chunk numeric with elements in registers and a dense LDS array of
// the chunk's output size indexed by bitmap rank.  Returns false (nothing
// launched) when the bin does not fit this kernel.
size_t direct_chunk_lds(bool f64, int32_t cap, int32_t words, int rpb);
bool launch_num_chunks_direct(const BinCfg& b, bool f64, const ChunkDesc* desc, int64_t n,
                              int32_t words, size_t ldsMax, const ChunkList& cl, int32_t* ccol,
                              void* cval, int32_t* err, hipStream_t s);
// sizeClass 0: chunks of <= 256 elements (4 per work group), 1: <= 4096, 2: larger.
void launch_sym_chunks_bitmap(int sizeClass, const ChunkDesc* desc, int64_t n, int32_t words,
                              const ChunkList& cl, hipStream_t s);
void launch_num_chunks_rank(const BinCfg& b, bool f64, const ChunkDesc* desc, int64_t n,
                            int32_t words, const ChunkList& cl, int32_t* ccol, void* cval,
                            int32_t* err, hipStream_t s);

// ---- k_prune.hip ----
void launch_prune_count(int64_t m, const void* rp, int rp64, const int32_t* col, const void* val,
                        bool f64, double thr, int64_t* keepCnt, double* colsum,
                        hipStream_t s);
// The count with its column sums sent through nb column buckets of
// 2^log2Cols columns (cap entries each: fill[nb * kFillStride] zeroed, bcol and bval
// nb * cap), then the buckets' sums added into colsum.  prune_buckets_fit
// gives the bucket geometry for n columns (false: too many columns, use
// launch_prune_count).
bool prune_buckets_fit(int64_t n, int* log2Cols, int32_t* nb);
// Bucket fill counters sit kFillStride apart (one 128-byte line each), so
// the reservations of different buckets do not contend for one line.
constexpr int kFillStride = 16;
void launch_prune_count_b(int64_t m, int64_t n, const void* rp, int rp64, const int32_t* col,
                          const void* val, bool f64, double thr, int64_t* keepCnt, double* colsum,
                          int32_t nb, int log2Cols, int64_t cap, unsigned long long* fill,
                          int32_t* bcol, double* bval, hipStream_t s);
// inv[j] = fp32 reciprocal of colsum[j] (0 for a zero sum).
void launch_colsum_recip(int64_t n, const double* colsum, float* inv, hipStream_t s);
// fp64 values are divided by colsum, fp32 ones multiplied by inv.
void launch_prune_fill(int64_t m, const void* rp, int rp64, const int32_t* col, const void* val,
                       bool f64, double thr, const int64_t* outOff, const double* colsum,
                       const float* inv, int32_t* ocol, void* oval, hipStream_t s);
// MCL inflation (normalise, drop below the threshold, square); column sums
// of all entries from launch_prune_count with threshold -inf.
void launch_mcl_count(int64_t m, const void* rp, int rp64, const int32_t* col, const void* val,
                      bool f64, double thr, const double* colsum, int64_t* keep, hipStream_t s);
void launch_mcl_fill(int64_t m, const void* rp, int rp64, const int32_t* col, const void* val,
                     bool f64, double thr, const int64_t* outOff, const double* colsum,
                     int32_t* ocol, void* oval, hipStream_t s);

// ---- k_transpose.hip ----
// Stable radix sort of A's entries on their column: `passes` digits of
// digitBits bits cover totalBits bits (2^totalBits >= n); every pass works on
// `tiles` tiles and histElems = 2^digitBits * tiles counters.
struct TransposePlan {
  int passes, digitBits, totalBits;
  int64_t tiles, histElems;
};
TransposePlan transpose_plan(int64_t n, int64_t nnz);
// rows[1] receives A's row indices; rows[0], keys[1] are needed when
// passes > 1, vals[0] when passes > 1 and values are given, vals[1] when
// passes > 2; keys[0] always (nnz > 0).  hist: histElems int32, off:
// histElems + 1 int64, scanTmp: scan_tmp_elems(histElems) int64.  aval null:
// pattern only.  err receives kErrCsr for a column outside [0, n).
void launch_transpose(const TransposePlan& tp, int64_t m, int64_t n, int64_t nnz, const void* arp,
                      int arp64, const int32_t* acol, const void* aval, int valBytes,
                      void* trp, int trp64, int32_t* tcol, void* tval, int32_t* rows[2],
                      uint32_t* keys[2], void* vals[2], int32_t* hist, int64_t* off,
                      int64_t* scanTmp, int32_t* err, hipStream_t s);

// ---- api.cpp: the transpose's host side, shared by both entry points ----
spgemm_status transpose_check_args(int64_t m, int64_t n, int64_t nnz, const void* dA_row_ptr,
                                   const int32_t* dA_col, const void* dA_val,
                                   spgemm_dtype dtype, void* dT_row_ptr, int32_t t_rowptr64,
                                   int32_t* dT_col, void* dT_val);
int64_t transpose_workspace_bytes(int64_t n, int64_t nnz, spgemm_dtype dtype, bool vals);
spgemm_status transpose_run(int64_t m, int64_t n, int64_t nnz, const void* dA_row_ptr,
                            int32_t a_rowptr64, const int32_t* dA_col, const void* dA_val,
                            spgemm_dtype dtype, void* dT_row_ptr, int32_t t_rowptr64,
                            int32_t* dT_col, void* dT_val, char* ws, hipStream_t s);
void set_thread_error(const char* msg);

// ---- k_estimate.hip ----
// Size prediction of light rows without the symbolic pass (upper bound or
// HyperLogLog estimate); lg = log2 of the registers per sketch (5 or 6), lc
// = M * ln(M / V) for V = 0..M (device), cap = reserved slots per light row.
void launch_hll_sketch(int64_t K, const int32_t* brp, const int32_t* bcol, int lg, uint8_t* regs,
                       hipStream_t s);
void launch_hll_capacity(int64_t m, const int32_t* arp, const int32_t* acol, const uint8_t* regs,
                         int lg, const double* lc, double coef, const int64_t* rowP,
                         const uint8_t* rowBin, int heavyBin, int64_t* cap, double* est,
                         hipStream_t s);
// Rows of more than maxP products get 0 (not estimated).
void launch_hll_rows_direct(int64_t ns, const int32_t* rows, const int32_t* arp,
                            const int32_t* acol, const int32_t* brp, const int32_t* bcol,
                            const int64_t* rowP, int64_t maxP, int lg, const double* lc,
                            double* est, hipStream_t s);
void launch_ub_capacity(int64_t m, const int64_t* rowP, const uint8_t* rowBin, int heavyBin,
                        int64_t* cap, hipStream_t s);
void launch_overflow_rows(int64_t m, const int64_t* cnt, const int64_t* rowP,
                          const uint8_t* rowBin, int heavyBin, int nbins, int64_t* cap2,
                          uint8_t* key, int32_t* nOver, hipStream_t s);
void launch_merge_counts(int64_t m, const uint8_t* rowBin, int heavyBin, const int64_t* cnt1,
                         const int64_t* cnt2, const int64_t* off2, int64_t* srcOff, int64_t* cnt,
                         hipStream_t s);
void launch_compact_rows(bool f64, int64_t m, const uint8_t* rowBin, int heavyBin,
                         const int64_t* srcOff, const int64_t* cnt, const int64_t* cRowOff,
                         const int32_t* col1, const void* val1, const int32_t* col2,
                         const void* val2, int32_t* ccol, void* cval, hipStream_t s);

}  // namespace sg
