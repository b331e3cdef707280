/*
 * spgemm.h -- C ABI of libspgemm.so: sparse general matrix-matrix product
 * C = A * B on CSR matrices, for one AMD Instinct MI355X (gfx950) GPU.
 *
 * Method (gMAGNUS page, "gMAGNUS: Fast SpGEMM on GPUs for Irregular Matrices
 * via Hierarchical Multisplit", §III, Algorithm 3):
 *   - rows whose intermediate product fits an on-chip accumulator ("light"
 *     rows, §II-B, §III-A) are computed row by row (Gustavson, Eq. 1) with LDS
 *     hash accumulators, binned by size (§III-E);
 *   - "heavy" rows are expanded by an outer product into an intermediate
 *     matrix C-hat (§III-B, Eq. 2), split by a hierarchical multisplit into
 *     column-range chunks (§III-C), and every chunk is accumulated entirely in
 *     LDS (dense accumulator for heavy chunks, hash for light ones, §III-E);
 *   - chunk count and levels come from C's column count and the LDS size
 *     (§III-D, Eq. 4-7).
 * The two-phase interface (symbolic computes C.rowPtr and nnz(C), numeric
 * fills C.col and C.val) follows §II-B of the same page and the
 * symbolic/numeric split described in §2 of the Ocean page.
 *
 * Conventions shared by every entry point
 *   - All matrix arrays are DEVICE pointers on the current HIP device; every
 *     size and count is a host integer.  `stream` is a hipStream_t passed as
 *     void* (NULL = the legacy default stream).
 *   - CSR: row_ptr (rows+1 entries, int32), col (nnz, int32), val (nnz, float
 *     or double per `dtype`).  Inputs must be canonical: row_ptr[0] == 0,
 *     row_ptr non-decreasing, 0 <= col < ncols, columns strictly increasing
 *     within a row.  opts->validate checks this on the device.
 *   - Output C is canonical CSR; an entry exists iff at least one stored
 *     pair A[i,k], B[k,j] exists (a computed 0.0 is kept).
 *   - Nothing is thrown across the ABI; every call returns spgemm_status.
 *   - Calls on one plan are not thread-safe; distinct plans are independent.
 */
#ifndef SPGEMM_H
#define SPGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum spgemm_status {
  SPGEMM_OK = 0,
  SPGEMM_ERR_INVALID_ARG = -1,    /* null pointer, negative size, bad dtype  */
  SPGEMM_ERR_INVALID_CSR = -2,    /* opts->validate found a non-canonical input */
  SPGEMM_ERR_INDEX_OVERFLOW = -3, /* int32 C.row_ptr requested, nnz(C) > INT32_MAX,
                                     or a size exceeds the int32 index range */
  SPGEMM_ERR_OOM = -4,            /* device allocation failed; C untouched   */
  SPGEMM_ERR_HIP = -5,            /* HIP runtime error; see spgemm_last_error */
  SPGEMM_ERR_STATE = -6,          /* call order violated or plan in error state */
  SPGEMM_ERR_INTERNAL = -7        /* a device-side capacity check tripped    */
} spgemm_status;

typedef enum spgemm_dtype { SPGEMM_F32 = 0, SPGEMM_F64 = 1 } spgemm_dtype;

/* Optional device allocator: return a device pointer of at least `bytes`
 * usable in stream order on `stream`, or NULL on failure.  With alloc == NULL
 * the library uses hipMallocAsync / hipFreeAsync on the plan's stream. */
typedef void *(*spgemm_alloc_fn)(size_t bytes, void *stream, void *ctx);
typedef void (*spgemm_free_fn)(void *ptr, void *stream, void *ctx);

/* Tuning and override knobs.  Zero-initialise, then set what you need; a zero
 * field means "automatic". */
typedef struct spgemm_options {
  int64_t lds_budget;           /* s_LM in bytes (gMAGNUS §III-D); 0 = LDS per
                                   work group of the device (160 KiB on gfx950) */
  int64_t heavy_threshold;      /* tau; 0 = derived from s_LM (Eq. 4 reading)   */
  int64_t dense_width;          /* final chunk width W (power of two); 0 = derived */
  int64_t mem_budget;           /* bytes for the heavy intermediate (the outer
                                   product and multisplit buffers, 8 (fp32) or
                                   12 (fp64) bytes per element, two buffers when
                                   there are levels); heavy rows are processed
                                   in batches of consecutive rows that fit it
                                   (at least one row a batch).  One batch keeps
                                   its expansion from symbolic to numeric;
                                   several batches expand again in numeric.
                                   0 = 45% of the device memory free at
                                   spgemm_symbolic, at least 1 GiB            */
  int32_t max_chunks_per_level; /* n_chunksMax (power of two >= 2); 0 = 32       */
  int32_t rowptr64;             /* 1: C.row_ptr is int64, else int32            */
  int32_t validate;             /* 1: check A and B are canonical CSR           */
  int32_t single_stream;        /* 1: light and heavy work on the caller's stream */
  int32_t profile;              /* 1: time each kernel phase with HIP events
                                   recorded on the stream it runs on; read the
                                   result from spgemm_stats.phase_ms           */
  int32_t histogram_from_data;  /* 1: count each level's (row, chunk) elements
                                   by reading the expanded columns (K6 as the
                                   gMAGNUS page prints it); 0: derive the same
                                   counts from the structure of A and of B's
                                   rows (default; the read pass is also used
                                   when n_req exceeds 8192)                    */
  spgemm_alloc_fn alloc;        /* optional allocator (see above)               */
  spgemm_free_fn free;
  void *alloc_ctx;
  int32_t expansion;            /* how the heavy rows' products reach their
                                   final chunks (the chunk tree, C and the
                                   parameters are the same in every mode):
                                   0 (default): one pass; every product
                                     is made from A and B row by row and
                                     written straight to its final chunk
                                     (needs the chunk counts from the
                                     structure and n_req <= 4096, else
                                     mode 2);
                                   1: as the gMAGNUS page prints it: masked
                                     CSC, outer product into C-hat, then one
                                     multisplit pass per level;
                                   2: the first multisplit level made from A
                                     and B row by row (C-hat never written),
                                     later levels as in mode 1              */
  int32_t heavy_row_threshold;  /* rows with more intermediate products than
                                   this take the heavy path; 0 = the
                                   heavy_threshold option if set, else
                                   floor(tau / 3): the largest light row whose
                                   numeric LDS table (2 slots per product)
                                   leaves room for three work groups per CU.
                                   Chunks keep tau (recursion, bins).        */
  int32_t light_hash_only;      /* 1: every light row takes the LDS hash
                                   accumulator; 0 (default): a light row whose
                                   products span at most 128 x its bin's
                                   product bound columns (at most 65536) takes
                                   the dense window: an LDS bitmap over the
                                   span, ranks by prefix popcount, values
                                   added at their rank (no hash, no sort);
                                   other rows of at least 512 products take a
                                   dense window over the 2048 columns around
                                   their diagonal position (row * n / m) plus
                                   an LDS hash table for the columns outside
                                   it, when those outliers fit half of the
                                   table (only the outliers are sorted)     */
  int32_t workflow;             /* how light rows get their output size (Ocean
                                   page, §3 and Table 1; heavy rows always take
                                   the exact chunk path):
                                   0 (default): symbolic pass (exact counts);
                                   1: upper bound: each light row reserves its
                                     product count P_i of output slots, is
                                     computed into them during
                                     spgemm_symbolic, and copied into C by
                                     spgemm_numeric;
                                   2: HyperLogLog estimate: per-B-row sketches
                                     merged per A row, min(P_i, ceil(coef*E))
                                     slots; rows that do not fit are computed
                                     again with P_i slots;
                                   3: choose by Table 1 (1 below 64 products
                                     per row, 2 when products / nnz(A) >= 8
                                     and the compression ratio of a 3% row
                                     sample is >= 8, else 0).
                                   C is the same in every mode. */
  int32_t hll_registers;        /* registers per sketch, 32 or 64; 0 = 32 when
                                   products / nnz(A) < 48, else 64          */
  int32_t hll_coef_pct;         /* estimate multiplier in percent; 0 = 200 with
                                   32 registers, 150 with 64               */
  int32_t light_no_esc;         /* 1: rows of at most 32 products take the LDS
                                   hash kernels; 0 (default): they take the
                                   expand-sort-compact kernel (32 lanes per
                                   row, sort by lane exchanges, no LDS;
                                   Ocean page, §3)                         */
  int64_t index_limit;          /* largest value accepted where an index is
                                   held in 32 bits: nnz(C) with an int32
                                   C.row_ptr, and a row's intermediate product
                                   count (its row-local product offsets are
                                   int32).  0 = INT32_MAX; a smaller value
                                   only serves tests of the overflow checks  */
  int64_t debug_device_error;   /* test hook, 0 in normal use: when nonzero,
                                   spgemm_numeric ends by storing this value
                                   in the plan's device status word on its
                                   stream, as a tripped device-side capacity
                                   check does, so that the reporting path
                                   (spgemm_wait, spgemm_get_stats) can be
                                   exercised from the host               */
  int64_t dense_direct;         /* 1: with expansion 0, dense chunks (W-wide
                                   slots of a heavy row holding more than
                                   min(tau, W/2) products) are accumulated
                                   straight from A and B (each entry's run of
                                   its B row inside the slot, found among B's
                                   per-slot runs) instead of from the expanded
                                   intermediate, which then holds only the
                                   light chunks' products; 0 (default): every
                                   product is expanded.  Same C either way.  */
  int64_t reserved[1];
} spgemm_options;

/* Parameters chosen by GetMagnusParams (gMAGNUS §III-D, Eq. 4-7). */
typedef struct spgemm_params {
  int64_t tau;              /* heavy threshold: a row/chunk is heavy iff its
                               element count exceeds tau                      */
  int64_t n_dense;          /* max dense accumulator width for numeric        */
  int64_t dense_width;      /* W = floor_pow2(n_dense): final chunk width     */
  int64_t chunks_required;  /* next_pow2(ceil(ncols / W)), at least 1         */
  int32_t chunks_max;       /* n_chunksMax                                    */
  int32_t levels;           /* multisplit levels (0 when chunks_required == 1) */
  int32_t v_chunks[8];      /* chunks per row at each level                   */
  int64_t level_width[8];   /* column width of a chunk after each level       */
} spgemm_params;

/* Kernel phases timed when spgemm_options.profile is set. */
typedef enum spgemm_phase {
  SPGEMM_PH_ROW_INFO = 0,        /* products per row, light/heavy bins (plan)   */
  SPGEMM_PH_SYM_LIGHT = 1,       /* light-row LDS hash symbolic                 */
  SPGEMM_PH_CSC = 2,             /* masked CSR->CSC and segment reservations   */
  SPGEMM_PH_OUTER_PRODUCT = 3,   /* C-hat expansion                             */
  SPGEMM_PH_HISTOGRAM = 4,       /* per-level (row, chunk) counts               */
  SPGEMM_PH_MULTISPLIT = 5,      /* per-level reorder into chunks              */
  SPGEMM_PH_SYM_CHUNK_HASH = 6,  /* light-chunk hash symbolic                   */
  SPGEMM_PH_SYM_CHUNK_DENSE = 7, /* heavy-chunk bitmap symbolic                 */
  SPGEMM_PH_ROWPTR = 8,          /* C.row_ptr scan and numeric binning          */
  SPGEMM_PH_NUM_LIGHT = 9,       /* light-row LDS hash numeric + sort           */
  SPGEMM_PH_NUM_CHUNK_HASH = 10, /* light-chunk hash numeric + sort             */
  SPGEMM_PH_NUM_CHUNK_DENSE = 11,/* heavy-chunk dense LDS numeric               */
  SPGEMM_PH_CHUNK_HIST = 12,     /* per-row W-wide chunk counts from structure  */
  SPGEMM_PH_EXPAND_SPLIT = 13,   /* first multisplit level fed from A and B     */
  SPGEMM_PH_EXPAND_FINAL = 14,   /* products made with values and written to
                                    their final chunks                          */
  SPGEMM_PH_SYM_HEAVY = 15,      /* heavy-row symbolic of the batched schedule,
                                    where values are not expanded in symbolic   */
  SPGEMM_PH_COUNT = 16
} spgemm_phase;

typedef struct spgemm_stats {
  int64_t products;           /* P = sum_i sum_{k in A_i} nnz(B_k); flops = 2P */
  int64_t max_row_products;
  int64_t light_rows;         /* rows with 0 < P_i <= tau                      */
  int64_t heavy_rows;         /* rows with P_i > tau                           */
  int64_t heavy_products;     /* P_h = nnz(C-hat)                              */
  int64_t heavy_a_nnz;        /* nnz of A restricted to heavy rows             */
  int64_t nnz_c;
  spgemm_params params;
  int64_t level_elems[8];     /* elements entering each multisplit level       */
  int64_t final_chunks;       /* non-empty chunks accumulated                  */
  int64_t dense_chunks;       /* of which in a dense LDS accumulator           */
  int64_t lds_hash_products;  /* products summed in LDS hash tables            */
  int64_t lds_dense_products; /* products summed in LDS dense accumulators     */
  int64_t global_products;    /* products summed in global memory (always 0)   */
  int64_t batches;            /* heavy-row batches (0 with no heavy rows)      */
  double ms_plan, ms_symbolic, ms_numeric; /* host wall time of each call      */
  double phase_ms[16];        /* GPU time of each spgemm_phase (with profile)  */
  int32_t phase_windows[16];  /* event-bracketed windows summed in phase_ms;
                                 a window holds one launch for the outer
                                 product, histogram, multisplit and dense
                                 phases (one per level for the per-level ones,
                                 and one per batch and expansion)           */
  int64_t device_errors;      /* device status bits seen (0 when all is well)  */
  int64_t heavy_row_threshold; /* rows above this many products were heavy     */
  int64_t chunk_col_bytes;    /* bytes of a column in the heavy intermediate:
                                 2 when it holds chunk-local 16-bit columns */
  int32_t workflow;           /* size prediction used (options.workflow 0-2) */
  int32_t hll_registers;      /* registers per sketch (workflow 2), else 0     */
  int64_t light_capacity;     /* output slots reserved for light rows (1, 2)   */
  int64_t overflow_rows;      /* light rows computed again with P_i slots      */
  double sampled_cr;          /* compression ratio of the row sample (mode 3)  */
  double phase_min_ms[16];    /* shortest window of each phase (with profile;
                                 0 for a phase with no window)              */
  int64_t hybrid_rows;        /* light rows accumulated in a dense window
                                 around their diagonal position plus an
                                 LDS hash table for the other columns     */
} spgemm_stats;

typedef struct spgemm_plan_s *spgemm_plan_t;
typedef struct spgemm_prune_s *spgemm_prune_t;

/* GetMagnusParams on the host; needs no GPU.  (gMAGNUS §III-D, Eq. 4-7.)
 * ncols = number of columns of C; lds_bytes = s_LM; val_bytes / col_bytes =
 * s_C.val / s_C.col; max_chunks_per_level = n_chunksMax (0 = 32);
 * dense_width = W override (0 = derived).  Where the printed formulas are
 * ambiguous, the readings taken are stated beside the code (params.cpp).
 * Errors: INVALID_ARG for non-positive sizes or a non-power-of-two
 * max_chunks_per_level / dense_width. */
spgemm_status spgemm_compute_params(int64_t ncols, int64_t lds_bytes,
                                    int32_t val_bytes, int32_t col_bytes,
                                    int32_t max_chunks_per_level,
                                    int64_t dense_width, spgemm_params *out);

/* Plan C = A * B (A: m x k, B: k x n).  Validates arguments, queries the
 * device, computes the parameters, counts intermediate products per row,
 * splits rows into light and heavy and bins them (gMAGNUS Algorithm 3,
 * setup phase).  Blocks once to read back the heavy count.  A and B are
 * borrowed until spgemm_destroy and must not change meanwhile.
 * Errors: INVALID_ARG, INDEX_OVERFLOW (nnz > INT32_MAX in an input),
 * INVALID_CSR (with validate), OOM, HIP; INDEX_OVERFLOW also when a row's
 * intermediate product count exceeds opts->index_limit (INT32_MAX).  On
 * error *out is NULL and nothing the caller owns was written. */
spgemm_status spgemm_plan(spgemm_plan_t *out, int64_t m, int64_t k, int64_t n,
                          const int32_t *dA_row_ptr, const int32_t *dA_col,
                          const void *dA_val, int64_t nnzA,
                          const int32_t *dB_row_ptr, const int32_t *dB_col,
                          const void *dB_val, int64_t nnzB, spgemm_dtype dtype,
                          const spgemm_options *opts, void *stream);

/* Symbolic phase: writes C.row_ptr (m+1 entries, int32, or int64 with
 * opts->rowptr64) into the caller's device buffer and returns nnz(C) on the
 * host (blocks once).  Heavy rows are expanded, multisplit and counted here;
 * the reordered intermediate is kept for numeric.  dC_row_ptr is written
 * last, only when the call succeeds.
 * Errors: STATE (not planned, or already run), INDEX_OVERFLOW (nnz(C) above
 * opts->index_limit, INT32_MAX by default, with an int32 C.row_ptr), OOM,
 * HIP, INVALID_CSR (with validate), INTERNAL (a device capacity check). */
spgemm_status spgemm_symbolic(spgemm_plan_t p, void *dC_row_ptr,
                              int64_t *nnzC);

/* Numeric phase: fills C.col (nnz(C) int32) and C.val (nnz(C), dtype),
 * columns sorted within each row.  Asynchronous on the plan's stream: the
 * kernels' own capacity checks (a numeric row or chunk whose size differs
 * from the symbolic count, a full hash table) are reported by spgemm_wait
 * or spgemm_get_stats, never by this call.  With a single heavy-row batch
 * (the symbolic expansion kept for numeric) this call allocates nothing, so
 * it cannot fail with OOM; with several batches each batch allocates its
 * chunk lists, and an OOM then leaves C.col/C.val partly written (C.row_ptr
 * from symbolic stays valid).
 * Errors: STATE (symbolic not run, or run twice), INVALID_ARG, OOM, HIP. */
spgemm_status spgemm_numeric(spgemm_plan_t p, int32_t *dC_col, void *dC_val);

/* Blocks until all work the plan has enqueued is done, then reports the
 * device status word: INTERNAL (with the check that tripped in
 * spgemm_last_error) when a device-side capacity check failed during
 * symbolic or numeric, in which case C must not be used; OK otherwise.  The
 * plan enters the error state on failure.  Call it (or spgemm_get_stats)
 * after spgemm_numeric before trusting C.
 * Errors: INVALID_ARG (NULL plan), INTERNAL, INVALID_CSR, HIP. */
spgemm_status spgemm_wait(spgemm_plan_t p);

spgemm_status spgemm_get_stats(spgemm_plan_t p, spgemm_stats *out);

/* Size prediction of the light rows (Ocean page, §3): after spgemm_symbolic
 * with options.workflow 1 or 2 (or 3 when it chose one of them), copies the
 * output slots reserved for every light row into dCap (m int64, device; 0
 * for other rows) and, with workflow 2, the HyperLogLog estimate of every
 * light row into dEst (m double, device).  Either pointer may be NULL.
 * Asynchronous on the plan's stream.  Errors: INVALID_ARG (NULL plan, dEst
 * without workflow 2), STATE (no symbolic yet, or workflow 0), HIP. */
spgemm_status spgemm_row_estimates(spgemm_plan_t p, int64_t *dCap, double *dEst);

/* Frees the plan's workspace (stream-ordered on the plan's stream). */
void spgemm_destroy(spgemm_plan_t p);

const char *spgemm_status_string(spgemm_status s);
/* Last error message of a plan, or of the calling thread when p == NULL. */
const char *spgemm_last_error(spgemm_plan_t p);

/* One Markov-clustering prune + column renormalisation of C (Trident page,
 * "Communication-Avoiding SpGEMM via Trident Partitioning", §5.7): keep
 * entries with C[i,j] >= threshold (compared in the value type), then divide
 * each kept entry by the fp64 sum of its column's kept entries, rounding once
 * to the value type.
 * Count call: computes the kept-entry row pointers into dOut_row_ptr (m+1;
 * int64 if out_rowptr64 else int32), the column sums, and returns the kept
 * count on the host (blocks once).  Fill call: writes dOut_col / dOut_val.
 * C is read through dC_row_ptr (int64 if c_rowptr64 else int32).
 * Errors: INVALID_ARG, INDEX_OVERFLOW, OOM, HIP, STATE. */
spgemm_status spgemm_prune_colnorm_count(
    spgemm_prune_t *out, int64_t m, int64_t n, const void *dC_row_ptr,
    int32_t c_rowptr64, const int32_t *dC_col, const void *dC_val,
    spgemm_dtype dtype, double threshold, void *dOut_row_ptr,
    int32_t out_rowptr64, int64_t *nnzOut, void *stream);
spgemm_status spgemm_prune_colnorm_fill(spgemm_prune_t p, int32_t *dOut_col,
                                        void *dOut_val);

/* The rest of one Markov-clustering iteration after the expansion C = A*A
 * (Trident page, §5.7: normalise the columns, prune entries below a
 * threshold, square the remaining entries).  With s_j the fp64 sum of all
 * entries of column j, y = C[i,j] / s_j is formed in fp64 and rounded once
 * to the value type (y = 0 when s_j = 0); entries with y >= threshold
 * (compared in the value type) are kept, with value y * y computed in the
 * value type.  Same two-call pattern, arguments, ownership and errors as
 * spgemm_prune_colnorm_count / _fill; the handle is released with
 * spgemm_prune_destroy. */
spgemm_status spgemm_mcl_inflate_count(
    spgemm_prune_t *out, int64_t m, int64_t n, const void *dC_row_ptr,
    int32_t c_rowptr64, const int32_t *dC_col, const void *dC_val,
    spgemm_dtype dtype, double threshold, void *dOut_row_ptr,
    int32_t out_rowptr64, int64_t *nnzOut, void *stream);
spgemm_status spgemm_mcl_inflate_fill(spgemm_prune_t p, int32_t *dOut_col,
                                      void *dOut_val);
void spgemm_prune_destroy(spgemm_prune_t p);

/* Transpose T = A^T of an m x n CSR matrix A into an n x m CSR matrix T, for
 * the rectangular products A * A^T that the Ocean page ("Ocean: Fast
 * Estimation-Based Sparse General Matrix-Matrix Multiplication on GPU",
 * evaluation on rectangular matrices) measures, and for restriction-type
 * operands (Trident page, §5.4).  T[j, i] = A[i, j] for every stored entry;
 * rows of T list their column indices in rising order (A's entries stored
 * row by row with rising rows; duplicates, if any, keep their storage
 * order), values are copied unchanged.
 * Inputs: dA_row_ptr (m+1; int64 if a_rowptr64 else int32), dA_col (nnz),
 * dA_val (nnz, float or double per dtype; NULL for the pattern only, then
 * dT_val is ignored).  Outputs, allocated by the caller: dT_row_ptr (n+1;
 * int64 if t_rowptr64 else int32), dT_col (nnz, int32), dT_val (nnz).
 * Temporaries (about 16 + 2*sizeof(value) bytes per entry) are allocated
 * with hipMallocAsync on `stream` and freed in stream order.  The call
 * blocks once, to read the device's column check.
 * Errors: INVALID_ARG (null pointer, negative size, bad dtype),
 * INDEX_OVERFLOW (m or n above INT32_MAX, or nnz above INT32_MAX with an
 * int32 dT_row_ptr), INVALID_CSR (a column index outside [0, n); T is then
 * undefined), OOM, HIP.  A's row pointers are trusted (row_ptr[0] == 0,
 * non-decreasing, row_ptr[m] == nnz). */
spgemm_status spgemm_transpose(int64_t m, int64_t n, int64_t nnz,
                               const void *dA_row_ptr, int32_t a_rowptr64,
                               const int32_t *dA_col, const void *dA_val,
                               spgemm_dtype dtype, void *dT_row_ptr,
                               int32_t t_rowptr64, int32_t *dT_col,
                               void *dT_val, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * transpose, arguments, outputs and errors as spgemm_transpose, with the
 * temporaries taken from a fixed 64 MiB device array inside the library
 * instead of hipMallocAsync (each GPU the library runs on holds its own
 * array until the process ends).  The call makes no device allocation.
 * The caller still allocates T.  About 16 + 2 * sizeof(value) bytes per
 * entry are needed (fewer for narrow column ranges); a call whose
 * temporaries exceed 64 MiB returns INVALID_ARG (message in
 * spgemm_last_error(NULL)) without touching T.  Calls on one GPU share the
 * array: calls in stream order are safe (every piece that must start at
 * zero is cleared by a kernel on `stream`), calls that overlap on one GPU
 * (other streams or host threads) race.  Blocks once, as spgemm_transpose
 * does. */
spgemm_status spgemm_transpose_noalloc(int64_t m, int64_t n, int64_t nnz,
                                       const void *dA_row_ptr, int32_t a_rowptr64,
                                       const int32_t *dA_col, const void *dA_val,
                                       spgemm_dtype dtype, void *dT_row_ptr,
                                       int32_t t_rowptr64, int32_t *dT_col,
                                       void *dT_val, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* SPGEMM_H */
